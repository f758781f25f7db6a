"""The ResidualKV write and read paths, as plain fp64 NumPy.

Source: the ResidualKV review page ("ResidualKV: 基于参考向量与残差的 KV Cache 压缩").
Each function names the passage it follows. Notation follows the page: kv_i is the
joint pre-RoPE K|V vector of token i (width 2*d_k, K heads first, section 2.1), the
reference pool holds every s-th token (section 2.6), k_i = min(k, |pool_i|)
(section 2.1 symbol table).

Readings where the page is silent (each is listed in the design notes):
* references sit at positions p = 0, s, 2s, ... and token i may use references
  with position < i;
* distances use the stored (FP8-dequantized) reference values, the same values the
  mean and the decoder use (section 2.5: encode and decode use numerically
  identical references);
* ties in distance are broken by the lower pool slot; the chosen slots are stored
  in ascending slot order;
* the reference mean is accumulated in fp32, in ascending slot order, then divided
  by k_i (IEEE fp32 division); the encoder sees it rounded to the KV dtype (bf16
  for bf16 KV), the decoder adds the fp32 mean; in the mean-projection form (an
  option, not on the page) the encoder instead takes f_c(mean)'s first-layer
  pre-activations as the average of the references' own, with no rounding of the mean;
* Swish is SiLU (beta = 1), no biases anywhere (section 2.3, section 2.5);
* a group is 32 consecutive latent coordinates; the two stored values are the step
  Delta and the group minimum; round() is round-half-to-even; codes are clamped to
  [0, 2^b - 1]; a group whose stored step is 0 stores code 0 (section 2.4);
* the code decision (min, max, step, (z - zmin)/step, rounding) is taken in fp32;
* RoPE is the half-split form: pair (j, j + D/2) of each key head rotates by
  p * theta^(-2j/D) at the token's own position p; values are not rotated
  (section 2.1, last paragraph);
* a reference token decodes to its stored value.
"""

from __future__ import annotations

import math
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

from .formats import bf16_round, fp16_round, fp8_e4m3fn_decode, fp8_e4m3fn_encode


# --------------------------------------------------------------------------------------
# single steps
# --------------------------------------------------------------------------------------


def topk_references(
    kv_i: np.ndarray,
    ref_val: np.ndarray,
    ref_pos: np.ndarray,
    count: int,
    pos_i: int,
    k: int,
) -> Tuple[np.ndarray, np.ndarray]:
    """Causal squared-L2 top-k_i over the reference pool (section 2.2, arg top-k_i equation).

    Returns (slots in ascending slot order, their squared distances). Only slots
    m < count with ref_pos[m] < pos_i are candidates; k_i = min(k, #candidates)
    (section 2.1, warm-up k_i).
    """
    cand = np.nonzero(ref_pos[:count] < pos_i)[0]
    if cand.size == 0:
        return np.zeros(0, dtype=np.int64), np.zeros(0)
    diff = ref_val[cand].astype(np.float64) - np.asarray(kv_i, dtype=np.float64)[None, :]
    d = np.sum(diff * diff, axis=1)
    order = np.lexsort((cand, d))  # by distance, then by slot
    k_i = min(k, cand.size)
    chosen = order[:k_i]
    slots = cand[chosen]
    dist = d[chosen]
    srt = np.argsort(slots, kind="stable")
    return slots[srt], dist[srt]


def reference_mean32(refs: np.ndarray) -> np.ndarray:
    """Arithmetic mean of the chosen references (section 2.2, mean equation).

    Accumulated in fp32 in the given (ascending slot) order, then divided by k_i
    with one IEEE fp32 division. An empty set gives the zero vector.
    """
    refs = np.asarray(refs)
    k_i = refs.shape[0]
    if k_i == 0:
        return np.zeros(refs.shape[1] if refs.ndim == 2 else 0, dtype=np.float32)
    s = np.zeros(refs.shape[1], dtype=np.float32)
    for j in range(k_i):
        s = (s + refs[j].astype(np.float32)).astype(np.float32)
    return (s / np.float32(k_i)).astype(np.float32)


def swiglu_compressor(x: np.ndarray, Wc1: np.ndarray, Wc2: np.ndarray, Wc3: np.ndarray) -> np.ndarray:
    """f_c(x) = (Swish(x W_c1) * x W_c2) W_c3 in fp64 (section 2.3, compressor equation).

    Weights in math layout: W_c1, W_c2 [2d_k, d_ff], W_c3 [d_ff, d_c]. Rows of x are tokens.
    """
    x = np.asarray(x, dtype=np.float64)
    a = x @ np.asarray(Wc1, dtype=np.float64)
    b = x @ np.asarray(Wc2, dtype=np.float64)
    swish = a / (1.0 + np.exp(-a))
    return (swish * b) @ np.asarray(Wc3, dtype=np.float64)


def reference_projections(refs: np.ndarray, Wc1: np.ndarray, Wc2: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """First-layer pre-activations of each reference, r_j W_c1 and r_j W_c2, in fp64.

    The mean-projection form of the encoder (not on the pages; an algebraic identity of
    the compressor of section 2.3): the first layer of f_c is linear, so the mean's
    pre-activations are the mean of the references' pre-activations,
    mean_i W = (1/k_i) sum_j r_j W, and r_j W can be computed once per reference when it
    enters the pool. refs: [k, 2d_k] stored reference values. Returns two [k, d_ff] arrays.
    """
    refs = np.asarray(refs, dtype=np.float64)
    return refs @ np.asarray(Wc1, dtype=np.float64), refs @ np.asarray(Wc2, dtype=np.float64)


def averaged_preactivations(p1: np.ndarray, p2: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """(1/k_i) sum_j of the chosen references' projections (ascending slot order), fp64.

    An empty set gives zeros (the zero mean of an empty pool)."""
    p1 = np.asarray(p1, dtype=np.float64)
    p2 = np.asarray(p2, dtype=np.float64)
    k_i = p1.shape[0]
    if k_i == 0:
        return np.zeros(p1.shape[1]), np.zeros(p2.shape[1])
    a1 = np.zeros(p1.shape[1])
    a2 = np.zeros(p2.shape[1])
    for j in range(k_i):
        a1 = a1 + p1[j]
        a2 = a2 + p2[j]
    return a1 / k_i, a2 / k_i


def swiglu_from_preactivations(a1: np.ndarray, a2: np.ndarray, Wc3: np.ndarray) -> np.ndarray:
    """(Swish(a1) * a2) W_c3 in fp64: the compressor of section 2.3 after its first layer."""
    a1 = np.asarray(a1, dtype=np.float64)
    a2 = np.asarray(a2, dtype=np.float64)
    swish = a1 / (1.0 + np.exp(-a1))
    return (swish * a2) @ np.asarray(Wc3, dtype=np.float64)


def linear_decoder(z: np.ndarray, Wd: np.ndarray) -> np.ndarray:
    """f_d(z) = z W_d, bias-free (section 2.5, decoder equation). W_d is [d_c, 2d_k]."""
    return np.asarray(z, dtype=np.float64) @ np.asarray(Wd, dtype=np.float64)


def group_quantize(z: np.ndarray, bits: int, group: int, store: str):
    """Per-token group quantizer (section 2.4, Delta / q / z-tilde equations).

    z: [n, d_c] latent residuals (fp64). store: 'f32' or 'f16' for the two per-group
    values. The code decision is taken in fp32. Returns (q uint8 [n, d_c],
    step [n, G], zmin [n, G]) with step/zmin as the stored values (float64).
    bits == 16 means quantization off: q is unused and the fp16 latent is returned
    in place of `step` (zmin is None).
    """
    z32 = np.asarray(z, dtype=np.float64).astype(np.float32)
    n, d_c = z32.shape
    if bits == 16:
        return None, fp16_round(z32.astype(np.float64)), None
    G = -(-d_c // group)
    levels = np.float32(2 ** bits - 1)
    q = np.zeros((n, d_c), dtype=np.uint8)
    step = np.zeros((n, G))
    zmin = np.zeros((n, G))
    rnd = fp16_round if store == "f16" else (lambda v: np.asarray(v, dtype=np.float32).astype(np.float64))
    for g in range(G):
        sl = slice(g * group, min(d_c, (g + 1) * group))
        zg = z32[:, sl]
        lo = zg.min(axis=1)
        hi = zg.max(axis=1)
        d32 = ((hi - lo).astype(np.float32) / levels).astype(np.float32)
        s_st = rnd(d32)
        m_st = rnd(lo)
        step[:, g] = s_st
        zmin[:, g] = m_st
        s32 = s_st.astype(np.float32)[:, None]
        m32 = m_st.astype(np.float32)[:, None]
        with np.errstate(divide="ignore", invalid="ignore"):
            t = ((zg - m32).astype(np.float32) / s32).astype(np.float32)
        qq = np.clip(np.rint(t), 0, 2 ** bits - 1)
        qq = np.where(s32 == 0, 0, qq)
        q[:, sl] = qq.astype(np.uint8)
    return q, step, zmin


def group_dequantize(q: np.ndarray, step: np.ndarray, zmin: np.ndarray, group: int) -> np.ndarray:
    """z~ = q * Delta + z_min per group (section 2.4), in fp64."""
    q = np.asarray(q, dtype=np.float64)
    n, d_c = q.shape
    g_of = np.arange(d_c) // group
    return q * step[:, g_of] + zmin[:, g_of]


def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    """omega_j = theta^(-2j/D), j < D/2, in fp64."""
    j = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * j / head_dim)


def rope_rotate(k: np.ndarray, pos: np.ndarray, n_heads: int, head_dim: int, theta: float) -> np.ndarray:
    """Standard (half-split) RoPE at each token's own position (section 2.1, last paragraph).

    k: [n, N*D] pre-RoPE keys; pos: [n] positions. Pair (j, j + D/2) of every head
    rotates by angle pos * theta^(-2j/D). Angles and rotation in fp64.
    """
    k = np.asarray(k, dtype=np.float64).reshape(-1, n_heads, head_dim)
    half = head_dim // 2
    ang = np.asarray(pos, dtype=np.float64)[:, None] * rope_inv_freq(head_dim, theta)[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1 = k[:, :, :half]
    x2 = k[:, :, half:]
    out = np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=2)
    return out.reshape(-1, n_heads * head_dim)


# --------------------------------------------------------------------------------------
# storage accounting (section 3.3)
# --------------------------------------------------------------------------------------


def group_storage_ratio(bits: int, group: int = 32) -> float:
    """Bytes of one quantized group (b-bit codes + two fp16 values) over its fp16 size."""
    payload_bits = bits * group + 2 * 16
    return payload_bits / (16.0 * group)


def keep_ratio(beta: float, rho_ref: float, q_full: float, q_res: float, d_c: int, two_dk: int) -> float:
    """KR = beta*q_full + (1-beta)*(rho_ref/2 + q_res*d_c/(2 d_k)) (section 3.3, KR equation).

    rho_ref/2: an FP8 reference costs half an fp16 row.
    """
    return beta * q_full + (1.0 - beta) * (0.5 * rho_ref + q_res * d_c / two_dk)


# --------------------------------------------------------------------------------------
# the cache and the whole codec
# --------------------------------------------------------------------------------------


class OracleCache:
    """Reference pool + per-token records of one sequence of one layer (review section 2.4/2.7)."""

    def __init__(self, two_dk: int, d_c: int, top_k: int, group: int, bits: int,
                 cap_ref: int, cap_tok: int, mode: str):
        self.two_dk, self.d_c, self.top_k, self.group, self.bits = two_dk, d_c, top_k, group, bits
        self.mode = mode
        G = -(-d_c // group)
        self.ref_code = np.zeros((cap_ref, two_dk), dtype=np.uint8)
        self.ref_val = np.zeros((cap_ref, two_dk), dtype=np.float64)
        self.ref_pos = np.full(cap_ref, -1, dtype=np.int32)
        self.ref_count = 0
        self.q = np.zeros((cap_tok, d_c), dtype=np.uint8)
        self.latent = np.zeros((cap_tok, d_c), dtype=np.float64)  # fp16 latent when bits == 16
        self.step = np.zeros((cap_tok, G), dtype=np.float64)
        self.zmin = np.zeros((cap_tok, G), dtype=np.float64)
        self.ref_idx = np.full((cap_tok, top_k), -1, dtype=np.int32)
        self.self_slot = np.full(cap_tok, -1, dtype=np.int32)
        self.ref_dist = np.full((cap_tok, top_k), np.nan)
        self.z = np.zeros((cap_tok, d_c), dtype=np.float64)  # unquantized latent, for checks
        # max |f_c(kv)| + max |f_c(mean)|: the magnitude the two encoder outputs have before
        # z takes their difference (the scale of the arithmetic error of any finite-precision
        # evaluation of z), for checks
        self.f_scale = np.zeros(cap_tok, dtype=np.float64)


class OracleCodec:
    """The write path (append / encode) and the read path (selected restore).

    weights: math layout, {'Wc1': [2dk, d_ff], 'Wc2': [2dk, d_ff], 'Wc3': [d_ff, d_c],
    'Wd': [d_c, 2dk]} (float arrays holding the stored weight values).
    mode: 'f32' (fp32 KV, fp32 references, fp32 step/min) or 'bf16' (bf16 KV, FP8
    references, fp16 step/min).
    mean_projection: the encoder's f_c(mean) takes its first-layer pre-activations as the
    average of the chosen references' own pre-activations (reference_projections), so
    the mean is never rounded to the KV dtype; otherwise (default) the encoder sees the
    fp32 mean rounded to the KV dtype.
    """

    def __init__(self, n_kv_heads: int, head_dim: int, d_ff: int, d_c: int, top_k: int,
                 bits: int, group: int, mode: str, rope_theta: float, weights: Dict[str, np.ndarray],
                 mean_projection: bool = False):
        self.mean_projection = bool(mean_projection)
        self.N, self.D = n_kv_heads, head_dim
        self.dk = n_kv_heads * head_dim
        self.two_dk = 2 * self.dk
        self.d_ff, self.d_c, self.top_k = d_ff, d_c, top_k
        self.bits, self.group, self.mode = bits, group, mode
        self.theta = rope_theta
        self.W = {k: np.asarray(v, dtype=np.float64) for k, v in weights.items()}

    @classmethod
    def from_workload(cls, cfg, weights, mean_projection: bool = False) -> "OracleCodec":
        return cls(cfg.n_kv_heads, cfg.head_dim, cfg.d_ff, cfg.d_c, cfg.top_k, cfg.bits,
                   cfg.group, cfg.mode, cfg.rope_theta, weights, mean_projection=mean_projection)

    def new_cache(self, cap_ref: int, cap_tok: int) -> OracleCache:
        return OracleCache(self.two_dk, self.d_c, self.top_k, self.group, self.bits,
                           cap_ref, cap_tok, self.mode)

    # ---- write path -------------------------------------------------------------------

    def append_ref(self, cache: OracleCache, kv: np.ndarray, pos: Sequence[int]) -> None:
        """Store tokens directly as references (section 2.7 step 4; FP8 storage, section 2.4)."""
        kv = np.asarray(kv, dtype=np.float64).reshape(-1, self.two_dk)
        for row, p in zip(kv, pos):
            m = cache.ref_count
            if m >= cache.ref_pos.shape[0]:
                raise ValueError("reference pool capacity exceeded")
            if self.mode == "bf16":
                code = fp8_e4m3fn_encode(row)
                cache.ref_code[m] = code
                cache.ref_val[m] = fp8_e4m3fn_decode(code)
            else:
                cache.ref_val[m] = row.astype(np.float32).astype(np.float64)
            cache.ref_pos[m] = p
            cache.self_slot[p] = m
            cache.ref_count = m + 1

    def encoder_input(self, mean32: np.ndarray) -> np.ndarray:
        """The mean as the encoder sees it: rounded to the KV dtype."""
        if self.mode == "bf16":
            return bf16_round(mean32).astype(np.float64)
        return mean32.astype(np.float64)

    def encode(self, cache: OracleCache, kv: np.ndarray, pos: Sequence[int],
               ref_override: Optional[Dict[int, Sequence[int]]] = None) -> None:
        """Search, average, encode, quantize each token (sections 2.2-2.4).

        ref_override maps a position to a given reference slot set (used to re-encode
        a token with another valid choice at a distance tie).
        """
        kv = np.asarray(kv, dtype=np.float64).reshape(-1, self.two_dk)
        pos = list(int(p) for p in pos)
        n = len(pos)
        W = self.W
        xbar = np.zeros((n, self.two_dk))
        a_mean = (np.zeros((n, self.d_ff)), np.zeros((n, self.d_ff)))
        for t, p in enumerate(pos):
            if ref_override is not None and p in ref_override:
                slots = np.sort(np.asarray(ref_override[p], dtype=np.int64))
                diff = cache.ref_val[slots] - kv[t][None, :]
                dist = np.sum(diff * diff, axis=1)
            else:
                slots, dist = topk_references(kv[t], cache.ref_val, cache.ref_pos,
                                              cache.ref_count, p, self.top_k)
            cache.ref_idx[p] = -1
            cache.ref_idx[p, : slots.size] = slots
            cache.ref_dist[p] = np.nan
            cache.ref_dist[p, : slots.size] = dist
            if self.mean_projection:
                p1, p2 = reference_projections(cache.ref_val[slots], W["Wc1"], W["Wc2"])
                a_mean[0][t], a_mean[1][t] = averaged_preactivations(p1, p2)
            else:
                mean32 = reference_mean32(cache.ref_val[slots]) if slots.size else np.zeros(self.two_dk, np.float32)
                xbar[t] = self.encoder_input(mean32)
        # average-then-encode: z = f_c(kv_i) - f_c(mean_i)  (section 2.3, boxed equation)
        f_kv = swiglu_compressor(kv, W["Wc1"], W["Wc2"], W["Wc3"])
        if self.mean_projection:
            f_mean = swiglu_from_preactivations(a_mean[0], a_mean[1], W["Wc3"])
        else:
            f_mean = swiglu_compressor(xbar, W["Wc1"], W["Wc2"], W["Wc3"])
        z = f_kv - f_mean
        store = "f16" if self.mode == "bf16" else "f32"
        q, step, zmin = group_quantize(z, self.bits, self.group, store)
        for t, p in enumerate(pos):
            cache.z[p] = z[t]
            cache.f_scale[p] = np.max(np.abs(f_kv[t])) + np.max(np.abs(f_mean[t]))
            if self.bits == 16:
                cache.latent[p] = step[t]
            else:
                cache.q[p] = q[t]
                cache.step[p] = step[t]
                cache.zmin[p] = zmin[t]

    # ---- read path --------------------------------------------------------------------

    def latent_tilde(self, cache: OracleCache, pos: Sequence[int]) -> np.ndarray:
        pos = np.asarray(pos, dtype=np.int64)
        if self.bits == 16:
            return cache.latent[pos].copy()
        return group_dequantize(cache.q[pos], cache.step[pos], cache.zmin[pos], self.group)

    def restore_prerope(self, cache: OracleCache, pos: Sequence[int]) -> np.ndarray:
        """KV-hat_i = f_d(z~_i) + mean_i (section 2.5, boxed equation); references: stored value."""
        pos = np.asarray(pos, dtype=np.int64)
        out = np.zeros((pos.size, self.two_dk))
        enc = [t for t, p in enumerate(pos) if cache.self_slot[p] < 0]
        if enc:
            zt = self.latent_tilde(cache, pos[enc])
            dec = linear_decoder(zt, self.W["Wd"])
            for r, t in enumerate(enc):
                slots = cache.ref_idx[pos[t]]
                slots = slots[slots >= 0]
                mean32 = reference_mean32(cache.ref_val[slots]) if slots.size else np.zeros(self.two_dk, np.float32)
                out[t] = dec[r] + mean32.astype(np.float64)
        for t, p in enumerate(pos):
            s = cache.self_slot[p]
            if s >= 0:
                out[t] = cache.ref_val[s]
        return out

    def decode_selected(self, cache: OracleCache, idx: Sequence[int]) -> np.ndarray:
        """Restore the selected tokens: K with RoPE at own position, V as is (section 2.7 step 2-3).

        Returns [m, 2*d_k] in fp64, K heads then V heads.
        """
        idx = np.asarray(idx, dtype=np.int64)
        v = self.restore_prerope(cache, idx)
        v[:, : self.dk] = rope_rotate(v[:, : self.dk], idx, self.N, self.D, self.theta)
        return v

    # ---- bulk helpers -------------------------------------------------------------------

    def prefill(self, kv: np.ndarray, stride: int, cap_ref: Optional[int] = None) -> OracleCache:
        """Append every stride-th token as a reference, then encode all others."""
        T = kv.shape[0]
        ref_pos = np.arange(0, T, stride)
        enc_pos = np.array([p for p in range(T) if p % stride != 0], dtype=np.int64)
        cache = self.new_cache(cap_ref or ref_pos.size, T)
        self.append_ref(cache, kv[ref_pos], ref_pos)
        if enc_pos.size:
            self.encode(cache, kv[enc_pos], enc_pos)
        return cache
