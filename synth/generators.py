"""Seeded generators: clustered pre-RoPE KV, codec weights, selected-token subsets.

Recipe (stands in for the real-model KV of the review page, section 1.2, Fig. 3,
where each token's best historical match is far away and highly similar):

* centres C ~ N(0, 1), shape [n_clusters, 2*d_k];
* each token picks a centre uniformly and independently, so its best matches are
  spread over the whole history rather than its neighbours;
* kv = C[c] + N(0, sigma^2) noise;
* optionally a seeded 2 % of channels is scaled by 4 (per-channel outliers, as in
  real K caches);
* finally the values are cast to the dtype the backbone hands over (fp32 or bf16,
  round to nearest even, via torch's CPU cast).

Weights are N(0, 1/fan_in) drawn in fp32 and cast to the codec dtype. They are
returned in the pages' math layout (x @ W): W_c1, W_c2 [2d_k, d_ff],
W_c3 [d_ff, d_c], W_d [d_c, 2d_k].

Seeds: the tiny case draws KV from default_rng(0) and weights from default_rng(1);
every other workload uses default_rng([workload_id, layer_or_sequence, stream])
with stream 0 = KV, 1 = weights, 2 = selected subset, 3 = appended tokens.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    """Cast float32 values to `dtype` ('f32' or 'bf16') and return them as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        import torch

        t = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32)
        return t.numpy()
    raise ValueError(f"unknown input dtype {dtype!r}")


def clustered_kv(
    T: int,
    dim: int,
    n_clusters: int,
    sigma: float,
    rng: np.random.Generator,
    outlier_frac: float = 0.0,
    outlier_scale: float = 1.0,
    dtype: str = "f32",
    chunk: int = 1 << 15,
) -> np.ndarray:
    """Clustered KV rows [T, dim] (float32 holding values exact in `dtype`)."""
    centres = rng.standard_normal((n_clusters, dim), dtype=np.float32)
    assign = rng.integers(0, n_clusters, size=T)
    n_out = int(round(outlier_frac * dim))
    scale = np.ones(dim, dtype=np.float32)
    if n_out > 0:
        ch = rng.choice(dim, size=n_out, replace=False)
        scale[ch] = outlier_scale
    out = np.empty((T, dim), dtype=np.float32)
    for s in range(0, T, chunk):
        e = min(T, s + chunk)
        noise = rng.standard_normal((e - s, dim), dtype=np.float32)
        blk = centres[assign[s:e]] + np.float32(sigma) * noise
        blk *= scale
        out[s:e] = _cast(blk, dtype)
    return out


def codec_weights(
    two_dk: int, d_ff: int, d_c: int, rng: np.random.Generator, dtype: str = "f32"
) -> Dict[str, np.ndarray]:
    """Codec weights N(0, 1/fan_in) in math layout (x @ W), float32 values exact in `dtype`."""

    def draw(fan_in: int, fan_out: int) -> np.ndarray:
        w = rng.standard_normal((fan_in, fan_out), dtype=np.float32) / np.float32(np.sqrt(fan_in))
        return _cast(w, dtype)

    return {
        "Wc1": draw(two_dk, d_ff),
        "Wc2": draw(two_dk, d_ff),
        "Wc3": draw(d_ff, d_c),
        "Wd": draw(d_c, two_dk),
    }


def selected_subset(T: int, frac: float, rng: np.random.Generator) -> np.ndarray:
    """Sorted subset of floor(frac*T) distinct token indices in [0, T)."""
    m = int(np.floor(frac * T))
    idx = rng.choice(T, size=m, replace=False)
    return np.sort(idx).astype(np.int32)


@dataclasses.dataclass(frozen=True)
class WorkloadConfig:
    """One synthetic workload: shapes, formats and generator parameters."""

    wid: int
    name: str
    T: int
    n_kv_heads: int
    head_dim: int
    d_ff: int
    d_c: int
    top_k: int
    bits: int  # 2 or 4 = INT codes; 16 = quantization off (fp16 latent)
    group: int
    stride: int  # a reference every `stride` tokens, starting at position 0
    n_clusters: int
    sigma: float
    outlier_frac: float
    outlier_scale: float
    mode: str  # 'f32' (fp32 KV, refs, weights, scales) or 'bf16' (bf16 KV/weights, FP8 refs, fp16 scales)
    rope_theta: float
    batch: int = 1
    select_frac: float = 0.3
    layers: int = 1

    @property
    def two_dk(self) -> int:
        return 2 * self.n_kv_heads * self.head_dim

    @property
    def in_dtype(self) -> str:
        return "f32" if self.mode == "f32" else "bf16"

    def replace(self, **kw) -> "WorkloadConfig":
        return dataclasses.replace(self, **kw)

    def kv_rng(self, seq: int = 0, layer: int = 0) -> np.random.Generator:
        if self.wid == 1:
            return np.random.default_rng(0)
        return np.random.default_rng([self.wid, layer * 1000 + seq, 0])

    def weight_rng(self, layer: int = 0) -> np.random.Generator:
        if self.wid == 1:
            return np.random.default_rng(1)
        return np.random.default_rng([self.wid, layer, 1])

    def subset_rng(self, step: int = 0, seq: int = 0, layer: int = 0) -> np.random.Generator:
        return np.random.default_rng([self.wid, layer * 1000 + seq, 2, step])

    def make_kv(self, seq: int = 0, layer: int = 0, T: Optional[int] = None) -> np.ndarray:
        return clustered_kv(
            self.T if T is None else T,
            self.two_dk,
            self.n_clusters,
            self.sigma,
            self.kv_rng(seq, layer),
            self.outlier_frac,
            self.outlier_scale,
            self.in_dtype,
        )

    def make_weights(self, layer: int = 0) -> Dict[str, np.ndarray]:
        return codec_weights(self.two_dk, self.d_ff, self.d_c, self.weight_rng(layer), self.in_dtype)

    def make_selected(self, T: Optional[int] = None, seq: int = 0, step: int = 0, layer: int = 0) -> np.ndarray:
        """Sorted random subset of floor(select_frac * T) token positions (the read set I_t)."""
        T = self.T if T is None else T
        if self.select_frac >= 1.0:
            return np.arange(T, dtype=np.int32)
        return selected_subset(T, self.select_frac, self.subset_rng(step, seq, layer))

    def ref_positions(self, T: Optional[int] = None) -> np.ndarray:
        T = self.T if T is None else T
        return np.arange(0, T, self.stride, dtype=np.int32)

    def enc_positions(self, T: Optional[int] = None) -> np.ndarray:
        T = self.T if T is None else T
        p = np.arange(T, dtype=np.int32)
        return p[p % self.stride != 0]


# The five workloads. Sizes come from the ResidualKV review page: Llama-3.1-8B has
# 8 KV heads x 128 (2*d_k = 2048, d_c = 512, section 2.3), Qwen2.5-7B has
# 4 KV heads x 128 (2*d_k = 1024). d_ff is not fixed by the pages for these
# runs; 1024 / 512 are used (Table I lists 3072 for the trained codecs).
WORKLOADS: Dict[int, WorkloadConfig] = {
    1: WorkloadConfig(
        wid=1, name="tiny-fp32", T=256, n_kv_heads=2, head_dim=64, d_ff=128, d_c=64,
        top_k=4, bits=4, group=32, stride=8, n_clusters=16, sigma=0.1,
        outlier_frac=0.0, outlier_scale=1.0, mode="f32", rope_theta=1.0e4,
        select_frac=1.0,
    ),
    2: WorkloadConfig(
        wid=2, name="llama3.1-8b-kv-prefill", T=32768, n_kv_heads=8, head_dim=128,
        d_ff=1024, d_c=512, top_k=4, bits=4, group=32, stride=8, n_clusters=256,
        sigma=0.15, outlier_frac=0.02, outlier_scale=4.0, mode="bf16", rope_theta=5.0e5,
    ),
    3: WorkloadConfig(
        wid=3, name="llama3.1-8b-kv-decode", T=131072, n_kv_heads=8, head_dim=128,
        d_ff=1024, d_c=512, top_k=4, bits=4, group=32, stride=8, n_clusters=256,
        sigma=0.15, outlier_frac=0.02, outlier_scale=4.0, mode="bf16", rope_theta=5.0e5,
        layers=32,
    ),
    4: WorkloadConfig(
        wid=4, name="qwen2.5-7b-kv-long-int2", T=262144, n_kv_heads=4, head_dim=128,
        d_ff=512, d_c=256, top_k=4, bits=2, group=32, stride=16, n_clusters=256,
        sigma=0.15, outlier_frac=0.02, outlier_scale=4.0, mode="bf16", rope_theta=1.0e6,
    ),
    5: WorkloadConfig(
        wid=5, name="llama3.1-8b-kv-batch16", T=32768, n_kv_heads=8, head_dim=128,
        d_ff=1024, d_c=512, top_k=4, bits=4, group=32, stride=8, n_clusters=256,
        sigma=0.15, outlier_frac=0.02, outlier_scale=4.0, mode="bf16", rope_theta=5.0e5,
        batch=16,
    ),
}


def workload(wid: int, **overrides) -> WorkloadConfig:
    """Workload `wid`, with fields overridden (e.g. a shorter T for parity runs)."""
    cfg = WORKLOADS[wid]
    return cfg.replace(**overrides) if overrides else cfg


# --------------------------------------------------------------------------------------
# near-duplicate and near-equidistant references (adversarial inputs of the top-k search)
# --------------------------------------------------------------------------------------


@dataclasses.dataclass
class NearTieCase:
    """kv rows [T, dim] with planted reference rows, and the tokens aimed at them.

    exact_tokens: positions whose nearest references tie exactly (equal rows, or a token
    halfway between two rows), so the lower-slot rule fixes the set; graded_tokens:
    positions whose nearest references differ by steps far larger than any rounding;
    below_fp32_tokens: positions whose k-th and (k+1)-th nearest references differ by
    about 3e-10 of the distance, the nearer one at the higher slot (fp32 sums cannot
    order them, fp64 can)."""

    kv: np.ndarray
    exact_tokens: np.ndarray
    graded_tokens: np.ndarray
    below_fp32_tokens: np.ndarray


def _fp8_base_row(dim: int, rng: np.random.Generator) -> np.ndarray:
    """A row of +-(1 + m/8), m = 0..6: exact in OCP e4m3 and bf16, and so is every
    value within 0.25 of it on the grid used below."""
    mag = 1.0 + rng.integers(0, 7, size=dim) / 8.0
    sgn = np.where(rng.random(dim) < 0.5, -1.0, 1.0)
    return (mag * sgn).astype(np.float32)


def near_tie_kv(base: np.ndarray, stride: int, ref_slots: Dict[str, int], tok_start: int,
                rng: np.random.Generator, n_dup: int = 12) -> NearTieCase:
    """Plant near-duplicate reference rows into `base` (clustered rows [T, dim], values
    exact in bf16), references at positions 0, stride, 2 stride, ...

    ref_slots gives the first pool slot of each planted group ('dup', 'graded', 'pairs');
    the tokens aimed at them take the non-reference positions from tok_start on (all
    after every planted reference). Groups:
      dup    - n_dup identical rows A, then n_dup rows A with one coordinate one FP8 step
               up; tokens equal to A, and halfway between A and a shifted row;
      graded - rows that agree with a token y on dim (10 + j) / 128 of its coordinates
               (slot order ascending in j, so later slots are nearer);
      pairs  - for 8 tokens: three rows nearer than a pair (P, Q) that differ only in
               coordinate 0 (2^-9 against 0); the token's coordinate 0 is 2^-10 - 2^-17,
               so Q (the higher slot) is nearer by 2^-25 at a distance near dim / 16.
    """
    kv = np.array(base, dtype=np.float32, copy=True)
    T, dim = kv.shape
    assert dim % 128 == 0 and dim >= 256
    slot_pos = lambda m: m * stride  # noqa: E731
    toks = [p for p in range(tok_start, T) if p % stride != 0]
    ti = iter(toks)
    exact, graded, below = [], [], []

    # dup group
    A = _fp8_base_row(dim, rng)
    s0 = ref_slots["dup"]
    for i in range(n_dup):
        kv[slot_pos(s0 + i)] = A
    for i in range(n_dup):
        j = 3 + 7 * i
        r = A.copy()
        r[j] = A[j] + np.sign(A[j]) * 0.125  # one e4m3 step in [1, 2)
        kv[slot_pos(s0 + n_dup + i)] = r
    for _ in range(4):
        p = next(ti)
        kv[p] = A
        exact.append(p)
    for i in range(4):
        j = 3 + 7 * i
        p = next(ti)
        y = A.copy()
        y[j] = A[j] + np.sign(A[j]) * 0.0625  # halfway to the shifted row
        kv[p] = y
        exact.append(p)

    # graded group
    Bg = _fp8_base_row(dim, rng)
    delta = np.where(rng.random(dim) < 0.5, -0.25, 0.25).astype(np.float32)
    y = Bg + delta  # |y| in [0.75, 2.0]: exact in e4m3 and bf16
    s0 = ref_slots["graded"]
    for i in range(12):
        r = Bg.copy()
        L = dim * (10 + i) // 128
        r[:L] = y[:L]
        kv[slot_pos(s0 + i)] = r
    p = next(ti)
    kv[p] = y
    graded.append(p)

    # below-fp32 pairs
    s0 = ref_slots["pairs"]
    for m in range(8):
        Bm = _fp8_base_row(dim, rng)
        dm = np.where(rng.random(dim) < 0.5, -0.25, 0.25).astype(np.float32)
        dm[:2] = 0.0
        x = Bm + dm
        x[0] = np.float32(2.0 ** -10 - 2.0 ** -17)
        rows = []
        for L in (dim * 75 // 256, dim * 62 // 256, dim * 50 // 256):  # nearer than the pair
            r = Bm.copy()
            r[2:2 + L] = x[2:2 + L]
            r[0] = 0.0
            rows.append(r)
        P = Bm.copy()
        P[0] = np.float32(2.0 ** -9)
        Q = Bm.copy()
        Q[0] = 0.0
        rows += [P, Q]
        for i, r in enumerate(rows):
            kv[slot_pos(s0 + 5 * m + i)] = r
        p = next(ti)
        kv[p] = x
        below.append(p)
    return NearTieCase(kv, np.array(exact, np.int64), np.array(graded, np.int64), np.array(below, np.int64))
