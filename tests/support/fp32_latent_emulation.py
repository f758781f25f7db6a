"""An fp32 evaluation of the latent residual, to derive the fp16-latent parity bar.

With quantization off the codec stores fp16(z), z = f_c(kv) - f_c(mean) (ResidualKV
review page, section 2.3 boxed equation; section 2.4: the quantizer is the identity when
off). Any implementation that accumulates in fp32 carries an absolute error on z at the
scale of the two encoder outputs it subtracts, not at the scale of z: a coordinate of z
near zero has an fp16 ulp far below that error. This module evaluates z with plain numpy
float32 arithmetic (BLAS sgemm for the three products, SiLU and the difference in fp32),
independently of the HIP path, so that the bar the GPU is held to is set by what fp32
arithmetic reaches on the CPU, not by the GPU's own results.
"""

from __future__ import annotations

import numpy as np

from oracle.codec import OracleCodec, reference_mean32
from oracle.formats import bf16_round, fp16_round

U32 = 2.0 ** -24


def fp16_ulp(x: np.ndarray) -> np.ndarray:
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - 10)


def hidden_f32(x: np.ndarray, W) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    a = x @ np.asarray(W["Wc1"], dtype=np.float32)
    b = x @ np.asarray(W["Wc2"], dtype=np.float32)
    return (a / (np.float32(1.0) + np.exp(-a))) * b


def projected_mean_hidden_f32(cache, enc, W) -> np.ndarray:
    """The mean's hidden values in the mean-projection form, in fp32: each reference's
    pre-activations r W_c1, r W_c2 (sgemm), summed over the token's references in
    ascending slot order, divided by k, then SiLU(a1) * a2."""
    W1 = np.asarray(W["Wc1"], dtype=np.float32)
    W2 = np.asarray(W["Wc2"], dtype=np.float32)
    out = np.zeros((len(enc), W1.shape[1]), dtype=np.float32)
    for t, p in enumerate(enc):
        sl = cache.ref_idx[p][cache.ref_idx[p] >= 0]
        if sl.size == 0:
            continue
        r = cache.ref_val[sl].astype(np.float32)
        p1, p2 = r @ W1, r @ W2
        a1 = np.zeros(W1.shape[1], dtype=np.float32)
        a2 = np.zeros(W1.shape[1], dtype=np.float32)
        for j in range(sl.size):
            a1 = a1 + p1[j]
            a2 = a2 + p2[j]
        a1 = a1 / np.float32(sl.size)
        a2 = a2 / np.float32(sl.size)
        out[t] = (a1 / (np.float32(1.0) + np.exp(-a1))) * a2
    return out


def emulate(wl, T: int, hidden_round=None, mean_projection: bool = False):
    """Oracle cache of the workload at T tokens, and the fp32 evaluation of z for its
    encoded tokens. hidden_round (optional) rounds the hidden difference before W_c3;
    mean_projection evaluates both with the encoder's mean-projection form.

    Returns (positions, z64 [n, d_c], z32 [n, d_c], f_scale [n])."""
    W = wl.make_weights()
    kv = wl.make_kv(T=T).astype(np.float64)
    codec = OracleCodec.from_workload(wl.replace(T=T), W, mean_projection=mean_projection)
    cache = codec.prefill(kv, wl.stride)
    enc = wl.enc_positions(T)
    if mean_projection:
        h_mean = projected_mean_hidden_f32(cache, enc, W)
    else:
        xbar = np.stack([codec.encoder_input(reference_mean32(cache.ref_val[cache.ref_idx[p][cache.ref_idx[p] >= 0]]))
                         for p in enc])
        h_mean = hidden_f32(xbar, W)
    dh = hidden_f32(kv[enc], W) - h_mean
    if hidden_round is not None:
        dh = hidden_round(dh.astype(np.float64)).astype(np.float32)
    z32 = (dh @ np.asarray(W["Wc3"], dtype=np.float32)).astype(np.float64)
    return enc, cache.z[enc], z32, cache.f_scale[enc]


def fp16_latent_bar(lat_a: np.ndarray, lat_b: np.ndarray, f_scale: np.ndarray, c: float) -> np.ndarray:
    """Largest allowed |lat_a - lat_b| per coordinate for two fp16 latents of the same z:
    one fp16 ulp at the larger magnitude (the two roundings) plus c * 2^-24 * f_scale of
    the token (the fp32 arithmetic error before rounding)."""
    big = np.maximum(np.abs(lat_a), np.abs(lat_b))
    return fp16_ulp(big) + c * U32 * np.asarray(f_scale, dtype=np.float64)[:, None]


def summarize(z64, z32, f_scale, c):
    """Statistics of fp16(z32) against fp16(z64)."""
    a, g = fp16_round(z64), fp16_round(z32)
    d = np.abs(a - g)
    pre = np.abs(z32 - z64) / (U32 * f_scale[:, None])
    return {
        "exact_frac": float(np.mean(d == 0)),
        "within_own_ulp_frac": float(np.mean(d <= fp16_ulp(a))),
        "max_pre_round_err_over_u_scale": float(pre.max()),
        "within_bar_frac": float(np.mean(d <= fp16_latent_bar(a, g, f_scale, c))),
    }


def quantized_agreement(z64, z32, f_scale, bits, store, c):
    """Codes and stored step/minimum of group_quantize on fp32 z against fp64 z: the code
    exact fraction, the largest code difference, and the largest ratio of a step / minimum
    difference to its bar (one storage ulp + 2 E / (2^b - 1), resp. + E, E = c 2^-24 f_scale)."""
    from oracle.codec import group_quantize

    qa, sa, ma = group_quantize(z64, bits, 32, store)
    qg, sg, mg = group_quantize(z32, bits, 32, store)
    E = c * U32 * np.asarray(f_scale, dtype=np.float64)[:, None]
    if store == "f16":
        ulp = fp16_ulp
    else:
        def ulp(x):
            a = np.abs(np.asarray(x, dtype=np.float64))
            return 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -126))) - 23)
    d = np.abs(qa.astype(int) - qg.astype(int))
    sbar = ulp(np.maximum(np.abs(sa), np.abs(sg))) + 2 * E / (2 ** bits - 1)
    mbar = ulp(np.maximum(np.abs(ma), np.abs(mg))) + E
    return {
        "code_exact_frac": float(np.mean(d == 0)),
        "code_max_diff": int(d.max()),
        "step_max_bar_ratio": float(np.max(np.abs(sa - sg) / sbar)),
        "zmin_max_bar_ratio": float(np.max(np.abs(ma - mg) / mbar)),
    }


def bf16_hidden(x):
    """The one-plane mistake: the hidden difference rounded to bf16 before W_c3."""
    return bf16_round(x)
