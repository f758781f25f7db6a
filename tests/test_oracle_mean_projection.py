"""Pins for the mean-projection form of the oracle's encoder.

The form is an algebraic identity of the compressor of section 2.3 of the ResidualKV
review page (not a step the page prints): the first layer of f_c is linear, so the
pre-activations of the reference mean are the mean of the references' pre-activations.
The oracle computes it as the steps of that shortcut (project each chosen reference,
average the projections, then SwiGLU and W_c3). These tests hold it to the definition it
must reproduce, f_c of the exact (unrounded) mean through the plain compressor, to the
special cases where it must coincide with the default form, and to the method's
degenerate case of a token equal to its mean.
"""

import numpy as np

from oracle import OracleCodec, swiglu_compressor
from oracle.codec import averaged_preactivations, reference_projections, swiglu_from_preactivations
from oracle.formats import bf16_round
from synth import codec_weights, workload


def make(mode="bf16", bits=4, k=4, N=2, D=16, d_ff=48, d_c=32, seed=5, proj=True):
    two_dk = 2 * N * D
    W = codec_weights(two_dk, d_ff, d_c, np.random.default_rng(seed), "bf16" if mode == "bf16" else "f32")
    return OracleCodec(N, D, d_ff, d_c, k, bits, 32, mode, 1e4, W, mean_projection=proj), W


def kv_of(codec, T, seed=2):
    kv = workload(seed).replace(n_kv_heads=codec.N, head_dim=codec.D).make_kv(T=T)
    return bf16_round(kv) if codec.mode == "bf16" else kv.astype(np.float32).astype(np.float64)


def test_projection_form_is_compressor_of_exact_mean():
    # z = f_c(kv) - f_c(mean) with mean the exact fp64 average of the stored references,
    # evaluated here by the plain compressor on that mean: an independent route to the
    # same number (a wrong slot, a swapped W_c1 / W_c2, a sum in place of the mean or a
    # missing W_c3 all fail it)
    codec, W = make()
    T, s = 150, 8
    kv = kv_of(codec, T)
    cache = codec.prefill(kv, s)
    checked = 0
    for p in range(1, T):
        if p % s == 0:
            continue
        sl = cache.ref_idx[p][cache.ref_idx[p] >= 0]
        mean64 = cache.ref_val[sl].mean(axis=0)
        z = (swiglu_compressor(kv[p][None], W["Wc1"], W["Wc2"], W["Wc3"])
             - swiglu_compressor(mean64[None], W["Wc1"], W["Wc2"], W["Wc3"]))[0]
        scale = cache.f_scale[p]
        assert np.max(np.abs(cache.z[p] - z)) <= 1e-12 * scale, p
        checked += 1
    assert checked > 100


def test_projection_form_searches_the_same_sets():
    # only the encoder's view of the mean changes: the reference sets are the search's
    codec, _ = make(proj=True)
    plain, _ = make(proj=False)
    kv = kv_of(codec, 120)
    a, b = codec.prefill(kv, 8), plain.prefill(kv, 8)
    assert np.array_equal(a.ref_idx, b.ref_idx)
    assert np.array_equal(a.ref_dist, b.ref_dist, equal_nan=True)
    assert not np.array_equal(a.z, b.z)  # the bf16 rounding of the mean is gone


def test_single_reference_coincides_with_default_form():
    # top_k = 1: the mean is the stored FP8 reference itself, which bf16 holds exactly, so
    # the default form's rounded mean is the same vector and both forms give the same bits
    codec, _ = make(k=1, proj=True)
    plain, _ = make(k=1, proj=False)
    kv = kv_of(codec, 100)
    a, b = codec.prefill(kv, 8), plain.prefill(kv, 8)
    for name in ("ref_idx", "z", "q", "step", "zmin"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name


def test_fp32_formats_differ_only_by_mean_rounding():
    # "f32" formats: the default form rounds the mean to fp32 only; the difference in z is
    # then bounded by the effect of a 2^-24 relative perturbation of the mean
    codec, W = make(mode="f32", bits=16, proj=True)
    plain, _ = make(mode="f32", bits=16, proj=False)
    kv = kv_of(codec, 120)
    a, b = codec.prefill(kv, 8), plain.prefill(kv, 8)
    enc = [p for p in range(1, 120) if p % 8]
    d = np.abs(a.z[enc] - b.z[enc])
    assert np.max(d / a.f_scale[enc][:, None]) < 1e-5
    assert np.max(d) > 0.0


def test_token_at_its_mean_has_zero_residual():
    # four identical references: their mean is exact in every format; a token equal to it
    # has z = 0 up to the fp64 rounding of the two routes (projection vs direct product)
    codec, _ = make(bits=4)
    rng = np.random.default_rng(3)
    r = bf16_round(rng.standard_normal(codec.two_dk).astype(np.float32) * 0.5)
    cache = codec.new_cache(8, 16)
    codec.append_ref(cache, np.stack([r] * 4), [0, 1, 2, 3])
    stored = cache.ref_val[0]
    codec.encode(cache, stored[None], [6])
    assert cache.ref_idx[6].tolist() == [0, 1, 2, 3]
    assert np.max(np.abs(cache.z[6])) <= 1e-12 * cache.f_scale[6]


def test_projection_helpers_closed_forms():
    rng = np.random.default_rng(8)
    refs = rng.standard_normal((3, 6))
    W1, W2 = rng.standard_normal((6, 5)), rng.standard_normal((6, 5))
    p1, p2 = reference_projections(refs, W1, W2)
    a1, a2 = averaged_preactivations(p1, p2)
    np.testing.assert_allclose(a1, refs.mean(axis=0) @ W1, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(a2, refs.mean(axis=0) @ W2, rtol=1e-13, atol=1e-13)
    e1, e2 = averaged_preactivations(np.zeros((0, 5)), np.zeros((0, 5)))
    assert np.all(e1 == 0) and np.all(e2 == 0)
    W3 = rng.standard_normal((5, 4))
    # Swish(0) = 0: zero pre-activations give f = 0; Swish(a) = a sigmoid(a) at a = 1
    assert np.all(swiglu_from_preactivations(np.zeros(5), np.ones(5), W3) == 0)
    one = swiglu_from_preactivations(np.ones(5), np.ones(5), np.eye(5))
    np.testing.assert_allclose(one, np.full(5, 1.0 / (1.0 + np.exp(-1.0))), rtol=1e-15)
