"""Pins for the CPU oracle of the ResidualKV codec.

Each test checks the oracle against something other than itself: values the
ResidualKV review page prints, closed forms, the page's exact identities and
bounds, special cases and brute force on tiny inputs. They are chosen so that a
plausible slip in the oracle (a dropped term, a swapped weight, a wrong index,
sign or order of operations) fails at least one of them.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import (
    OracleCodec,
    group_dequantize,
    group_quantize,
    group_storage_ratio,
    keep_ratio,
    linear_decoder,
    reference_mean32,
    rope_rotate,
    swiglu_compressor,
    topk_references,
)
from oracle.formats import bf16_round, fp8_e4m3fn_decode, fp8_e4m3fn_encode
from synth import codec_weights, workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_values.json")


def small_codec(mode="bf16", bits=4, N=2, D=16, d_ff=48, d_c=32, k=4, theta=1e4, seed=5, weights=None):
    two_dk = 2 * N * D
    W = weights or codec_weights(two_dk, d_ff, d_c, np.random.default_rng(seed), "bf16" if mode == "bf16" else "f32")
    return OracleCodec(N, D, d_ff, d_c, k, bits, 32, mode, theta, W), W


# ---------------------------------------------------------------- search (section 2.2)


def test_topk_brute_force_tiny_pools():
    rng = np.random.default_rng(11)
    for trial in range(60):
        n_ref = int(rng.integers(1, 11))
        dim = int(rng.integers(2, 9))
        k = int(rng.integers(1, 6))
        ref_val = rng.standard_normal((n_ref, dim))
        ref_pos = rng.permutation(40)[:n_ref].astype(np.int32)
        pos_i = int(rng.integers(0, 45))
        kv = rng.standard_normal(dim)
        slots, dist = topk_references(kv, ref_val, ref_pos, n_ref, pos_i, k)
        cand = [m for m in range(n_ref) if ref_pos[m] < pos_i]
        k_i = min(k, len(cand))
        assert slots.size == k_i
        if k_i == 0:
            continue
        # the chosen set minimises the mean squared distance rho^2 over all k_i-subsets
        best = min(
            itertools.combinations(cand, k_i),
            key=lambda S: sum(float(np.sum((kv - ref_val[m]) ** 2)) for m in S),
        )
        assert sorted(best) == slots.tolist()
        assert np.all(np.diff(slots) > 0)
        assert np.all(ref_pos[slots] < pos_i)
        np.testing.assert_allclose(dist, [np.sum((kv - ref_val[m]) ** 2) for m in slots])


def test_topk_tie_prefers_lower_slot():
    ref_val = np.array([[1.0, 0.0], [0.0, 1.0], [-1.0, 0.0], [3.0, 3.0]])
    ref_pos = np.array([0, 1, 2, 3], dtype=np.int32)
    slots, _ = topk_references(np.zeros(2), ref_val, ref_pos, 4, 10, 2)
    assert slots.tolist() == [0, 1]


def test_warmup_k_i():
    codec, _ = small_codec()
    cfg_T, s = 72, 8
    kv = np.random.default_rng(0).standard_normal((cfg_T, codec.two_dk)).astype(np.float32)
    kv = bf16_round(kv)
    cache = codec.prefill(kv, s)
    for p in range(cfg_T):
        if p % s == 0:
            continue
        k_i = int(np.sum(cache.ref_idx[p] >= 0))
        assert k_i == min(4, (p - 1) // s + 1), p
        assert np.all(cache.ref_pos[cache.ref_idx[p][cache.ref_idx[p] >= 0]] < p)


# ------------------------------------------------------------ mean, Theorem IV.1 (section 2.8)


def test_theorem_iv1_distance_decomposition():
    codec, _ = small_codec()
    kv = bf16_round(workload(1).make_kv(T=160)[:, : codec.two_dk])
    cache = codec.prefill(kv, 8)
    checked = 0
    for p in range(1, 160):
        if p % 8 == 0:
            continue
        sl = cache.ref_idx[p][cache.ref_idx[p] >= 0]
        R = cache.ref_val[sl]
        mean = R.mean(axis=0)
        rho2 = np.mean(np.sum((kv[p] - R) ** 2, axis=1))
        delta2 = np.sum((kv[p] - mean) ** 2)
        V = np.mean(np.sum((R - mean) ** 2, axis=1))
        assert rho2 == pytest.approx(delta2 + V, rel=1e-12)
        # the stored distances are the ones the theorem talks about
        assert np.mean(cache.ref_dist[p][: sl.size]) == pytest.approx(rho2, rel=1e-12)
        checked += 1
    assert checked > 100


def test_mean32_exact_for_fp8_references():
    # a sum of at most four FP8 values needs at most 23 significant bits: the fp32
    # accumulation is exact, so mean32 is the exact mean rounded once to fp32
    rng = np.random.default_rng(2)
    for _ in range(200):
        k = int(rng.integers(1, 5))
        R = fp8_e4m3fn_decode(fp8_e4m3fn_encode(rng.standard_normal((k, 64)) * 8))
        m32 = reference_mean32(R)
        exact = (R.sum(axis=0) / k).astype(np.float32)
        assert np.array_equal(m32.view(np.uint32), exact.view(np.uint32))
    assert reference_mean32(np.zeros((0, 5))).tolist() == [0.0] * 5


# -------------------------------------------------------------- encoder (section 2.3)


def test_swiglu_closed_form_and_operand_roles():
    # W_c1 = I goes through Swish, W_c2 = 2I is the gate, W_c3 = I: f(x) = Swish(x) * 2x
    I = np.eye(3)
    x = np.array([[1.0, 0.0, -1.0]])
    f = swiglu_compressor(x, I, 2 * I, I)
    # Swish(1) = 1/(1+e^-1) = 0.7310585786300049, Swish(-1) = -0.2689414213699951
    np.testing.assert_allclose(f, [[2 * 0.7310585786300049, 0.0, 2 * 0.2689414213699951]], rtol=1e-15)
    # swapping the roles of W_c1 and W_c2 gives Swish(2x) * x, which differs
    g = swiglu_compressor(x, 2 * I, I, I)
    assert abs(g[0, 0] - f[0, 0]) > 0.2
    # large positive pre-activation: Swish(a) -> a
    big = swiglu_compressor(np.array([[40.0]]), np.eye(1), np.eye(1), np.eye(1))
    assert big[0, 0] == pytest.approx(1600.0, rel=1e-15)


def test_average_then_encode_order():
    codec, W = small_codec(mode="f32", bits=16)
    rng = np.random.default_rng(9)
    dim = codec.two_dk
    a, b, c = (rng.standard_normal(dim) for _ in range(3))
    kv = rng.standard_normal(dim)

    def z_with_refs(refs, kv_row):
        cache = codec.new_cache(8, 16)
        codec.append_ref(cache, np.asarray(refs), list(range(len(refs))))
        codec.encode(cache, kv_row[None, :], [10])
        return cache.z[10].copy()

    # (1) two reference pairs with the same mean give the same z: z depends on the
    # references only through their mean (rules out encode-then-average)
    z1 = z_with_refs([a, b], kv)
    z2 = z_with_refs([a + c, b - c], kv)
    # mean32 of the two pairs differs only by fp32 rounding
    np.testing.assert_allclose(z1, z2, atol=1e-5)
    fa, fb = swiglu_compressor(np.stack([a, b]), W["Wc1"], W["Wc2"], W["Wc3"])
    enc_then_avg = swiglu_compressor(kv[None], W["Wc1"], W["Wc2"], W["Wc3"])[0] - (fa + fb) / 2
    assert np.max(np.abs(enc_then_avg - z1)) > 1e-2
    # (2) shifting the token and its references together changes z: z is not f_c(kv - mean)
    u = 3.0 * rng.standard_normal(dim)
    z3 = z_with_refs([a + u, b + u], kv + u)
    assert np.max(np.abs(z3 - z1)) > 1e-2


def test_zero_residual_when_token_equals_reference_mean():
    codec, _ = small_codec(mode="bf16", bits=4)
    rng = np.random.default_rng(4)
    refs = bf16_round(rng.standard_normal((4, codec.two_dk)).astype(np.float32))
    cache = codec.new_cache(8, 16)
    codec.append_ref(cache, refs, [0, 1, 2, 3])
    mean32 = reference_mean32(cache.ref_val[:4])
    kv = bf16_round(mean32)  # the token equals the encoder's view of its reference mean
    codec.encode(cache, kv[None, :], [6])
    assert cache.ref_idx[6].tolist() == [0, 1, 2, 3]
    assert np.all(cache.z[6] == 0.0)
    assert np.all(cache.q[6] == 0) and np.all(cache.step[6] == 0.0) and np.all(cache.zmin[6] == 0.0)
    # decode restores the fp32 reference mean exactly (RoPE at position 6 on K only)
    pre = codec.restore_prerope(cache, [6])[0]
    assert np.array_equal(pre, mean32.astype(np.float64))


def test_zero_compressor_gives_mean():
    codec, W = small_codec(mode="f32")
    W0 = dict(W)
    W0["Wc1"] = np.zeros_like(W["Wc1"])  # Swish(0) = 0 so f_c is identically 0
    codec0 = OracleCodec(codec.N, codec.D, codec.d_ff, codec.d_c, 4, 4, 32, "f32", 1e4, W0)
    kv = workload(1).make_kv(T=40)[:, : codec.two_dk]
    cache = codec0.prefill(kv, 8)
    for p in range(1, 40):
        if p % 8:
            assert np.all(cache.z[p] == 0.0)
            sl = cache.ref_idx[p][cache.ref_idx[p] >= 0]
            np.testing.assert_array_equal(codec0.restore_prerope(cache, [p])[0], reference_mean32(cache.ref_val[sl]))


# -------------------------------------------------------------- quantizer (section 2.4)


@pytest.mark.parametrize("bits", [2, 4])
def test_quantizer_bounds_fp32_storage(bits):
    rng = np.random.default_rng(bits)
    z = rng.standard_normal((300, 96)) * rng.uniform(0.01, 10, (300, 1))
    q, step, zmin = group_quantize(z, bits, 32, "f32")
    zt = group_dequantize(q, step, zmin, 32)
    z32 = z.astype(np.float32).astype(np.float64)
    g_of = np.arange(96) // 32
    # per coordinate |z~ - z| <= Delta/2 (the first step of the page's error bound)
    err = np.abs(zt - z32)
    assert np.all(err <= step[:, g_of] / 2 * (1 + 1e-5) + 1e-12)
    # group-norm bound and its relaxation: ||e|| <= sqrt(sum |G| range^2)/(2(2^b-1)) <= sqrt(g/2)/(2^b-1) ||z||
    rng_g = np.stack([np.ptp(z32[:, g * 32:(g + 1) * 32], axis=1) for g in range(3)], axis=1)
    e = np.linalg.norm(zt - z32, axis=1)
    b1 = np.sqrt(np.sum(32 * rng_g ** 2, axis=1)) / (2 * (2 ** bits - 1))
    b2 = np.sqrt(32 / 2) / (2 ** bits - 1) * np.linalg.norm(z32, axis=1)
    assert np.all(e <= b1 * (1 + 1e-5)) and np.all(b1 <= b2 * (1 + 1e-12))
    # group minimum -> code 0, group maximum -> code 2^b - 1
    for g in range(3):
        sl = slice(g * 32, (g + 1) * 32)
        rows = np.arange(300)
        assert np.all(q[rows, g * 32 + np.argmin(z32[:, sl], axis=1)] == 0)
        assert np.all(q[rows, g * 32 + np.argmax(z32[:, sl], axis=1)] == 2 ** bits - 1)


def test_quantizer_constant_group_passes_through():
    z = np.zeros((2, 64))
    z[0, :32] = 0.3125
    z[0, 32:] = np.linspace(-1, 1, 32)
    z[1, :] = -7.25
    q, step, zmin = group_quantize(z, 4, 32, "f32")
    zt = group_dequantize(q, step, zmin, 32)
    assert step[0, 0] == 0.0 and step[1, 0] == 0.0 and step[1, 1] == 0.0
    np.testing.assert_array_equal(zt[0, :32], z[0, :32])
    np.testing.assert_array_equal(zt[1], z[1])


def test_quantizer_fp16_storage_bound():
    rng = np.random.default_rng(1)
    z = rng.standard_normal((500, 64)) * 0.3
    for bits in (2, 4):
        q, step, zmin = group_quantize(z, bits, 32, "f16")
        zt = group_dequantize(q, step, zmin, 32)
        z32 = z.astype(np.float32).astype(np.float64)
        g_of = np.arange(64) // 32
        lo = np.stack([z32[:, :32].min(1), z32[:, 32:].min(1)], 1)
        d32 = np.stack([np.ptp(z32[:, :32], 1), np.ptp(z32[:, 32:], 1)], 1) / (2 ** bits - 1)
        slack = np.abs(lo - zmin) + (2 ** bits - 1) * np.abs(d32 - step)
        assert np.all(np.abs(zt - z32) <= (step / 2 + slack)[:, g_of] + 1e-7)
        assert np.all(q <= 2 ** bits - 1)


def test_quantization_off_is_fp16_identity():
    z = np.random.default_rng(0).standard_normal((4, 64))
    _, lat, _ = group_quantize(z, 16, 32, "f16")
    np.testing.assert_array_equal(lat, z.astype(np.float32).astype(np.float16).astype(np.float64))


# -------------------------------------------------------------- decoder (section 2.5)


def test_decoder_linear_and_error_propagation():
    codec, W = small_codec(mode="f32")
    Wd = W["Wd"]
    z = np.random.default_rng(3).standard_normal((10, codec.d_c))
    assert np.all(linear_decoder(np.zeros((1, codec.d_c)), Wd) == 0)
    np.testing.assert_allclose(linear_decoder(2 * z[:5] - z[5:], Wd),
                               2 * linear_decoder(z[:5], Wd) - linear_decoder(z[5:], Wd), atol=1e-12)
    kv = workload(1).make_kv(T=64)[:, : codec.two_dk]
    cache = codec.prefill(kv, 8)
    opn = np.linalg.norm(Wd, 2)
    for p in range(1, 64):
        if p % 8 == 0:
            continue
        pre = codec.restore_prerope(cache, [p])[0]
        sl = cache.ref_idx[p][cache.ref_idx[p] >= 0]
        exact = linear_decoder(cache.z[p][None], Wd)[0] + reference_mean32(cache.ref_val[sl])
        eq = codec.latent_tilde(cache, [p])[0] - cache.z[p]
        assert np.linalg.norm(pre - exact) <= opn * np.linalg.norm(eq) * (1 + 1e-9) + 1e-12


def test_reference_tokens_decode_to_stored_value():
    codec, _ = small_codec(mode="bf16")
    kv = bf16_round(np.random.default_rng(1).standard_normal((24, codec.two_dk)).astype(np.float32) * 3)
    cache = codec.prefill(kv, 8)
    out = codec.decode_selected(cache, [0, 8, 16])
    # position 0: RoPE is the identity, the output is exactly the FP8 round trip of the token
    np.testing.assert_array_equal(out[0], fp8_e4m3fn_decode(fp8_e4m3fn_encode(kv[0])))
    # V half is never rotated
    np.testing.assert_array_equal(out[1, codec.dk:], cache.ref_val[1, codec.dk:])


# ------------------------------------------------------------------ RoPE (section 2.1)


def test_rope_half_split_known_values():
    # D = 4, theta = 1e4: omega = [1, 0.01]; pairs are (0, 2) and (1, 3)
    k = np.array([[1.0, 0.0, 0.0, 0.0], [0.0, 1.0, 0.0, 0.0]])
    out = rope_rotate(k, np.array([1, 1]), 1, 4, 1e4)
    np.testing.assert_allclose(out[0], [0.5403023058681398, 0.0, 0.8414709848078965, 0.0], rtol=1e-15, atol=1e-16)
    np.testing.assert_allclose(out[1], [0.0, math.cos(0.01), 0.0, math.sin(0.01)], rtol=1e-15, atol=1e-16)


def test_rope_identities():
    rng = np.random.default_rng(0)
    N, D, th = 3, 8, 5e5
    q = rng.standard_normal((1, N * D))
    k = rng.standard_normal((1, N * D))
    assert np.array_equal(rope_rotate(k, np.array([0]), N, D, th), k)
    a, b = 131071, 77
    r = rope_rotate(k, np.array([a]), N, D, th).reshape(N, D)
    kk = k.reshape(N, D)
    # norms of every rotated pair are preserved
    np.testing.assert_allclose(r[:, :4] ** 2 + r[:, 4:] ** 2, kk[:, :4] ** 2 + kk[:, 4:] ** 2, rtol=1e-12)
    # relative position: <R_a q, R_b k> = <R_(a-b) q, k>, head by head
    lhs = np.sum(rope_rotate(q, np.array([a]), N, D, th).reshape(N, D) *
                 rope_rotate(k, np.array([b]), N, D, th).reshape(N, D), axis=1)
    rhs = np.sum(rope_rotate(q, np.array([a - b]), N, D, th).reshape(N, D) * kk, axis=1)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-9, atol=1e-9)


def test_restored_key_rotates_at_own_position():
    codec, _ = small_codec(mode="f32", bits=16)
    rng = np.random.default_rng(8)
    refs = rng.standard_normal((4, codec.two_dk)).astype(np.float32)
    cache = codec.new_cache(8, 64)
    codec.append_ref(cache, refs, [0, 8, 16, 24])
    kv = reference_mean32(cache.ref_val[:4]).astype(np.float64)
    codec.encode(cache, kv[None], [37])
    out = codec.decode_selected(cache, [37])[0]
    want_k = rope_rotate(kv[None, : codec.dk], np.array([37]), codec.N, codec.D, codec.theta)[0]
    np.testing.assert_array_equal(out[: codec.dk], want_k)
    np.testing.assert_array_equal(out[codec.dk:], kv[codec.dk:])
    wrong = rope_rotate(kv[None, : codec.dk], np.array([24]), codec.N, codec.D, codec.theta)[0]
    assert np.max(np.abs(out[: codec.dk] - wrong)) > 1e-3


# ---------------------------------------------------------- streaming = bulk (section 2.7)


def test_streaming_equals_bulk():
    codec, _ = small_codec(mode="bf16", bits=4)
    T, s = 90, 8
    kv = bf16_round(workload(2).replace(n_kv_heads=2, head_dim=16).make_kv(T=T))
    bulk = codec.prefill(kv, s)
    stream = codec.new_cache(bulk.ref_pos.shape[0], T)
    for p in range(T):
        if p % s == 0:
            codec.append_ref(stream, kv[p][None], [p])
        else:
            codec.encode(stream, kv[p][None], [p])
    for name in ("ref_code", "ref_pos", "q", "step", "zmin", "ref_idx", "self_slot"):
        assert np.array_equal(getattr(bulk, name), getattr(stream, name)), name
    np.testing.assert_array_equal(codec.decode_selected(bulk, np.arange(T)), codec.decode_selected(stream, np.arange(T)))


# ------------------------------------------------- re-encoding with given reference sets


def test_ref_override_with_own_sets_reproduces_records():
    # the parity tests re-encode a token with the GPU's (equally near) reference set; with
    # the oracle's own sets that re-encode must reproduce its records bit for bit
    codec, _ = small_codec(mode="bf16", bits=4)
    T, s = 120, 8
    kv = bf16_round(workload(2).replace(n_kv_heads=2, head_dim=16).make_kv(T=T))
    bulk = codec.prefill(kv, s)
    pos = np.array([p for p in range(1, T) if p % s][::3])
    again = codec.prefill(kv, s)
    codec.encode(again, kv[pos], pos, ref_override={int(p): bulk.ref_idx[p][bulk.ref_idx[p] >= 0] for p in pos})
    for name in ("q", "step", "zmin", "ref_idx", "ref_dist", "z"):
        assert np.array_equal(getattr(bulk, name), getattr(again, name), equal_nan=True), name


def test_ref_override_uses_the_given_slots():
    # another set than the search's: the stored slots, their distances and the mean the
    # encoder sees all come from the given slots (section 2.2 mean equation, section 2.3)
    codec, W = small_codec(mode="bf16", bits=4)
    T, s = 120, 8
    kv = bf16_round(workload(2).replace(n_kv_heads=2, head_dim=16).make_kv(T=T))
    cache = codec.prefill(kv, s)
    p = 101
    given = [0, 3, 7, 11]  # descending order on purpose: stored ascending
    codec.encode(cache, kv[p][None], [p], ref_override={p: given[::-1]})
    assert cache.ref_idx[p].tolist() == given
    np.testing.assert_array_equal(cache.ref_dist[p], np.sum((cache.ref_val[given] - kv[p][None]) ** 2, axis=1))
    xbar = bf16_round(reference_mean32(cache.ref_val[given])).astype(np.float64)
    z = (swiglu_compressor(kv[p][None], W["Wc1"], W["Wc2"], W["Wc3"])
         - swiglu_compressor(xbar[None], W["Wc1"], W["Wc2"], W["Wc3"]))[0]
    np.testing.assert_array_equal(cache.z[p], z)
    searched = codec.prefill(kv, s)
    assert not np.array_equal(searched.ref_idx[p], cache.ref_idx[p])
    assert not np.array_equal(searched.z[p], cache.z[p])


def test_near_tie_generator_plants_what_it_says():
    # the adversarial search inputs of the GPU parity tests: planted rows are exact in FP8,
    # equal rows tie at distance 0 (lower slots win), and each planted pair puts its nearer
    # row at the higher slot, 2^-25 nearer
    from synth import near_tie_kv

    wl = workload(2, T=2200, stride=2)
    c = near_tie_kv(wl.make_kv(), 2, {"dup": 600, "graded": 40, "pairs": 1030}, 2110, np.random.default_rng(7))
    refp = np.arange(0, wl.T, 2)
    rv = fp8_e4m3fn_decode(fp8_e4m3fn_encode(c.kv[refp]))
    for m in list(range(600, 624)) + list(range(40, 52)) + list(range(1030, 1070)):
        np.testing.assert_array_equal(rv[m], c.kv[refp[m]])
    assert np.array_equal(bf16_round(c.kv), c.kv)
    for p in c.exact_tokens:
        slots, _ = topk_references(c.kv[p], rv, refp, refp.size, p, 4)
        assert slots.tolist() == [600, 601, 602, 603]
    slots, d = topk_references(c.kv[c.graded_tokens[0]], rv, refp, refp.size, c.graded_tokens[0], 4)
    assert slots.tolist() == [48, 49, 50, 51] and np.all(np.diff(d) == -1.0)
    for m, p in enumerate(c.below_fp32_tokens):
        slots, _ = topk_references(c.kv[p], rv, refp, refp.size, p, 4)
        base = 1030 + 5 * m
        assert slots.tolist() == [base, base + 1, base + 2, base + 4]
        dP = np.sum((rv[base + 3] - c.kv[p]) ** 2)
        dQ = np.sum((rv[base + 4] - c.kv[p]) ** 2)
        assert dP - dQ == 2.0 ** -25


# ------------------------------------------------------------ storage accounting (section 3.3)


def test_storage_ratios_match_printed_values():
    g = json.load(open(GOLDEN))
    q = g["group_storage_ratio"]
    assert group_storage_ratio(4, q["group"]) == q["q4"]
    assert group_storage_ratio(2, q["group"]) == q["q2"]
    for key in ("keep_ratio_llama", "keep_ratio_llama_4_full"):
        e = g[key]
        kr = keep_ratio(e["beta"], e["rho_ref"], q["q4"], q["q4"], e["d_c"], e["two_dk"])
        assert abs(100 * kr - e["printed_percent"]) <= e["printed_tolerance_percent"], (key, kr)
    lw = g["llama_latent_width"]
    assert 2 * lw["n_kv_heads"] * lw["head_dim"] == lw["two_dk"] == workload(2).two_dk
    assert lw["d_c"] == workload(2).d_c


def test_record_bytes_reproduce_sparse_layer_term():
    # INT4 record of d_c = 512: 256 code bytes + 16 groups x two fp16 = 320 B, which
    # over an fp16 K|V row (2 * 2048 B) is q_4 * d_c / (2 d_k); an FP8 reference row is half
    cfg = workload(2)
    rec = cfg.d_c * cfg.bits // 8 + (cfg.d_c // cfg.group) * 2 * 2
    assert rec == 320
    assert rec / (2 * cfg.two_dk) == group_storage_ratio(4) * cfg.d_c / cfg.two_dk
    assert cfg.two_dk * 1 / (2 * cfg.two_dk) == 0.5


# ------------------------------------------------------------------ tiny whole pipeline


def test_tiny_workload_pipeline_runs_and_is_sane():
    cfg = workload(1)
    kv = cfg.make_kv()
    W = cfg.make_weights()
    codec = OracleCodec.from_workload(cfg, W)
    cache = codec.prefill(kv, cfg.stride)
    out = codec.decode_selected(cache, np.arange(cfg.T))
    pre = codec.restore_prerope(cache, np.arange(cfg.T))
    # the nearest reference of a clustered token is close to it (same cluster)
    enc = np.array([p for p in range(4 * cfg.stride, cfg.T) if p % cfg.stride])
    best = np.array([min(np.linalg.norm(kv[p] - cache.ref_val[m]) for m in cache.ref_idx[p] if m >= 0) for p in enc])
    assert np.median(best / np.linalg.norm(kv[enc], axis=1)) < 0.3
    assert np.all(np.isfinite(out))
    # RoPE keeps the norm of every rotated pair
    np.testing.assert_allclose(np.linalg.norm(out[:, : codec.dk].reshape(-1, 2, 2, 32), axis=2),
                               np.linalg.norm(pre[:, : codec.dk].reshape(-1, 2, 2, 32), axis=2), rtol=1e-12)
