"""GPU parity of the HIP codec (through the C ABI) against the CPU oracle.

Sizes: the tiny fp32 workload in full; the Llama-3.1-8B and Qwen2.5-7B KV shapes
and the batched workload at shortened histories that the oracle finishes in
seconds but that still span several tiles and a ragged tail; and the two bulk
workloads at their full sizes, in the launch configuration the benchmark times,
on sampled tokens the oracle computes one by one.
"""

import numpy as np
import pytest
import torch

from kv_cache_compression_residualkv_amd import binding as B
from oracle import OracleCodec
from oracle.formats import FP8_E4M3FN_VALUES, fp8_e4m3fn_encode
from parity_util import (
    GpuCodec,
    assert_codes_ok,
    assert_end_to_end,
    assert_kv_ok,
    compare_codes,
    compare_refsets,
    kv_errors,
    mirror_cache,
)
from synth import workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    B.load_library()  # raises if librkv.so is missing: no fallback


def _banner(msg):
    print(f"\n[parity] {msg}", flush=True)


# ------------------------------------------------------------------ references


def test_fp8_append_is_bit_exact():
    wl = workload(2, T=64)
    _banner("fp8 append: all codes, ties, saturation")
    gpu = GpuCodec(wl, wl.make_weights(), cap_ref=4, cap_tok=64)
    vals = FP8_E4M3FN_VALUES[np.isfinite(FP8_E4M3FN_VALUES)]  # 254 finite values
    pos_vals = FP8_E4M3FN_VALUES[:0x7F]
    mids = (pos_vals[:-1] + pos_vals[1:]) / 2  # exact ties, bf16-representable
    extra = np.array([448.0, 460.0, 464.0, 500.0, 1e4, -1e4, -0.0, 0.0, 2.0 ** -10, -(2.0 ** -10), 2.0 ** -11])
    rng = np.random.default_rng(0)
    row = np.concatenate([vals, mids, -mids, extra])
    row = np.concatenate([row, rng.standard_normal(wl.two_dk - row.size) * 6])
    kv = np.stack([row, rng.standard_normal(wl.two_dk) * 20]).astype(np.float32)
    kv = torch.from_numpy(kv).to(torch.bfloat16).float().numpy()
    kv_dev = gpu.to_dev(kv)
    rows = torch.tensor([[0, 1]], dtype=torch.int32, device="cuda")
    posv = torch.tensor([[0, 5]], dtype=torch.int32, device="cuda")
    B.rkv_append_ref(gpu.cfg, gpu.cache, kv_dev, rows, posv)
    torch.cuda.synchronize()
    got = gpu.cache.ref_vals[0, :2].cpu().numpy()
    want = fp8_e4m3fn_encode(kv)
    assert np.array_equal(got, want), np.nonzero(got != want)
    assert gpu.cache.ref_count.item() == 2
    assert gpu.cache.ref_pos[0, :2].tolist() == [0, 5]
    assert gpu.cache.self_slot[0, 0].item() == 0 and gpu.cache.self_slot[0, 5].item() == 1
    norm = np.sum(FP8_E4M3FN_VALUES[want] ** 2, axis=1)
    np.testing.assert_allclose(gpu.cache.ref_norm2[0, :2].cpu().numpy(), norm, rtol=1e-6)
    # a reference decodes to its stored value; at position 0 RoPE is the identity
    out = gpu.decode(np.array([0, 5]))
    np.testing.assert_array_equal(out[0, 0], FP8_E4M3FN_VALUES[want[0]])
    oc = OracleCodec.from_workload(wl, wl.make_weights())
    ocache = oc.new_cache(4, 64)
    oc.append_ref(ocache, kv, [0, 5])
    assert_kv_ok(out[0], oc.decode_selected(ocache, [0, 5]), "reference decode")
    assert gpu.cache.error_bits() == 0


# ------------------------------------------------------------------ whole pipeline

CASES = {
    "tiny-fp32": (1, dict()),
    "llama-shape": (2, dict(T=2000)),
    "qwen-shape-int2": (4, dict(T=3000)),
    "batch3-int4": (5, dict(T=600, batch=3)),
    "batch2-fp16-latent": (5, dict(T=520, batch=2, bits=16)),
    "llama-shape-k2-fp16-latent": (2, dict(T=700, top_k=2, bits=16)),
    # the largest k the boundary accepts: k_i up to 8 references, means of up to 8 FP8
    # rows (k = 5, 6, 7 divide exactly), the restore form for k > 4
    "llama-shape-k8": (2, dict(T=900, top_k=8)),
    # the trained codecs' shapes of Table I: Llama-3.1-8B d_ff = 3072, Qwen2.5-7B d_c = 384
    # and d_ff = 3072 (a partial last quantizer tile, 12 latent K-steps in the restore),
    # Qwen2.5-32B d_ff = 4096
    "llama-table1-dff3072": (2, dict(T=1200, d_ff=3072)),
    "qwen-table1-dc384-int2": (4, dict(T=1600, d_ff=3072, d_c=384)),
    "qwen-table1-dc384-int4-batch2": (4, dict(T=700, d_ff=3072, d_c=384, bits=4, batch=2)),
    "qwen32b-table1-dff4096": (2, dict(T=800, d_ff=4096)),
    # d_c = 128: the quantizer's narrow 512-token x 128-column tiles alone (no 256-wide
    # tile), 4 latent K-steps in the restore
    "llama-shape-dc128": (2, dict(T=1300, d_c=128)),
    # d_c = 64 in the bf16 formats: narrow quantizer tiles with half their columns past d_c,
    # and the restore's general kernel (the token-tile restore takes multiples of 128)
    "llama-shape-dc64": (2, dict(T=900, d_c=64)),
    # head_dim 64 in the bf16 formats (16 KV heads x 64: the 2048-wide joint vector, RoPE
    # pairs (j, j + 32), the restore's 64-column passes)
    "d64-bf16-int4": (2, dict(T=1100, n_kv_heads=16, head_dim=64)),
    "d64-bf16-fp16-latent": (2, dict(T=700, n_kv_heads=8, head_dim=64, d_c=256, bits=16)),
}


@pytest.mark.parametrize("case", list(CASES))
def test_pipeline_parity(case):
    wid, over = CASES[case]
    wl = workload(wid, **over)
    T = wl.T
    W = wl.make_weights()
    _banner(f"pipeline {case}: wid={wid} T={T} B={wl.batch} 2dk={wl.two_dk} bits={wl.bits}")
    gpu = GpuCodec(wl, W)
    kvs = [wl.make_kv(seq=b) for b in range(wl.batch)]
    kv_dev = gpu.to_dev(np.stack(kvs))
    gpu.prefill(kv_dev, T)
    torch.cuda.synchronize()
    assert gpu.cache.error_bits() == 0
    codec = OracleCodec.from_workload(wl, W)
    enc_pos = wl.enc_positions()
    sel = np.stack([wl.make_selected(T, seq=b) for b in range(wl.batch)]).astype(np.int32)
    out_all = gpu.decode(np.tile(np.arange(T, dtype=np.int32), (wl.batch, 1)))
    out_sel = gpu.decode(sel)
    # the prepared decoder (rkv_prepare_decoder) gives the same bits
    assert np.array_equal(gpu.decode(np.tile(np.arange(T, dtype=np.int32), (wl.batch, 1)), prepared=True), out_all)
    assert np.array_equal(gpu.decode(sel, prepared=True), out_sel)
    for b in range(wl.batch):
        orc = codec.prefill(kvs[b], wl.stride, cap_ref=gpu.cap_ref)
        gpc = mirror_cache(codec, gpu, b)
        # the pool is bit-exact
        assert gpc.ref_count == orc.ref_count
        if wl.mode == "bf16":
            assert np.array_equal(gpc.ref_code, orc.ref_code)
        else:
            assert np.array_equal(gpc.ref_val, orc.ref_val)
        assert np.array_equal(gpc.self_slot, orc.self_slot)
        ties, hard = compare_refsets(lambda p: kvs[b][p], orc, gpc, enc_pos)
        assert not hard, (case, b, hard[:10])
        if ties:
            codec.encode(orc, kvs[b][ties], ties, ref_override={p: gpc.ref_idx[p][gpc.ref_idx[p] >= 0] for p in ties})
        st = compare_codes(codec, orc, gpc, enc_pos)
        st["ties"] = len(ties)
        print(f"[parity] {case} seq {b}: {st}", flush=True)
        assert_codes_ok(st)
        # decode kernel against the oracle on the GPU's own records
        assert_kv_ok(out_all[b], codec.decode_selected(gpc, np.arange(T)), "decode-all on gpu records")
        assert_kv_ok(out_sel[b], codec.decode_selected(gpc, sel[b]), "decode-sel on gpu records")
        # end to end against the oracle's records
        ma, rr, nd = assert_end_to_end(codec, out_all[b], orc, gpc, np.arange(T), "end-to-end")
        print(f"[parity] {case} seq {b}: end-to-end max_abs(agreeing records)={ma:.3g} rms_rel={rr:.3g} "
              f"tokens with a code difference={nd}", flush=True)


def test_bf16_output_is_rounded_fp32_output():
    wl = workload(2, T=400)
    gpu = GpuCodec(wl, wl.make_weights())
    gpu.prefill(gpu.to_dev(wl.make_kv()[None]), wl.T)
    idx = np.arange(wl.T, dtype=np.int32)[None]
    for prepared in (False, True):
        f = gpu.decode(idx, torch.float32, prepared=prepared)
        h = gpu.decode(idx, torch.bfloat16, prepared=prepared)
        want = torch.from_numpy(f).to(torch.bfloat16).float().numpy()
        assert np.array_equal(h.view(np.uint32), want.view(np.uint32))


def test_streaming_equals_bulk_and_is_deterministic():
    wl = workload(2, T=160)
    W = wl.make_weights()
    kv = wl.make_kv()
    _banner("streaming vs bulk, 160 single-token calls")
    bulk = GpuCodec(wl, W)
    kv_dev = bulk.to_dev(kv[None])
    bulk.prefill(kv_dev, wl.T)
    again = GpuCodec(wl, W)
    again.prefill(kv_dev, wl.T)
    stream = GpuCodec(wl, W)
    for p in range(wl.T):
        t = torch.tensor([[p]], dtype=torch.int32, device="cuda")
        if p % wl.stride == 0:
            B.rkv_append_ref(stream.cfg, stream.cache, kv_dev, t, t)
        else:
            B.rkv_encode(stream.cfg, stream.W, stream.cache, kv_dev, t, t)
    torch.cuda.synchronize()
    for name in ("ref_vals", "ref_pos", "ref_count", "codes", "scale", "zmin", "ref_idx", "self_slot"):
        a = getattr(bulk.cache, name)
        assert torch.equal(a, getattr(stream.cache, name)), name
        assert torch.equal(a, getattr(again.cache, name)), name


# ------------------------------------------------------------------ edge cases


def test_few_token_calls_equal_bulk_batched():
    """Calls with at most 4 tokens per sequence (pool scan, one-wavefront GEMMs) write the
    same records as one bulk call (tiled search and GEMMs), batch of 3, INT4 and INT2, at
    Table I's Qwen2.5-7B codec shape (d_c = 384, d_ff = 3072: 256-wide and narrow quantizer
    tiles) and at d_c = 128 (narrow quantizer tiles alone)."""
    for wid, T, bits, over in ((5, 300, 4, {}), (4, 400, 2, {}), (4, 260, 2, dict(d_ff=3072, d_c=384)),
                               (5, 300, 4, dict(d_c=128))):
        wl = workload(wid, T=T, batch=3, bits=bits, **over)
        W = wl.make_weights()
        _banner(f"few-token calls vs bulk: wid={wid} T={T} B=3 bits={bits}")
        kvs = np.stack([wl.make_kv(seq=b) for b in range(3)])
        bulk = GpuCodec(wl, W)
        kv_dev = bulk.to_dev(kvs)
        bulk.prefill(kv_dev, T)
        small = GpuCodec(wl, W)
        refp = torch.from_numpy(np.tile(wl.ref_positions(), (3, 1))).cuda().contiguous()
        B.rkv_append_ref(small.cfg, small.cache, kv_dev, refp, refp)
        encp = wl.enc_positions()
        for k in range(0, encp.size, 4):
            p = torch.from_numpy(np.tile(encp[k:k + 4], (3, 1)).astype(np.int32)).cuda().contiguous()
            B.rkv_encode(small.cfg, small.W, small.cache, kv_dev, p, p)
        torch.cuda.synchronize()
        assert small.cache.error_bits() == 0
        for name in ("codes", "scale", "zmin", "ref_idx"):
            assert torch.equal(getattr(bulk.cache, name), getattr(small.cache, name)), name


def test_empty_pool_and_range_errors():
    wl = workload(2, T=64)
    W = wl.make_weights()
    gpu = GpuCodec(wl, W, cap_ref=8, cap_tok=64)
    kv = wl.make_kv()
    kv_dev = gpu.to_dev(kv[None])
    # token 3 with an empty pool: no references, zero mean, flagged
    t = torch.tensor([[3]], dtype=torch.int32, device="cuda")
    B.rkv_encode(gpu.cfg, gpu.W, gpu.cache, kv_dev, t, t)
    torch.cuda.synchronize()
    assert gpu.cache.error_bits() & B.DEVERR_EMPTY_POOL
    assert gpu.cache.ref_idx[0, 3].tolist() == [-1] * wl.top_k
    codec = OracleCodec.from_workload(wl, W)
    orc = codec.new_cache(8, 64)
    codec.encode(orc, kv[[3]], [3])
    gpc = mirror_cache(codec, gpu)
    assert_codes_ok(compare_codes(codec, orc, gpc, [3]))
    assert_kv_ok(gpu.decode(np.array([3]))[0], codec.decode_selected(orc, [3]), "empty pool decode")
    # decode of an index outside the cache: zeros and a flag
    gpu.cache.err_word.zero_()
    out = gpu.decode(np.array([1, 64, -5, 3], dtype=np.int32))
    assert np.all(out[0, 1] == 0) and np.all(out[0, 2] == 0)
    assert gpu.cache.error_bits() & B.DEVERR_IDX_RANGE
    # encode at a position outside the records: skipped and flagged
    gpu.cache.err_word.zero_()
    bad = torch.tensor([[70]], dtype=torch.int32, device="cuda")
    row = torch.tensor([[5]], dtype=torch.int32, device="cuda")
    B.rkv_encode(gpu.cfg, gpu.W, gpu.cache, kv_dev, row, bad)
    torch.cuda.synchronize()
    assert gpu.cache.error_bits() & B.DEVERR_POS_RANGE
    # a full pool: the device sees the overflow (the host cannot: the count lives on
    # the device); the slots past capacity are skipped and flagged
    gpu.cache.err_word.zero_()
    r5 = torch.arange(0, 40, 8, dtype=torch.int32, device="cuda")[None]
    B.rkv_append_ref(gpu.cfg, gpu.cache, kv_dev, r5, r5)
    torch.cuda.synchronize()
    assert gpu.cache.error_bits() == 0 and gpu.cache.ref_count.item() == 5
    B.rkv_append_ref(gpu.cfg, gpu.cache, kv_dev, r5 + 1, r5 + 1)
    torch.cuda.synchronize()
    assert gpu.cache.error_bits() & B.DEVERR_REF_CAPACITY
    assert gpu.cache.ref_count.item() == 8
    assert gpu.cache.ref_pos[0].tolist() == [0, 8, 16, 24, 32, 1, 9, 17]


def test_empty_calls_change_nothing():
    """Calls with no tokens (append and encode with n = 0, restore with m = 0) return
    success and leave the cache as it was."""
    wl = workload(2, T=256)
    W = wl.make_weights()
    gpu = GpuCodec(wl, W)
    kv = wl.make_kv()
    kv_dev = gpu.to_dev(kv[None])
    gpu.prefill(kv_dev, wl.T)
    torch.cuda.synchronize()
    names = ("ref_vals", "ref_pos", "ref_norm2", "ref_count", "codes", "scale", "zmin", "ref_idx", "self_slot")
    before = {n: getattr(gpu.cache, n).clone() for n in names}
    none = torch.zeros((1, 0), dtype=torch.int32, device="cuda")
    B.rkv_append_ref(gpu.cfg, gpu.cache, kv_dev, none, none)
    B.rkv_encode(gpu.cfg, gpu.W, gpu.cache, kv_dev, none, none)
    out = gpu.decode(np.zeros((1, 0), dtype=np.int32))
    torch.cuda.synchronize()
    assert out.shape == (1, 0, wl.two_dk)
    assert gpu.cache.error_bits() == 0
    for n in names:
        assert torch.equal(before[n], getattr(gpu.cache, n)), n


# ------------------------------------------------------------------ full sizes, sampled


@pytest.mark.parametrize("wid", [2, 4])
def test_full_size_sampled(wid):
    wl = workload(wid)
    T = wl.T
    W = wl.make_weights()
    _banner(f"full size wid={wid} T={T}: generating")
    kv = wl.make_kv()
    gpu = GpuCodec(wl, W)
    kv_dev = gpu.to_dev(kv[None])
    _banner(f"full size wid={wid}: GPU prefill")
    gpu.prefill(kv_dev, T)
    torch.cuda.synchronize()
    assert gpu.cache.error_bits() == 0
    codec = OracleCodec.from_workload(wl, W)
    orc = codec.new_cache(gpu.cap_ref, T)
    refp = wl.ref_positions()
    codec.append_ref(orc, kv[refp], refp)
    gpc = mirror_cache(codec, gpu)
    assert np.array_equal(gpc.ref_code, orc.ref_code)
    rng = np.random.default_rng([wid, 99])
    enc = wl.enc_positions()
    # 256 tokens: at d_c = 512 that is 131072 codes, enough that the 99.99 % code bar
    # (13 differing codes) is not decided by two or three near-boundary values
    sample = np.unique(np.concatenate([enc[:16], enc[-16:], rng.choice(enc, 224, replace=False)]))
    _banner(f"full size wid={wid}: oracle on {sample.size} sampled tokens")
    codec.encode(orc, kv[sample], sample)
    ties, hard = compare_refsets(lambda p: kv[p], orc, gpc, sample)
    assert not hard, hard
    if ties:
        codec.encode(orc, kv[ties], ties, ref_override={p: gpc.ref_idx[p][gpc.ref_idx[p] >= 0] for p in ties})
    st = compare_codes(codec, orc, gpc, sample)
    print(f"[parity] full wid={wid}: {st} ties={len(ties)}", flush=True)
    assert_codes_ok(st)
    sel = np.sort(np.concatenate([sample, rng.choice(refp, 8, replace=False)]))
    out = gpu.decode(sel[None].astype(np.int32))
    assert_kv_ok(out[0], codec.decode_selected(gpc, sel), "full-size decode on gpu records")
    assert np.array_equal(gpu.decode(sel[None].astype(np.int32), prepared=True), out)
    ma, rr, nd = assert_end_to_end(codec, out[0], orc, gpc, sel, "full-size end to end")
    print(f"[parity] full wid={wid}: end-to-end max_abs={ma:.3g} rms_rel={rr:.3g} code-diff tokens={nd}", flush=True)
