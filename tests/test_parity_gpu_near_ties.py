"""GPU parity of the reference search on near-duplicate and near-equidistant references.

The search keeps, per pool chunk, the chunk's best 8 candidates by an approximate score
(ResidualKV review page, section 2.2: arg top-k_i of the negative squared distance; ties
go to the lower slot). These cases plant, inside one chunk, twelve identical FP8 rows
and rows one FP8 step apart, tokens equal to them and halfway between them (exact ties
that the lower-slot rule decides), rows at distances graded in slot order, and pairs of
rows whose distances differ by 2^-25 at a distance near 128 (fp32 sums cannot order
them). A chunk list full of equal scores may have dropped a member of the set, so these
tokens take the select step's exact rescan, which the test counts.

Bars: exact ties and graded distances give exactly the oracle's slots; the pairs may
give the other, equally near set (a tie within 1e-5 relative), which the oracle then
re-encodes (ref_override) before the codes are compared; codes, steps and minima, and the
restored K|V, are held to the usual bars. A token equal to its reference mean must store
the zero residual exactly (every group constant).
"""

import numpy as np
import pytest
import torch

from kv_cache_compression_residualkv_amd import binding as B
from oracle import OracleCodec
from parity_util import (
    GpuCodec,
    assert_codes_ok,
    assert_end_to_end,
    compare_codes,
    compare_refsets,
    mirror_cache,
)
from synth import near_tie_kv, workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    B.load_library()  # raises if librkv.so is missing: no fallback


def _banner(msg):
    print(f"\n[parity] {msg}", flush=True)


# (workload id, overrides, first slot of each planted group, first token position)
CASES = {
    # 1100 references: three chunks of 512 slots in the tiled search; the groups sit in
    # different chunks
    "llama-shape": (2, dict(T=2200, stride=2), {"dup": 600, "graded": 40, "pairs": 1030}, 2110),
    "qwen-shape-int2": (4, dict(T=2200, stride=2), {"dup": 300, "graded": 700, "pairs": 1040}, 2110),
    # fp32 formats: the register-staged search, 128-slot blocks
    "tiny-fp32": (1, dict(T=1200, stride=2), {"dup": 100, "graded": 300, "pairs": 520}, 1110),
}


def _run(case, few_token):
    wid, over, slots, tok_start = CASES[case]
    wl = workload(wid, **over)
    T = wl.T
    W = wl.make_weights()
    planted = near_tie_kv(wl.make_kv(), wl.stride, slots, tok_start, np.random.default_rng(wid))
    kv = planted.kv
    _banner(f"near ties {case}: T={T} stride={wl.stride} 2dk={wl.two_dk} few_token={few_token}")
    gpu = GpuCodec(wl, W)
    kv_dev = gpu.to_dev(kv[None])
    gpu.prefill(kv_dev, T)
    special = np.concatenate([planted.exact_tokens, planted.graded_tokens, planted.below_fp32_tokens])
    if few_token:
        # encode the planted tokens again, at most 4 per call: the pool scan path
        gpu.cache.stats.zero_()
        for i in range(0, special.size, 3):
            p = torch.from_numpy(special[i:i + 3].astype(np.int32)).cuda()[None]
            B.rkv_encode(gpu.cfg, gpu.W, gpu.cache, kv_dev, p, p)
    torch.cuda.synchronize()
    assert gpu.cache.error_bits() == 0
    stats = gpu.cache.encode_stats()
    print(f"[parity] {case}: encode stats {stats}", flush=True)

    codec = OracleCodec.from_workload(wl, W)
    orc = codec.new_cache(gpu.cap_ref, T)
    refp = wl.ref_positions()
    codec.append_ref(orc, kv[refp], refp)
    rng = np.random.default_rng(11)
    others = np.sort(rng.choice(wl.enc_positions()[wl.enc_positions() < tok_start], 48, replace=False))
    sample = np.concatenate([special, others])
    codec.encode(orc, kv[sample], sample)
    gpc = mirror_cache(codec, gpu)
    kv_of = lambda p: kv[p].astype(np.float64)  # noqa: E731
    ties, hard = compare_refsets(kv_of, orc, gpc, sample)
    print(f"[parity] {case}: {len(ties)} ties {ties}, hard {hard}", flush=True)
    assert not hard, hard
    # exact ties and graded distances: exactly the oracle's slots (lower-slot rule)
    for p in np.concatenate([planted.exact_tokens, planted.graded_tokens]):
        assert np.array_equal(orc.ref_idx[p], gpc.ref_idx[p]), (p, orc.ref_idx[p], gpc.ref_idx[p])
    # the pairs below fp32's resolution: the GPU may take the lower slot of the pair,
    # which is a tie; at least one does, so the re-encode path below runs
    assert set(ties) <= set(planted.below_fp32_tokens.tolist()), ties
    assert len(ties) >= 1
    # a chunk list full of equal scores sends its token to the exact rescan
    assert stats["exact_rescan"] >= 1, stats
    if ties:
        codec.encode(orc, kv[ties], ties, ref_override={p: gpc.ref_idx[p][gpc.ref_idx[p] >= 0] for p in ties})
        for p in ties:
            assert np.array_equal(orc.ref_idx[p], gpc.ref_idx[p])
    # a token equal to its reference mean has z = 0 (section 2.3 boxed equation): every
    # group constant, stored step and minimum 0, codes 0, exactly as the oracle has it
    for p in planted.exact_tokens[:4]:
        assert np.all(orc.z[p] == 0.0)
        if codec.bits == 16:
            assert np.all(gpc.latent[p] == 0.0), p
        else:
            assert np.all(gpc.q[p] == 0) and np.all(gpc.step[p] == 0.0) and np.all(gpc.zmin[p] == 0.0), (
                p, gpc.step[p], gpc.zmin[p])
    st = compare_codes(codec, orc, gpc, sample)
    print(f"[parity] {case}: codes {st}", flush=True)
    if codec.bits != 16:
        for p in sample:
            d = np.abs(orc.q[p].astype(int) - gpc.q[p].astype(int))
            if d.any():
                print(f"[parity] {case}: token {p} codes differ at {int((d > 0).sum())} coordinates (max {d.max()}), "
                      f"ref_idx {gpc.ref_idx[p].tolist()}, step ulps "
                      f"{float(np.max(np.abs(orc.step[p] - gpc.step[p]) / np.maximum(orc.step[p], 1e-30))):.3g}",
                      flush=True)
    assert_codes_ok(st)
    out = gpu.decode(sample[None].astype(np.int32))[0]
    ma, rr, nd = assert_end_to_end(codec, out, orc, gpc, sample, case)
    print(f"[parity] {case}: restore max_abs={ma:.3g} rms_rel={rr:.3g} differing records={nd}", flush=True)


@pytest.mark.parametrize("case", list(CASES))
def test_near_ties_bulk(case):
    _run(case, few_token=False)


@pytest.mark.parametrize("case", ["llama-shape", "qwen-shape-int2"])
def test_near_ties_few_token(case):
    _run(case, few_token=True)
