"""rkv_encode_noalloc (the encode on the library's static device scratch) against
rkv_encode (caller workspace): bit-identical records on two calls in a row, the second
with fewer tokens, and a clear error for a call larger than the scratch."""

import numpy as np
import pytest
import torch

from kv_cache_compression_residualkv_amd import binding as B
from synth import workload

pytestmark = pytest.mark.gpu

RECORDS = ("codes", "scale", "zmin", "ref_idx", "self_slot", "ref_vals", "ref_pos", "ref_norm2", "ref_count")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    B.load_library()  # raises if librkv.so is missing: no fallback


def _cache(wl):
    cfg = B.CodecConfig.from_workload(wl)
    cap_ref = (wl.T + wl.stride - 1) // wl.stride
    return cfg, B.CodecCache(cfg, wl.batch, cap_ref, wl.T, "cuda")


def test_noalloc_encode_equals_workspace_encode():
    wl = workload(2, T=1300, batch=1)
    W = wl.make_weights()
    kv = torch.from_numpy(wl.make_kv()).to(torch.bfloat16).cuda()[None].contiguous()
    cfg, ref = _cache(wl)
    _, got = _cache(wl)
    weights = B.CodecWeights.from_math(W, cfg, "cuda")
    refp = torch.from_numpy(wl.ref_positions()).cuda()[None]
    enc = wl.enc_positions()
    first = torch.from_numpy(enc[: enc.size - 40]).cuda()[None].contiguous()  # bulk: 1097 tokens
    second = torch.from_numpy(enc[enc.size - 3:]).cuda()[None].contiguous()  # 3 tokens: the pool-scan path
    need = B.rkv_encode_workspace_bytes(cfg, 1, first.shape[1], ref.cap_ref)
    print(f"\n[no-alloc] first call {first.shape[1]} tokens, {need} workspace bytes of "
          f"{B.RKV_NOALLOC_SCRATCH_BYTES}", flush=True)
    assert need <= B.RKV_NOALLOC_SCRATCH_BYTES
    for cache in (ref, got):
        B.rkv_append_ref(cfg, cache, kv, refp, refp)
    for call in (first, second):
        B.rkv_encode(cfg, weights, ref, kv, call, call)
        B.rkv_encode_noalloc(cfg, weights, got, kv, call, call)
        torch.cuda.synchronize()
        for name in RECORDS:
            assert torch.equal(getattr(ref, name), getattr(got, name)), (call.shape, name)
    assert got.error_bits() == 0 and ref.error_bits() == 0
    # every encoded token got at least one reference (k_i = min(k, pool) >= 1 from position 1 on)
    done = torch.cat([first[0], second[0]]).long()
    assert bool((got.ref_idx[0, done, 0] >= 0).all())
    # a call needing more than the scratch is refused before anything runs
    big = torch.from_numpy(np.tile(enc, 4)[:4000].astype(np.int32)).cuda()[None].contiguous()
    wl_big = workload(2, T=4096)
    cfg_b, cache_b = _cache(wl_big)
    assert B.rkv_encode_workspace_bytes(cfg_b, 1, 4000, cache_b.cap_ref) > B.RKV_NOALLOC_SCRATCH_BYTES
    codes_before = cache_b.codes.clone()
    with pytest.raises(B.RkvError) as e:
        B.rkv_encode_noalloc(cfg_b, weights, cache_b, kv, big, big)
    assert e.value.status == -6
    torch.cuda.synchronize()
    assert torch.equal(cache_b.codes, codes_before)
