"""Host-only checks of the C ABI: librkv loads, exports every declared entry point,
and its argument checks return the documented status without touching a GPU."""

import ctypes
import os
import re

import pytest
import torch

from kv_cache_compression_residualkv_amd import binding as B
from synth import workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rkv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rkv_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from kv_cache_compression_residualkv_amd.build import build

        build()
    return B.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(B.EXPORTED)
    for name in names:
        assert hasattr(lib, name), name
    assert lib.rkv_abi_version() == 4


def test_prepared_decoder_bytes(lib):
    for wid in (2, 4):
        cfg = B.CodecConfig.from_workload(workload(wid))
        assert B.rkv_prepared_decoder_bytes(cfg) == 2 * cfg.two_dk * cfg.d_c
    f32 = B.CodecConfig.from_workload(workload(1))
    assert B.rkv_prepared_decoder_bytes(f32) == 0
    assert lib.rkv_prepare_decoder(ctypes.byref(f32.c_struct()), None, None, None) in (-1, -2)


def test_status_strings(lib):
    for code, text in B.STATUS.items():
        assert lib.rkv_status_string(code).decode() == text
    assert lib.rkv_status_string(-99).decode() == "unknown status"


@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_workload_configs_are_supported(lib, wid):
    cfg = B.CodecConfig.from_workload(workload(wid))
    assert B.rkv_validate_config(cfg) == 0


def test_config_validation(lib):
    base = B.CodecConfig.from_workload(workload(2))
    bad = [
        (dict(n_kv_heads=0), -1),
        (dict(head_dim=-4), -1),
        (dict(head_dim=63), -1),
        (dict(rope_theta=0.0), -1),
        (dict(bits=3), -2),
        (dict(bits=8), -2),
        (dict(top_k=9), -2),
        (dict(group=16), -2),
        (dict(d_c=640), -2),
        (dict(d_c=96), -2),
        (dict(d_c=192), -2),
        (dict(d_ff=1000), -2),
        (dict(head_dim=256, n_kv_heads=4), -2),
        (dict(n_kv_heads=3, head_dim=32), -2),
        (dict(n_kv_heads=4, head_dim=32), -2),
    ]
    for kw, want in bad:
        assert B.rkv_validate_config(B.dataclasses.replace(base, **kw)) == want, kw
    c = base.c_struct()
    c.ref_dtype = B.RKV_BF16  # bf16 references are a valid dtype but not a supported combination
    assert lib.rkv_validate_config(ctypes.byref(c)) == -2
    c = base.c_struct()
    c.kv_dtype = 17
    assert lib.rkv_validate_config(ctypes.byref(c)) == -1
    assert lib.rkv_validate_config(None) == -1


def test_record_bytes(lib):
    rb = B.rkv_record_bytes(B.CodecConfig.from_workload(workload(2)))
    # INT4, d_c = 512: 256 code bytes, 16 groups of fp16 step and min, 4 int32 reference slots
    assert rb == dict(codes=256, scale=32, zmin=32, ref_idx=16, self_slot=4, ref_row=2048)
    rb4 = B.rkv_record_bytes(B.CodecConfig.from_workload(workload(4)))
    assert rb4["codes"] == 64 and rb4["scale"] == 16 and rb4["ref_row"] == 1024
    off = B.CodecConfig.from_workload(workload(5, bits=16))
    assert B.rkv_record_bytes(off)["codes"] == 1024 and B.rkv_record_bytes(off)["scale"] == 0
    tiny = B.rkv_record_bytes(B.CodecConfig.from_workload(workload(1)))
    assert tiny == dict(codes=32, scale=8, zmin=8, ref_idx=16, self_slot=4, ref_row=1024)


def test_workspace_bytes(lib):
    cfg = B.CodecConfig.from_workload(workload(2))
    w = B.rkv_encode_workspace_bytes(cfg, 1, 28672, 4096)
    # at least the mean rows (bf16) and the hidden difference (fp32)
    assert w >= 28672 * (2048 * 2 + 1024 * 4)
    assert w % 256 == 0
    assert B.rkv_encode_workspace_bytes(cfg, 1, 0, 4096) >= 0
    assert B.rkv_encode_workspace_bytes(cfg, 0, 10, 4096) == 0
    assert B.rkv_encode_workspace_bytes(B.dataclasses.replace(cfg, bits=5), 1, 10, 4096) == 0


def test_entry_points_reject_bad_arguments_on_host(lib):
    cfg = B.CodecConfig.from_workload(workload(1))
    c = cfg.c_struct()
    cache = B._Cache()
    # null cache / null config
    assert lib.rkv_append_ref(ctypes.byref(c), None, None, 0, None, None, 1, None) == -1
    assert lib.rkv_append_ref(None, ctypes.byref(cache), None, 0, None, None, 1, None) == -1
    # a cache with capacities but missing arrays
    cache.batch, cache.cap_ref, cache.cap_tok = 1, 8, 8
    assert lib.rkv_encode(ctypes.byref(c), None, ctypes.byref(cache), None, 0, None, None, 1, None, 0, None) == -1
    # fake but aligned addresses: host checks only, nothing is launched
    fake = 1 << 20
    for f in ("ref_vals", "ref_pos", "ref_norm2", "ref_count", "codes", "scale", "zmin", "ref_idx", "self_slot"):
        setattr(cache, f, fake)
    w = B._Weights(fake, fake, fake, fake)
    # the prepared decoder ("bf16" formats only): argument checks; a misaligned prepared
    # copy is refused by the restore
    c2 = B.CodecConfig.from_workload(workload(2)).c_struct()
    assert lib.rkv_prepare_decoder(ctypes.byref(c), ctypes.byref(w), fake, None) == -2
    assert lib.rkv_prepare_decoder(ctypes.byref(c2), None, fake, None) == -1
    assert lib.rkv_prepare_decoder(ctypes.byref(c2), ctypes.byref(w), None, None) == -1
    assert lib.rkv_prepare_decoder(ctypes.byref(c2), ctypes.byref(w), fake + 8, None) == -4
    wp = B._Weights(fake, fake, fake, fake, fake + 8)
    assert lib.rkv_decode_selected(ctypes.byref(c2), ctypes.byref(wp), ctypes.byref(cache), fake, 4, fake, 1, None) == -4
    # negative sizes
    assert lib.rkv_encode(ctypes.byref(c), ctypes.byref(w), ctypes.byref(cache), fake, 4, fake, fake, -1, fake, 1 << 30, None) == -1
    assert lib.rkv_decode_selected(ctypes.byref(c), ctypes.byref(w), ctypes.byref(cache), fake, -2, fake, 0, None) == -1
    # n above capacity
    assert lib.rkv_encode(ctypes.byref(c), ctypes.byref(w), ctypes.byref(cache), fake, 16, fake, fake, 9, fake, 1 << 30, None) == -3
    assert lib.rkv_append_ref(ctypes.byref(c), ctypes.byref(cache), fake, 16, fake, fake, 9, None) == -3
    # missing / small workspace
    assert lib.rkv_encode(ctypes.byref(c), ctypes.byref(w), ctypes.byref(cache), fake, 8, fake, fake, 4, None, 0, None) == -6
    assert lib.rkv_encode(ctypes.byref(c), ctypes.byref(w), ctypes.byref(cache), fake, 8, fake, fake, 4, fake, 16, None) == -6
    # misaligned pointers
    assert lib.rkv_append_ref(ctypes.byref(c), ctypes.byref(cache), fake + 4, 8, fake, fake, 2, None) == -4
    assert lib.rkv_decode_selected(ctypes.byref(c), ctypes.byref(w), ctypes.byref(cache), fake, 3, fake + 2, 0, None) == -4
    cache.codes = fake + 8
    assert lib.rkv_decode_selected(ctypes.byref(c), ctypes.byref(w), ctypes.byref(cache), fake, 3, fake, 0, None) == -4
    cache.codes = fake
    # unsupported output dtype
    assert lib.rkv_decode_selected(ctypes.byref(c), ctypes.byref(w), ctypes.byref(cache), fake, 3, fake, B.RKV_F16, None) == -2
    # empty calls succeed without launching anything
    assert lib.rkv_append_ref(ctypes.byref(c), ctypes.byref(cache), fake, 8, fake, fake, 0, None) == 0
    assert lib.rkv_encode(ctypes.byref(c), ctypes.byref(w), ctypes.byref(cache), fake, 8, fake, fake, 0, None, 0, None) == 0
    assert lib.rkv_decode_selected(ctypes.byref(c), ctypes.byref(w), ctypes.byref(cache), fake, 0, fake, 0, None) == 0


@pytest.mark.parametrize(
    "limit,s0,n_sink,num,den",
    [(262144 - 256, 10, 0, 0, 1), (262144 - 256, 10, 0, 1, 1000), (262144 - 256, 10, 0, 2, 100),
     (262144 - 256, 10, 0, 5, 100), (262144 - 256, 10, 0, 1, 10), (131072, 16, 4, 1, 1000),
     (40, 3, 2, 1, 2), (300, 100, 0, 29, 100), (5, 8, 7, 1, 3), (0, 1, 0, 0, 1), (1, 1, 0, 0, 1),
     (2 ** 31 - 1, 1000000, 0, 1, 1)],
)
def test_reference_schedule_matches_oracle(lib, limit, s0, n_sink, num, den):
    from oracle.schedule import dynamic_reference_positions

    got = B.rkv_reference_schedule(limit, s0, n_sink, num, den)
    want = dynamic_reference_positions(limit, s0, n_sink, f"{num}/{den}")
    assert got.dtype == torch.int32 and got.tolist() == want


def test_reference_schedule_statuses(lib):
    n = ctypes.c_int32(-1)
    buf = (ctypes.c_int32 * 4)()
    assert lib.rkv_reference_schedule(100, 10, 0, 0, 1, None, 0, ctypes.byref(n)) == -3 and n.value == 10
    assert lib.rkv_reference_schedule(100, 10, 0, 0, 1, buf, 4, ctypes.byref(n)) == -3 and n.value == 10
    assert list(buf) == [0, 10, 20, 30]
    assert lib.rkv_reference_schedule(0, 10, 0, 0, 1, None, 0, ctypes.byref(n)) == 0 and n.value == 0
    for args in [(-1, 10, 0, 0, 1), (100, 0, 0, 0, 1), (100, 10, -1, 0, 1), (100, 10, 0, -1, 1), (100, 10, 0, 1, 0)]:
        assert lib.rkv_reference_schedule(*args, None, 0, ctypes.byref(n)) == -1, args
    assert lib.rkv_reference_schedule(100, 10, 0, 0, 1, None, 4, ctypes.byref(n)) == -1
    assert lib.rkv_reference_schedule(100, 10, 0, 0, 1, buf, -1, ctypes.byref(n)) == -1
    assert lib.rkv_reference_schedule(100, 10, 0, 0, 1, buf, 4, None) == -1


def test_decode_attend_host_checks(lib):
    cfg = B.CodecConfig.from_workload(workload(2))
    w = B.rkv_decode_attend_workspace_bytes(cfg, 1, 39321, 32)
    # the fused restore + attention keeps the restored rows on chip: the workspace holds
    # the per-tile partial outputs (308 tiles of 128 tokens x 8 KV heads x 8 query-head
    # slots x (D + 2) floats) and room for the fp16 decoder (2 * 2d_k * d_c bytes)
    up = lambda v: (v + 255) // 256 * 256  # noqa: E731
    tiles = (39321 + 127) // 128
    assert w == up(tiles * 8 * 8 * 128 * 4) + up(tiles * 8 * 8 * 2 * 4) + up(2 * cfg.two_dk * cfg.d_c)
    assert w < 39321 * cfg.two_dk * 2 // 10
    # k = 8 is outside the token-tile restore: the rows go through the workspace
    cfg8 = B.CodecConfig.from_workload(workload(2, top_k=8))
    assert B.rkv_decode_attend_workspace_bytes(cfg8, 1, 39321, 32) >= 39321 * cfg.two_dk * 2
    assert B.rkv_decode_attend_workspace_bytes(cfg, 1, 0, 32) == 0
    assert B.rkv_decode_attend_workspace_bytes(cfg, 1, 100, 30) == 0  # not a multiple of 8 KV heads
    assert B.rkv_decode_attend_workspace_bytes(cfg, 1, 100, 72) == 0  # 9 query heads per KV head
    assert B.rkv_decode_attend_workspace_bytes(B.CodecConfig.from_workload(workload(1)), 1, 100, 4) == 0
    # argument checks run before anything touches a device: an empty cache struct
    empty = B._Cache()
    assert lib.rkv_decode_attend(ctypes.byref(cfg.c_struct()), None, ctypes.byref(empty), None, 4, None, 32,
                                 ctypes.c_float(0.1), None, None, 0, None) == -1


def test_encode_noalloc_host_checks(lib):
    # argument checks before any device work: no configuration, no cache, a bad configuration
    cfg = B.CodecConfig.from_workload(workload(2))
    assert lib.rkv_encode_noalloc(None, None, None, None, 0, None, None, 1, None) == -1
    assert lib.rkv_encode_noalloc(ctypes.byref(cfg.c_struct()), None, None, None, 0, None, None, 1, None) == -1
    bad = cfg.c_struct()
    bad.group = 16
    c = B._Cache()
    c.batch, c.cap_ref, c.cap_tok = 1, 8, 8
    assert lib.rkv_encode_noalloc(ctypes.byref(bad), None, ctypes.byref(c), None, 0, None, None, 1, None) == -2
    # the static scratch bounds the calls it serves
    assert B.RKV_NOALLOC_SCRATCH_BYTES == 16 << 20
    assert B.rkv_encode_workspace_bytes(cfg, 1, 1400, 4096) <= B.RKV_NOALLOC_SCRATCH_BYTES
    assert B.rkv_encode_workspace_bytes(cfg, 1, 4000, 4096) > B.RKV_NOALLOC_SCRATCH_BYTES


def test_mean_projection_flag_host_checks(lib):
    # RKV_FLAG_MEAN_PROJECTION: "bf16" formats only; unknown flag bits are invalid
    cfg = B.CodecConfig.from_workload(workload(2), mean_projection=True)
    assert B.rkv_validate_config(cfg) == 0
    f32 = B.CodecConfig.from_workload(workload(1), mean_projection=True)
    assert B.rkv_validate_config(f32) == -2
    bad = B.CodecConfig.from_workload(workload(2)).c_struct()
    bad.flags = 2
    assert lib.rkv_validate_config(ctypes.byref(bad)) == -1
    # no mean rows in the workspace: smaller by n * 2 d_k bf16 values (up to alignment)
    plain = B.CodecConfig.from_workload(workload(2))
    wp, wq = B.rkv_encode_workspace_bytes(plain, 1, 28672, 4096), B.rkv_encode_workspace_bytes(cfg, 1, 28672, 4096)
    assert wp - wq == 28672 * 2048 * 2
    # the encode needs ref_proj and proj_count, 16-byte aligned, before anything is launched
    fake = 1 << 20
    cache = B._Cache()
    cache.batch, cache.cap_ref, cache.cap_tok = 1, 8, 8
    for f in ("ref_vals", "ref_pos", "ref_norm2", "ref_count", "codes", "scale", "zmin", "ref_idx", "self_slot"):
        setattr(cache, f, fake)
    w = B._Weights(fake, fake, fake, fake)
    c = cfg.c_struct()
    args = (ctypes.byref(c), ctypes.byref(w), ctypes.byref(cache), fake, 4, fake, fake, 2, fake, 1 << 30, None)
    assert lib.rkv_encode(*args) == -1
    cache.ref_proj, cache.proj_count = fake + 8, fake
    assert lib.rkv_encode(*args) == -4
    cache.ref_proj, cache.proj_count = fake, None
    assert lib.rkv_encode(*args) == -1

