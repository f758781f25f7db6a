"""Thin ctypes binding of librkv (include/rkv.h).

Argument marshalling only: torch tensors supply device memory and the current
stream; every step of the codec runs in the HIP kernels behind the C ABI. There
is no fallback: if librkv.so is missing or a call fails, an exception is raised.

The functions keep the C names (rkv_append_ref, rkv_encode, rkv_decode_selected,
...). The helper classes build the C structs from torch tensors:

* CodecConfig  -> rkv_config
* CodecWeights -> rkv_weights (nn.Linear layout [out, in], contiguous, on the GPU)
* CodecCache   -> rkv_cache (allocates the caller-owned cache arrays with torch)
"""

from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Dict, Optional

import torch

from .build import LIB_PATH

RKV_F32, RKV_BF16, RKV_F16, RKV_FP8_E4M3 = 0, 1, 2, 3
STATUS = {
    0: "ok",
    -1: "invalid argument",
    -2: "unsupported configuration",
    -3: "capacity exceeded",
    -4: "pointer not 16-byte aligned",
    -5: "HIP runtime error",
    -6: "workspace missing or too small",
}
RKV_ENCODE_PHASES = 4
RKV_STATS_WORDS = 2
RKV_NOALLOC_SCRATCH_BYTES = 16 << 20
ABI_VERSION = 4
RKV_FLAG_MEAN_PROJECTION = 1
DEVERR_EMPTY_POOL, DEVERR_POS_RANGE, DEVERR_REF_CAPACITY, DEVERR_IDX_RANGE, DEVERR_ROW_RANGE = 1, 2, 4, 8, 16

EXPORTED = (
    "rkv_abi_version",
    "rkv_status_string",
    "rkv_validate_config",
    "rkv_record_bytes",
    "rkv_encode_workspace_bytes",
    "rkv_reference_schedule",
    "rkv_append_ref",
    "rkv_encode",
    "rkv_encode_ex",
    "rkv_encode_noalloc",
    "rkv_decode_selected",
    "rkv_decode_attend_workspace_bytes",
    "rkv_decode_attend",
    "rkv_prepared_decoder_bytes",
    "rkv_prepare_decoder",
)


class RkvError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS.get(status, 'unknown')} ({status})")
        self.status = status


class _Config(ctypes.Structure):
    _fields_ = [
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("d_ff", ctypes.c_int32),
        ("d_c", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("bits", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("ref_dtype", ctypes.c_int32),
        ("scale_dtype", ctypes.c_int32),
        ("weight_dtype", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("rope_theta", ctypes.c_double),
    ]


class _Weights(ctypes.Structure):
    _fields_ = [("w_c1", ctypes.c_void_p), ("w_c2", ctypes.c_void_p), ("w_c3", ctypes.c_void_p), ("w_d", ctypes.c_void_p),
                ("w_d_f16", ctypes.c_void_p)]


class _Cache(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("cap_ref", ctypes.c_int32),
        ("cap_tok", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("ref_vals", ctypes.c_void_p),
        ("ref_pos", ctypes.c_void_p),
        ("ref_norm2", ctypes.c_void_p),
        ("ref_count", ctypes.c_void_p),
        ("codes", ctypes.c_void_p),
        ("scale", ctypes.c_void_p),
        ("zmin", ctypes.c_void_p),
        ("ref_idx", ctypes.c_void_p),
        ("self_slot", ctypes.c_void_p),
        ("err_word", ctypes.c_void_p),
        ("stats", ctypes.c_void_p),
        ("ref_proj", ctypes.c_void_p),
        ("proj_count", ctypes.c_void_p),
    ]


_LIB: Optional[ctypes.CDLL] = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load librkv.so (built in-tree by build.py); raises if it is missing."""
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build the HIP library first (__graft_entry__.build())")
    lib = ctypes.CDLL(p)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    cfg_p, w_p, c_p = ctypes.POINTER(_Config), ctypes.POINTER(_Weights), ctypes.POINTER(_Cache)
    lib.rkv_abi_version.restype = i32
    lib.rkv_status_string.restype = ctypes.c_char_p
    lib.rkv_status_string.argtypes = [ctypes.c_int]
    lib.rkv_validate_config.restype = ctypes.c_int
    lib.rkv_validate_config.argtypes = [cfg_p]
    lib.rkv_record_bytes.restype = ctypes.c_int
    lib.rkv_record_bytes.argtypes = [cfg_p, ctypes.POINTER(sz)]
    lib.rkv_encode_workspace_bytes.restype = sz
    lib.rkv_encode_workspace_bytes.argtypes = [cfg_p, i32, i32, i32]
    lib.rkv_reference_schedule.restype = ctypes.c_int
    lib.rkv_reference_schedule.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(i32), i32, ctypes.POINTER(i32)]
    lib.rkv_append_ref.restype = ctypes.c_int
    lib.rkv_append_ref.argtypes = [cfg_p, c_p, vp, i32, vp, vp, i32, vp]
    lib.rkv_encode.restype = ctypes.c_int
    lib.rkv_encode.argtypes = [cfg_p, w_p, c_p, vp, i32, vp, vp, i32, vp, sz, vp]
    lib.rkv_encode_ex.restype = ctypes.c_int
    lib.rkv_encode_ex.argtypes = [cfg_p, w_p, c_p, vp, i32, vp, vp, i32, vp, sz, vp, ctypes.POINTER(vp)]
    lib.rkv_encode_noalloc.restype = ctypes.c_int
    lib.rkv_encode_noalloc.argtypes = [cfg_p, w_p, c_p, vp, i32, vp, vp, i32, vp]
    lib.rkv_decode_selected.restype = ctypes.c_int
    lib.rkv_decode_selected.argtypes = [cfg_p, w_p, c_p, vp, i32, vp, i32, vp]
    lib.rkv_decode_attend_workspace_bytes.restype = sz
    lib.rkv_decode_attend_workspace_bytes.argtypes = [cfg_p, i32, i32, i32]
    lib.rkv_decode_attend.restype = ctypes.c_int
    lib.rkv_decode_attend.argtypes = [cfg_p, w_p, c_p, vp, i32, vp, i32, ctypes.c_float, vp, vp, sz, vp]
    lib.rkv_prepared_decoder_bytes.restype = sz
    lib.rkv_prepared_decoder_bytes.argtypes = [cfg_p]
    lib.rkv_prepare_decoder.restype = ctypes.c_int
    lib.rkv_prepare_decoder.argtypes = [cfg_p, w_p, vp, vp]
    if path is None:
        _LIB = lib
    return lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise RkvError(fn, status)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to librkv must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


# ------------------------------------------------------------------------------ config


@dataclasses.dataclass(frozen=True)
class CodecConfig:
    n_kv_heads: int
    head_dim: int
    d_ff: int
    d_c: int
    top_k: int = 4
    bits: int = 4
    group: int = 32
    mode: str = "bf16"  # 'bf16': bf16 KV/weights, FP8 refs, fp16 scale/min; 'f32': all fp32
    rope_theta: float = 1.0e4
    mean_projection: bool = False  # RKV_FLAG_MEAN_PROJECTION

    @classmethod
    def from_workload(cls, w, mean_projection: bool = False) -> "CodecConfig":
        return cls(w.n_kv_heads, w.head_dim, w.d_ff, w.d_c, w.top_k, w.bits, w.group, w.mode, w.rope_theta,
                   mean_projection)

    @property
    def two_dk(self) -> int:
        return 2 * self.n_kv_heads * self.head_dim

    @property
    def kv_torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.mode == "f32" else torch.bfloat16

    @property
    def ref_torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.mode == "f32" else torch.uint8

    @property
    def scale_torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.mode == "f32" else torch.float16

    def c_struct(self) -> _Config:
        f32 = self.mode == "f32"
        return _Config(
            self.n_kv_heads, self.head_dim, self.d_ff, self.d_c, self.top_k, self.bits, self.group,
            RKV_F32 if f32 else RKV_BF16,
            RKV_F32 if f32 else RKV_FP8_E4M3,
            RKV_F32 if f32 else RKV_F16,
            RKV_F32 if f32 else RKV_BF16,
            RKV_FLAG_MEAN_PROJECTION if self.mean_projection else 0,
            float(self.rope_theta),
        )


def rkv_abi_version() -> int:
    return int(load_library().rkv_abi_version())


def rkv_validate_config(cfg: CodecConfig) -> int:
    return int(load_library().rkv_validate_config(ctypes.byref(cfg.c_struct())))


def rkv_record_bytes(cfg: CodecConfig) -> Dict[str, int]:
    out = (ctypes.c_size_t * 6)()
    _check("rkv_record_bytes", load_library().rkv_record_bytes(ctypes.byref(cfg.c_struct()), out))
    return dict(zip(("codes", "scale", "zmin", "ref_idx", "self_slot", "ref_row"), (int(v) for v in out)))


def rkv_encode_workspace_bytes(cfg: CodecConfig, batch: int, n: int, cap_ref: int) -> int:
    return int(load_library().rkv_encode_workspace_bytes(ctypes.byref(cfg.c_struct()), batch, n, cap_ref))


def rkv_reference_schedule(limit: int, s0: int, n_sink: int, alpha_num: int, alpha_den: int) -> torch.Tensor:
    """Reference positions of the dynamic stride (host int32 tensor, ascending)."""
    lib = load_library()
    count = ctypes.c_int32(0)
    st = lib.rkv_reference_schedule(limit, s0, n_sink, alpha_num, alpha_den, None, 0, ctypes.byref(count))
    if st not in (0, -3):
        _check("rkv_reference_schedule", st)
    out = torch.empty(count.value, dtype=torch.int32)
    buf = ctypes.cast(out.data_ptr(), ctypes.POINTER(ctypes.c_int32)) if count.value else None
    _check("rkv_reference_schedule",
           lib.rkv_reference_schedule(limit, s0, n_sink, alpha_num, alpha_den, buf, count.value, ctypes.byref(count)))
    return out


def rkv_prepared_decoder_bytes(cfg: CodecConfig) -> int:
    return int(load_library().rkv_prepared_decoder_bytes(ctypes.byref(cfg.c_struct())))


# ------------------------------------------------------------------------------ weights / cache


class CodecWeights:
    """Codec weights on the GPU in nn.Linear layout ([out, in]).

    from_math() takes the pages' math layout (x @ W, W [in, out]) and transposes."""

    def __init__(self, w_c1: torch.Tensor, w_c2: torch.Tensor, w_c3: torch.Tensor, w_d: torch.Tensor):
        self.w_c1, self.w_c2, self.w_c3, self.w_d = (t.contiguous() for t in (w_c1, w_c2, w_c3, w_d))
        self.w_d_f16: Optional[torch.Tensor] = None
        self._c = _Weights(_ptr(self.w_c1), _ptr(self.w_c2), _ptr(self.w_c3), _ptr(self.w_d), None)

    def prepare_decoder(self, cfg: "CodecConfig", stream=None) -> "CodecWeights":
        """Fill the optional prepared decoder (rkv_prepare_decoder) and use it from now on."""
        n = rkv_prepared_decoder_bytes(cfg)
        if n == 0:
            raise RkvError("rkv_prepare_decoder", -2)
        buf = torch.empty((n,), dtype=torch.uint8, device=self.w_d.device)
        _check("rkv_prepare_decoder", load_library().rkv_prepare_decoder(
            ctypes.byref(cfg.c_struct()), ctypes.byref(self._c), _ptr(buf), _stream(stream)))
        self.w_d_f16 = buf
        self._c.w_d_f16 = _ptr(buf)
        return self

    def drop_prepared_decoder(self) -> None:
        self.w_d_f16 = None
        self._c.w_d_f16 = None

    @classmethod
    def from_math(cls, W: Dict, cfg: CodecConfig, device="cuda") -> "CodecWeights":
        dt = cfg.kv_torch_dtype

        def tr(a):
            return torch.as_tensor(a).to(torch.float32).t().contiguous().to(dt).to(device)

        return cls(tr(W["Wc1"]), tr(W["Wc2"]), tr(W["Wc3"]), tr(W["Wd"]))


class CodecCache:
    """Caller-owned cache arrays of one layer (torch tensors) + the rkv_cache struct."""

    def __init__(self, cfg: CodecConfig, batch: int, cap_ref: int, cap_tok: int, device="cuda",
                 err_word: bool = True, stats: bool = True):
        rb = rkv_record_bytes(cfg)
        self.cfg, self.batch, self.cap_ref, self.cap_tok = cfg, batch, cap_ref, cap_tok
        W2 = cfg.two_dk
        G = cfg.d_c // cfg.group
        self.ref_vals = torch.zeros((batch, cap_ref, W2), dtype=cfg.ref_torch_dtype, device=device)
        self.ref_pos = torch.full((batch, cap_ref), -1, dtype=torch.int32, device=device)
        self.ref_norm2 = torch.zeros((batch, cap_ref), dtype=torch.float32, device=device)
        self.ref_count = torch.zeros((batch,), dtype=torch.int32, device=device)
        self.codes = torch.zeros((batch, cap_tok, rb["codes"]), dtype=torch.uint8, device=device)
        self.scale = torch.zeros((batch, cap_tok, G), dtype=cfg.scale_torch_dtype, device=device)
        self.zmin = torch.zeros_like(self.scale)
        self.ref_idx = torch.full((batch, cap_tok, cfg.top_k), -1, dtype=torch.int32, device=device)
        self.self_slot = torch.full((batch, cap_tok), -1, dtype=torch.int32, device=device)
        self.err_word = torch.zeros((1,), dtype=torch.int32, device=device) if err_word else None
        self.stats = torch.zeros((RKV_STATS_WORDS,), dtype=torch.int32, device=device) if stats else None
        # the mean-projection form's per-reference projections and their count
        self.ref_proj = (torch.zeros((batch, cap_ref, cfg.d_ff, 2), dtype=torch.float32, device=device)
                         if cfg.mean_projection else None)
        self.proj_count = torch.zeros((batch,), dtype=torch.int32, device=device) if cfg.mean_projection else None
        self._c = _Cache(
            batch, cap_ref, cap_tok, 0,
            _ptr(self.ref_vals), _ptr(self.ref_pos), _ptr(self.ref_norm2), _ptr(self.ref_count),
            _ptr(self.codes), _ptr(self.scale), _ptr(self.zmin), _ptr(self.ref_idx), _ptr(self.self_slot),
            _ptr(self.err_word), _ptr(self.stats), _ptr(self.ref_proj), _ptr(self.proj_count),
        )

    def error_bits(self) -> int:
        return int(self.err_word.item()) if self.err_word is not None else 0

    def encode_stats(self) -> Dict[str, int]:
        """The encode's counters (rkv_cache.stats): tokens whose set boundary needed exact
        distances, and tokens re-searched exactly over whole pool chunks."""
        if self.stats is None:
            return {"exact_boundary": 0, "exact_rescan": 0}
        v = self.stats.cpu().tolist()
        return {"exact_boundary": int(v[0]), "exact_rescan": int(v[1])}


# ------------------------------------------------------------------------------ entry points


def _rows_pos(kv: torch.Tensor, rows: torch.Tensor, pos: torch.Tensor, batch: int):
    if kv.dim() == 2:
        kv = kv.unsqueeze(0)
    rows = rows.reshape(batch, -1).to(torch.int32).contiguous()
    pos = pos.reshape(batch, -1).to(torch.int32).contiguous()
    if rows.shape != pos.shape:
        raise ValueError("rows and pos must have the same shape")
    return kv.contiguous(), rows, pos


def rkv_append_ref(cfg: CodecConfig, cache: CodecCache, kv: torch.Tensor, rows: torch.Tensor, pos: torch.Tensor,
                   stream=None) -> None:
    """Append tokens to the reference pool. kv [B, L, 2dk]; rows/pos [B, n] int32 on the GPU."""
    kv, rows, pos = _rows_pos(kv, rows, pos, cache.batch)
    st = load_library().rkv_append_ref(ctypes.byref(cfg.c_struct()), ctypes.byref(cache._c), _ptr(kv), kv.shape[1],
                                       _ptr(rows), _ptr(pos), rows.shape[1], _stream(stream))
    _check("rkv_append_ref", st)


def rkv_encode(cfg: CodecConfig, weights: CodecWeights, cache: CodecCache, kv: torch.Tensor, rows: torch.Tensor,
               pos: torch.Tensor, workspace: Optional[torch.Tensor] = None, stream=None, events=None) -> torch.Tensor:
    """Encode tokens into residual records. Returns the workspace used (allocated if None).

    events: optional sequence of RKV_ENCODE_PHASES + 1 raw hipEvent_t handles (ints, or
    None to skip that mark); when given, rkv_encode_ex records them between the encode's
    kernels."""
    kv, rows, pos = _rows_pos(kv, rows, pos, cache.batch)
    n = rows.shape[1]
    need = rkv_encode_workspace_bytes(cfg, cache.batch, n, cache.cap_ref)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=kv.device)
    lib = load_library()
    args = (ctypes.byref(cfg.c_struct()), ctypes.byref(weights._c), ctypes.byref(cache._c), _ptr(kv), kv.shape[1],
            _ptr(rows), _ptr(pos), n, _ptr(workspace), workspace.numel(), _stream(stream))
    if events is None:
        _check("rkv_encode", lib.rkv_encode(*args))
    else:
        if len(events) != RKV_ENCODE_PHASES + 1:
            raise ValueError(f"need {RKV_ENCODE_PHASES + 1} events")
        arr = (ctypes.c_void_p * len(events))(*events)
        _check("rkv_encode_ex", lib.rkv_encode_ex(*args, arr))
    return workspace


def rkv_encode_noalloc(cfg: CodecConfig, weights: CodecWeights, cache: CodecCache, kv: torch.Tensor,
                       rows: torch.Tensor, pos: torch.Tensor, stream=None) -> None:
    """rkv_encode with the library's static device scratch instead of a workspace (no
    allocation by the library; the argument tensors are the caller's)."""
    kv, rows, pos = _rows_pos(kv, rows, pos, cache.batch)
    st = load_library().rkv_encode_noalloc(ctypes.byref(cfg.c_struct()), ctypes.byref(weights._c),
                                           ctypes.byref(cache._c), _ptr(kv), kv.shape[1], _ptr(rows), _ptr(pos),
                                           rows.shape[1], _stream(stream))
    _check("rkv_encode_noalloc", st)


def rkv_decode_selected(cfg: CodecConfig, weights: CodecWeights, cache: CodecCache, idx: torch.Tensor,
                        out: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.float32,
                        stream=None) -> torch.Tensor:
    """Restore selected tokens. idx [B, m] int32 on the GPU; returns out [B, m, 2dk]."""
    idx = idx.reshape(cache.batch, -1).to(torch.int32).contiguous()
    m = idx.shape[1]
    if out is None:
        out = torch.empty((cache.batch, m, cfg.two_dk), dtype=out_dtype, device=idx.device)
    odt = RKV_F32 if out.dtype == torch.float32 else RKV_BF16
    st = load_library().rkv_decode_selected(ctypes.byref(cfg.c_struct()), ctypes.byref(weights._c),
                                            ctypes.byref(cache._c), _ptr(idx), m, _ptr(out), odt, _stream(stream))
    _check("rkv_decode_selected", st)
    return out


def rkv_decode_attend_workspace_bytes(cfg: CodecConfig, batch: int, m: int, n_q_heads: int) -> int:
    return int(load_library().rkv_decode_attend_workspace_bytes(ctypes.byref(cfg.c_struct()), batch, m, n_q_heads))


def rkv_decode_attend(cfg: CodecConfig, weights: CodecWeights, cache: CodecCache, idx: torch.Tensor,
                      q: torch.Tensor, scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, stream=None):
    """Attention of q [B, H_q, D] (bf16, on the GPU) over the restored tokens idx [B, m].
    Returns (out [B, H_q, D] fp32, the workspace used)."""
    idx = idx.reshape(cache.batch, -1).to(torch.int32).contiguous()
    m = idx.shape[1]
    q = q.contiguous()
    hq = q.shape[1]
    if scale is None:
        scale = 1.0 / float(cfg.head_dim) ** 0.5
    if out is None:
        out = torch.empty((cache.batch, hq, cfg.head_dim), dtype=torch.float32, device=q.device)
    need = rkv_decode_attend_workspace_bytes(cfg, cache.batch, m, hq)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=q.device)
    st = load_library().rkv_decode_attend(ctypes.byref(cfg.c_struct()), ctypes.byref(weights._c),
                                          ctypes.byref(cache._c), _ptr(idx), m, _ptr(q), hq, float(scale), _ptr(out),
                                          _ptr(workspace), workspace.numel(), _stream(stream))
    _check("rkv_decode_attend", st)
    return out, workspace
