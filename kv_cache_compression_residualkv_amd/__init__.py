"""ResidualKV cache codec for AMD MI355X (gfx950).

The codec runs in hand-written HIP kernels behind a C ABI (include/rkv.h,
librkv.so); this package holds the kernels' sources (csrc/), the in-tree build
(build.py) and a thin ctypes binding (binding.py). PyTorch only provides device
memory and streams.
"""

from .binding import (  # noqa: F401
    CodecCache,
    CodecConfig,
    CodecWeights,
    RkvError,
    load_library,
    rkv_abi_version,
    rkv_append_ref,
    rkv_decode_attend,
    rkv_decode_attend_workspace_bytes,
    rkv_decode_selected,
    rkv_encode,
    rkv_encode_noalloc,
    rkv_encode_workspace_bytes,
    rkv_prepared_decoder_bytes,
    rkv_record_bytes,
    rkv_reference_schedule,
    rkv_validate_config,
)
