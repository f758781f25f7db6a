"""CPU oracle for the ResidualKV cache codec (test infrastructure only).

A plain, slow, obviously correct NumPy implementation of what the codec computes,
written from the ResidualKV review page ("ResidualKV: 基于参考向量与残差的 KV Cache
压缩", arXiv 2602.08005v2 review). Floating point is fp64 except at the storage
points the method defines (FP8 references, fp16 scale/min, fp16 latent) and at
the points where floating point decides an integer (the quantization code), which
are taken in fp32, the precision of the GPU kernels.

Only the tests, the package's smoke check and the benchmark's CPU-baseline leg may
import this package. The GPU product path never calls it, and it shares no code
with the HIP kernels; the only thing both sides share is the seeded input
generator package `synth`, which holds none of the codec's arithmetic.

Parity status: every function here is pinned by tests/test_oracle_pins.py against
values the pages print, closed forms, invariants and brute force. The composed
pipeline on real model data is "parity unpinned": the pages print no worked
z, codes or restored K/V, and no trained codec is available.
"""

from .formats import (  # noqa: F401
    FP8_E4M3FN_VALUES,
    fp8_e4m3fn_decode,
    fp8_e4m3fn_encode,
    bf16_round,
    fp16_round,
    pack_codes,
    unpack_codes,
)
from .codec import (  # noqa: F401
    OracleCodec,
    OracleCache,
    swiglu_compressor,
    linear_decoder,
    group_quantize,
    group_dequantize,
    rope_rotate,
    topk_references,
    reference_mean32,
    rope_inv_freq,
    keep_ratio,
    group_storage_ratio,
)
