"""Seeded synthetic inputs for the ResidualKV codec.

This package is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark. It holds none of the codec's arithmetic: it only draws random numbers
and casts inputs to the dtype they arrive in (the backbone's KV and the codec
weights). Everything the codec computes from these inputs lives elsewhere.

Workload shapes follow the ResidualKV review page ("ResidualKV: 基于参考向量与残差的
KV Cache 压缩"): the joint pre-RoPE K|V vector of width 2*d_k = 2*N*D (section 2.1),
a fixed reference stride (section 2.6), k = 4 (section 2.2), group size 32
(section 2.4) and a 30 % attention-compute ratio (section 3.3, Table III).
"""

from .generators import (  # noqa: F401
    WorkloadConfig,
    clustered_kv,
    codec_weights,
    selected_subset,
    workload,
    WORKLOADS,
    NearTieCase,
    near_tie_kv,
)
