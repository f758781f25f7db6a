"""Attention over the selected tokens (test infrastructure only, like the rest of the oracle).

ResidualKV review page, section 2.7 (division of labour with sparse attention): a
sparse attention method chooses which history tokens a layer reads, and the codec
restores exactly those; the layer then attends over the restored keys and values.
The page does not restate attention itself; this is textbook scaled dot-product
attention with softmax, for one decoding query per head:

    out_h = sum_j softmax_j(scale * q_h . k_{j, g(h)}) v_{j, g(h)}

over the selected tokens j, with grouped-query heads: query head h reads KV head
g(h) = h // (H_q / N), consecutive query heads sharing one KV head (the layout of
Llama-3.1-8B's 32 query / 8 KV heads and Qwen2.5-7B's 28 / 4).

Readings: the query already carries its rotary embedding (the restored keys carry
theirs, section 2.5); an empty selection gives a zero output.

Parity: pinned by tests/test_oracle_attention.py (single token, identical keys,
two tokens in closed form, permutation invariance, dominance of one score, the
grouped-head mapping).
"""

from __future__ import annotations

import numpy as np


def sparse_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """q [H_q, D]; k, v [m, N, D] (the restored keys and values of the m selected
    tokens); returns [H_q, D] in fp64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Hq, D = q.shape
    m, N, _ = k.shape
    if Hq % N:
        raise ValueError("query heads must be a multiple of the KV heads")
    G = Hq // N
    out = np.zeros((Hq, D))
    if m == 0:
        return out
    for h in range(Hq):
        g = h // G
        s = scale * (k[:, g, :] @ q[h])  # [m]
        w = np.exp(s - s.max())
        out[h] = (w @ v[:, g, :]) / w.sum()
    return out
