#!/usr/bin/env python3
"""Benchmark of the ResidualKV codec hot path on one MI355X.

One step = one pass of the whole path over the Llama-3.1-8B KV shape (one layer,
batch 1, T = 32768 tokens, 8 KV heads x 128, d_c = 512, d_ff = 1024, INT4 g32,
FP8 references every 8th token):
  rkv_append_ref   4096 reference tokens  (FP8 store)
  rkv_encode       28672 tokens           (search, select + mean, SwiGLU, W_c3 + quantize)
  rkv_decode_selected all 32768 tokens    (dequantize, z W_d + mean, RoPE), bf16 out
Every token is written and restored once per step: value = T / step time.
Inputs (synthetic, seeded) are resident in HBM before the timed region.

Printed: one JSON line with the metric, the dominant kernel's roofline (kernel
time measured with HIP events recorded between the encode's kernels on the
stream they run on) and the CPU oracle timed on a bounded sample on the host.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published peaks (dense): bf16/fp16 MFMA 2.5 PFLOP/s, HBM3E 8 TB/s
PEAK_MFMA_BF16 = 2.5e15
PEAK_HBM = 8.0e12
METRIC = "tokens/s encoded and decoded at Llama-3.1-8B KV shape; % of MFMA/HBM roofline"
PHASES = ("append", "search", "select", "compress", "quantize", "decode")
KERNEL_NAMES = {
    "append": "append_ref_kernel",
    "search": "search_ring_kernel",
    "select": "select_kernel",
    "compress": "swiglu_ring_kernel",
    "quantize": "latent_quant_ring_kernel",
    "decode": "decode_tiles_dl_kernel",
}


def algorithmic_work(wl, n_enc_decoded: int):
    """Algorithmic flops and bytes per launch of each kernel for one step."""
    T, W2, d_ff, d_c, s = wl.T, wl.two_dk, wl.d_ff, wl.d_c, wl.stride
    refp = np.arange(0, T, s)
    encp = np.array([p for p in range(T) if p % s])
    n_ref, n = refp.size, encp.size
    visible = np.searchsorted(refp, encp, side="left")  # references with position < token
    rec = d_c * wl.bits // 8 + (d_c // wl.group) * 4 + wl.top_k * 4
    work = {
        "append": dict(flops=0.0, bytes=n_ref * W2 * (2 + 1)),
        "search": dict(flops=2.0 * W2 * float(visible.sum()), bytes=n * W2 * 2 + n_ref * W2),
        "select": dict(flops=0.0, bytes=n * (W2 * 2 + wl.top_k * W2 + W2 * 2)),
        "compress": dict(flops=2.0 * (2 * n) * W2 * (2 * d_ff), bytes=2 * n * W2 * 2 + 2 * W2 * d_ff * 2 + n * d_ff * 4),
        "quantize": dict(flops=2.0 * n * d_ff * d_c, bytes=n * d_ff * 4 + d_ff * d_c * 2 + n * rec),
        "decode": dict(flops=2.0 * n_enc_decoded * d_c * W2,
                       bytes=T * W2 * 2 + n_enc_decoded * rec + n_ref * W2 + W2 * d_c * 2),
    }
    return work


def roofline(work, ms):
    """Binding roof (the larger time at peak) and the achieved fraction."""
    t = ms * 1e-3
    t_mfma = work["flops"] / PEAK_MFMA_BF16
    t_hbm = work["bytes"] / PEAK_HBM
    if t_mfma >= t_hbm:
        ach = work["flops"] / t / 1e12
        return dict(bound="mfma", achieved=round(ach, 2), peak=PEAK_MFMA_BF16 / 1e12, unit="TFLOP/s",
                    frac=round(ach / (PEAK_MFMA_BF16 / 1e12), 4))
    ach = work["bytes"] / t / 1e9
    return dict(bound="hbm", achieved=round(ach, 1), peak=PEAK_HBM / 1e9, unit="GB/s",
                frac=round(ach / (PEAK_HBM / 1e9), 4))


def source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "kv_cache_compression_residualkv_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they match this source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except Exception:
        return None
    e = d.get(kernel)
    if not e or e.get("source_digest") != source_digest():
        return None
    return e.get("bytes_per_launch")


def cpu_baseline(wl, kv, W, n_enc_sample=96, n_dec_sample=2048):
    """The oracle, untuned, on a bounded sample of the same step; scaled to tokens/s."""
    from oracle import OracleCodec

    try:
        from threadpoolctl import threadpool_info

        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        cores = int(blas[0]["num_threads"]) if blas else 1
    except Exception:
        cores = 1
    codec = OracleCodec.from_workload(wl, W)
    refp = wl.ref_positions()
    encp = wl.enc_positions()
    cache = codec.new_cache(refp.size, wl.T)
    t0 = time.perf_counter()
    codec.append_ref(cache, kv[refp], refp)
    t_app = time.perf_counter() - t0
    sel = encp[np.linspace(0, encp.size - 1, n_enc_sample).astype(np.int64)]
    t0 = time.perf_counter()
    codec.encode(cache, kv[sel], sel)
    t_enc = (time.perf_counter() - t0) / sel.size
    dec = np.unique(np.concatenate([sel, refp[:: max(1, refp.size // 256)]]))[:n_dec_sample]
    t0 = time.perf_counter()
    codec.decode_selected(cache, dec)
    t_dec = (time.perf_counter() - t0) / dec.size
    step = t_app + encp.size * t_enc + wl.T * t_dec
    return dict(
        value=round(wl.T / step, 2),
        unit="tokens/s",
        cores=cores,
        kind="oracle",
        sample=(f"all {refp.size} reference appends, {sel.size} evenly spaced encodes (full causal pool each) "
                f"and {dec.size} restores of one T={wl.T} step; step time = appends + {encp.size} x mean encode "
                f"+ {wl.T} x mean restore; NumPy fp64, BLAS threads = {cores}, elementwise parts single-threaded"),
        seconds=round(t_app + t_enc * sel.size + t_dec * dec.size, 1),
    )


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--select-frac", type=float, default=0.3, help="read fraction for the extra selected-restore rate")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (HBM counter calibration)")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch

        src = torch.ones(args.copy_calibration << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": src.numel() * 4, "launches": 5}))
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the codec runs on one GPU, "
              "see the multi-GPU notes in DESIGN.md)", file=sys.stderr)
        return 2

    import torch

    import kv_cache_compression_residualkv_amd as rkv
    from synth import workload

    dev = "cuda"
    torch.cuda.set_device(0)
    wl = workload(2)
    T, W2 = wl.T, wl.two_dk
    print(f"[bench] generating {wl.name}: T={T} 2dk={W2}", file=sys.stderr, flush=True)
    kv_np = wl.make_kv()
    W = wl.make_weights()
    cfg = rkv.CodecConfig.from_workload(wl)
    weights = rkv.CodecWeights.from_math(W, cfg, dev)
    # the decoder's fp16 copy is prepared once with the weights (rkv_prepare_decoder)
    weights.prepare_decoder(cfg)
    n_ref = (T + wl.stride - 1) // wl.stride
    cache = rkv.CodecCache(cfg, 1, n_ref, T, dev)
    kv = torch.from_numpy(kv_np).to(torch.bfloat16).to(dev)[None].contiguous()
    refp = torch.from_numpy(wl.ref_positions()).to(dev)[None].contiguous()
    encp = torch.from_numpy(wl.enc_positions()).to(dev)[None].contiguous()
    idx_all = torch.arange(T, dtype=torch.int32, device=dev)[None].contiguous()
    sel_np = wl.make_selected(T) if args.select_frac == wl.select_frac else np.sort(
        np.random.default_rng(7).choice(T, int(args.select_frac * T), replace=False)).astype(np.int32)
    idx_sel = torch.from_numpy(sel_np).to(dev)[None].contiguous()
    out = torch.empty((1, T, W2), dtype=torch.bfloat16, device=dev)
    out_sel = torch.empty((1, idx_sel.shape[1], W2), dtype=torch.bfloat16, device=dev)
    ws = torch.empty((rkv.rkv_encode_workspace_bytes(cfg, 1, encp.shape[1], n_ref),), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def new_events():
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(PHASES) + 1)]
        for e in evs:
            e.record(stream)  # create the underlying hipEvent
        return evs

    def step(evs=None):
        cache.ref_count.zero_()
        if evs is not None:
            evs[0].record(stream)
        rkv.rkv_append_ref(cfg, cache, kv, refp, refp, stream=stream)
        enc_events = None if evs is None else [e.cuda_event for e in evs[1:6]]
        rkv.rkv_encode(cfg, weights, cache, kv, encp, encp, ws, stream=stream, events=enc_events)
        rkv.rkv_decode_selected(cfg, weights, cache, idx_all, out=out, stream=stream)
        if evs is not None:
            evs[6].record(stream)

    ev_sets = [new_events() for _ in range(args.steps)]
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert cache.error_bits() == 0, cache.error_bits()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for k in range(args.steps):
        step(ev_sets[k])
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / args.steps
    # per-kernel averages: events[i] .. events[i+1] bracket phase i
    phase_ms = {}
    for i, name in enumerate(PHASES):
        phase_ms[name] = float(np.mean([ev[i].elapsed_time(ev[i + 1]) for ev in ev_sets]))

    # the read path alone on the pages' 30 % attention-compute subset
    sel_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for _ in range(3):
        rkv.rkv_decode_selected(cfg, weights, cache, idx_sel, out=out_sel, stream=stream)
    sel_ev[0].record(stream)
    for _ in range(20):
        rkv.rkv_decode_selected(cfg, weights, cache, idx_sel, out=out_sel, stream=stream)
    sel_ev[1].record(stream)
    torch.cuda.synchronize()
    sel_ms = sel_ev[0].elapsed_time(sel_ev[1]) / 20

    n_enc = int(encp.shape[1])
    work = algorithmic_work(wl, n_enc)
    dominant = max((p for p in PHASES), key=lambda p: phase_ms[p])
    roof = roofline(work[dominant], phase_ms[dominant])
    roof["kernel"] = KERNEL_NAMES[dominant]
    roof["kernel_ms"] = round(phase_ms[dominant], 4)
    roof["work"] = {k: float(v) for k, v in work[dominant].items()}
    tr = measured_traffic(KERNEL_NAMES[dominant])
    roof["traffic"] = tr
    per_kernel = {p: dict(ms=round(phase_ms[p], 4), **{k: v for k, v in roofline(work[p], phase_ms[p]).items()
                                                       if k in ("bound", "achieved", "unit", "frac")})
                  for p in PHASES}

    result = {
        "metric": METRIC,
        "value": round(T / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "llama3.1-8b-kv-prefill-and-restore: one layer, batch 1, T=32768, 8 KV heads x 128 "
                        "(2d_k=2048), d_ff=1024, d_c=512, k=4, INT4 g32 fp16 step/min, FP8 e4m3 refs every 8th "
                        "token; step = append 4096 refs + encode 28672 tokens + restore all 32768 (bf16 out)",
            "T": T, "two_dk": W2, "d_ff": wl.d_ff, "d_c": wl.d_c, "top_k": wl.top_k, "bits": wl.bits,
            "stride": wl.stride, "global_batch": 1, "seq_len": T, "parallelism": "single-gpu",
        },
        "roofline": roof,
        "encode_tok_s": round(n_enc / (sum(phase_ms[p] for p in ("search", "select", "compress", "quantize")) * 1e-3), 1),
        "write_tok_s": round(T / (sum(phase_ms[p] for p in PHASES[:5]) * 1e-3), 1),
        "decode_tok_s": round(T / (phase_ms["decode"] * 1e-3), 1),
        "decode_selected_tok_s": round(idx_sel.shape[1] / (sel_ms * 1e-3), 1),
        "decode_selected_frac": args.select_frac,
        "per_kernel": per_kernel,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(wl, kv_np, W)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
