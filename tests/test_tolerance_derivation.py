"""Derivation of the fp16-latent parity bar (quantization off, review page section 2.4).

An fp32 evaluation of z on the CPU (tests/support/fp32_latent_emulation.py, numpy
float32, no GPU code) shows what fp32 arithmetic reaches against the fp64 oracle:
* fewer than 99.99 % of the fp16 latents land within one fp16 ulp of their own value:
  a coordinate near zero has an ulp far below the arithmetic error of the difference
  f_c(kv) - f_c(mean), which is set by the two outputs' magnitude; so a bar of one own
  ulp on 99.99 % of coordinates cannot be met by any fp32 implementation;
* the error before rounding stays below 16 * 2^-24 * (max|f_c(kv)| + max|f_c(mean)|).
The parity bar is therefore one fp16 ulp at the larger of the two latents plus
C * 2^-24 * (max|f_c(kv)| + max|f_c(mean)|) with C = 64, four times the worst the
emulation shows; a planted mistake (the hidden difference rounded to bf16 before W_c3)
fails it on most coordinates. The stored step and minimum of the quantized formats take
the same arithmetic term (2E/(2^b - 1) and E) on top of one storage ulp.
"""

import numpy as np

from support.fp32_latent_emulation import bf16_hidden, emulate, quantized_agreement, summarize
from synth import workload

C_BAR = 64.0


def test_fp32_pipeline_misses_own_ulp_bar_and_meets_derived_bar():
    wl = workload(2, bits=16)
    _, z64, z32, fs = emulate(wl, 700)
    st = summarize(z64, z32, fs, C_BAR)
    print(st)
    assert st["within_own_ulp_frac"] < 0.9999, st
    assert st["max_pre_round_err_over_u_scale"] <= C_BAR / 2, st
    assert st["within_bar_frac"] == 1.0, st


def test_derived_bar_rejects_bf16_hidden():
    wl = workload(2, bits=16)
    _, z64, z32, fs = emulate(wl, 300, hidden_round=bf16_hidden)
    st = summarize(z64, z32, fs, C_BAR)
    print(st)
    assert st["within_bar_frac"] < 0.9, st


def test_qwen_shape_meets_derived_bar():
    wl = workload(4, bits=16)
    _, z64, z32, fs = emulate(wl, 900)
    st = summarize(z64, z32, fs, C_BAR)
    print(st)
    assert st["max_pre_round_err_over_u_scale"] <= C_BAR / 2, st
    assert st["within_bar_frac"] == 1.0, st


def test_stored_step_and_minimum_bars_hold_for_fp32_pipeline():
    # the same arithmetic error carried into the quantizer's stored values: an fp32
    # evaluation keeps step and minimum within one storage ulp + 2E/(2^b - 1), resp. + E,
    # and its codes within the code bar (INT4 / fp16 storage at the Llama shape; INT4 /
    # fp32 storage at the tiny fp32 workload)
    for wl, T, store in ((workload(2), 600, "f16"), (workload(1), 256, "f32")):
        _, z64, z32, fs = emulate(wl, T)
        st = quantized_agreement(z64, z32, fs, wl.bits, store, C_BAR)
        print(wl.name, st)
        assert st["code_exact_frac"] >= 0.9999 and st["code_max_diff"] <= 1, st
        assert st["step_max_bar_ratio"] <= 1.0 and st["zmin_max_bar_ratio"] <= 1.0, st


def test_mean_projection_form_meets_the_same_bars():
    # the encoder's mean-projection form (the mean's pre-activations averaged from the
    # references' own, no rounding of the mean): an fp32 evaluation of it stays within
    # the same derived bars, for the fp16 latent and for the quantized records
    wl = workload(2, bits=16)
    _, z64, z32, fs = emulate(wl, 500, mean_projection=True)
    st = summarize(z64, z32, fs, C_BAR)
    print(st)
    assert st["max_pre_round_err_over_u_scale"] <= C_BAR / 2, st
    assert st["within_bar_frac"] == 1.0, st
    wl = workload(2)
    _, z64, z32, fs = emulate(wl, 500, mean_projection=True)
    st = quantized_agreement(z64, z32, fs, wl.bits, "f16", C_BAR)
    print(st)
    assert st["code_exact_frac"] >= 0.9999 and st["code_max_diff"] <= 1, st
    assert st["step_max_bar_ratio"] <= 1.0 and st["zmin_max_bar_ratio"] <= 1.0, st
