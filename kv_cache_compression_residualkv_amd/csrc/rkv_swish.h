// Swish (SiLU) of the SwiGLU encoder (ResidualKV review page, section 2.3: the
// compressor's activation), in fp32.
#pragma once

#include <hip/hip_runtime.h>

namespace rkv {

// Swish(a) = a / (1 + e^-a), built from the hardware 2^x and reciprocal:
//  * e^-a = 2^t with t = -a log2(e). log2(e) is held as two fp32 constants L + Lc
//    (the constant split of Cody and Waite's argument reduction), and the rounding
//    error of the product -a L is recovered exactly by an FMA (the FMA form of the exact
//    product, as in Dekker's and Ogita-Rump-Oishi's error-free transformations), so
//    t + tl carries the exponent to about 2^-40 relative. 2^(t + tl) is taken as
//    2^t (v_exp_f32) times the first-order term 1 + tl ln 2 (|tl| < 2^-15).
//  * The quotient a / d, d = 1 + e^-a, starts from the hardware reciprocal r ~ 1/d
//    (v_rcp_f32, about 1 ulp) and takes one correction of the residual,
//    q' = q + (a - q d) r with q = a r (a Newton-Raphson step on the quotient in the
//    form Markstein gives for FMA hardware).
// The error against the exactly rounded Swish is bounded by a test over [-87, 88]
// (tests/test_swish_accuracy_gpu.py). Below a = -87 the value is under 1e-35 in
// magnitude; the argument is clamped there so that 1 + e^-a stays finite.
// Every fused operation is written out and contraction is off, so the function rounds
// the same wherever it is inlined (the kernels and the accuracy probe alike).
__device__ inline float silu(float a) {
#pragma clang fp contract(off)
    a = fmaxf(a, -87.0f);
    const float L = 1.44269502f, Lc = 1.92596299e-8f;
    const float t = -a * L;
    const float tl = fmaf(-a, Lc, fmaf(-a, L, -t));
    const float d = fmaf(__builtin_amdgcn_exp2f(t), fmaf(tl, 0.693147181f, 1.0f), 1.0f);
    const float r = __builtin_amdgcn_rcpf(d);
    const float q = a * r;
    return fmaf(fmaf(-q, d, a), r, q);
}

// One hidden value h = Swish(a) * g, rounded on its own: written as a plain product, the
// compiler may fuse it into the difference h(kv) - h(mean) that follows (an FMA rounds
// only once), so that one side is rounded and the other is not, and a token equal to its
// reference mean would get a nonzero residual. The review page's z = f_c(kv) - f_c(mean)
// (section 2.3) is exactly zero there, and so is this.
__device__ inline float swiglu_h(float a, float g) {
#pragma clang fp contract(off)
    return silu(a) * g;
}

}  // namespace rkv
