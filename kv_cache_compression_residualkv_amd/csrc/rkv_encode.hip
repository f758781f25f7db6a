// SwiGLU residual encoder and per-token group quantizer.
//
// ResidualKV review page, section 2.3: f_c(x) = (Swish(x W_c1) * x W_c2) W_c3 and the
// stored residual is z = f_c(kv_i) - f_c(mean_i) (average first, then encode);
// section 2.4: per-token groups of 32 latent coordinates with
// Delta = (max - min)/(2^b - 1), q = round((z - min)/Delta).
//
// Since W_c3 is linear, z = (h(kv_i) - h(mean_i)) W_c3 with h(x) = Swish(x W_c1) * x W_c2.
//   swiglu_kernel       rows of a tile alternate kv_i / mean_i of the same token, so
//                       the epilogue holds h of both in one lane and writes
//                       dH = h(kv_i) - h(mean_i) in fp32 (one row per token).
//   latent_quant_kernel z = dH W_c3. dH is split into three bf16 terms
//                       (hi + mid + lo carries 24 significant bits), each multiplied
//                       by the bf16 W_c3 on MFMA; the epilogue reduces each group's
//                       min/max across the 16 lanes that hold it, stores Delta and
//                       min, and packs the codes.
#include <float.h>

#include "rkv_device.h"
#include "rkv_internal.h"

namespace rkv {

namespace {

constexpr int kThreads = 256;
constexpr int kKC = 64;

// ---------------------------------------------------------------- GEMM 1
// tile: 128 rows (64 tokens x {kv, mean}) x 128 columns (64 of W_c1 and the same 64 of
// W_c2). Waves in a 2 x 2 layout: wave (wm, wn) owns rows [64 wm, +64) and W_c1/W_c2
// columns [32 wn, +32); its 4 x 4 MFMA tiles are (row tile) x (c1, c1, c2, c2).
constexpr int kBM1 = 128;
constexpr int kBN1 = 128;

template <typename T>
struct Gemm1Smem {
    static constexpr int P = Pitch<T, kKC>::value;
    static constexpr size_t bytes = (size_t)(kBM1 + kBN1) * P * sizeof(T);
};

// copy 32 elements (compute type == storage type here)
template <typename T>
struct Copy32 {
    static constexpr int kWords = 32 * (int)sizeof(T) / 16;
    uint4 w[kWords];
    __device__ inline void load(const T* p) {
#pragma unroll
        for (int i = 0; i < kWords; ++i) w[i] = reinterpret_cast<const uint4*>(p)[i];
    }
    __device__ inline void zero() {
#pragma unroll
        for (int i = 0; i < kWords; ++i) w[i] = make_uint4(0, 0, 0, 0);
    }
    __device__ inline void store(T* p) const {
#pragma unroll
        for (int i = 0; i < kWords; ++i) reinterpret_cast<uint4*>(p)[i] = w[i];
    }
};

__device__ inline float silu(float a) { return a / (1.0f + expf(-a)); }

template <typename T>
__global__ __launch_bounds__(kThreads) void swiglu_kernel(const T* __restrict__ kv, int kv_len,
                                                          const int* __restrict__ rows, int n,
                                                          const T* __restrict__ xbar, const T* __restrict__ w1,
                                                          const T* __restrict__ w2, int W2, int d_ff,
                                                          float* __restrict__ dh) {
    constexpr int P = Gemm1Smem<T>::P;
    extern __shared__ __align__(16) unsigned char smem[];
    T* sA = reinterpret_cast<T*>(smem);
    T* sB = sA + kBM1 * P;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int b = blockIdx.z;
    const int tok0 = blockIdx.x * (kBM1 / 2);
    const int j0 = blockIdx.y * (kBN1 / 2);

    // staging: thread -> (row, 32-column half)
    const int st_row = tid >> 1, st_col = (tid & 1) * 32;
    const T* a_src = nullptr;
    {
        const int t = tok0 + (st_row >> 1);
        if (t < n) {
            if (st_row & 1) {
                a_src = xbar + ((size_t)b * n + t) * W2;
            } else {
                const int r = rows[(size_t)b * n + t];
                if (r >= 0 && r < kv_len) a_src = kv + ((size_t)b * kv_len + r) * W2;
            }
        }
    }
    const T* b_src = (st_row < 64) ? w1 + (size_t)(j0 + st_row) * W2 : w2 + (size_t)(j0 + st_row - 64) * W2;

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = zero4();

    Copy32<T> ra, rb;
    if (a_src) ra.load(a_src + st_col); else ra.zero();
    rb.load(b_src + st_col);
    const int nk = W2 / kKC;
    for (int kc = 0; kc < nk; ++kc) {
        __syncthreads();
        ra.store(sA + st_row * P + st_col);
        rb.store(sB + st_row * P + st_col);
        __syncthreads();
        if (kc + 1 < nk) {
            const int off = (kc + 1) * kKC + st_col;
            if (a_src) ra.load(a_src + off);
            rb.load(b_src + off);
        }
#pragma unroll
        for (int ks = 0; ks < kKC / 32; ++ks) {
            const int kof = ks * 32 + 8 * (lane >> 4);
            typename Mma<T>::frag fa[4], fb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) fa[i] = lds_frag<T>(sA + (64 * wm + 16 * i + (lane & 15)) * P + kof);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = (j < 2) ? (32 * wn + 16 * j) : (64 + 32 * wn + 16 * (j - 2));
                fb[j] = lds_frag<T>(sB + (col + (lane & 15)) * P + kof);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = Mma<T>::step(acc[i][j], fa[i], fb[j]);
        }
    }
    // epilogue: rows 4g+0/4g+1 are kv/mean of one token, 4g+2/4g+3 of the next
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int tok = tok0 + 32 * wm + 8 * i + 2 * (lane >> 4);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const f32x4 a = acc[i][c];
            const f32x4 g = acc[i][c + 2];
            const float h0 = silu(a[0]) * g[0];
            const float h1 = silu(a[1]) * g[1];
            const float h2 = silu(a[2]) * g[2];
            const float h3 = silu(a[3]) * g[3];
            const int j = j0 + 32 * wn + 16 * c + (lane & 15);
            if (tok < n) dh[((size_t)b * n + tok) * d_ff + j] = h0 - h1;
            if (tok + 1 < n) dh[((size_t)b * n + tok + 1) * d_ff + j] = h2 - h3;
        }
    }
}

// ---------------------------------------------------------------- GEMM 2 + quantizer
// tile: 128 tokens x 64 latent columns (two groups). Wave w owns tokens [32 w, +32)
// and all 64 columns: 2 x 4 MFMA tiles per split term.
constexpr int kBM2 = 128;
constexpr int kBN2 = 64;

template <typename T, int NS>
struct Gemm2Smem {
    static constexpr int P = Pitch<T, kKC>::value;
    static constexpr size_t bytes = (size_t)(NS * kBM2 + kBN2) * P * sizeof(T);
};

template <typename T, int NS>
struct Split;

template <>
struct Split<bf16_t, 3> {
    // x = hi + mid + lo, each bf16; the remainders are exact in fp32
    static __device__ inline void run(const float* x, bf16_t* d0, bf16_t* d1, bf16_t* d2) {
        bf16_t a[8], m[8], l[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const bf16_t hi = (bf16_t)x[i];
            const float r1 = x[i] - (float)hi;
            const bf16_t mi = (bf16_t)r1;
            const float r2 = r1 - (float)mi;
            a[i] = hi;
            m[i] = mi;
            l[i] = (bf16_t)r2;
        }
        *reinterpret_cast<uint4*>(d0) = *reinterpret_cast<uint4*>(a);
        *reinterpret_cast<uint4*>(d1) = *reinterpret_cast<uint4*>(m);
        *reinterpret_cast<uint4*>(d2) = *reinterpret_cast<uint4*>(l);
    }
};

template <>
struct Split<float, 1> {
    static __device__ inline void run(const float* x, float* d0, float*, float*) {
        *reinterpret_cast<float4*>(d0) = make_float4(x[0], x[1], x[2], x[3]);
        *reinterpret_cast<float4*>(d0 + 4) = make_float4(x[4], x[5], x[6], x[7]);
    }
};

template <typename ScT>
__device__ inline float store_scalar(ScT* p, float v);
template <>
__device__ inline float store_scalar<float>(float* p, float v) {
    *p = v;
    return v;
}
template <>
__device__ inline float store_scalar<f16_t>(f16_t* p, float v) {
    const f16_t h = (f16_t)v;
    *p = h;
    return (float)h;
}
template <typename ScT>
__device__ inline float round_scalar(float v);
template <>
__device__ inline float round_scalar<float>(float v) { return v; }
template <>
__device__ inline float round_scalar<f16_t>(float v) { return (float)(f16_t)v; }

template <typename T, int NS, typename ScT>
__global__ __launch_bounds__(kThreads) void latent_quant_kernel(const float* __restrict__ dh, int n,
                                                                const T* __restrict__ w3, int d_ff, int d_c,
                                                                int bits, const int* __restrict__ pos, int cap_tok,
                                                                uint8_t* __restrict__ codes, size_t code_bytes,
                                                                ScT* __restrict__ scale, ScT* __restrict__ zmin) {
    constexpr int P = Gemm2Smem<T, NS>::P;
    extern __shared__ __align__(16) unsigned char smem[];
    T* sA = reinterpret_cast<T*>(smem);  // NS planes of [kBM2][P]
    T* sB = sA + NS * kBM2 * P;          // [kBN2][P]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.z;
    const int t0 = blockIdx.x * kBM2;
    const int c0 = blockIdx.y * kBN2;

    // staging: A 128 rows x 64 fp32 -> each thread 32 values of one row;
    // B 64 rows x 64 -> threads 0..127 each 32 values of one row
    const int st_row = tid >> 1, st_col = (tid & 1) * 32;
    const float* a_src = (t0 + st_row < n) ? dh + ((size_t)b * n + t0 + st_row) * d_ff : nullptr;
    const T* b_src = (tid < 128) ? w3 + (size_t)(c0 + st_row) * d_ff : nullptr;

    f32x4 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = zero4();

    float4 ra[8];
    Copy32<T> rb;
    auto load_a = [&](int off) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            ra[i] = a_src ? reinterpret_cast<const float4*>(a_src + off)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    };
    load_a(st_col);
    if (b_src) rb.load(b_src + st_col);
    const int nk = d_ff / kKC;
    for (int kc = 0; kc < nk; ++kc) {
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float* x = reinterpret_cast<const float*>(&ra[2 * q]);
            T* d0 = sA + st_row * P + st_col + 8 * q;
            Split<T, NS>::run(x, d0, d0 + (NS > 1 ? kBM2 * P : 0), d0 + (NS > 2 ? 2 * kBM2 * P : 0));
        }
        if (b_src) rb.store(sB + st_row * P + st_col);
        __syncthreads();
        if (kc + 1 < nk) {
            const int off = (kc + 1) * kKC + st_col;
            load_a(off);
            if (b_src) rb.load(b_src + off);
        }
#pragma unroll
        for (int ks = 0; ks < kKC / 32; ++ks) {
            const int kof = ks * 32 + 8 * (lane >> 4);
            typename Mma<T>::frag fb[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) fb[j] = lds_frag<T>(sB + (16 * j + (lane & 15)) * P + kof);
#pragma unroll
            for (int sp = 0; sp < NS; ++sp) {
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const typename Mma<T>::frag fa =
                        lds_frag<T>(sA + sp * kBM2 * P + (32 * wave + 16 * i + (lane & 15)) * P + kof);
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[i][j] = Mma<T>::step(acc[i][j], fa, fb[j]);
                }
            }
        }
    }

    // epilogue: lane holds z[token 32 w + 16 i + 4 (lane/16) + e][col 16 j + lane%16];
    // group gr of the tile = columns j in {2 gr, 2 gr + 1}
    const float levels = (float)((1 << (bits == 16 ? 1 : bits)) - 1);
    const int G = d_c / 32;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = t0 + 32 * wave + 16 * i + 4 * (lane >> 4) + e;
            const bool tv = t < n;
            int p = tv ? pos[(size_t)b * n + t] : -1;
            const bool ok = tv && p >= 0 && p < cap_tok;
            uint8_t* rec = codes + ((size_t)b * cap_tok + (ok ? p : 0)) * code_bytes;
            if (bits == 16) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int col = c0 + 16 * j + (lane & 15);
                    if (ok) reinterpret_cast<f16_t*>(rec)[col] = (f16_t)acc[i][j][e];
                }
                continue;
            }
#pragma unroll
            for (int gr = 0; gr < 2; ++gr) {
                const float v0 = acc[i][2 * gr][e];
                const float v1 = acc[i][2 * gr + 1][e];
                const float lo = seg16_min(fminf(v0, v1));
                const float hi = seg16_max(fmaxf(v0, v1));
                const float delta = (hi - lo) / levels;
                const float st = round_scalar<ScT>(delta);
                const float zm = round_scalar<ScT>(lo);
                const int g = (c0 >> 5) + gr;
                if (ok && (lane & 15) == 0) {
                    store_scalar<ScT>(scale + ((size_t)b * cap_tok + p) * G + g, delta);
                    store_scalar<ScT>(zmin + ((size_t)b * cap_tok + p) * G + g, lo);
                }
                float q0 = 0.f, q1 = 0.f;
                if (st != 0.f) {
                    q0 = fminf(fmaxf(__builtin_rintf((v0 - zm) / st), 0.f), levels);
                    q1 = fminf(fmaxf(__builtin_rintf((v1 - zm) / st), 0.f), levels);
                }
                const uint32_t iq0 = (uint32_t)q0, iq1 = (uint32_t)q1;
                // column of v0 = 32 g + lane%16, of v1 = 32 g + 16 + lane%16
                if (bits == 4) {
                    const uint32_t n0 = __shfl_xor((int)iq0, 1, 64);
                    const uint32_t n1 = __shfl_xor((int)iq1, 1, 64);
                    if (ok && (lane & 1) == 0) {
                        rec[(32 * g + (lane & 15)) >> 1] = (uint8_t)(iq0 | (n0 << 4));
                        rec[(32 * g + 16 + (lane & 15)) >> 1] = (uint8_t)(iq1 | (n1 << 4));
                    }
                } else {  // bits == 2: four consecutive coordinates per byte
                    uint32_t b0 = iq0 << (2 * (lane & 3));
                    uint32_t b1 = iq1 << (2 * (lane & 3));
                    b0 |= __shfl_xor((int)b0, 1, 64);
                    b1 |= __shfl_xor((int)b1, 1, 64);
                    b0 |= __shfl_xor((int)b0, 2, 64);
                    b1 |= __shfl_xor((int)b1, 2, 64);
                    if (ok && (lane & 3) == 0) {
                        rec[(32 * g + (lane & 15)) >> 2] = (uint8_t)b0;
                        rec[(32 * g + 16 + (lane & 15)) >> 2] = (uint8_t)b1;
                    }
                }
            }
        }
    }
}

}  // namespace

template <typename T>
static hipError_t swiglu_impl(const Shape& s, const CacheView& c, const EncodePlan& p, const void* kv, int kv_len,
                              const int* rows, int n, const void* w1, const void* w2, void* ws, hipStream_t st) {
    const size_t smem = Gemm1Smem<T>::bytes;
    auto kern = swiglu_kernel<T>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    char* w = static_cast<char*>(ws);
    const dim3 grid((2 * n + kBM1 - 1) / kBM1, s.d_ff / (kBN1 / 2), c.B);
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), smem, st, static_cast<const T*>(kv), kv_len, rows, n,
                       reinterpret_cast<const T*>(w + p.off_xbar), static_cast<const T*>(w1),
                       static_cast<const T*>(w2), s.W2, s.d_ff, reinterpret_cast<float*>(w + p.off_dh));
    return hipGetLastError();
}

hipError_t launch_swiglu(const Shape& s, const CacheView& c, const EncodePlan& p, const void* kv, int kv_len,
                         const int* rows, int n, const void* w1, const void* w2, void* ws, hipStream_t st) {
    if (s.f32) return swiglu_impl<float>(s, c, p, kv, kv_len, rows, n, w1, w2, ws, st);
    return swiglu_impl<bf16_t>(s, c, p, kv, kv_len, rows, n, w1, w2, ws, st);
}

template <typename T, int NS, typename ScT>
static hipError_t latent_impl(const Shape& s, const CacheView& c, const EncodePlan& p, const int* pos, int n,
                              const void* w3, void* ws, hipStream_t st) {
    const size_t smem = Gemm2Smem<T, NS>::bytes;
    auto kern = latent_quant_kernel<T, NS, ScT>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    char* w = static_cast<char*>(ws);
    const dim3 grid((n + kBM2 - 1) / kBM2, s.d_c / kBN2, c.B);
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), smem, st, reinterpret_cast<const float*>(w + p.off_dh), n,
                       static_cast<const T*>(w3), s.d_ff, s.d_c, s.bits, pos, c.cap_tok, c.codes, c.code_bytes,
                       static_cast<ScT*>(c.scale), static_cast<ScT*>(c.zmin));
    return hipGetLastError();
}

hipError_t launch_latent_quant(const Shape& s, const CacheView& c, const EncodePlan& p, const int* pos, int n,
                               const void* w3, void* ws, hipStream_t st) {
    if (s.f32) return latent_impl<float, 1, float>(s, c, p, pos, n, w3, ws, st);
    return latent_impl<bf16_t, 3, f16_t>(s, c, p, pos, n, w3, ws, st);
}

}  // namespace rkv
