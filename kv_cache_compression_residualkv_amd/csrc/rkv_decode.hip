// Selected-token restore.
//
// ResidualKV review page, section 2.5 (boxed equation): KV-hat_i = z~_i W_d + mean_i
// with the bias-free linear decoder; section 2.4: z~ = q Delta + z_min per group;
// section 2.7 steps 2-3: only the selected tokens are read and restored; section 2.1
// (last paragraph): the restored pre-RoPE key is rotated at the token's own position.
//
// A workgroup owns one 128-column slice of the K|V output (one head at D = 128) and
// keeps that slice of W_d resident in LDS; it walks a range of selected tokens, 128
// at a time (32 per wavefront). The MFMA computes out^T = W_d^T z~^T: the W_d slice is
// the A operand (from LDS), the dequantized latents are the B operand, built in
// registers straight from the packed codes. Each lane ends up with 4 consecutive
// output columns of one token, which makes the reference-mean gather (4 bytes per
// reference row) and the RoPE pairing (column j with j + D/2, same lane) local.
#include <math.h>

#include "rkv_device.h"
#include "rkv_internal.h"

namespace rkv {

namespace {

constexpr int kThreads = 256;
constexpr int kCols = 128;       // output columns per workgroup
constexpr int kWaveTok = 32;     // tokens per wavefront pass
constexpr int kPassTok = 4 * kWaveTok;

struct RopeFreq {
    double rev[64];  // theta^(-2j/D) / (2 pi): revolutions per position, j < D/2
};

template <typename T>
struct DecSmem {
    static __host__ __device__ inline int pitch(int d_c) { return d_c + 16 / (int)sizeof(T); }
    static inline size_t bytes(int d_c) { return (size_t)kCols * pitch(d_c) * sizeof(T); }
};

// latent fragment of one token: 8 consecutive coordinates starting at k (a multiple of 8)
template <typename T, typename ScT>
struct Latent;

template <typename ScT>
__device__ inline float ld_scalar(const ScT* p);
template <>
__device__ inline float ld_scalar<float>(const float* p) { return *p; }
template <>
__device__ inline float ld_scalar<f16_t>(const f16_t* p) { return (float)*p; }

template <typename T, typename ScT>
__device__ inline typename Mma<T>::frag latent_frag(const uint8_t* rec, const ScT* sc, const ScT* zm, int k,
                                                    int bits) {
    float v[8];
    if (bits == 16) {
        const uint4 w = *reinterpret_cast<const uint4*>(rec + 2 * k);
        const f16_t* h = reinterpret_cast<const f16_t*>(&w);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (float)h[i];
    } else {
        const int g = k >> 5;
        const float s = ld_scalar<ScT>(sc + g);
        const float m = ld_scalar<ScT>(zm + g);
        uint32_t q;
        if (bits == 4) {
            q = *reinterpret_cast<const uint32_t*>(rec + (k >> 1));
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = fmaf((float)((q >> (4 * i)) & 0xFu), s, m);
        } else {
            q = *reinterpret_cast<const uint16_t*>(rec + (k >> 2));
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = fmaf((float)((q >> (2 * i)) & 0x3u), s, m);
        }
    }
    return Mma<T>::from_float(v);
}

template <typename OutT>
__device__ inline void store_out4(OutT* p, float a, float b, float c, float d);
template <>
__device__ inline void store_out4<float>(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}
template <>
__device__ inline void store_out4<bf16_t>(bf16_t* p, float a, float b, float c, float d) {
    bf16_t t[4] = {(bf16_t)a, (bf16_t)b, (bf16_t)c, (bf16_t)d};
    *reinterpret_cast<uint2*>(p) = *reinterpret_cast<uint2*>(t);
}

// grid: (W2 / 128 column slices, token ranges, batch)
template <typename T, typename RefT, typename ScT, typename WT, typename OutT>
__global__ __launch_bounds__(kThreads) void decode_kernel(
    const int* __restrict__ idx, int m, int tok_per_wg, const RefT* __restrict__ ref_vals,
    const int* __restrict__ self_slot, const int* __restrict__ ref_idx, const uint8_t* __restrict__ codes,
    size_t code_bytes, const ScT* __restrict__ scale, const ScT* __restrict__ zmin, const WT* __restrict__ wd,
    int W2, int dk, int D, int d_c, int bits, int top_k, int cap_ref, int cap_tok, RopeFreq freq,
    OutT* __restrict__ out, int* err) {
    extern __shared__ __align__(16) unsigned char smem[];
    T* sW = reinterpret_cast<T*>(smem);
    const int P = DecSmem<T>::pitch(d_c);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col0 = blockIdx.x * kCols;
    const int b = blockIdx.z;
    const int G = d_c / 32;

    // W_d slice [128 output columns][d_c] -> LDS in the compute type
    for (int e = tid * 8; e < kCols * d_c; e += kThreads * 8) {
        const int r = e / d_c, k = e - r * d_c;
        float v[8];
        Load8<WT>::run(wd + (size_t)(col0 + r) * d_c + k, v);
        lds_store8<T>(sW + r * P + k, v);
    }
    __syncthreads();

    const bool rope = col0 < dk;
    const int half = D / 2;
    const int pair_tiles = half / 16;  // row tiles between a column and its partner
    const int t_begin = blockIdx.y * tok_per_wg;
    const int t_end = min(m, t_begin + tok_per_wg);
    const RefT* pool = ref_vals + (size_t)b * cap_ref * W2;

    for (int tp = t_begin + wave * kWaveTok; tp < t_end; tp += kPassTok) {
        // per-token metadata for this lane's two tokens (lane%16 of each 16-token tile)
        int tokp[2], nref[2], rs[2][8];
        bool is_enc[2];
        const uint8_t* rec[2];
        const ScT* sc[2];
        const ScT* zm[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int t = tp + 16 * j + (lane & 15);
            int p = -1;
            if (t < t_end) p = idx[(size_t)b * m + t];
            const bool ok = p >= 0 && p < cap_tok;
            if (t < t_end && !ok && lane < 16 && blockIdx.x == 0) flag_error(err, DEVERR_IDX_RANGE);
            tokp[j] = ok ? p : 0;
            const int ss = ok ? self_slot[(size_t)b * cap_tok + p] : -1;
            is_enc[j] = ok && ss < 0;
            int cnt = 0;
#pragma unroll
            for (int q = 0; q < 8; ++q) rs[j][q] = 0;
            if (ok && ss >= 0) {
                rs[j][0] = min(ss, cap_ref - 1);
                cnt = 1;
            } else if (ok) {
                const int* ri = ref_idx + ((size_t)b * cap_tok + p) * top_k;
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    if (q < top_k) {
                        const int v = ri[q];
                        if (v >= 0) {
                            rs[j][cnt < 8 ? cnt : 7] = min(v, cap_ref - 1);
                            ++cnt;
                        }
                    }
                }
            }
            nref[j] = ok ? cnt : 0;
            const size_t ro = (size_t)b * cap_tok + (ok ? p : 0);
            rec[j] = codes + ro * code_bytes;
            sc[j] = scale + ro * G;
            zm[j] = zmin + ro * G;
        }

        f32x4 acc[8][2];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            acc[i][0] = zero4();
            acc[i][1] = zero4();
        }
        for (int k0 = 0; k0 < d_c; k0 += 32) {
            const int kof = k0 + 8 * (lane >> 4);
            typename Mma<T>::frag fz[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                if (is_enc[j]) {
                    fz[j] = latent_frag<T, ScT>(rec[j], sc[j], zm[j], kof, bits);
                } else {
                    float zz[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                    fz[j] = Mma<T>::from_float(zz);
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const typename Mma<T>::frag fw = lds_frag<T>(sW + (16 * i + (lane & 15)) * P + kof);
                acc[i][0] = Mma<T>::step(acc[i][0], fw, fz[0]);
                acc[i][1] = Mma<T>::step(acc[i][1], fw, fz[1]);
            }
        }

        // epilogue: lane holds columns col0 + 16 i + 4 (lane/16) + e of token j
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int t = tp + 16 * j + (lane & 15);
            // reference mean: fp32 sum in ascending slot order, one IEEE division
            const float kf = (float)nref[j];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int c = col0 + 16 * i + 4 * (lane >> 4);
                float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    if (q < nref[j]) {
                        const float4 v = Load4<RefT>::run(pool + (size_t)rs[j][q] * W2 + c);
                        s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
                    }
                }
                if (nref[j] > 1) {
                    s.x = __fdiv_rn(s.x, kf); s.y = __fdiv_rn(s.y, kf);
                    s.z = __fdiv_rn(s.z, kf); s.w = __fdiv_rn(s.w, kf);
                }
                acc[i][j][0] += s.x;
                acc[i][j][1] += s.y;
                acc[i][j][2] += s.z;
                acc[i][j][3] += s.w;
            }
            if (rope) {
                // RoPE at the token's own position: angle p * theta^(-2j/D); the phase is
                // reduced to one revolution in fp64, then sin/cos in fp32
                const double pp = (double)tokp[j];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int cl = (16 * i) % D;  // head-local column of this row tile
                    if (cl >= half) continue;
                    const int ip = i + pair_tiles;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int jj = cl + 4 * (lane >> 4) + e;
                        const double r = pp * freq.rev[jj];
                        const float fr = (float)(r - rint(r));
                        float sn, cs;
                        __sincosf(6.283185307179586f * fr, &sn, &cs);
                        const float x1 = acc[i][j][e], x2 = acc[ip][j][e];
                        acc[i][j][e] = x1 * cs - x2 * sn;
                        acc[ip][j][e] = x2 * cs + x1 * sn;
                    }
                }
            }
            if (t < t_end) {
                OutT* o = out + ((size_t)b * m + t) * W2;
                const bool ok = tokp[j] >= 0 && (is_enc[j] || nref[j] > 0);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int c = col0 + 16 * i + 4 * (lane >> 4);
                    if (ok)
                        store_out4<OutT>(o + c, acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
                    else
                        store_out4<OutT>(o + c, 0.f, 0.f, 0.f, 0.f);
                }
            }
        }
    }
}

}  // namespace

template <typename T, typename RefT, typename ScT, typename WT, typename OutT>
static hipError_t decode_impl(const Shape& s, const CacheView& c, const int* idx, int m, const void* wd, void* out,
                              hipStream_t st) {
    const size_t smem = DecSmem<T>::bytes(s.d_c);
    auto kern = decode_kernel<T, RefT, ScT, WT, OutT>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    RopeFreq f{};
    for (int j = 0; j < s.D / 2 && j < 64; ++j)
        f.rev[j] = std::pow(s.theta, -2.0 * j / (double)s.D) / 6.283185307179586;
    const int slices = s.W2 / kCols;
    // aim at about two workgroups per CU in total
    int ranges = (512 + slices * c.B - 1) / (slices * c.B);
    int per = (m + ranges - 1) / ranges;
    per = ((per + kPassTok - 1) / kPassTok) * kPassTok;
    if (per < kPassTok) per = kPassTok;
    ranges = (m + per - 1) / per;
    const dim3 grid(slices, ranges, c.B);
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), smem, st, idx, m, per, static_cast<const RefT*>(c.ref_vals),
                       c.self_slot, c.ref_idx, c.codes, c.code_bytes, static_cast<const ScT*>(c.scale),
                       static_cast<const ScT*>(c.zmin), static_cast<const WT*>(wd), s.W2, s.dk, s.D, s.d_c, s.bits,
                       s.top_k, c.cap_ref, c.cap_tok, f, static_cast<OutT*>(out), c.err);
    return hipGetLastError();
}

hipError_t launch_decode(const Shape& s, const CacheView& c, const int* idx, int m, const void* wd, void* out,
                         int out_dtype, hipStream_t st) {
    if (s.f32) {
        if (out_dtype == RKV_F32) return decode_impl<float, float, float, float, float>(s, c, idx, m, wd, out, st);
        return decode_impl<float, float, float, float, bf16_t>(s, c, idx, m, wd, out, st);
    }
    if (out_dtype == RKV_F32) return decode_impl<f16_t, fp8_t, f16_t, bf16_t, float>(s, c, idx, m, wd, out, st);
    return decode_impl<f16_t, fp8_t, f16_t, bf16_t, bf16_t>(s, c, idx, m, wd, out, st);
}

}  // namespace rkv
