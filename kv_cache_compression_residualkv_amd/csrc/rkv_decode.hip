// Selected-token restore.
//
// ResidualKV review page, section 2.5 (boxed equation): KV-hat_i = z~_i W_d + mean_i
// with the bias-free linear decoder; section 2.4: z~ = q Delta + z_min per group;
// section 2.7 steps 2-3: only the selected tokens are read and restored; section 2.1
// (last paragraph): the restored pre-RoPE key is rotated at the token's own position.
//
// A workgroup owns one 128-column slice of the K|V output (one head at D = 128) and
// keeps that slice of W_d resident in LDS; each wavefront restores 32 tokens per
// pass. The MFMA computes out^T = W_d^T z~^T (W_d slice = A operand from LDS, the
// dequantized latents = B operand built in registers). The K order is permuted so
// that lane group g (lane / 16) supplies the contiguous quarter
// [g d_c / 4, (g + 1) d_c / 4) of each token's latent over the K-steps, and the LDS
// reads of W_d use the same permutation: a token's packed codes then arrive in a few
// 16-byte loads, issued one pass ahead. Each lane ends with 4 consecutive output
// columns of one token, which keeps the reference-mean gather (4 bytes per reference
// row) and the RoPE pairing (column j with j + D/2, same lane) local; bf16 output rows
// are staged through LDS and written as whole 256-byte row segments.
#include <math.h>

#include "rkv_device.h"
#include "rkv_internal.h"

namespace rkv {

namespace {

constexpr int kThreads = 256;
constexpr int kCols = 128;     // output columns per workgroup
constexpr int kWaveTok = 32;   // tokens per wavefront pass
constexpr int kPassTok = 4 * kWaveTok;
constexpr int kMaxK = 8;       // references per token kept in registers

template <typename T, typename OutT>
struct DecSmem {
    static __host__ __device__ inline int pitch(int d_c) { return d_c + 16 / (int)sizeof(T); }
    // bf16 output: 16 tokens x 128 columns staged per wavefront (row pitch 272 B)
    static constexpr int kStagePitch = 272;
    static constexpr bool kStage = sizeof(OutT) == 2;
    static inline size_t bytes(int d_c) {
        return (size_t)kCols * pitch(d_c) * sizeof(T) + (kStage ? (size_t)4 * 16 * kStagePitch : 0);
    }
};

template <typename ScT>
__device__ inline float ld_scalar(const ScT* p);
template <>
__device__ inline float ld_scalar<float>(const float* p) { return *p; }
template <>
__device__ inline float ld_scalar<f16_t>(const f16_t* p) { return (float)*p; }

// Everything a lane needs for one token of a pass.
template <typename ScT>
struct TokMeta {
    int p;        // position, -1 if none
    int enc;      // 1: encoded token with a record; 0: reference or invalid
    int nref;     // references averaged (a reference token averages itself)
    int ref[kMaxK];
    int g0;       // first group the lane's quarter touches
    uint4 q[4];   // this lane's quarter of the packed codes (bits <= 4)
    float sc[4], zm[4];  // step and minimum of the quarter's groups
};

// Loads everything one token needs for the next pass. All loads depend only on the
// position p (read two passes earlier), so they issue together.
template <typename ScT>
__device__ inline void load_meta(TokMeta<ScT>& M, int p, int b, const int* self_slot, const int* ref_idx,
                                 const uint8_t* codes, size_t code_bytes, const ScT* scale, const ScT* zmin,
                                 int top_k, int cap_ref, int cap_tok, int d_c, int bits, int g) {
    M.p = p;
    M.enc = 0;
    M.nref = 0;
#pragma unroll
    for (int q = 0; q < kMaxK; ++q) M.ref[q] = 0;
    M.g0 = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        M.q[u] = make_uint4(0, 0, 0, 0);
        M.sc[u] = 0.f;
        M.zm[u] = 0.f;
    }
    if (p < 0) return;
    const size_t ro = (size_t)b * cap_tok + p;
    const int ss = self_slot[ro];
    // the chosen slots come first (ascending), then -1 padding
    const int* ri = ref_idx + ro * top_k;
    int rv[kMaxK];
#pragma unroll
    for (int q = 0; q < kMaxK; ++q) rv[q] = (q < top_k) ? ri[q] : -1;
    if (bits != 16) {
        const int quarter = d_c >> 2;
        const int nbytes = quarter * bits / 8;  // this lane's code bytes (<= 64)
        const uint8_t* rec = codes + ro * code_bytes + (size_t)g * nbytes;
        if ((nbytes & 15) == 0) {
#pragma unroll
            for (int u = 0; u < 4; ++u)
                M.q[u] = (16 * u < nbytes) ? reinterpret_cast<const uint4*>(rec)[u] : make_uint4(0, 0, 0, 0);
        } else {
            uint32_t wv[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) wv[u] = (4 * u < nbytes) ? reinterpret_cast<const uint32_t*>(rec)[u] : 0u;
#pragma unroll
            for (int u = 0; u < 4; ++u) M.q[u] = make_uint4(wv[4 * u], wv[4 * u + 1], wv[4 * u + 2], wv[4 * u + 3]);
        }
        const int G = d_c / 32;
        const int g0 = (g * quarter) >> 5;
        const int g1 = ((g + 1) * quarter - 1) >> 5;
        M.g0 = g0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const bool ok = g0 + u <= g1;
            M.sc[u] = ok ? ld_scalar<ScT>(scale + ro * G + g0 + u) : 0.f;
            M.zm[u] = ok ? ld_scalar<ScT>(zmin + ro * G + g0 + u) : 0.f;
        }
    }
    if (ss >= 0) {  // a reference token restores its stored row (no latent term)
        M.nref = 1;
        M.ref[0] = min(ss, cap_ref - 1);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            M.q[u] = make_uint4(0, 0, 0, 0);
            M.sc[u] = 0.f;
            M.zm[u] = 0.f;
        }
        return;
    }
    M.enc = 1;
    int cnt = 0;
#pragma unroll
    for (int q = 0; q < kMaxK; ++q) {
        M.ref[q] = rv[q] >= 0 ? min(rv[q], cap_ref - 1) : 0;
        cnt += rv[q] >= 0 ? 1 : 0;
    }
    M.nref = cnt;
}

// Position of token t of the range, -1 when outside it or invalid (flagged).
__device__ inline int load_pos(const int* idx, int t, int t_end, int m, int b, int cap_tok, int* err, bool flag) {
    if (t >= t_end) return -1;
    const int p = idx[(size_t)b * m + t];
    if (p < 0 || p >= cap_tok) {
        if (flag) flag_error(err, DEVERR_IDX_RANGE);
        return -1;
    }
    return p;
}

// First references of a token gathered ahead of the epilogue: 4 consecutive FP8 values
// of reference q at the lane's columns of row tile i.
constexpr int kGatherRefs = 4;
template <typename RefT>
struct Gather {
    uint32_t v[8][kGatherRefs];
};

template <typename RefT, typename ScT>
__device__ inline void issue_gather(Gather<RefT>& G, const TokMeta<ScT>& M, const RefT* pool, int W2, int col0, int g) {
    if constexpr (std::is_same<RefT, fp8_t>::value) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int q = 0; q < kGatherRefs; ++q)
                G.v[i][q] = (q < M.nref)
                                ? *reinterpret_cast<const uint32_t*>(pool + (size_t)M.ref[q] * W2 + col0 + 16 * i + 4 * g)
                                : 0u;
    }
}

// 8 consecutive latent values (quarter-relative offset 8 ks) of a token as an MFMA fragment.
template <typename T, typename ScT, int BITS>
__device__ inline typename Mma<T>::frag latent_frag(const TokMeta<ScT>& M, int ks, int bits_rt, const uint8_t* rec16) {
    const int bits = BITS ? BITS : bits_rt;  // compile-time for the bf16 formats
    typename Mma<T>::frag f;
    // tokens without a record (references, invalid positions) carry zero codes, step and
    // minimum, so the quantized path yields zeros without a branch
    if (bits == 16) {
        uint4 w = *reinterpret_cast<const uint4*>(rec16 + 16 * ks);
        if (!M.enc) w = make_uint4(0, 0, 0, 0);
        const f16_t* h = reinterpret_cast<const f16_t*>(&w);
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = (T)h[i];
        return f;
    }
    // a quarter starts on a group boundary (d_c / 4 is 16 or a multiple of 32), so K-step
    // ks lies in the quarter's group ks / 4: a compile-time index once ks is unrolled
    const float s = M.sc[ks >> 2], z = M.zm[ks >> 2];
    uint32_t w;
    if (bits == 4) {
        const int word = ks;  // 8 nibbles per 32-bit word
        const uint4 v = M.q[word >> 2];
        const int c = word & 3;
        w = c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w;
    } else {
        const int word = ks >> 1;  // 16 two-bit codes per word, 8 per K-step
        const uint4 v = M.q[word >> 2];
        const int c = word & 3;
        const uint32_t ww = c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w;
        w = (ks & 1) ? (ww >> 16) : (ww & 0xFFFFu);
    }
    if constexpr (std::is_same<T, f16_t>::value) {
        // (0x6400 | q) is the fp16 number 1024 + q: subtract 1024, then one fp16 FMA
        const f16x2 off = {(f16_t)1024.0f, (f16_t)1024.0f};
        const f16x2 sv = {(f16_t)s, (f16_t)s};
        const f16x2 zv = {(f16_t)z, (f16_t)z};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t a, bq;
            if (bits == 4) {
                a = (w >> (8 * i)) & 0xFu;
                bq = (w >> (8 * i + 4)) & 0xFu;
            } else {
                a = (w >> (4 * i)) & 0x3u;
                bq = (w >> (4 * i + 2)) & 0x3u;
            }
            const uint32_t pk = 0x64006400u | a | (bq << 16);
            f16x2 x = *reinterpret_cast<const f16x2*>(&pk);
            x = x - off;
            x = __builtin_elementwise_fma(x, sv, zv);
            f[2 * i] = x[0];
            f[2 * i + 1] = x[1];
        }
    } else {
        const int sh = bits;
        const uint32_t mask = (1u << bits) - 1u;
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = (T)fmaf((float)((w >> (sh * i)) & mask), s, z);
    }
    return f;
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

// Epilogue of 16 tokens (lane: token tbase + lane % 16, columns col0 + 16 i + 4 g + e):
// add the reference mean, rotate the key columns, store.
template <typename RefT, typename ScT, typename OutT, int D>
__device__ inline void finish_tokens(const TokMeta<ScT>& M, const Gather<RefT>& Gt, f32x4 (&acc)[8], int tbase,
                                     int t_end, bool rope, const RefT* pool, int W2, int col0,
                                     const double (&rev)[D / 32][4], unsigned char* sO, OutT* out, int m, int b) {
    typedef DecSmem<f16_t, OutT> SM;
    constexpr int half = D / 2, pair_tiles = half / 16, tpd = D / 16;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, mrow = lane & 15;
    // reference mean: fp32 sum in ascending slot order, one correctly rounded division
    const float kf = (float)M.nref;
    const float rk = __fdiv_rn(1.0f, kf > 0.f ? kf : 1.0f);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = col0 + 16 * i + 4 * g;
        float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int q = 0; q < kMaxK; ++q) {
            if (q < M.nref) {
                float4 v;
                if constexpr (std::is_same<RefT, fp8_t>::value) {
                    if (q < kGatherRefs) v = fp8x4_to_f32(Gt.v[i][q]);
                    else v = Load4<RefT>::run(pool + (size_t)M.ref[q] * W2 + c);
                } else {
                    v = Load4<RefT>::run(pool + (size_t)M.ref[q] * W2 + c);
                }
                s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
            }
        }
        if (M.nref > 1) {
            if constexpr (std::is_same<RefT, fp8_t>::value) {
                s.x = div_small(s.x, kf, rk); s.y = div_small(s.y, kf, rk);
                s.z = div_small(s.z, kf, rk); s.w = div_small(s.w, kf, rk);
            } else {  // fp32 references: general sums, IEEE division
                s.x = __fdiv_rn(s.x, kf); s.y = __fdiv_rn(s.y, kf);
                s.z = __fdiv_rn(s.z, kf); s.w = __fdiv_rn(s.w, kf);
            }
        }
        acc[i][0] += s.x;
        acc[i][1] += s.y;
        acc[i][2] += s.z;
        acc[i][3] += s.w;
    }
    if (rope && M.p >= 0) {
        // RoPE at the token's own position: the phase p theta^(-2j/D) in revolutions is
        // reduced to [-1/2, 1/2] in fp64, then sin/cos in fp32
        const double pp = (double)M.p;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int jt = i % tpd;
            if (jt >= pair_tiles) continue;
            const int ip = i + pair_tiles;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const double r = pp * rev[jt][e];
                const float fr = (float)(r - rint(r));
                const float sn = __builtin_amdgcn_sinf(fr);
                const float cs = __builtin_amdgcn_cosf(fr);
                const float x1 = acc[i][e], x2 = acc[ip][e];
                acc[i][e] = x1 * cs - x2 * sn;
                acc[ip][e] = x2 * cs + x1 * sn;
            }
        }
    }
    const bool valid = M.p >= 0;
    if constexpr (SM::kStage) {
        // stage 16 tokens x 128 columns, then write whole row segments
        unsigned char* st = sO + (size_t)wave * 16 * SM::kStagePitch;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            OutT* d = reinterpret_cast<OutT*>(st + mrow * SM::kStagePitch) + 16 * i + 4 * g;
            if (valid) store_out4<OutT>(d, acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
            else store_out4<OutT>(d, 0.f, 0.f, 0.f, 0.f);
        }
        __builtin_amdgcn_wave_barrier();
        // each token row: 128 columns x 2 bytes = 16 chunks of 16 bytes
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int ch = lane + 64 * r;
            const int tr = ch >> 4, cc = ch & 15;
            const int t = tbase + tr;
            if (t < t_end) {
                const uint4 v = *reinterpret_cast<const uint4*>(st + tr * SM::kStagePitch + 16 * cc);
                *reinterpret_cast<uint4*>(out + ((size_t)b * m + t) * W2 + col0 + 8 * cc) = v;
            }
        }
        __builtin_amdgcn_wave_barrier();
    } else {
        const int t = tbase + mrow;
        if (t < t_end) {
            OutT* o = out + ((size_t)b * m + t) * W2;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int c = col0 + 16 * i + 4 * g;
                if (valid) store_out4<OutT>(o + c, acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
                else store_out4<OutT>(o + c, 0.f, 0.f, 0.f, 0.f);
            }
        }
    }
}

// grid: (W2 / 128 column slices, token ranges, batch). NKS = d_c / 32 K-steps (each lane
// group covers d_c / 4 latent coordinates, 8 per step); D = head dimension. Both are
// compile-time so every register array is indexed statically.
template <typename T, typename RefT, typename ScT, typename WT, typename OutT, int NKS, int D, int BITS>
__global__ __launch_bounds__(kThreads) void decode_kernel(
    const int* __restrict__ idx, int m, int tok_per_wg, const RefT* __restrict__ ref_vals,
    const int* __restrict__ self_slot, const int* __restrict__ ref_idx, const uint8_t* __restrict__ codes,
    size_t code_bytes, const ScT* __restrict__ scale, const ScT* __restrict__ zmin, const WT* __restrict__ wd,
    int W2, int dk, int bits, int top_k, int cap_ref, int cap_tok, double theta, OutT* __restrict__ out,
    int* err) {
    constexpr int d_c = 32 * NKS;
    typedef DecSmem<T, OutT> SM;
    extern __shared__ __align__(16) unsigned char smem[];
    T* sW = reinterpret_cast<T*>(smem);
    const int P = SM::pitch(d_c);
    unsigned char* sO = smem + (size_t)kCols * P * sizeof(T);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, mrow = lane & 15;
    const int col0 = blockIdx.x * kCols;
    const int b = blockIdx.z;
    constexpr int quarter = d_c / 4;
    constexpr int half = D / 2;
    constexpr int pair_tiles = half / 16;  // row tiles between a column and its RoPE partner

    // revolutions per position of the RoPE pairs this lane rotates: j = 16 jt + 4 g + e
    double rev[D / 32][4];
#pragma unroll
    for (int jt = 0; jt < pair_tiles; ++jt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            rev[jt][e] = pow(theta, -2.0 * (double)(16 * jt + 4 * g + e) / (double)D) * 0.15915494309189535;

    // W_d slice [128 output columns][d_c] -> LDS in the compute type, 8 loads in flight
    // per thread before they are converted and stored
    {
        constexpr int kIters = kCols * d_c / (kThreads * 8);
#pragma unroll
        for (int it0 = 0; it0 < kIters; it0 += 8) {
            float v[8][8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (it0 + u < kIters) {
                    const int e = (it0 + u) * kThreads * 8 + tid * 8;
                    const int r = e / d_c, k = e - r * d_c;
                    Load8<WT>::run(wd + (size_t)(col0 + r) * d_c + k, v[u]);
                }
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (it0 + u < kIters) {
                    const int e = (it0 + u) * kThreads * 8 + tid * 8;
                    const int r = e / d_c, k = e - r * d_c;
                    lds_store8<T>(sW + r * P + k, v[u]);
                }
            }
        }
    }

    const bool rope = col0 < dk;
    const int t_begin = blockIdx.y * tok_per_wg;
    const int t_end = min(m, t_begin + tok_per_wg);
    const RefT* pool = ref_vals + (size_t)b * cap_ref * W2;
    const bool flag = blockIdx.x == 0 && g == 0;

    // pipeline: positions two passes ahead, records one pass ahead, reference rows of
    // the current pass gathered before its MFMA loop
    int tp = t_begin + wave * kWaveTok;
    TokMeta<ScT> cur0, cur1, nxt0, nxt1;
    auto meta = [&](TokMeta<ScT>& M, int p) {
        load_meta<ScT>(M, p, b, self_slot, ref_idx, codes, code_bytes, scale, zmin, top_k, cap_ref, cap_tok, d_c,
                       BITS ? BITS : bits, g);
    };
    meta(cur0, load_pos(idx, tp + mrow, t_end, m, b, cap_tok, err, flag));
    meta(cur1, load_pos(idx, tp + 16 + mrow, t_end, m, b, cap_tok, err, flag));
    int pn0 = load_pos(idx, tp + kPassTok + mrow, t_end, m, b, cap_tok, err, flag);
    int pn1 = load_pos(idx, tp + kPassTok + 16 + mrow, t_end, m, b, cap_tok, err, flag);
    __syncthreads();  // W_d slice in LDS

    for (; tp < t_end; tp += kPassTok) {
        Gather<RefT> ga0, ga1;
        issue_gather<RefT, ScT>(ga0, cur0, pool, W2, col0, g);
        issue_gather<RefT, ScT>(ga1, cur1, pool, W2, col0, g);
        meta(nxt0, pn0);
        meta(nxt1, pn1);
        pn0 = load_pos(idx, tp + 2 * kPassTok + mrow, t_end, m, b, cap_tok, err, flag);
        pn1 = load_pos(idx, tp + 2 * kPassTok + 16 + mrow, t_end, m, b, cap_tok, err, flag);
        const uint8_t* rec0 =
            codes + ((size_t)b * cap_tok + (cur0.p >= 0 ? cur0.p : 0)) * code_bytes + (size_t)g * quarter * 2;
        const uint8_t* rec1 =
            codes + ((size_t)b * cap_tok + (cur1.p >= 0 ? cur1.p : 0)) * code_bytes + (size_t)g * quarter * 2;

        f32x4 acc0[8], acc1[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            acc0[i] = zero4();
            acc1[i] = zero4();
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const typename Mma<T>::frag f0 = latent_frag<T, ScT, BITS>(cur0, ks, bits, rec0);
            const typename Mma<T>::frag f1 = latent_frag<T, ScT, BITS>(cur1, ks, bits, rec1);
            const int kof = g * quarter + 8 * ks;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const typename Mma<T>::frag fw = lds_frag<T>(sW + (16 * i + mrow) * P + kof);
                acc0[i] = Mma<T>::step(acc0[i], fw, f0);
                acc1[i] = Mma<T>::step(acc1[i], fw, f1);
            }
        }
        finish_tokens<RefT, ScT, OutT, D>(cur0, ga0, acc0, tp, t_end, rope, pool, W2, col0, rev, sO, out, m, b);
        finish_tokens<RefT, ScT, OutT, D>(cur1, ga1, acc1, tp + 16, t_end, rope, pool, W2, col0, rev, sO, out, m, b);
        cur0 = nxt0;
        cur1 = nxt1;
    }
}

}  // namespace

template <typename T, typename RefT, typename ScT, typename WT, typename OutT, int NKS, int D, int BITS>
static hipError_t decode_impl(const Shape& s, const CacheView& c, const int* idx, int m, const void* wd, void* out,
                              hipStream_t st) {
    const size_t smem = DecSmem<T, OutT>::bytes(s.d_c);
    auto kern = decode_kernel<T, RefT, ScT, WT, OutT, NKS, D, BITS>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    const int slices = s.W2 / kCols;
    // one workgroup per CU (the W_d slice fills most of LDS)
    int ranges = (256 + slices * c.B - 1) / (slices * c.B);
    int per = (m + ranges - 1) / ranges;
    per = ((per + kPassTok - 1) / kPassTok) * kPassTok;
    if (per < kPassTok) per = kPassTok;
    ranges = (m + per - 1) / per;
    const dim3 grid(slices, ranges, c.B);
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), smem, st, idx, m, per, static_cast<const RefT*>(c.ref_vals),
                       c.self_slot, c.ref_idx, c.codes, c.code_bytes, static_cast<const ScT*>(c.scale),
                       static_cast<const ScT*>(c.zmin), static_cast<const WT*>(wd), s.W2, s.dk, s.bits, s.top_k,
                       c.cap_ref, c.cap_tok, s.theta, static_cast<OutT*>(out), c.err);
    return hipGetLastError();
}

template <typename T, typename RefT, typename ScT, typename WT, typename OutT, int D, int BITS>
static hipError_t decode_dc(const Shape& s, const CacheView& c, const int* idx, int m, const void* wd, void* out,
                            hipStream_t st) {
    switch (s.d_c / 32) {
        case 2: return decode_impl<T, RefT, ScT, WT, OutT, 2, D, BITS>(s, c, idx, m, wd, out, st);
        case 4: return decode_impl<T, RefT, ScT, WT, OutT, 4, D, BITS>(s, c, idx, m, wd, out, st);
        case 8: return decode_impl<T, RefT, ScT, WT, OutT, 8, D, BITS>(s, c, idx, m, wd, out, st);
        case 12: return decode_impl<T, RefT, ScT, WT, OutT, 12, D, BITS>(s, c, idx, m, wd, out, st);
        case 16: return decode_impl<T, RefT, ScT, WT, OutT, 16, D, BITS>(s, c, idx, m, wd, out, st);
        default: return hipErrorInvalidValue;
    }
}

// bf16 formats: the code width is a compile-time parameter; fp32 formats read it at run time
template <typename T, typename RefT, typename ScT, typename WT, typename OutT, int D>
static hipError_t decode_bits(const Shape& s, const CacheView& c, const int* idx, int m, const void* wd, void* out,
                              hipStream_t st) {
    if constexpr (std::is_same<T, float>::value) {
        return decode_dc<T, RefT, ScT, WT, OutT, D, 0>(s, c, idx, m, wd, out, st);
    } else {
        if (s.bits == 4) return decode_dc<T, RefT, ScT, WT, OutT, D, 4>(s, c, idx, m, wd, out, st);
        if (s.bits == 2) return decode_dc<T, RefT, ScT, WT, OutT, D, 2>(s, c, idx, m, wd, out, st);
        return decode_dc<T, RefT, ScT, WT, OutT, D, 16>(s, c, idx, m, wd, out, st);
    }
}

template <typename T, typename RefT, typename ScT, typename WT, typename OutT>
static hipError_t decode_d(const Shape& s, const CacheView& c, const int* idx, int m, const void* wd, void* out,
                           hipStream_t st) {
    if (s.D == 64) return decode_bits<T, RefT, ScT, WT, OutT, 64>(s, c, idx, m, wd, out, st);
    if (s.D == 128) return decode_bits<T, RefT, ScT, WT, OutT, 128>(s, c, idx, m, wd, out, st);
    return hipErrorInvalidValue;
}

hipError_t launch_decode(const Shape& s, const CacheView& c, const int* idx, int m, const void* wd, const void* wd16,
                         void* out, int out_dtype, hipStream_t st) {
    if (decode_tiles_supported(s)) return launch_decode_tiles(s, c, idx, m, wd, wd16, out, out_dtype, st);
    if (s.f32) {
        if (out_dtype == RKV_F32) return decode_d<float, float, float, float, float>(s, c, idx, m, wd, out, st);
        return decode_d<float, float, float, float, bf16_t>(s, c, idx, m, wd, out, st);
    }
    if (out_dtype == RKV_F32) return decode_d<f16_t, fp8_t, f16_t, bf16_t, float>(s, c, idx, m, wd, out, st);
    return decode_d<f16_t, fp8_t, f16_t, bf16_t, bf16_t>(s, c, idx, m, wd, out, st);
}

}  // namespace rkv
