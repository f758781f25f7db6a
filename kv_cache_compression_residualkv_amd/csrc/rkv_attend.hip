// Attention of one decoding query per head over the restored selected tokens
// (ResidualKV review page, section 2.7: the sparse attention method picks the tokens,
// the codec restores them, the layer attends over them).
//
//   out[b, h] = sum_j softmax_j(scale * q[b, h] . K[b, j, g]) V[b, j, g],  g = h / G,
//
// G = H_q / N query heads per KV head. Where the token-tile restore applies, the
// attention runs inside it (restore_attend_kernel, rkv_decode_tiles.hip: no restored row
// leaves the chip) and leaves one partial per token tile; otherwise the selected tokens
// are restored into the workspace and split over tokens (each workgroup one chunk of
// kChunk tokens of one KV head). Then one combine pass per (sequence, query head):
//   chunk pass: scores of the chunk's tokens for the G query heads (one thread per
//     token reads its key row; the queries sit in LDS and are read as broadcasts),
//     the chunk maximum and exp weights per head, then P V with 16 lanes per token
//     row (16-byte value loads, 4 rows per wavefront at a time); writes the chunk's
//     unnormalised output, maximum and weight sum;
//   combine pass (one workgroup per query head and 32 dimensions): rescales the chunks
//     to the overall maximum and divides by the sum.
// The key/value rows are bf16 [B, m, 2 d_k] (K heads, then V heads), as the restore
// writes them. The pass reads each row once: it is bound by HBM bandwidth.
#include <hip/hip_runtime.h>

#include <cfloat>

#include "rkv_device.h"
#include "rkv_internal.h"

namespace rkv {
namespace {

constexpr int kChunk = 256;   // tokens per workgroup
constexpr int kThreads = 256;  // one thread per token in the score pass
constexpr int kMaxG = kAttendMaxG;  // query heads per KV head

template <int D, int G>
__global__ __launch_bounds__(kThreads) void attend_chunk_kernel(const bf16_t* __restrict__ kv, int m, int W2, int dk,
                                                                const bf16_t* __restrict__ q, int Hq, float scale,
                                                                float* __restrict__ part_o,
                                                                float* __restrict__ part_ml, int nch) {
    static_assert(D == 64 || D == 128, "head dimension");
    static_assert(G >= 1 && G <= kMaxG, "query heads per KV head");
    __shared__ float sQ[kMaxG][D];
    __shared__ float sP[kMaxG][kChunk];
    __shared__ float sO[4][kMaxG][D];
    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int j0 = c * kChunk;
    for (int e = tid; e < G * D; e += kThreads) {
        const int h = e / D, d = e - h * D;
        sQ[h][d] = (float)q[((size_t)b * Hq + (size_t)g * G + h) * D + d];
    }
    __syncthreads();

    // scores: thread t takes token j0 + t
    {
        const int j = j0 + tid;
        float s[G];
#pragma unroll
        for (int h = 0; h < G; ++h) s[h] = 0.f;
        // rows past m read row m - 1 (their scores are replaced below): all loads in flight
        const bf16_t* krow = kv + ((size_t)b * m + min(j, m - 1)) * W2 + (size_t)g * D;
        uint4 raw[D / 8];
#pragma unroll
        for (int u = 0; u < D / 8; ++u) raw[u] = *reinterpret_cast<const uint4*>(krow + 8 * u);
#pragma unroll
        for (int u = 0; u < D / 8; ++u) {
            const uint32_t w4[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float kf = __uint_as_float((e & 1) ? (w4[e >> 1] & 0xFFFF0000u) : (w4[e >> 1] << 16));
#pragma unroll
                for (int h = 0; h < G; ++h) s[h] = fmaf(kf, sQ[h][8 * u + e], s[h]);
            }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) sP[h][tid] = j < m ? s[h] * scale : -INFINITY;
    }
    // P V operands: lane group r = lane / 16 takes row 16 i + 4 wave + r, lane % 16 its 8
    // dims (D = 64: lanes with (lane % 16) >= 8 hold no dims). The value loads do not
    // depend on the scores, so they are issued here and land during the softmax pass;
    // rows past m read row m - 1 with weight 0 (sP is 0 there).
    const int r = lane >> 4, dl = 8 * (lane & 15);
    uint4 vraw[kChunk / 16];
    if (dl < D) {
#pragma unroll
        for (int i = 0; i < kChunk / 16; ++i) {
            const int j = min(j0 + 16 * i + 4 * wave + r, m - 1);
            vraw[i] = *reinterpret_cast<const uint4*>(kv + ((size_t)b * m + j) * W2 + dk + (size_t)g * D + dl);
        }
    }
    __syncthreads();

    // per head: chunk maximum, weights exp(s - max), their sum (wave w: heads w, w + 4)
    for (int h = wave; h < G; h += 4) {
        float mx = -INFINITY;
        for (int t = lane; t < kChunk; t += 64) mx = fmaxf(mx, sP[h][t]);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
        float sum = 0.f;
        for (int t = lane; t < kChunk; t += 64) {
            const float p = j0 + t < m ? expf(sP[h][t] - mx) : 0.f;
            sP[h][t] = p;
            sum += p;
        }
        sum = wave_sum(sum);
        if (lane == 0) {
            float* ml = part_ml + ((((size_t)b * (W2 / (2 * D)) + g) * nch + c) * kMaxG + h) * 2;
            ml[0] = mx;
            ml[1] = sum;
        }
    }
    __syncthreads();

    float acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    if (dl < D) {
#pragma unroll
        for (int i = 0; i < kChunk / 16; ++i) {
            const int t = 16 * i + 4 * wave + r;
            const uint32_t w4[4] = {vraw[i].x, vraw[i].y, vraw[i].z, vraw[i].w};
            float v8[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) v8[e] = __uint_as_float((e & 1) ? (w4[e >> 1] & 0xFFFF0000u) : (w4[e >> 1] << 16));
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float p = sP[h][t];
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(p, v8[e], acc[h][e]);
            }
        }
    }
    // the four row groups of the wavefront, then the four wavefronts through LDS
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float v = acc[h][e];
            v += __shfl_xor(v, 16, 64);
            v += __shfl_xor(v, 32, 64);
            acc[h][e] = v;
        }
    if (r == 0 && dl < D) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) sO[wave][h][dl + e] = acc[h][e];
    }
    __syncthreads();
    for (int e = tid; e < G * D; e += kThreads) {
        const int h = e / D, d = e - h * D;
        const float o = (sO[0][h][d] + sO[1][h][d]) + (sO[2][h][d] + sO[3][h][d]);
        part_o[((((size_t)b * (W2 / (2 * D)) + g) * nch + c) * kMaxG + h) * D + d] = o;
    }
}

// out[b, hq, d] for query head hq = g G + h and 32 dimensions d0 .. d0 + 31 per workgroup
// (no chunks, m = 0: zeros). The chunks' weights exp(m_c - M) and weighted sums l_c
// exp(m_c - M) are formed once in LDS (M: the largest m_c); then thread (slice, d) adds
// the chunks slice, slice + S, ... of dimension d (S = kCombThreads / 32 slices) and the
// slices meet through LDS.
constexpr int kCombThreads = 1024;
constexpr int kCombDims = 32;
constexpr int kCombMaxChunks = 2048;  // chunks whose weights fit the LDS table; more are recomputed

template <int D>
__global__ __launch_bounds__(kCombThreads) void attend_combine_kernel(const float* __restrict__ part_o,
                                                                      const float* __restrict__ part_ml, int N,
                                                                      int nch, int Hq, int G, float* __restrict__ out) {
    constexpr int S = kCombThreads / kCombDims;
    __shared__ float sMax[kCombThreads / 64];
    __shared__ float sW[kCombMaxChunks];
    __shared__ float sNum[S][kCombDims];
    __shared__ float sDen[kCombThreads / 64];
    const int hq = blockIdx.x, b = blockIdx.y, d0 = kCombDims * blockIdx.z;
    const int g = hq / G, h = hq - g * G;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t base = ((size_t)b * N + g) * nch;
    float mx = -INFINITY;
    for (int c = tid; c < nch; c += kCombThreads) mx = fmaxf(mx, part_ml[((base + c) * kMaxG + h) * 2]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    if (lane == 0) sMax[wave] = mx;
    __syncthreads();
    mx = sMax[0];
#pragma unroll
    for (int w = 1; w < kCombThreads / 64; ++w) mx = fmaxf(mx, sMax[w]);
    // chunk weights and the denominator
    float den = 0.f;
    for (int c = tid; c < nch; c += kCombThreads) {
        const float* ml = part_ml + ((base + c) * kMaxG + h) * 2;
        const float w = expf(ml[0] - mx);
        if (c < kCombMaxChunks) sW[c] = w;
        den = fmaf(ml[1], w, den);
    }
    den = wave_sum(den);
    if (lane == 0) sDen[wave] = den;
    __syncthreads();
    const int d = tid % kCombDims, sl = tid / kCombDims;
    float num = 0.f;
#pragma unroll 4
    for (int c = sl; c < nch; c += S) {
        const float w = c < kCombMaxChunks ? sW[c] : expf(part_ml[((base + c) * kMaxG + h) * 2] - mx);
        num = fmaf(part_o[((base + c) * kMaxG + h) * D + d0 + d], w, num);
    }
    sNum[sl][d] = num;
    __syncthreads();
    if (tid < kCombDims) {
        float n = 0.f;
#pragma unroll
        for (int k = 0; k < S; ++k) n += sNum[k][tid];
        float dd = 0.f;
#pragma unroll
        for (int w = 0; w < kCombThreads / 64; ++w) dd += sDen[w];
        out[((size_t)b * Hq + hq) * D + d0 + tid] = dd > 0.f ? n / dd : 0.f;
    }
}

template <int D, int G>
hipError_t chunk_launch(dim3 grid, hipStream_t st, const bf16_t* kv, int m, int W2, int dk, const void* q, int Hq,
                        float scale, float* part_o, float* part_ml, int nch) {
    hipLaunchKernelGGL((attend_chunk_kernel<D, G>), grid, dim3(kThreads), 0, st, kv, m, W2, dk,
                       static_cast<const bf16_t*>(q), Hq, scale, part_o, part_ml, nch);
    return hipSuccess;
}

template <int D>
hipError_t chunk_g(int G, dim3 grid, hipStream_t st, const bf16_t* kv, int m, int W2, int dk, const void* q, int Hq,
                   float scale, float* part_o, float* part_ml, int nch) {
    switch (G) {
        case 1: return chunk_launch<D, 1>(grid, st, kv, m, W2, dk, q, Hq, scale, part_o, part_ml, nch);
        case 2: return chunk_launch<D, 2>(grid, st, kv, m, W2, dk, q, Hq, scale, part_o, part_ml, nch);
        case 3: return chunk_launch<D, 3>(grid, st, kv, m, W2, dk, q, Hq, scale, part_o, part_ml, nch);
        case 4: return chunk_launch<D, 4>(grid, st, kv, m, W2, dk, q, Hq, scale, part_o, part_ml, nch);
        case 5: return chunk_launch<D, 5>(grid, st, kv, m, W2, dk, q, Hq, scale, part_o, part_ml, nch);
        case 6: return chunk_launch<D, 6>(grid, st, kv, m, W2, dk, q, Hq, scale, part_o, part_ml, nch);
        case 7: return chunk_launch<D, 7>(grid, st, kv, m, W2, dk, q, Hq, scale, part_o, part_ml, nch);
        case 8: return chunk_launch<D, 8>(grid, st, kv, m, W2, dk, q, Hq, scale, part_o, part_ml, nch);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

// The fused path (restore_attend_kernel, then the combine) serves every shape the
// token-tile restore takes; other shapes restore into the workspace and run the chunk
// kernel over the rows.
static bool attend_fused(const Shape& s) { return decode_tiles_supported(s); }

struct AttendWs {
    size_t rows, part_o, part_ml, wprep, total;
    int nch;
};
static AttendWs attend_ws(const Shape& s, int B, int m) {
    auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
    AttendWs w{};
    if (m <= 0) return w;  // nothing restored: the combine writes zeros
    const bool fused = attend_fused(s);
    w.nch = fused ? restore_attend_tiles(m) : (m + kChunk - 1) / kChunk;
    size_t off = 0;
    w.rows = off;
    if (!fused) off += up((size_t)B * m * s.W2 * sizeof(bf16_t));
    w.part_o = off;
    off += up((size_t)B * s.N * w.nch * kMaxG * s.D * sizeof(float));
    w.part_ml = off;
    off += up((size_t)B * s.N * w.nch * kMaxG * 2 * sizeof(float));
    w.wprep = off;  // the fused path's prepared decoder when the caller has none
    if (fused) off += up((size_t)2 * s.W2 * s.d_c);
    w.total = off;
    return w;
}

size_t attend_workspace_bytes(const Shape& s, int B, int m) { return attend_ws(s, B, m).total; }

bool attend_supported(const Shape& s, int Hq) {
    return !s.f32 && (s.D == 64 || s.D == 128) && Hq > 0 && Hq % s.N == 0 && Hq / s.N <= kMaxG;
}

hipError_t launch_attend(const Shape& s, const CacheView& c, const int* idx, int m, const void* wd,
                         const void* wd16, const void* q, int Hq, float scale, float* out, void* ws, hipStream_t st) {
    const int B = c.B, G = Hq / s.N;
    const AttendWs L = attend_ws(s, B, m);
    const int nch = L.nch;
    char* w = static_cast<char*>(ws);
    float* part_o = reinterpret_cast<float*>(w + L.part_o);
    float* part_ml = reinterpret_cast<float*>(w + L.part_ml);
    if (m > 0) {
        hipError_t e;
        if (attend_fused(s)) {
            if (!wd16) {
                e = launch_prepare_decoder(s, wd, w + L.wprep, st);
                if (e != hipSuccess) return e;
                wd16 = w + L.wprep;
            }
            e = launch_restore_attend(s, c, idx, m, wd16, q, Hq, scale, part_o, part_ml, st);
        } else {
            bf16_t* kv = reinterpret_cast<bf16_t*>(w + L.rows);
            e = launch_decode(s, c, idx, m, wd, wd16, kv, RKV_BF16, st);
            if (e != hipSuccess) return e;
            e = s.D == 64 ? chunk_g<64>(G, dim3(nch, s.N, B), st, kv, m, s.W2, s.dk, q, Hq, scale, part_o, part_ml, nch)
                          : chunk_g<128>(G, dim3(nch, s.N, B), st, kv, m, s.W2, s.dk, q, Hq, scale, part_o, part_ml,
                                         nch);
            if (e == hipSuccess) e = hipGetLastError();
        }
        if (e != hipSuccess) return e;
    }
    const dim3 cgrid(Hq, B, s.D / kCombDims);
    if (s.D == 64)
        hipLaunchKernelGGL(attend_combine_kernel<64>, cgrid, dim3(kCombThreads), 0, st, part_o, part_ml, s.N, nch, Hq,
                           G, out);
    else
        hipLaunchKernelGGL(attend_combine_kernel<128>, cgrid, dim3(kCombThreads), 0, st, part_o, part_ml, s.N, nch, Hq,
                           G, out);
    return hipGetLastError();
}

}  // namespace rkv
