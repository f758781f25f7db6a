// Causal sparse reference search and reference mean.
//
// ResidualKV review page, section 2.2: each non-reference token picks the k_i
// references of its causal pool with the smallest squared L2 distance
// (arg top-k_i of -||kv_i - kv_j||^2, k_i = min(k, |pool|)) and averages them.
//
// Two kernels:
//   search_kernel  - one workgroup scores a tile of 128 tokens against one chunk of
//                    the pool. Scores ||r||^2 - 2 x.r come from MFMA (x bf16, r FP8
//                    widened exactly to bf16, fp32 accumulation) with the pool as
//                    the A operand so that each lane owns tokens; each lane keeps a
//                    sorted top-8 of (score, slot) per token in registers, and the
//                    workgroup merges its lanes' lists into one top-8 per token and
//                    chunk.
//   select_kernel  - one wavefront per token merges the chunks' lists, decides the
//                    k_i references (exact fp32 distances are computed only when the
//                    approximate scores of the boundary candidates are closer than
//                    their rounding bound), writes them in ascending slot order and
//                    writes the reference mean row the encoder consumes.
#include <float.h>
#include <limits.h>

#include "rkv_device.h"
#include "rkv_internal.h"

namespace rkv {

namespace {

constexpr int kTok = 128;   // tokens per search tile
constexpr int kSlot = 128;  // pool slots per block
constexpr int kKC = 64;     // K elements per LDS stage
constexpr int kTop = 8;     // candidates kept per token
constexpr int kThreads = 256;

// 32 consecutive elements of storage type S held as raw 16-byte words.
template <typename S>
struct Raw32 {
    static constexpr int kWords = 32 * (int)sizeof(S) / 16;
    uint4 w[kWords];
    __device__ inline void load(const S* p) {
#pragma unroll
        for (int i = 0; i < kWords; ++i) w[i] = reinterpret_cast<const uint4*>(p)[i];
    }
    __device__ inline void zero() {
#pragma unroll
        for (int i = 0; i < kWords; ++i) w[i] = make_uint4(0, 0, 0, 0);
    }
    __device__ inline void get8(int j, float* o) const;
};

template <>
__device__ inline void Raw32<fp8_t>::get8(int j, float* o) const {
    const uint4 v = w[j >> 1];
    const uint32_t a = (j & 1) ? v.z : v.x;
    const uint32_t b = (j & 1) ? v.w : v.y;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = fp8_to_f32((a >> (8 * i)) & 0xFFu);
#pragma unroll
    for (int i = 0; i < 4; ++i) o[4 + i] = fp8_to_f32((b >> (8 * i)) & 0xFFu);
}

template <>
__device__ inline void Raw32<bf16_t>::get8(int j, float* o) const {
    const uint4 v = w[j];
    const uint32_t x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[2 * i] = __uint_as_float(x[i] << 16);
        o[2 * i + 1] = __uint_as_float(x[i] & 0xFFFF0000u);
    }
}

template <>
__device__ inline void Raw32<float>::get8(int j, float* o) const {
    const uint4 a = w[2 * j], b = w[2 * j + 1];
    o[0] = __uint_as_float(a.x); o[1] = __uint_as_float(a.y); o[2] = __uint_as_float(a.z); o[3] = __uint_as_float(a.w);
    o[4] = __uint_as_float(b.x); o[5] = __uint_as_float(b.y); o[6] = __uint_as_float(b.z); o[7] = __uint_as_float(b.w);
}

template <typename T, typename S>
__device__ inline void stage32(T* dst, const Raw32<S>& r) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float v[8];
        r.get8(j, v);
        lds_store8<T>(dst + 8 * j, v);
    }
}

// Sorted (ascending) insertion into a per-lane top-8 list.
__device__ inline void top_insert(float (&ls)[kTop], int (&li)[kTop], float s, int id) {
    if (s < ls[kTop - 1]) {
        ls[kTop - 1] = s;
        li[kTop - 1] = id;
#pragma unroll
        for (int j = kTop - 1; j > 0; --j) {
            const bool sw = ls[j] < ls[j - 1];
            const float a = ls[j], c = ls[j - 1];
            const int ia = li[j], ic = li[j - 1];
            ls[j] = sw ? c : a;
            ls[j - 1] = sw ? a : c;
            li[j] = sw ? ic : ia;
            li[j - 1] = sw ? ia : ic;
        }
    }
}

template <typename T>
struct SearchSmem {
    static constexpr int P = Pitch<T, kKC>::value;
    static constexpr size_t kOperands = (size_t)(kSlot + kTok) * P * sizeof(T);
    static constexpr size_t kMerge = (size_t)kTok * 8 * kTop * (sizeof(float) + sizeof(int));
    static constexpr size_t kMain = kOperands > kMerge ? kOperands : kMerge;
    static constexpr size_t kMeta = kTok * sizeof(int) + kSlot * (sizeof(int) + sizeof(float));
    static constexpr size_t bytes = kMain + kMeta;
};

// grid: (token tiles, pool chunks, batch); 256 threads = 4 waves in a 2 x 2 layout:
// wave (ws, wt) scores slots [64 ws, 64 ws + 64) of the block against tokens
// [64 wt, 64 wt + 64) of the tile (4 x 4 MFMA tiles of 16 x 16).
template <typename T, typename KvT, typename RefT>
__global__ __launch_bounds__(kThreads) void search_kernel(
    const KvT* __restrict__ kv, int kv_len, const int* __restrict__ rows, const int* __restrict__ pos, int n,
    const RefT* __restrict__ ref_vals, const int* __restrict__ ref_pos, const float* __restrict__ ref_norm2,
    const int* __restrict__ ref_count, int W2, int cap_ref, int chunk_slots, int nsplit,
    float* __restrict__ part_score, int* __restrict__ part_slot) {
    typedef SearchSmem<T> SM;
    constexpr int P = SM::P;
    extern __shared__ __align__(16) unsigned char smem[];
    T* sA = reinterpret_cast<T*>(smem);  // pool rows   [kSlot][P]
    T* sB = sA + kSlot * P;              // token rows  [kTok][P]
    float* mS = reinterpret_cast<float*>(smem);              // merge scores [kTok][8][kTop]
    int* mI = reinterpret_cast<int*>(mS + kTok * 8 * kTop);  // merge slots
    int* s_tokpos = reinterpret_cast<int*>(smem + SM::kMain);
    int* s_refpos = s_tokpos + kTok;
    float* s_norm = reinterpret_cast<float*>(s_refpos + kSlot);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int ws = wave >> 1, wt = wave & 1;
    const int tile = blockIdx.x, split = blockIdx.y, b = blockIdx.z;
    const int t0 = tile * kTok;
    const int count = min(ref_count[b], cap_ref);
    const int s_begin = split * chunk_slots;
    const int s_end = min(count, s_begin + chunk_slots);

    if (tid < kTok) {
        const int t = t0 + tid;
        s_tokpos[tid] = (t < n) ? pos[(size_t)b * n + t] : INT_MIN;
    }
    __syncthreads();
    int tile_maxpos = INT_MIN;
    for (int i = 0; i < kTok; ++i) tile_maxpos = max(tile_maxpos, s_tokpos[i]);

    // token row pointer for this thread's staging row
    const int st_row = tid >> 1;
    const int st_col = (tid & 1) * 32;
    const KvT* tok_src = nullptr;
    {
        const int t = t0 + st_row;
        if (t < n) {
            const int r = rows[(size_t)b * n + t];
            if (r >= 0 && r < kv_len) tok_src = kv + ((size_t)b * kv_len + r) * W2;
        }
    }

    float ls[4][kTop];
    int li[4][kTop];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < kTop; ++j) {
            ls[q][j] = FLT_MAX;
            li[q][j] = -1;
        }

    int tokpos_l[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) tokpos_l[tt] = s_tokpos[64 * wt + 16 * tt + (lane & 15)];

    const int nk = W2 / kKC;
    for (int sb = s_begin; sb < s_end; sb += kSlot) {
        __syncthreads();
        if (tid < kSlot) {
            const int m = sb + tid;
            const bool ok = m < s_end;
            s_refpos[tid] = ok ? ref_pos[(size_t)b * cap_ref + m] : INT_MAX;
            s_norm[tid] = ok ? ref_norm2[(size_t)b * cap_ref + m] : 0.f;
        }
        __syncthreads();
        const int live = __syncthreads_or(tid < kSlot && s_refpos[tid] < tile_maxpos);
        if (!live) continue;

        const int slot_row = sb + st_row;
        const RefT* ref_src =
            (slot_row < s_end) ? ref_vals + ((size_t)b * cap_ref + slot_row) * W2 : nullptr;

        f32x4 acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = zero4();

        Raw32<RefT> ra;
        Raw32<KvT> rb;
        if (ref_src) ra.load(ref_src + st_col); else ra.zero();
        if (tok_src) rb.load(tok_src + st_col); else rb.zero();
        for (int kc = 0; kc < nk; ++kc) {
            __syncthreads();
            stage32<T>(sA + st_row * P + st_col, ra);
            stage32<T>(sB + st_row * P + st_col, rb);
            __syncthreads();
            if (kc + 1 < nk) {
                const int off = (kc + 1) * kKC + st_col;
                if (ref_src) ra.load(ref_src + off);
                if (tok_src) rb.load(tok_src + off);
            }
#pragma unroll
            for (int ks = 0; ks < kKC / 32; ++ks) {
                const int kof = ks * 32 + 8 * (lane >> 4);
                typename Mma<T>::frag fa[4], fb[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) fa[i] = lds_frag<T>(sA + (64 * ws + 16 * i + (lane & 15)) * P + kof);
#pragma unroll
                for (int j = 0; j < 4; ++j) fb[j] = lds_frag<T>(sB + (64 * wt + 16 * j + (lane & 15)) * P + kof);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[i][j] = Mma<T>::step(acc[i][j], fa[i], fb[j]);
            }
        }
        // epilogue: score = ||r||^2 - 2 x.r for causal slots, into the per-token lists
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int sl = 64 * ws + 16 * i + 4 * (lane >> 4) + e;
                const int rp = s_refpos[sl];
                const float nr = s_norm[sl];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (rp < tokpos_l[j]) top_insert(ls[j], li[j], fmaf(-2.f, acc[i][j][e], nr), sb + sl);
                }
            }
        }
    }

    // merge the 8 lists of every token (4 lane groups x 2 slot halves)
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int tl = 64 * wt + 16 * j + (lane & 15);
        const int src = ws * 4 + (lane >> 4);
        float* ps = mS + ((size_t)tl * 8 + src) * kTop;
        int* pi = mI + ((size_t)tl * 8 + src) * kTop;
#pragma unroll
        for (int q = 0; q < kTop; ++q) {
            ps[q] = ls[j][q];
            pi[q] = li[j][q];
        }
    }
    __syncthreads();
    if (tid < kTok && t0 + tid < n) {
        float bs[kTop];
        int bi[kTop];
#pragma unroll
        for (int q = 0; q < kTop; ++q) {
            bs[q] = FLT_MAX;
            bi[q] = -1;
        }
        const float* ps = mS + (size_t)tid * 8 * kTop;
        const int* pi = mI + (size_t)tid * 8 * kTop;
        for (int c = 0; c < 8 * kTop; ++c) {
            if (pi[c] >= 0) top_insert(bs, bi, ps[c], pi[c]);
        }
        const size_t o = (((size_t)b * n + t0 + tid) * nsplit + split) * kTop;
#pragma unroll
        for (int q = 0; q < kTop; ++q) {
            part_score[o + q] = bs[q];
            part_slot[o + q] = bi[q];
        }
    }
}

// ------------------------------------------------------------------ select + mean

template <typename XT>
__device__ inline void store4(XT* p, float4 v);
template <>
__device__ inline void store4<float>(float* p, float4 v) {
    *reinterpret_cast<float4*>(p) = v;
}
template <>
__device__ inline void store4<bf16_t>(bf16_t* p, float4 v) {
    bf16_t t[4] = {(bf16_t)v.x, (bf16_t)v.y, (bf16_t)v.z, (bf16_t)v.w};
    *reinterpret_cast<uint2*>(p) = *reinterpret_cast<uint2*>(t);
}

// One wavefront per token; 4 tokens per block.
template <typename KvT, typename RefT>
__global__ __launch_bounds__(kThreads) void select_kernel(
    const KvT* __restrict__ kv, int kv_len, const int* __restrict__ rows, const int* __restrict__ pos, int n,
    const RefT* __restrict__ ref_vals, const float* __restrict__ ref_norm2, const float* __restrict__ part_score,
    const int* __restrict__ part_slot, int nsplit, int W2, int cap_ref, int cap_tok, int top_k,
    int* __restrict__ ref_idx, KvT* __restrict__ xbar, int* err) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int b = blockIdx.y;
    if (t >= n) return;
    const int row = rows[(size_t)b * n + t];
    const int p = pos[(size_t)b * n + t];
    const bool row_ok = row >= 0 && row < kv_len;
    const bool pos_ok = p >= 0 && p < cap_tok;
    KvT* xrow = xbar + ((size_t)b * n + t) * W2;
    if (!row_ok || !pos_ok) {
        if (lane == 0) flag_error(err, (row_ok ? 0 : DEVERR_ROW_RANGE) | (pos_ok ? 0 : DEVERR_POS_RANGE));
        for (int c = 4 * lane; c < W2; c += 256) store4<KvT>(xrow + c, make_float4(0.f, 0.f, 0.f, 0.f));
        return;
    }
    const KvT* x = kv + ((size_t)b * kv_len + row) * W2;
    const RefT* pool = ref_vals + (size_t)b * cap_ref * W2;

    // gather the chunks' candidates, one per lane
    const int ncand = nsplit * kTop;  // <= 64
    float s = FLT_MAX;
    int id = -1;
    if (lane < ncand) {
        const size_t o = ((size_t)b * n + t) * nsplit * kTop + lane;
        id = part_slot[o];
        s = (id >= 0) ? part_score[o] : FLT_MAX;
    }
    // rank by (score, slot); invalid candidates carry FLT_MAX and slot -1 -> INT_MAX
    const int key_id = id >= 0 ? id : INT_MAX;
    int rank = 0;
    for (int j = 0; j < ncand; ++j) {
        const float sj = __shfl(s, j, 64);
        const int ij = __shfl(key_id, j, 64);
        rank += (sj < s || (sj == s && ij < key_id)) ? 1 : 0;
    }
    const unsigned long long valid_mask = __ballot(id >= 0);
    const int nvalid = __popcll(valid_mask);
    const int k_i = min(top_k, nvalid);

    // rounding bound of an approximate score: 2^-17 (||x||^2 + ||r||^2)
    float xn = 0.f;
    for (int c = 4 * lane; c < W2; c += 256) {
        const float4 v = Load4<KvT>::run(x + c);
        xn = fmaf(v.x, v.x, fmaf(v.y, v.y, fmaf(v.z, v.z, fmaf(v.w, v.w, xn))));
    }
    xn = wave_sum(xn);
    const float nr = (id >= 0) ? ref_norm2[(size_t)b * cap_ref + id] : 0.f;
    const float margin = 7.62939453125e-06f * (xn + nr);  // 2^-17
    const bool in_set = id >= 0 && rank < k_i;
    // highest (score + margin) inside the set vs lowest (score - margin) outside it
    float hi_in = in_set ? s + margin : -FLT_MAX;
    float lo_out = (id >= 0 && !in_set) ? s - margin : FLT_MAX;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        hi_in = fmaxf(hi_in, __shfl_xor(hi_in, o, 64));
        lo_out = fminf(lo_out, __shfl_xor(lo_out, o, 64));
    }
    bool chosen = in_set;
    if (k_i > 0 && lo_out <= hi_in) {
        // ambiguous boundary: exact fp32 squared distances of the best 8 candidates
        const bool cand = id >= 0 && rank < kTop;
        float dist = FLT_MAX;
        for (int q = 0; q < kTop; ++q) {
            const unsigned long long mq = __ballot(rank == q && id >= 0);
            if (mq == 0ull) break;
            const int sq = __shfl(id, __ffsll((long long)mq) - 1, 64);
            float acc = 0.f;
            const RefT* r = pool + (size_t)sq * W2;
            for (int c = 4 * lane; c < W2; c += 256) {
                const float4 xv = Load4<KvT>::run(x + c);
                const float4 rv = Load4<RefT>::run(r + c);
                const float d0 = xv.x - rv.x, d1 = xv.y - rv.y, d2 = xv.z - rv.z, d3 = xv.w - rv.w;
                acc += (d0 * d0 + d1 * d1) + (d2 * d2 + d3 * d3);
            }
            acc = wave_sum(acc);
            if (cand && rank == q) dist = acc;
        }
        // rank the candidates by (exact distance, slot)
        int erank = 0;
        for (int j = 0; j < kTop; ++j) {
            const int src_lane = __ffsll((long long)__ballot(rank == j && id >= 0)) - 1;
            if (src_lane < 0) break;
            const float dj = __shfl(dist, src_lane, 64);
            const int ij = __shfl(key_id, src_lane, 64);
            erank += (dj < dist || (dj == dist && ij < key_id)) ? 1 : 0;
        }
        chosen = cand && erank < k_i;
    }
    // chosen slots in ascending slot order
    int srank = 0;
    const unsigned long long cm = __ballot(chosen);
    for (int j = 0; j < 64; ++j) {
        if (!((cm >> j) & 1ull)) continue;
        const int ij = __shfl(id, j, 64);
        srank += (chosen && ij < id) ? 1 : 0;
    }
    // broadcast the chosen slots in order
    int slots[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const unsigned long long mq = __ballot(chosen && srank == q);
        slots[q] = mq ? __shfl(id, __ffsll((long long)mq) - 1, 64) : -1;
    }
    int* out_idx = ref_idx + ((size_t)b * cap_tok + p) * top_k;
    if (lane < top_k) {
        int v = -1;
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (q == lane) v = slots[q];
        out_idx[lane] = v;
    }
    if (k_i == 0 && lane == 0) flag_error(err, DEVERR_EMPTY_POOL);

    // reference mean: fp32 sum in ascending slot order, one IEEE division, rounded to
    // the KV dtype for the encoder
    const float kf = (float)k_i;
    for (int c = 4 * lane; c < W2; c += 256) {
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            if (q < k_i) {
                const float4 v = Load4<RefT>::run(pool + (size_t)slots[q] * W2 + c);
                acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
            }
        }
        if (k_i > 0) {
            acc.x = __fdiv_rn(acc.x, kf); acc.y = __fdiv_rn(acc.y, kf);
            acc.z = __fdiv_rn(acc.z, kf); acc.w = __fdiv_rn(acc.w, kf);
        }
        store4<KvT>(xrow + c, acc);
    }
}

}  // namespace

EncodePlan plan_encode(const Shape& s, int B, int n, int cap_ref) {
    EncodePlan p{};
    const int tiles = (n + kTok - 1) / kTok;
    const int nblocks = (cap_ref + kSlot - 1) / kSlot;
    int nsplit = (1024 + tiles * B - 1) / (tiles * B > 0 ? tiles * B : 1);
    nsplit = nsplit < 1 ? 1 : nsplit;
    nsplit = nsplit > 8 ? 8 : nsplit;
    nsplit = nsplit > nblocks ? (nblocks > 0 ? nblocks : 1) : nsplit;
    const int per = (nblocks + nsplit - 1) / nsplit;
    p.nsplit = nsplit;
    p.chunk_slots = (per > 0 ? per : 1) * kSlot;
    const size_t tok = (size_t)B * n;
    auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
    size_t off = 0;
    p.off_part_score = off;
    off = up(off + tok * nsplit * kTop * sizeof(float));
    p.off_part_slot = off;
    off = up(off + tok * nsplit * kTop * sizeof(int));
    p.off_xbar = off;
    off = up(off + tok * s.W2 * (s.f32 ? 4 : 2));
    p.off_dh = off;
    off = up(off + tok * s.d_ff * sizeof(float));
    p.total = off;
    return p;
}

template <typename T, typename KvT, typename RefT>
static hipError_t search_impl(const Shape& s, const CacheView& c, const EncodePlan& p, const void* kv, int kv_len,
                              const int* rows, const int* pos, int n, void* ws, hipStream_t st) {
    const size_t smem = SearchSmem<T>::bytes;
    auto kern = search_kernel<T, KvT, RefT>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    char* w = static_cast<char*>(ws);
    const dim3 grid((n + kTok - 1) / kTok, p.nsplit, c.B);
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), smem, st, static_cast<const KvT*>(kv), kv_len, rows, pos, n,
                       static_cast<const RefT*>(c.ref_vals), c.ref_pos, c.ref_norm2, c.ref_count, s.W2, c.cap_ref,
                       p.chunk_slots, p.nsplit, reinterpret_cast<float*>(w + p.off_part_score),
                       reinterpret_cast<int*>(w + p.off_part_slot));
    return hipGetLastError();
}

hipError_t launch_search(const Shape& s, const CacheView& c, const EncodePlan& p, const void* kv, int kv_len,
                         const int* rows, const int* pos, int n, void* ws, hipStream_t st) {
    if (s.f32) return search_impl<float, float, float>(s, c, p, kv, kv_len, rows, pos, n, ws, st);
    return search_impl<bf16_t, bf16_t, fp8_t>(s, c, p, kv, kv_len, rows, pos, n, ws, st);
}

template <typename KvT, typename RefT>
static hipError_t select_impl(const Shape& s, const CacheView& c, const EncodePlan& p, const void* kv, int kv_len,
                              const int* rows, const int* pos, int n, void* ws, hipStream_t st) {
    char* w = static_cast<char*>(ws);
    const dim3 grid((n + 3) / 4, c.B);
    hipLaunchKernelGGL((select_kernel<KvT, RefT>), grid, dim3(kThreads), 0, st, static_cast<const KvT*>(kv), kv_len,
                       rows, pos, n, static_cast<const RefT*>(c.ref_vals), c.ref_norm2,
                       reinterpret_cast<const float*>(w + p.off_part_score),
                       reinterpret_cast<const int*>(w + p.off_part_slot), p.nsplit, s.W2, c.cap_ref, c.cap_tok,
                       s.top_k, c.ref_idx, reinterpret_cast<KvT*>(w + p.off_xbar), c.err);
    return hipGetLastError();
}

hipError_t launch_select(const Shape& s, const CacheView& c, const EncodePlan& p, const void* kv, int kv_len,
                         const int* rows, const int* pos, int n, void* ws, hipStream_t st) {
    if (s.f32) return select_impl<float, float>(s, c, p, kv, kv_len, rows, pos, n, ws, st);
    return select_impl<bf16_t, fp8_t>(s, c, p, kv, kv_len, rows, pos, n, ws, st);
}

}  // namespace rkv
