// Causal sparse reference search and reference mean.
//
// ResidualKV review page, section 2.2: each non-reference token picks the k_i
// references of its causal pool with the smallest squared L2 distance
// (arg top-k_i of -||kv_i - kv_j||^2, k_i = min(k, |pool|)) and averages them.
//
// Kernels:
//   plan + queue   - per token tile, the pool blocks it has to read (those whose first
//                    position lies below the tile's last token; the pool is
//                    position-ordered), cut into chunks; one work queue per XCD.
//   search kernel  - persistent, one workgroup per CU: each item scores a tile of 128
//                    tokens against a chunk of pool blocks (256 slots each). Scores
//                    ||r||^2 - 2 x.r come from
//                    MFMA (x bf16, r FP8 widened exactly to bf16, fp32 accumulation)
//                    with the pool as the A operand so that each lane owns tokens.
//                    The pool and token rows stream through an LDS ring filled by
//                    direct global->LDS loads (the K stages of consecutive pool blocks
//                    form one pipelined sequence). After each pool block every lane
//                    folds its scores into a sorted per-token top-8 held in registers
//                    with a sorting network and bitonic merges on 64-bit (score, slot)
//                    keys (no divergence, no per-candidate insertion). The workgroup
//                    finally merges its lanes' lists into one top-8 per token and chunk.
//                    Single slots are masked by position.
//   select_kernel  - one wavefront per token merges the chunks' lists, decides the
//                    k_i references (exact fp32 distances are computed only when the
//                    approximate scores of the boundary candidates are closer than
//                    their rounding bound), writes them in ascending slot order and
//                    writes the reference mean row the encoder consumes.
// The fp32 formats (small parity configurations) use a register-staged variant of
// the search with fp32 MFMA and per-candidate insertion.
#include <float.h>
#include <limits.h>

#include <algorithm>

#include <type_traits>

#include "rkv_device.h"
#include "rkv_gemm.h"
#include "rkv_internal.h"
#include "rkv_pipe.h"

namespace rkv {

namespace {

constexpr int kThreads = 256;
constexpr int kTop = 8;  // candidates kept per token
constexpr int kTok = 128;  // tokens per search tile

// select's rescan queue (int words of the workspace): [0] queued tokens, [1] spare,
// [2, 2 + kRqPar) arrival counters of the parallel rescans, then two words per queued
// token from kRqHead. The first kRqPar queued tokens are rescanned in kRqParts parts, one
// workgroup each, whose partial top-8 lists (off_rescan_part) the last part merges.
constexpr int kRqPar = 64;
constexpr int kRqParts = 64;
constexpr int kRqHead = 2 + kRqPar;
// clears the queue head and the arrival counters (block (0, 0) of the first kernel of an
// encode; at least kRqHead threads)
__device__ inline void reset_rescan(int* rescan) {
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < kRqHead) rescan[threadIdx.x] = 0;
}

template <typename T>
struct SC {
    static constexpr int BM = std::is_same<T, float>::value ? 128 : 256;  // pool slots per block
    static constexpr int BN = kTok;
    static constexpr int WM = BM / 2, WN = 64;
    static constexpr int P = Pitch<T, kKC>::value;
    static constexpr size_t kPipe = (size_t)2 * (BM + BN) * P * sizeof(T);
    static constexpr size_t kMerge = (size_t)kTok * 8 * kTop * (sizeof(float) + sizeof(int));
    static constexpr size_t kMain = kPipe > kMerge ? kPipe : kMerge;
    static constexpr size_t bytes = kMain + 16;
};

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

// A operand: rows of the pool block of the current stage (FP8 or fp32 storage).
template <typename T, typename RefT, int BM>
struct PoolLoader {
    static constexpr int kUnits = BM / 128;
    Raw32<RefT> raw[kUnits];
    const RefT* pool;
    int W2, nk, blk0, count;
    __device__ inline void load(int s) {
        const int blk = blk0 + s / nk;
        const int k0 = (s % nk) * kKC + (threadIdx.x & 1) * 32;
#pragma unroll
        for (int u = 0; u < kUnits; ++u) {
            const int slot = blk * BM + (threadIdx.x >> 1) + 128 * u;
            if (slot < count) raw[u].load(pool + (size_t)slot * W2 + k0);
            else raw[u].zero();
        }
    }
    __device__ inline void store(T* lds, int P) const {
#pragma unroll
        for (int u = 0; u < kUnits; ++u)
            stage32<T>(lds + ((threadIdx.x >> 1) + 128 * u) * P + (threadIdx.x & 1) * 32, raw[u]);
    }
};

// B operand: the tile's token rows; the same K stage repeats for every pool block.
template <typename T, typename KvT>
struct TokLoader {
    RowTile<T, KvT, kTok> t;
    const KvT* row[1];
    int nk;
    __device__ inline void load(int s) { t.load_rows(row, (s % nk) * kKC); }
    __device__ inline void store(T* lds, int P) const { t.store(lds, P); }
};

// grid: (8 * per, batch) blocks over logical tiles (token tile, chunk), chunks fastest.
template <typename T, typename KvT, typename RefT>
__global__ __launch_bounds__(kThreads) void search_kernel(
    const KvT* __restrict__ kv, int kv_len, const int* __restrict__ rows, const int* __restrict__ pos, int n,
    const RefT* __restrict__ ref_vals, const int* __restrict__ ref_pos, const float* __restrict__ ref_norm2,
    const int* __restrict__ ref_count, int W2, int cap_ref, int blocks_per_chunk, int nsplit, int ntiles, int per,
    float* __restrict__ part_score, int* __restrict__ part_slot, int* __restrict__ rescan) {
    typedef SC<T> C;
    reset_rescan(rescan);
    extern __shared__ __align__(16) unsigned char smem_u8[];
    unsigned char* smem = smem_u8;
    T* lds = reinterpret_cast<T*>(smem);
    int* s_vis = reinterpret_cast<int*>(smem + C::kMain);
    // Causal work grows with the token position, so token tiles are dealt round-robin
    // over the 8 XCDs (block b runs on XCD b mod 8), latest (heaviest) tiles first; the
    // pool chunks of one tile run back to back on the same XCD and share its L2.
    const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int tl = j / nsplit, split = j - tl * nsplit;
    const int tiles_x = (ntiles - x + 7) / 8;  // tiles owned by XCD x: x, x + 8, ...
    if (tl >= tiles_x) return;
    const int tile = x + 8 * (tiles_x - 1 - tl);
    const int b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ws = wave >> 1, wt = wave & 1;
    const int t0 = tile * kTok;
    const int count = max(0, min(ref_count[b], cap_ref));
    const int* rp = ref_pos + (size_t)b * cap_ref;
    const float* rn = ref_norm2 + (size_t)b * cap_ref;

    int tokpos_l[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int t = t0 + 64 * wt + 16 * j + (lane & 15);
        tokpos_l[j] = (t < n) ? pos[(size_t)b * n + t] : INT_MIN;
    }
    if (tid == 0) {
        // visible pool prefix: slots with position < the tile's largest position
        int mx = INT_MIN;
        for (int i = 0; i < kTok && t0 + i < n; ++i) mx = max(mx, pos[(size_t)b * n + t0 + i]);
        int lo = 0, hi = count;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (rp[mid] < mx) lo = mid + 1;
            else hi = mid;
        }
        s_vis[0] = lo;
    }
    __syncthreads();
    const int visible = s_vis[0];
    const int nblk = (visible + C::BM - 1) / C::BM;
    const int blk0 = split * blocks_per_chunk;
    const int blk1 = min(nblk, blk0 + blocks_per_chunk);
    const int nk = W2 / kKC;

    float ls[4][kTop];
    int li[4][kTop];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < kTop; ++j) {
            ls[q][j] = FLT_MAX;
            li[q][j] = -1;
        }

    if (blk1 > blk0) {
        PoolLoader<T, RefT, C::BM> la;
        la.pool = ref_vals + (size_t)b * cap_ref * W2;
        la.W2 = W2;
        la.nk = nk;
        la.blk0 = blk0;
        la.count = visible;
        TokLoader<T, KvT> lb;
        lb.nk = nk;
        {
            const int t = t0 + (tid >> 1);
            const KvT* p = nullptr;
            if (t < n) {
                const int r = rows[(size_t)b * n + t];
                if (r >= 0 && r < kv_len) p = kv + ((size_t)b * kv_len + r) * W2;
            }
            lb.row[0] = p;
        }
        f32x4 acc[C::WM / 16][C::WN / 16];
        auto fold = [&](int bi, f32x4(&a)[C::WM / 16][C::WN / 16]) {
            const int base = (blk0 + bi) * C::BM + C::WM * ws + 4 * (lane >> 4);
            // A candidate can only matter if it beats the 8th best of every lane holding
            // the same token (lanes l, l^16, l^32, l^48): the smallest of those four
            // 8th-best scores bounds the token's 8th best from above. Candidates are
            // gated four at a time against it before any insertion work.
            float thr[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float t = ls[j][kTop - 1];
                t = fminf(t, __shfl_xor(t, 16, 64));
                t = fminf(t, __shfl_xor(t, 32, 64));
                thr[j] = t;
            }
#pragma unroll
            for (int i = 0; i < C::WM / 16; ++i) {
                int p[4];
                float nr[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int slot = base + 16 * i + e;
                    const bool ok = slot < visible;
                    p[e] = ok ? rp[slot] : INT_MAX;
                    nr[e] = ok ? rn[slot] : 0.f;
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float sc[4];
                    float mn = FLT_MAX;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        sc[e] = (p[e] < tokpos_l[j]) ? fmaf(-2.f, a[i][j][e], nr[e]) : FLT_MAX;
                        mn = fminf(mn, sc[e]);
                    }
                    if (mn < fminf(thr[j], ls[j][kTop - 1])) {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (sc[e] < thr[j]) top_insert(ls[j], li[j], sc[e], base + 16 * i + e);
                    }
                }
            }
        };
        mainloop<T, C::BM, C::BN, C::WM, C::WN>(la, lb, (blk1 - blk0) * nk, nk, lds, C::WM * ws, 64 * wt, acc, fold);
    }

    // merge the 8 lists of every token (4 lane groups x 2 slot halves)
    __syncthreads();
    float* mS = reinterpret_cast<float*>(smem);
    int* mI = reinterpret_cast<int*>(mS + kTok * 8 * kTop);
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

// ------------------------------------------------------------------ bf16 / FP8 search

// Workgroup of 8 wavefronts: wavefront w owns pool slots 64 (w % 4) .. +64 of each
// block and tokens 64 (w / 4) .. +64 of the tile, as 2 x 2 output tiles of one
// v_mfma_f32_32x32x16_bf16 each. Every lane then holds 2 tokens x 32 slots of a block,
// and every FP8 pool value is widened by two wavefronts (not four, as with 16-row
// tiles) at the same LDS read traffic.
namespace s2 {
constexpr int kThreads = 512;
constexpr int BM = 256;                    // pool slots per block
constexpr int BN = kTok;                   // tokens per tile
constexpr int NST = 4;                     // LDS ring stages
constexpr int kStageA = BM * kStageK;      // FP8 pool stage bytes
constexpr int kStageB = BN * kStageK * 2;  // bf16 token stage bytes
constexpr int kSlot = kStageA + kStageB;
constexpr int kRing = NST * kSlot;
constexpr int kMeta = BM * 8;              // positions, then norms, of one pool block
constexpr int kMetaBufs = 4;               // blocks whose metadata may be resident
constexpr int kMerge = kTok * 8 * kTop * 8;  // 8 lists of 8 keys per token
constexpr int kOffMeta = kRing;
constexpr int kOffRed = kOffMeta + kMetaBufs * kMeta;
constexpr int kMain = kOffRed + 64;
constexpr size_t bytes = (size_t)(kMain > kMerge ? kMain : kMerge);
static_assert(bytes <= 160 * 1024, "LDS budget");
constexpr int kLoadsA = BM / 16 / 8;       // 1 KB pool blocks per wavefront and stage
constexpr int kLoadsB = BN / 8 / 8;        // 1 KB token blocks per wavefront and stage
constexpr int kPer = kLoadsA + kLoadsB;    // direct loads per wavefront and stage (+1 with metadata)
}  // namespace s2

// A candidate as one 64-bit key: the score's bits mapped to an order-preserving
// unsigned integer in the high word, the slot in the low word. Unsigned order of keys
// is the lexicographic (score, slot) order, so a compare-exchange is one 64-bit
// compare and four selects (no scalar mask arithmetic). Masked candidates carry
// kNoKey (score FLT_MAX, slot -1) and sort last.
__device__ inline uint64_t score_key(float sc, int slot) {
    uint32_t b = __float_as_uint(sc);
    b ^= (b & 0x80000000u) ? 0xFFFFFFFFu : 0x80000000u;
    return ((uint64_t)b << 32) | (uint32_t)slot;
}
__device__ inline float key_score(uint64_t k) {
    uint32_t b = (uint32_t)(k >> 32);
    b ^= (b & 0x80000000u) ? 0x80000000u : 0xFFFFFFFFu;
    return __uint_as_float(b);
}
__device__ inline int key_slot(uint64_t k) { return (int)(uint32_t)k; }
constexpr uint64_t kNoKey = ((uint64_t)(0x7F7FFFFFu ^ 0x80000000u) << 32) | 0xFFFFFFFFull;

__device__ inline void cas(uint64_t& a, uint64_t& b) {
    const bool sw = b < a;
    const uint64_t ta = sw ? b : a, tb = sw ? a : b;
    a = ta;
    b = tb;
}

// 19-comparator sorting network for 8 elements
__device__ inline void sort8(uint64_t (&k)[8]) {
#define RKV_C(x, y) cas(k[x], k[y])
    RKV_C(0, 2); RKV_C(1, 3); RKV_C(4, 6); RKV_C(5, 7);
    RKV_C(0, 4); RKV_C(1, 5); RKV_C(2, 6); RKV_C(3, 7);
    RKV_C(0, 1); RKV_C(2, 3); RKV_C(4, 5); RKV_C(6, 7);
    RKV_C(2, 4); RKV_C(3, 5);
    RKV_C(1, 4); RKV_C(3, 6);
    RKV_C(1, 2); RKV_C(3, 4); RKV_C(5, 6);
#undef RKV_C
}

// a <- the 8 smallest of two sorted lists a, b, sorted (bitonic merge)
__device__ inline void merge8(uint64_t (&a)[8], const uint64_t (&b)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = b[7 - i] < a[i] ? b[7 - i] : a[i];
#define RKV_C(x, y) cas(a[x], a[y])
    RKV_C(0, 4); RKV_C(1, 5); RKV_C(2, 6); RKV_C(3, 7);
    RKV_C(0, 2); RKV_C(1, 3); RKV_C(4, 6); RKV_C(5, 7);
    RKV_C(0, 1); RKV_C(2, 3); RKV_C(4, 5); RKV_C(6, 7);
#undef RKV_C
}

// The same networks on 32-bit keys (a compare-exchange is one min and one max)
__device__ inline void cas32(uint32_t& a, uint32_t& b) {
    const uint32_t lo = min(a, b), hi = max(a, b);
    a = lo;
    b = hi;
}
__device__ inline void sort8_32(uint32_t (&k)[8]) {
#define RKV_C(x, y) cas32(k[x], k[y])
    RKV_C(0, 2); RKV_C(1, 3); RKV_C(4, 6); RKV_C(5, 7);
    RKV_C(0, 4); RKV_C(1, 5); RKV_C(2, 6); RKV_C(3, 7);
    RKV_C(0, 1); RKV_C(2, 3); RKV_C(4, 5); RKV_C(6, 7);
    RKV_C(2, 4); RKV_C(3, 5);
    RKV_C(1, 4); RKV_C(3, 6);
    RKV_C(1, 2); RKV_C(3, 4); RKV_C(5, 6);
#undef RKV_C
}
__device__ inline void merge8_32(uint32_t (&a)[8], const uint32_t (&b)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = min(a[i], b[7 - i]);
#define RKV_C(x, y) cas32(a[x], a[y])
    RKV_C(0, 4); RKV_C(1, 5); RKV_C(2, 6); RKV_C(3, 7);
    RKV_C(0, 2); RKV_C(1, 3); RKV_C(4, 6); RKV_C(5, 7);
    RKV_C(0, 1); RKV_C(2, 3); RKV_C(4, 5); RKV_C(6, 7);
#undef RKV_C
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// 4-byte direct load (lane l lands at byte 4 l of the LDS destination)
__device__ inline void dma4(const void* g, void* lds) {
    __builtin_amdgcn_global_load_lds(g, (RKV_LDS void*)lds, 4, 0, 0);
}


// LDS layout of a ring slot: the FP8 pool stage (256 rows x 64 K bytes) as 16 blocks of
// 16 rows at a 64-byte pitch, the 16-byte granule m of row r at position m ^ h(r); the
// bf16 token stage (128 rows x 64 K) as 16 blocks (row group g, K half q) = 2 g + q,
// the 8-value chunk c at position c ^ h(r). One direct load fills one block, four
// consecutive lanes fetching one contiguous 64-byte row segment.
//
// Fragments. A K-half p (32 K values) of a stage is consumed by two MFMAs (sub-steps
// e = 0, 1). Lanes 0-31 supply K values 32 p + 8 e .. +8 and lanes 32-63 supply
// 32 p + 16 + 8 e .. +8, in both operands (one consistent assignment of K to MFMA
// slots, so the products are unchanged). A lane therefore reads its pool row's whole
// granule 2 p + (lane / 32) once (one 16-byte read, both sub-steps), and its token
// row's chunk 4 p + 2 (lane / 32) + e per sub-step; every 16 lanes of a read cover all
// 64 LDS banks once.
struct SFrag {
    u32x4 a[2];    // the wavefront's 2 pool row tiles (raw FP8, 16 K values)
    bf16x8 b[2][2];  // [token tile][sub-step]
};

// ---- work plan of the bf16 / FP8 search -------------------------------------------------
// Pool blocks a token tile has to read: those whose first slot's position lies below the
// tile's largest token position (the pool is appended in position order). One
// wavefront per (tile, sequence).
__global__ __launch_bounds__(256) void search_plan_kernel(const int* __restrict__ pos, int n,
                                                          const int* __restrict__ ref_pos,
                                                          const int* __restrict__ ref_count, int cap_ref, int ntiles,
                                                          int* __restrict__ tile_nblk, int* __restrict__ rescan) {
    reset_rescan(rescan);
    const int lane = threadIdx.x & 63;
    const int tile = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int b = blockIdx.y;
    if (tile >= ntiles) return;
    const int t0 = tile * kTok;
    int mp = INT_MIN;
    for (int j = lane; j < kTok; j += 64)
        if (t0 + j < n) mp = max(mp, pos[(size_t)b * n + t0 + j]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mp = max(mp, __shfl_xor(mp, o, 64));
    const int count = max(0, min(ref_count[b], cap_ref));
    const int nbp = (count + s2::BM - 1) / s2::BM;
    int v = 0;
    for (int bb = lane; bb < nbp; bb += 64) v += ref_pos[(size_t)b * cap_ref + (size_t)bb * s2::BM] < mp ? 1 : 0;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    if (lane == 0) tile_nblk[(size_t)b * ntiles + tile] = v;
}

// Work queues: tile u (u = 0 .. B ntiles - 1; sequence u % B, tile ntiles - 1 - u / B, so the
// latest and heaviest tiles come first) contributes one item (u, c) per chunk c of bpc pool
// blocks it reads, to queue u % 8 (one queue per XCD: the chunks of a tile share its token
// rows in that XCD's L2). Wavefront q builds queue q and resets its counter.
__global__ __launch_bounds__(512) void search_queue_kernel(const int* __restrict__ tile_nblk, int B, int ntiles,
                                                           int bpc, int cap_q, int* __restrict__ items,
                                                           int* __restrict__ ctr) {
    const int lane = threadIdx.x & 63, q = threadIdx.x >> 6;
    const int U = B * ntiles;
    int base = 0;
    // pass 0: the full chunks of every tile; pass 1: the shorter last chunks (the queue ends
    // on the smallest items, which evens out when the workgroups finish)
    for (int pass = 0; pass < 2; ++pass) {
        for (int k0 = 0; q + 8 * k0 < U; k0 += 64) {
            const int u = q + 8 * (k0 + lane);
            int c0 = 0, nch = 0;
            if (u < U) {
                const int b = u % B, tile = ntiles - 1 - u / B;
                const int nb = tile_nblk[(size_t)b * ntiles + tile];
                const int full = nb / bpc;
                if (pass == 0) {
                    nch = full;
                } else {
                    c0 = full;
                    nch = (nb - full * bpc) > 0 ? 1 : 0;
                }
            }
            int incl = nch;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int t = __shfl_up(incl, o, 64);
                if (lane >= o) incl += t;
            }
            const int off = base + incl - nch;
            for (int c = 0; c < nch; ++c) items[(size_t)q * cap_q + off + c] = u * 16 + c0 + c;
            base += __shfl(incl, 63, 64);
        }
    }
    if (lane == 0) {
        ctr[2 * q] = 0;
        ctr[2 * q + 1] = base;
    }
}

// ---- few tokens per sequence (decode-time appends) --------------------------------------
// A token against its whole pool on the MFMA tiles leaves most of a 128-token tile empty and
// reads the pool through eight workgroups; with at most 4 tokens per sequence the pool is
// scanned instead by one wavefront per 16 slots, scores in fp32 FMAs (bf16 x FP8 products
// are exact in fp32, as in the MFMA path), then one workgroup per token keeps its 8 best.
// Row columns: chunk c (1024 columns), lane l holds columns 1024 c + 16 l .. +16.
// slots scored per wavefront by the pool scan (all their loads in flight at once)
constexpr int kScanSlots = 8;

template <int NC>
__global__ __launch_bounds__(256) void search_scan_kernel(const bf16_t* __restrict__ kv, int kv_len,
                                                          const int* __restrict__ rows, const int* __restrict__ pos,
                                                          int n, const fp8_t* __restrict__ ref_vals,
                                                          const int* __restrict__ ref_pos,
                                                          const float* __restrict__ ref_norm2,
                                                          const int* __restrict__ ref_count, int cap_ref,
                                                          float* __restrict__ scores, int* __restrict__ rescan) {
    constexpr int W2 = 1024 * NC;
    reset_rescan(rescan);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int b = blockIdx.y;
    const int count = max(0, min(ref_count[b], cap_ref));
    const int s0 = kScanSlots * (4 * blockIdx.x + wave);
    if (s0 >= count) return;
    float x[4][NC][16];
    int tp[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        tp[t] = INT_MIN;
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int e = 0; e < 16; ++e) x[t][c][e] = 0.f;
        if (t < n) {
            tp[t] = pos[(size_t)b * n + t];
            int kr = rows[(size_t)b * n + t];
            kr = (kr >= 0 && kr < kv_len) ? kr : 0;
            const bf16_t* xr = kv + ((size_t)b * kv_len + kr) * W2;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                Load8<bf16_t>::run(xr + 1024 * c + 16 * lane, &x[t][c][0]);
                Load8<bf16_t>::run(xr + 1024 * c + 16 * lane + 8, &x[t][c][8]);
            }
        }
    }
    const fp8_t* pool = ref_vals + (size_t)b * cap_ref * W2;
    float res[4] = {0.f, 0.f, 0.f, 0.f};  // lane r: dots of slot s0 + r
#pragma unroll
    for (int r = 0; r < kScanSlots; ++r) {
        const int sl = min(s0 + r, count - 1);
        float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const u32x4 raw = *reinterpret_cast<const u32x4*>(pool + (size_t)sl * W2 + 1024 * c + 16 * lane);
            float v[16];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float4 f = fp8x4_to_f32(raw[w]);
                v[4 * w] = f.x; v[4 * w + 1] = f.y; v[4 * w + 2] = f.z; v[4 * w + 3] = f.w;
            }
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int e = 0; e < 16; ++e) part[t] = fmaf(x[t][c][e], v[e], part[t]);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if (t < n) {
                const float d = wave_sum(part[t]);
                if (lane == r) res[t] = d;
            }
        }
    }
    const int sl = s0 + lane;
    if (lane < kScanSlots && sl < count) {
        const int rpos = ref_pos[(size_t)b * cap_ref + sl];
        const float nr = ref_norm2[(size_t)b * cap_ref + sl];
#pragma unroll
        for (int t = 0; t < 4; ++t)
            if (t < n) scores[((size_t)b * n + t) * cap_ref + sl] = rpos < tp[t] ? fmaf(-2.f, res[t], nr) : FLT_MAX;
    }
}

// The 8 best (score, slot) keys of one token over chunk blockIdx.x of its scanned pool (one
// workgroup per token and chunk; the pool is cut into gridDim.x equal chunks and each chunk's
// list goes to its own split, as the tiled search leaves them): each thread ranks its strided
// candidates in groups of 8, the lists merge across the lanes of a wavefront, then across the
// four wavefronts. Masked slots (FLT_MAX) leave as empty entries.
__global__ __launch_bounds__(256) void search_small_topk_kernel(const float* __restrict__ scores, int n,
                                                                const int* __restrict__ ref_count, int cap_ref,
                                                                int nsplit, float* __restrict__ part_score,
                                                                int* __restrict__ part_slot) {
    __shared__ uint64_t s_l[4][kTop];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ck = blockIdx.x, t = blockIdx.y, b = blockIdx.z;
    const int count = max(0, min(ref_count[b], cap_ref));
    const int cs = (count + gridDim.x - 1) / gridDim.x;
    const int c0 = ck * cs, c1 = min(count, c0 + cs);
    const float* sc = scores + ((size_t)b * n + t) * cap_ref;
    uint64_t lk[kTop];
#pragma unroll
    for (int q = 0; q < kTop; ++q) lk[q] = kNoKey;
    for (int g0 = c0; g0 < c1; g0 += 8 * 256) {
        uint64_t gk[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int sl = g0 + 256 * e + tid;
            gk[e] = sl < c1 ? score_key(sc[sl], sl) : kNoKey;
        }
        sort8(gk);
        merge8(lk, gk);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        uint64_t ok[kTop];
#pragma unroll
        for (int q = 0; q < kTop; ++q) {
            const int lo = __shfl_xor((int)(uint32_t)lk[q], o, 64);
            const int hi = __shfl_xor((int)(uint32_t)(lk[q] >> 32), o, 64);
            ok[q] = ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
        }
        merge8(lk, ok);
    }
    if (lane == 0) {
#pragma unroll
        for (int q = 0; q < kTop; ++q) s_l[wave][q] = lk[q];
    }
    __syncthreads();
    if (tid == 0) {
        uint64_t ak[kTop], bk[kTop];
#pragma unroll
        for (int q = 0; q < kTop; ++q) ak[q] = s_l[0][q];
#pragma unroll
        for (int w = 1; w < 4; ++w) {
#pragma unroll
            for (int q = 0; q < kTop; ++q) bk[q] = s_l[w][q];
            merge8(ak, bk);
        }
        const size_t o = (((size_t)b * n + t) * nsplit + ck) * kTop;
#pragma unroll
        for (int q = 0; q < kTop; ++q) {
            const float v = key_score(ak[q]);
            part_score[o + q] = v;
            part_slot[o + q] = v < FLT_MAX ? key_slot(ak[q]) : -1;
        }
    }
}

// Persistent search: one workgroup per CU takes items from its XCD's queue (blockIdx.x % 8,
// the hardware's round-robin placement), then from the other queues; an item scores token
// tile u against pool blocks c bpc .. + bpc and leaves one sorted top-8 per token.
template <typename KvT>
__global__ __launch_bounds__(s2::kThreads) void search_ring_kernel(
    const KvT* __restrict__ kv, int kv_len, const int* __restrict__ rows, const int* __restrict__ pos, int n,
    const fp8_t* __restrict__ ref_vals, const int* __restrict__ ref_pos, const float* __restrict__ ref_norm2,
    const int* __restrict__ ref_count, int W2, int cap_ref, int bpc, int nsplit, int ntiles, int B,
    const int* __restrict__ tile_nblk, const int* __restrict__ items, int cap_q, int* __restrict__ ctr,
    float* __restrict__ part_score, int* __restrict__ part_slot) {
    extern __shared__ __align__(16) unsigned char smem_u8[];
    char* smem = reinterpret_cast<char*>(smem_u8);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wq = wave & 3, wh = wave >> 2, hl = lane >> 5, l32 = lane & 31;
    const int wv = wave_id();
    const int nk = W2 / kStageK;
    int* s_item = reinterpret_cast<int*>(smem + s2::kOffRed);

    // next item code from queue q onwards (wavefront 0 claims, the workgroup reads it after
    // a barrier). `it` is an index already taken from queue q (the claim for the next item
    // is issued when an item starts, so its latency hides behind the item). When queue q is
    // exhausted, lanes 0-7 read all eight queues' counters at once (atomic loads: the
    // counters move under other CUs' claims) and the claim moves to the next one that still
    // holds items; a failed attempt only raises that queue's counter, so every workgroup
    // leaves once all queues are exhausted.
    int q = blockIdx.x & 7;
    int tot_q = ctr[2 * q + 1];
    auto claim = [&](int it) {
        if (tid < 64) {
            int code = -1;
            it = __shfl(it, 0, 64);
            bool done = false;
            if (it < tot_q) {
                code = items[(size_t)q * cap_q + it];
                done = true;
            }
            while (!done) {
                bool rem = false;
                if (lane < 8)
                    rem = __hip_atomic_load(&ctr[2 * lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
                          ctr[2 * lane + 1];
                const uint32_t m = (uint32_t)__ballot(rem) & 0xFFu;
                if (m == 0u) break;
                const uint32_t rot = ((m >> q) | (m << (8 - q))) & 0xFFu;
                q = (q + __ffs(rot) - 1) & 7;
                tot_q = ctr[2 * q + 1];
                int it2 = 0;
                if (lane == 0) it2 = atomicAdd(&ctr[2 * q], 1);
                it2 = __shfl(it2, 0, 64);
                if (it2 < tot_q) {
                    code = items[(size_t)q * cap_q + it2];
                    done = true;
                }
            }
            if (lane == 0) s_item[0] = code;
        }
    };
    int pend = 0;
    if (tid == 0) pend = atomicAdd(&ctr[2 * q], 1);
    claim(pend);
    __syncthreads();
    int code = s_item[0];

    while (code >= 0) {
        if (tid == 0) pend = atomicAdd(&ctr[2 * q], 1);
        const int u = code >> 4, split = code & 15;
        const int b = u % B, tile = ntiles - 1 - u / B;
        const int t0 = tile * kTok;
        const int count = max(0, min(ref_count[b], cap_ref));
        const int* rp = ref_pos + (size_t)b * cap_ref;
        const float* rn = ref_norm2 + (size_t)b * cap_ref;
        const int nblk = tile_nblk[(size_t)b * ntiles + tile];
        const int blk0 = split * bpc;
        const int blk1 = min(nblk, blk0 + bpc);

        int tokpos_l[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int t = t0 + 64 * wh + 32 * tt + l32;
            tokpos_l[tt] = (t < n) ? pos[(size_t)b * n + t] : INT_MIN;
        }
        uint64_t lk[2][kTop];  // per-token sorted lists of candidate keys
#pragma unroll
        for (int qq = 0; qq < 2; ++qq)
#pragma unroll
            for (int j = 0; j < kTop; ++j) lk[qq][j] = kNoKey;

        const char* pool = reinterpret_cast<const char*>(ref_vals + (size_t)b * cap_ref * W2);
        // pool loads: load u of wave w fills block w + 8 u (rows 16 (w + 8 u) ..), lane ->
        // row lane / 4 of it, granule position lane % 4
        int rowa[s2::kLoadsA];
        int cha[s2::kLoadsA];
#pragma unroll
        for (int v = 0; v < s2::kLoadsA; ++v) {
            rowa[v] = 16 * (wv + 8 * v) + (lane >> 2);
            cha[v] = 16 * swz(lane >> 2, lane & 3);
        }
        // token loads: load u of wave w fills block w + 8 u = 2 g + q
        const char* srcb[s2::kLoadsB];
#pragma unroll
        for (int v = 0; v < s2::kLoadsB; ++v) {
            const int blk = wv + 8 * v;
            const int r = 16 * (blk >> 1) + (lane >> 2);
            const int t = min(t0 + r, n - 1);
            int kr = rows[(size_t)b * n + t];
            kr = (kr >= 0 && kr < kv_len) ? kr : 0;
            srcb[v] = reinterpret_cast<const char*>(kv + ((size_t)b * kv_len + kr) * W2) + 64 * (blk & 1) +
                      16 * swz(lane >> 2, lane & 3);
        }
        // metadata loads (stage 0 of each block): waves 0-3 positions, 4-7 norms, 64 slots each
        const int msl = 64 * (wv & 3) + lane;
        const char* msrc = (wv < 4) ? reinterpret_cast<const char*>(rp) : reinterpret_cast<const char*>(rn);
        const int moff = (wv < 4 ? 0 : 1024) + 256 * (wv & 3);

        // issue cursor: next stage to load (block ib relative to blk0, K stage ik, ring slot is)
        int ib = 0, ik = 0, is = 0;
        const char* arow[s2::kLoadsA];
        auto set_block = [&](int bi) {
            const int base = (blk0 + bi) * s2::BM;
#pragma unroll
            for (int v = 0; v < s2::kLoadsA; ++v)
                arow[v] = pool + (size_t)min(base + rowa[v], cap_ref - 1) * W2 + cha[v];
        };
        set_block(0);
        auto issue = [&]() {
            char* sl = smem + is * s2::kSlot;
#pragma unroll
            for (int v = 0; v < s2::kLoadsA; ++v) dma16(arow[v] + ik * kStageK, sl + 1024 * (wv + 8 * v));
#pragma unroll
            for (int v = 0; v < s2::kLoadsB; ++v)
                dma16(srcb[v] + (size_t)ik * (kStageK * 2), sl + s2::kStageA + 1024 * (wv + 8 * v));
            if (ik == 0) {
                const int sl_m = min((blk0 + ib) * s2::BM + msl, cap_ref - 1);
                dma4(msrc + 4 * (size_t)sl_m, smem + s2::kOffMeta + (ib & (s2::kMetaBufs - 1)) * s2::kMeta + moff);
            }
            is = is + 1 == s2::NST ? 0 : is + 1;
            if (++ik == nk) {
                ik = 0;
                ++ib;
                set_block(ib);
            }
        };

        f32x16 acc[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

        // fragment reads of K half p of the stage in ring slot sl
        auto load = [&](SFrag& f, int sl, int p) {
            const char* sa = smem + sl * s2::kSlot;
            const char* sb = sa + s2::kStageA;
            const int r = l32 & 15;
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                const int g = 4 * wq + 2 * st + (l32 >> 4);
                f.a[st] = lds_load<u32x4>(sa + 1024 * g + 64 * r + 16 * swz(r, 2 * p + hl));
            }
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const int g = 4 * wh + 2 * tt + (l32 >> 4);
#pragma unroll
                for (int e = 0; e < 2; ++e)
                    f.b[tt][e] = lds_load<bf16x8>(sb + 1024 * (2 * g + p) + 64 * r + 16 * swz(r, 2 * hl + e));
            }
        };
        auto mma = [&](const SFrag& f) {
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
                for (int st = 0; st < 2; ++st) {
                    const bf16x8 wa = widen8(f.a[st][2 * e], f.a[st][2 * e + 1]);
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt)
                        acc[st][tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa, f.b[tt][e], acc[st][tt], 0, 0, 0);
                }
        };
        // lane's slots of a block: 64 wq + 32 st + 8 i + 4 hl + j (accumulator element 4 i + j)
        // A block's 32 candidates of a token are first ranked on 32-bit keys: the score's
        // order-preserving bits with the low 5 replaced by the candidate's index in the lane
        // (8 g + c, unique, slot order), i.e. scores rounded down by less than 32 ulps; a
        // masked candidate is 0xFFFFFFFF. The block's best 8 then join the token's list as
        // 64-bit (score, slot) keys. The select step widens its rounding margin to match.
        auto fold = [&](int bi) {
            const int blk = blk0 + bi;
            const char* mb = smem + s2::kOffMeta + (bi & (s2::kMetaBufs - 1)) * s2::kMeta;
            const int* m_pos = reinterpret_cast<const int*>(mb);
            const float* m_nrm = reinterpret_cast<const float*>(mb + 1024);
            const int lim = count - blk * s2::BM;  // slots at this offset and beyond are past the pool
            uint32_t bk[2][8];
            // The block's candidates as keys, best 8 per token. MASKED: with the causal mask
            // and the pool's end; without it when every candidate is visible to every token
            // of this wavefront (the block is full and its last slot, whose position is the
            // block's largest, lies before the wavefront's earliest token).
            auto block_keys = [&](auto masked) {
                constexpr bool kMasked = decltype(masked)::value;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    // group g: slot tile st = g / 2, rows i = 2 (g % 2) + {0, 1}
                    const int st = g >> 1;
                    int pe[8];
                    float ne[8];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int i = 2 * (g & 1) + h;
                        const int off = 64 * wq + 32 * st + 8 * i + 4 * hl;
                        const f32x4 n4 = lds_load<f32x4>(m_nrm + off);
                        if constexpr (kMasked) {
                            const i32x4 p4 = lds_load<i32x4>(m_pos + off);
#pragma unroll
                            for (int j = 0; j < 4; ++j) pe[4 * h + j] = (off + j < lim) ? p4[j] : INT_MAX;
                        }
#pragma unroll
                        for (int j = 0; j < 4; ++j) ne[4 * h + j] = n4[j];
                    }
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt) {
                        uint32_t gk[8];
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const int i = 2 * (g & 1) + h;
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                const int c = 4 * h + j;
                                uint32_t hb = __float_as_uint(fmaf(-2.f, acc[st][tt][4 * i + j], ne[c]));
                                hb ^= (uint32_t)((int)hb >> 31) | 0x80000000u;
                                const uint32_t key = (hb & ~31u) | (uint32_t)(8 * g + c);
                                if constexpr (kMasked) gk[c] = pe[c] < tokpos_l[tt] ? key : 0xFFFFFFFFu;
                                else gk[c] = key;
                            }
                        }
                        sort8_32(gk);
                        if (g == 0) {
#pragma unroll
                            for (int qq = 0; qq < 8; ++qq) bk[tt][qq] = gk[qq];
                        } else {
                            merge8_32(bk[tt], gk);
                        }
                    }
                    // keep each group's LDS reads next to their use
                    __builtin_amdgcn_sched_barrier(0);
                }
            };
            const bool vis =
                __all(lim >= s2::BM && m_pos[s2::BM - 1] < min(tokpos_l[0], tokpos_l[1]));
            if (vis) block_keys(std::false_type{});
            else block_keys(std::true_type{});
            // lane-local index x -> slot offset 64 wq + 4 (lane / 32) + 32 st + 8 i + j
            const uint32_t sbase = (uint32_t)(blk * s2::BM + 64 * wq + 4 * hl);
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                uint64_t gk[8];
#pragma unroll
                for (int qq = 0; qq < 8; ++qq) {
                    const uint32_t k = bk[tt][qq], x = k & 31u;
                    gk[qq] = k == 0xFFFFFFFFu ? kNoKey
                                              : ((uint64_t)(k & ~31u) << 32) | (sbase + x + (x & 0x1Cu));
                }
                if (bi == 0) {
#pragma unroll
                    for (int qq = 0; qq < kTop; ++qq) lk[tt][qq] = gk[qq];
                } else {
                    merge8(lk[tt], gk);
                }
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
        };

        // ring: stage s + NST is issued right after the barrier that follows the wait for
        // stage s + 1, into the slot stage s used (the LDS reads of one K half overlap the
        // MFMAs of the other)
        const int n_st = (blk1 - blk0) * nk;
        for (int p = 0; p < s2::NST; ++p)
            if (p < n_st) issue();
        if (n_st >= s2::NST) {
            wait_vmcnt<(s2::NST - 1) * s2::kPer>();
        } else {
            wait_vmcnt<0>();
        }
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        SFrag f0, f1;
        load(f0, 0, 0);
        int slot = 0, kin = 0, bi = 0;
        for (int s = 0; s + 1 < n_st; ++s) {
            load(f1, slot, 1);
            mma(f0);
            const int next = slot + 1 == s2::NST ? 0 : slot + 1;
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            wait_lgkm0();
            const int ahead = min(s2::NST - 2, n_st - 2 - s);
            if (ahead >= 2) {
                wait_vmcnt<2 * s2::kPer>();
            } else if (ahead == 1) {
                wait_vmcnt<s2::kPer>();
            } else {
                wait_vmcnt<0>();
            }
            __builtin_amdgcn_s_barrier();
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            if (s + s2::NST < n_st) issue();
            load(f0, next, 0);
            mma(f1);
            slot = next;
            if (++kin == nk) {
                kin = 0;
                fold(bi);
                ++bi;
            }
        }
        load(f1, slot, 1);
        mma(f0);
        mma(f1);
        fold(bi);

        // the next item is claimed while the lists are merged
        __syncthreads();
        claim(pend);
        // lanes l and l ^ 32 hold the same tokens: merge their lists in registers
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            uint64_t ok[kTop];
#pragma unroll
            for (int qq = 0; qq < kTop; ++qq) {
                const int lo = __shfl_xor((int)(uint32_t)lk[tt][qq], 32, 64);
                const int hi = __shfl_xor((int)(uint32_t)(lk[tt][qq] >> 32), 32, 64);
                ok[qq] = ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
            }
            merge8(lk[tt], ok);
        }
        // then the 4 slot quarters' lists through LDS, pairwise
        uint64_t* mK = reinterpret_cast<uint64_t*>(smem);
        if (hl == 0) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const int tk = 64 * wh + 32 * tt + l32;
#pragma unroll
                for (int qq = 0; qq < kTop; ++qq) mK[(wq * kTop + qq) * kTok + tk] = lk[tt][qq];
            }
        }
        __syncthreads();
        if (tid < 2 * kTok) {
            const int tk = tid & (kTok - 1), l0 = 2 * (tid >> 7);
            uint64_t ak[kTop], bk[kTop];
#pragma unroll
            for (int qq = 0; qq < kTop; ++qq) {
                ak[qq] = mK[(l0 * kTop + qq) * kTok + tk];
                bk[qq] = mK[((l0 + 1) * kTop + qq) * kTok + tk];
            }
            merge8(ak, bk);
#pragma unroll
            for (int qq = 0; qq < kTop; ++qq) mK[(l0 * kTop + qq) * kTok + tk] = ak[qq];
        }
        __syncthreads();
        if (tid < kTok && t0 + tid < n) {
            uint64_t ak[kTop], bk[kTop];
#pragma unroll
            for (int qq = 0; qq < kTop; ++qq) {
                ak[qq] = mK[qq * kTok + tid];
                bk[qq] = mK[(2 * kTop + qq) * kTok + tid];
            }
            merge8(ak, bk);
            const size_t o = (((size_t)b * n + t0 + tid) * nsplit + split) * kTop;
#pragma unroll
            for (int qq = 0; qq < kTop; ++qq) {
                const float sc = key_score(ak[qq]);
                part_score[o + qq] = sc;
                part_slot[o + qq] = sc < FLT_MAX ? key_slot(ak[qq]) : -1;
            }
        }
        code = s_item[0];
        __syncthreads();
    }
}

// ------------------------------------------------------------------ select + mean

// 8 consecutive values stored from floats (one 16-byte store for bf16, two for fp32)
template <typename XT>
__device__ inline void gstore8(XT* p, const float* v);
template <>
__device__ inline void gstore8<float>(float* p, const float* v) {
    reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}
template <>
__device__ inline void gstore8<bf16_t>(bf16_t* p, const float* v) {
    *reinterpret_cast<bf16x8*>(p) = Mma<bf16_t>::from_float(v);
}

// 64-bit minimum over the wavefront
__device__ inline uint64_t wave_min_u64(uint64_t v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, o, 64);
        const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), o, 64);
        const uint64_t w = ((uint64_t)hi << 32) | lo;
        v = w < v ? w : v;
    }
    // the same in every lane: keep it in scalar registers
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Squared L2 distance of one reference row to the token row, summed by one lane alone
// (eight partial sums over the columns, combined in a fixed tree): equal rows get equal
// distances, so an exact tie is left to the slot order.
template <typename KvT, typename RefT>
__device__ inline float lane_dist(const KvT* __restrict__ x, const RefT* __restrict__ r, int W2) {
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
    for (int c = 0; c < W2; c += 8) {
        float xv[8], rv[8];
        Load8<KvT>::run(x + c, xv);
        Load8<RefT>::run(r + c, rv);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float d = xv[e] - rv[e];
            a[e] = fmaf(d, d, a[e]);
        }
    }
    return ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
}

// 8 ints in ascending order (the 19-comparator network)
__device__ inline void sort8_i32(int (&k)[8]) {
#define RKV_C(x, y)                          \
    {                                        \
        const int lo = min(k[x], k[y]);      \
        const int hi = max(k[x], k[y]);      \
        k[x] = lo;                           \
        k[y] = hi;                           \
    }
    RKV_C(0, 2); RKV_C(1, 3); RKV_C(4, 6); RKV_C(5, 7);
    RKV_C(0, 4); RKV_C(1, 5); RKV_C(2, 6); RKV_C(3, 7);
    RKV_C(0, 1); RKV_C(2, 3); RKV_C(4, 5); RKV_C(6, 7);
    RKV_C(2, 4); RKV_C(3, 5);
    RKV_C(1, 4); RKV_C(3, 6);
    RKV_C(1, 2); RKV_C(3, 4); RKV_C(5, 6);
#undef RKV_C
}

// Reference mean of one token by one wavefront: fp32 sum in ascending slot order, one
// correctly rounded division, rounded to the KV dtype for the encoder. slots[0..k_i-1]
// hold the chosen slots in ascending order (the same in every lane). A null row: the
// encoder takes the mean from the references' projections and needs no mean row.
template <typename KvT, typename RefT>
__device__ inline void write_mean(const RefT* __restrict__ pool, const int (&slots)[8], int k_i, int W2,
                                  KvT* __restrict__ xrow, int lane) {
    if (!xrow) return;
    const float kf = (float)k_i;
    const float rk = __fdiv_rn(1.0f, k_i > 0 ? kf : 1.0f);
#pragma unroll 2
    for (int c = 8 * lane; c < W2; c += 512) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            if (q < k_i) {
                float v[8];
                Load8<RefT>::run(pool + (size_t)slots[q] * W2 + c, v);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] += v[e];
            }
        }
        if (k_i > 1) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if constexpr (std::is_same<RefT, fp8_t>::value) {
                    acc[e] = div_small(acc[e], kf, rk);
                } else {  // fp32 references: general sums, IEEE division
                    acc[e] = __fdiv_rn(acc[e], kf);
                }
            }
        }
        gstore8<KvT>(xrow + c, acc);
    }
}

// One wavefront per token; 4 tokens per block. Row accesses take 8 columns per lane
// (chunks of 512 columns).
//
// Every chunk list holds the chunk's best 8 candidates by approximate score (rounded
// down, ties by slot). Three cases decide the set:
//  * the approximate boundary is clear of the rounding bound and no list can have
//    dropped a member: the k_i best candidates by approximate score;
//  * the boundary is ambiguous among the stored candidates: exact distances for the
//    candidates the bounds cannot place (counted in stats[0]);
//  * a full list's 8th score comes within the bound of the set's largest exact
//    distance, so a slot the list dropped could belong to the set: the token goes to
//    the rescan queue (two words from rescan[kRqHead]: the token, and the mask of such
//    lists | the number of lists << 8), and rescan_kernel writes its references and
//    mean row (counted in stats[1]).
template <typename KvT, typename RefT>
__global__ __launch_bounds__(kThreads) void select_kernel(
    const KvT* __restrict__ kv, int kv_len, const int* __restrict__ rows, const int* __restrict__ pos, int n,
    const RefT* __restrict__ ref_vals, const float* __restrict__ ref_norm2, const float* __restrict__ part_score,
    const int* __restrict__ part_slot, int nsplit, int nch_fixed, const int* __restrict__ tile_nblk, int bpc, int W2,
    int cap_ref, int cap_tok, int top_k, int* __restrict__ ref_idx, KvT* __restrict__ xbar, int* rescan, int* err,
    int* stats) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int b = blockIdx.y;
    if (t >= n) return;
    const int row = rows[(size_t)b * n + t];
    const int p = pos[(size_t)b * n + t];
    const bool row_ok = row >= 0 && row < kv_len;
    const bool pos_ok = p >= 0 && p < cap_tok;
    KvT* xrow = xbar ? xbar + ((size_t)b * n + t) * W2 : nullptr;
    if (!row_ok || !pos_ok) {
        if (lane == 0) flag_error(err, (row_ok ? 0 : DEVERR_ROW_RANGE) | (pos_ok ? 0 : DEVERR_POS_RANGE));
        const float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int c = 8 * lane; c < W2; c += 512) gstore8<KvT>(xrow + c, z);
        return;
    }
    const KvT* x = kv + ((size_t)b * kv_len + row) * W2;
    const RefT* pool = ref_vals + (size_t)b * cap_ref * W2;
    // the first chunks of the token's row are loaded before the candidates are ranked, so
    // their latency overlaps the ranking
    constexpr int kPre = 4;
    float xv[kPre][8];
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
        const int c = 8 * lane + 512 * u;
        if (c < W2) {
            Load8<KvT>::run(x + c, xv[u]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) xv[u][e] = 0.f;
        }
    }

    // gather the chunks' candidates, one per lane (with a work plan, only the chunks of
    // pool blocks the token's tile read hold lists)
    int nch = nch_fixed;
    if (tile_nblk) {
        const int ntiles = (n + kTok - 1) / kTok;
        nch = min(nsplit, (tile_nblk[(size_t)b * ntiles + t / kTok] + bpc - 1) / bpc);
    }
    const int ncand = nch * kTop;  // <= 64
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
        const float sj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), j));
        const int ij = __builtin_amdgcn_readlane(key_id, j);
        rank += (sj < s || (sj == s && ij < key_id)) ? 1 : 0;
    }
    const unsigned long long valid_mask = __ballot(id >= 0);
    const int nvalid = __popcll(valid_mask);
    const int k_i = min(top_k, nvalid);

    // bound on the error of an approximate score: 2^-17 (||x||^2 + ||r||^2) for the fp32
    // accumulation of the MFMA path, and as much again for the 32-ulp rounding of its
    // block-level ranking keys (|score| <= 2 (||x||^2 + ||r||^2))
    float xn = 0.f;
#pragma unroll
    for (int u = 0; u < kPre; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) xn = fmaf(xv[u][e], xv[u][e], xn);
    for (int c = 8 * lane + 512 * kPre; c < W2; c += 512) {
        float v[8];
        Load8<KvT>::run(x + c, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) xn = fmaf(v[e], v[e], xn);
    }
    xn = wave_sum(xn);
    const float nr = (id >= 0) ? ref_norm2[(size_t)b * cap_ref + id] : 0.f;
    const float margin = 1.52587890625e-05f * (xn + nr);  // 2^-16
    const bool in_set = id >= 0 && rank < k_i;
    // highest (score + margin) inside the set vs lowest (score - margin) outside it
    float hi_in = in_set ? s + margin : -FLT_MAX;
    float lo_out = (id >= 0 && !in_set) ? s - margin : FLT_MAX;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        hi_in = fmaxf(hi_in, __shfl_xor(hi_in, o, 64));
        lo_out = fminf(lo_out, __shfl_xor(lo_out, o, 64));
    }

    // A slot a full list dropped ranks after the list's 8th on the same rounded-down keys,
    // so its approximate score is at least the 8th's stored score, and its exact score at
    // least that minus its accumulation error, 2^-17 (||x||^2 + ||r||^2). If it could
    // belong to the set its exact score is at most hi_in, so its distance is at most
    // dmax = hi_in + ||x||^2 and ||r||^2 <= 2 ||x||^2 + 2 dmax. A list whose 8th score minus
    // 2^-17 (3 ||x||^2 + 2 dmax) (rounded up to 1e-5, for the score's own rounding) stays
    // above hi_in cannot hide a member of the set.
    bool hides = false;
    if (k_i > 0 && lane < ncand && (lane & (kTop - 1)) == kTop - 1 && id >= 0) {
        const float dmax = fmaxf(hi_in + xn, 0.f);
        hides = s - 1.0e-5f * (3.f * xn + 2.f * dmax) <= hi_in;
    }
    const unsigned long long hide_mask = __ballot(hides);

    if (hide_mask) {
        // the exact search over whole chunks runs in rescan_kernel, which then writes this
        // token's references and mean row
        if (lane == 0) {
            const int slot = atomicAdd(&rescan[0], 1);
            rescan[kRqHead + 2 * slot] = b * n + t;
            uint32_t cm = 0;
#pragma unroll
            for (int c = 0; c < 8; ++c) cm |= ((hide_mask >> (kTop * c + kTop - 1)) & 1ull) ? (1u << c) : 0u;
            rescan[kRqHead + 1 + 2 * slot] = (int)(cm | ((uint32_t)nch << 8));
            if (stats) atomicAdd(&stats[1], 1);
        }
        return;
    }
    int slots[8];  // the chosen slots in ascending order, -1 padded (the same in every lane)
    {
        bool chosen = in_set;
        if (k_i > 0 && lo_out <= hi_in) {
            // ambiguous boundary. A candidate of the set whose score plus margin lies below
            // every outside candidate's score minus margin is closer than all of them in
            // exact arithmetic too, so it stays; one outside whose score minus margin lies
            // above every set member's score plus margin has k_i closer candidates and
            // stays out. The rest get exact fp32 squared distances; the free places of the
            // set go to the best of them by (exact distance, slot).
            if (lane == 0 && stats) atomicAdd(&stats[0], 1);
            const bool sure_in = in_set && s + margin < lo_out;
            const bool sure_out = !in_set && s - margin > hi_in;
            const bool amb = id >= 0 && !sure_in && !sure_out;
            const unsigned long long am = __ballot(amb);
            float dist = FLT_MAX;
            for (unsigned long long mq = am; mq; mq &= mq - 1) {
                const int src = __ffsll((long long)mq) - 1;
                const int sq = __shfl(id, src, 64);
                float acc = 0.f;
                const RefT* r = pool + (size_t)sq * W2;
                for (int c = 4 * lane; c < W2; c += 256) {
                    const float4 xv = Load4<KvT>::run(x + c);
                    const float4 rv = Load4<RefT>::run(r + c);
                    const float d0 = xv.x - rv.x, d1 = xv.y - rv.y, d2 = xv.z - rv.z, d3 = xv.w - rv.w;
                    acc += (d0 * d0 + d1 * d1) + (d2 * d2 + d3 * d3);
                }
                acc = wave_sum(acc);
                if (lane == src) dist = acc;
            }
            int arank = 0;
            for (unsigned long long mq = am; mq; mq &= mq - 1) {
                const int src = __ffsll((long long)mq) - 1;
                const float dj = __shfl(dist, src, 64);
                const int ij = __shfl(key_id, src, 64);
                arank += (dj < dist || (dj == dist && ij < key_id)) ? 1 : 0;
            }
            const int nsure = __popcll(__ballot(sure_in));
            chosen = sure_in || (amb && arank < k_i - nsure);
        }
        // chosen slots in ascending slot order
        int srank = 0;
        const unsigned long long cm = __ballot(chosen);
        for (int j = 0; j < 64; ++j) {
            if (!((cm >> j) & 1ull)) continue;
            const int ij = __shfl(id, j, 64);
            srank += (chosen && ij < id) ? 1 : 0;
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const unsigned long long mq = __ballot(chosen && srank == q);
            slots[q] = mq ? __shfl(id, __ffsll((long long)mq) - 1, 64) : -1;
        }
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
    write_mean<KvT, RefT>(pool, slots, k_i, W2, xrow, lane);
}

// wave-uniform ascending list best[0..7] of (distance, slot) keys: merge one key per lane
__device__ inline void offer_keys(uint64_t (&best)[8], uint64_t mine) {
    uint64_t kth = best[7];
    // keys enter in ascending order, so at most 8 of them enter per call
    for (;;) {
        const uint64_t m = wave_min_u64(mine);
        if (m >= kth) break;
        uint64_t v = m;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const uint64_t lo = best[q] < v ? best[q] : v;
            const uint64_t hi = best[q] < v ? v : best[q];
            best[q] = lo;
            v = hi;
        }
        if (mine == m) mine = ~0ull;
        kth = best[7];
    }
}

// exact (distance, slot) key of one reference row, or none
template <typename KvT, typename RefT>
__device__ inline uint64_t exact_key(bool ok, const KvT* x, const RefT* pool, int slot, int W2) {
    if (!ok) return ~0ull;
    const float d = lane_dist<KvT, RefT>(x, pool + (size_t)slot * W2, W2);
    return ((uint64_t)__float_as_uint(d) << 32) | (uint32_t)slot;
}

// the four wavefronts' lists merged through LDS; the result in wavefront 0
__device__ inline void merge_waves(uint64_t (&best)[8], uint64_t (*s_best)[8]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane < 8) {
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (q == lane) s_best[wave][q] = best[q];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int q = 0; q < 8; ++q) best[q] = ~0ull;
        offer_keys(best, lane < 32 ? s_best[lane >> 3][lane & 7] : ~0ull);
    }
}

// The token's references (the top_k smallest keys of `best`, in ascending slot order) and
// mean row, by wavefront 0.
template <typename KvT, typename RefT>
__device__ inline void write_set(const uint64_t (&best)[8], int top_k, const RefT* pool, int W2, int* out_idx,
                                 KvT* xrow) {
    const int lane = threadIdx.x & 63;
    int sl8[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) sl8[q] = (q < top_k && best[q] != ~0ull) ? (int)(uint32_t)best[q] : INT_MAX;
    sort8_i32(sl8);
    int slots[8];
    int kk = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        slots[q] = sl8[q] == INT_MAX ? -1 : sl8[q];
        kk += slots[q] >= 0 ? 1 : 0;
    }
    if (lane < top_k) {
        int v = -1;
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (q == lane) v = slots[q];
        out_idx[lane] = v;
    }
    write_mean<KvT, RefT>(pool, slots, kk, W2, xrow, lane);
}

// Exact search of the tokens select_kernel queued: exact squared distances (one lane per
// reference row, lane_dist) over every visible slot of the chunks whose lists could hide
// a member of the set and over the stored candidates of the other chunks; the top_k
// smallest (distance, slot) keys are the token's references (ascending slot) and give its
// mean row. A chunk list that could hide a member holds 8 visible slots, so k_i = top_k.
//   queued tokens 0 .. kRqPar - 1: kRqParts parts each (work item = token x part, spread
//     over the grid); a part scans its share of the slots and writes its best 8 keys to
//     part_keys; the part that arrives last (an atomic counter per token, after a device
//     fence) merges the kRqParts lists and writes the result;
//   later queued tokens: one workgroup each scans all of the token's slots.
template <typename KvT, typename RefT>
__global__ __launch_bounds__(256) void rescan_kernel(
    const KvT* __restrict__ kv, int kv_len, const int* __restrict__ rows, const int* __restrict__ pos, int n,
    const RefT* __restrict__ ref_vals, const int* __restrict__ ref_pos, const int* __restrict__ ref_count,
    const int* __restrict__ part_slot, int nsplit, int chunk_len, int W2, int cap_ref, int cap_tok, int top_k,
    int* __restrict__ ref_idx, KvT* __restrict__ xbar, int* __restrict__ rescan, uint64_t* __restrict__ part_keys) {
    __shared__ uint64_t s_best[4][8];
    __shared__ int s_last;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nq = rescan[0];
    const int npar = min(nq, kRqPar);

    // the scan of queued token e: its chunks' slots as one list of S slots (hiding chunks in
    // order), parts [part S / P, (part + 1) S / P); part 0 also offers the stored candidates
    struct Tok {
        int b, t, p, nch, cl, count;
        uint32_t hmask;
        const KvT* x;
        const RefT* pool;
        const int* rp;
    };
    auto token = [&](int e) {
        Tok k;
        const int code = rescan[kRqHead + 2 * e];
        const uint32_t info = (uint32_t)rescan[kRqHead + 1 + 2 * e];
        k.b = code / n;
        k.t = code - k.b * n;
        const int row = rows[(size_t)k.b * n + k.t];
        k.p = pos[(size_t)k.b * n + k.t];
        k.x = kv + ((size_t)k.b * kv_len + row) * W2;  // select queued only tokens with valid rows
        k.pool = ref_vals + (size_t)k.b * cap_ref * W2;
        k.rp = ref_pos + (size_t)k.b * cap_ref;
        k.hmask = info & 0xFFu;
        k.nch = (int)(info >> 8);
        k.count = max(0, min(ref_count[k.b], cap_ref));
        k.cl = chunk_len > 0 ? chunk_len : (k.count + k.nch - 1) / max(k.nch, 1);
        return k;
    };
    auto scan_len = [&](const Tok& k) {
        int S = 0;
        for (uint32_t mq = k.hmask; mq; mq &= mq - 1) {
            const int c = __ffs(mq) - 1;
            S += max(0, min(k.count, (c + 1) * k.cl) - c * k.cl);
        }
        return S;
    };
    // slot of position i of the scan list
    auto scan_slot = [&](const Tok& k, int i) {
        for (uint32_t mq = k.hmask; mq; mq &= mq - 1) {
            const int c = __ffs(mq) - 1;
            const int len = max(0, min(k.count, (c + 1) * k.cl) - c * k.cl);
            if (i < len) return c * k.cl + i;
            i -= len;
        }
        return -1;
    };
    auto offer_stored = [&](const Tok& k, uint64_t (&best)[8]) {
        // stored candidates of the lists that cannot hide a member (wavefront 0, a lane each)
        if (wave == 0) {
            const int c = lane / kTop;
            const bool ok = lane < k.nch * kTop && !((k.hmask >> c) & 1u);
            const int id = ok ? part_slot[((size_t)k.b * n + k.t) * nsplit * kTop + lane] : -1;
            offer_keys(best, exact_key<KvT, RefT>(id >= 0, k.x, k.pool, id, W2));
        }
    };
    auto scan = [&](const Tok& k, int lo, int hi, uint64_t (&best)[8]) {
        for (int i0 = lo + 64 * wave; i0 < hi; i0 += 256) {
            const int i = i0 + lane;
            const int sl = i < hi ? scan_slot(k, i) : -1;
            offer_keys(best, exact_key<KvT, RefT>(sl >= 0 && k.rp[sl] < k.p, k.x, k.pool, sl, W2));
        }
    };

    // parallel rescans
    for (int w = blockIdx.x; w < npar * kRqParts; w += gridDim.x) {
        const int e = w / kRqParts, part = w - e * kRqParts;
        const Tok k = token(e);
        const int S = scan_len(k);
        uint64_t best[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) best[q] = ~0ull;
        if (part == 0) offer_stored(k, best);
        scan(k, (int)((long long)S * part / kRqParts), (int)((long long)S * (part + 1) / kRqParts), best);
        merge_waves(best, s_best);
        uint64_t* mine = part_keys + ((size_t)e * kRqParts + part) * 8;
        if (wave == 0 && lane < 8) {
#pragma unroll
            for (int q = 0; q < 8; ++q)
                if (q == lane) mine[q] = best[q];
        }
        __threadfence();
        __syncthreads();
        if (tid == 0) s_last = atomicAdd(&rescan[2 + e], 1) == kRqParts - 1;
        __syncthreads();
        if (s_last) {
            __threadfence();
            if (wave == 0) {
#pragma unroll
                for (int q = 0; q < 8; ++q) best[q] = ~0ull;
                const uint64_t* all = part_keys + (size_t)e * kRqParts * 8;
                for (int j = 0; j < kRqParts * 8; j += 64) offer_keys(best, all[j + lane]);
                write_set<KvT, RefT>(best, top_k, k.pool, W2, ref_idx + ((size_t)k.b * cap_tok + k.p) * top_k,
                                     xbar ? xbar + ((size_t)k.b * n + k.t) * W2 : nullptr);
            }
        }
        __syncthreads();
    }
    // later queued tokens: one workgroup each
    for (int e = npar + blockIdx.x; e < nq; e += gridDim.x) {
        const Tok k = token(e);
        uint64_t best[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) best[q] = ~0ull;
        offer_stored(k, best);
        scan(k, 0, scan_len(k), best);
        merge_waves(best, s_best);
        if (wave == 0)
            write_set<KvT, RefT>(best, top_k, k.pool, W2, ref_idx + ((size_t)k.b * cap_tok + k.p) * top_k,
                                 xbar ? xbar + ((size_t)k.b * n + k.t) * W2 : nullptr);
        __syncthreads();
    }
}

}  // namespace

EncodePlan plan_encode(const Shape& s, int B, int n, int cap_ref) {
    EncodePlan p{};
    const int BM = s.f32 ? SC<float>::BM : SC<bf16_t>::BM;
    const int nblocks = (cap_ref + BM - 1) / BM;
    int bpc = (nblocks + 7) / 8;
    if (bpc < 2) bpc = 2;
    int nsplit = (nblocks + bpc - 1) / bpc;
    if (nsplit < 1) nsplit = 1;
    p.nsplit = nsplit;
    p.chunk_slots = bpc;  // pool blocks per chunk
    const size_t tok = (size_t)B * n;
    auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
    size_t off = 0;
    // work plan of the bf16 search: blocks per tile, 8 item queues, their counters
    const size_t units = (size_t)B * ((n + kTok - 1) / kTok);
    p.cap_q = (int)((units + 7) / 8) * nsplit;
    p.off_tile_nblk = off;
    off = up(off + units * sizeof(int));
    p.off_items = off;
    off = up(off + (size_t)8 * p.cap_q * sizeof(int));
    p.off_ctr = off;
    off = up(off + 16 * sizeof(int));
    // few tokens per sequence: the pool is scanned (scores [B][n][cap_ref] fp32)
    p.small = !s.f32 && n <= 4 && (s.W2 == 1024 || s.W2 == 2048);
    p.off_scores = off;
    if (p.small) off = up(off + (size_t)B * n * cap_ref * sizeof(float));
    p.off_part_score = off;
    off = up(off + tok * nsplit * kTop * sizeof(float));
    p.off_part_slot = off;
    off = up(off + tok * nsplit * kTop * sizeof(int));
    p.off_rescan = off;  // select's rescan queue (kRqHead words, then 2 per token)
    off = up(off + (kRqHead + 2 * tok) * sizeof(int));
    p.off_rescan_part = off;  // partial lists of the parallel rescans
    off = up(off + (size_t)kRqPar * kRqParts * 8 * sizeof(uint64_t));
    p.off_xbar = off;  // mean rows (none in the mean-projection form)
    if (!s.mproj) off = up(off + tok * s.W2 * (s.f32 ? 4 : 2));
    p.off_dh = off;
    // dH: fp32 rows (fp32 formats) or three bf16 planes per row (bf16 formats)
    off = up(off + tok * s.d_ff * (s.f32 ? 4 : 6));
    p.total = off;
    return p;
}

template <typename T, typename KvT, typename RefT>
static hipError_t search_impl(const Shape& s, const CacheView& c, const EncodePlan& p, const void* kv, int kv_len,
                              const int* rows, const int* pos, int n, void* ws, hipStream_t st) {
    const size_t smem = SC<T>::bytes;
    auto kern = search_kernel<T, KvT, RefT>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    char* w = static_cast<char*>(ws);
    const int ntiles = (n + kTok - 1) / kTok;
    const int per = ((ntiles + 7) / 8) * p.nsplit;  // blocks per XCD
    hipLaunchKernelGGL(kern, dim3(8 * per, c.B), dim3(kThreads), smem, st, static_cast<const KvT*>(kv), kv_len, rows,
                       pos, n, static_cast<const RefT*>(c.ref_vals), c.ref_pos, c.ref_norm2, c.ref_count, s.W2,
                       c.cap_ref, p.chunk_slots, p.nsplit, ntiles, per, reinterpret_cast<float*>(w + p.off_part_score),
                       reinterpret_cast<int*>(w + p.off_part_slot), reinterpret_cast<int*>(w + p.off_rescan));
    return hipGetLastError();
}

// compute units of the current device (cached per device)
static int device_cus() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
        cus[dev] = v;
    }
    return cus[dev];
}

static hipError_t search_ring_impl(const Shape& s, const CacheView& c, const EncodePlan& p, const void* kv,
                                   int kv_len, const int* rows, const int* pos, int n, void* ws, hipStream_t st) {
    const size_t smem = s2::bytes;
    auto kern = search_ring_kernel<bf16_t>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    char* w = static_cast<char*>(ws);
    const int ntiles = (n + kTok - 1) / kTok;
    int* tile_nblk = reinterpret_cast<int*>(w + p.off_tile_nblk);
    int* items = reinterpret_cast<int*>(w + p.off_items);
    int* ctr = reinterpret_cast<int*>(w + p.off_ctr);
    hipLaunchKernelGGL(search_plan_kernel, dim3((ntiles + 3) / 4, c.B), dim3(256), 0, st, pos, n, c.ref_pos,
                       c.ref_count, c.cap_ref, ntiles, tile_nblk, reinterpret_cast<int*>(w + p.off_rescan));
    hipLaunchKernelGGL(search_queue_kernel, dim3(1), dim3(512), 0, st, tile_nblk, c.B, ntiles, p.chunk_slots, p.cap_q,
                       items, ctr);
    // one workgroup per CU (the LDS of one fills a CU), never more than there are items
    const long long max_items = (long long)c.B * ntiles * p.nsplit;
    const int grid = (int)std::min<long long>(device_cus(), max_items);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(s2::kThreads), smem, st, static_cast<const bf16_t*>(kv), kv_len, rows,
                       pos, n, static_cast<const fp8_t*>(c.ref_vals), c.ref_pos, c.ref_norm2, c.ref_count, s.W2,
                       c.cap_ref, p.chunk_slots, p.nsplit, ntiles, c.B, tile_nblk, items, p.cap_q, ctr,
                       reinterpret_cast<float*>(w + p.off_part_score), reinterpret_cast<int*>(w + p.off_part_slot));
    return hipGetLastError();
}

// pool chunks of the few-token top-k: as many as the candidate splits allow, at most 8
// (the select step merges at most 64 candidates)
static int small_chunks(const EncodePlan& p) { return max(1, min(8, p.nsplit)); }

static hipError_t search_small_impl(const Shape& s, const CacheView& c, const EncodePlan& p, const void* kv,
                                    int kv_len, const int* rows, const int* pos, int n, void* ws, hipStream_t st) {
    char* w = static_cast<char*>(ws);
    float* scores = reinterpret_cast<float*>(w + p.off_scores);
    const dim3 grid((c.cap_ref + 4 * kScanSlots - 1) / (4 * kScanSlots), c.B);
    if (s.W2 == 2048) {
        hipLaunchKernelGGL(search_scan_kernel<2>, grid, dim3(256), 0, st, static_cast<const bf16_t*>(kv), kv_len, rows,
                           pos, n, static_cast<const fp8_t*>(c.ref_vals), c.ref_pos, c.ref_norm2, c.ref_count,
                           c.cap_ref, scores, reinterpret_cast<int*>(w + p.off_rescan));
    } else {
        hipLaunchKernelGGL(search_scan_kernel<1>, grid, dim3(256), 0, st, static_cast<const bf16_t*>(kv), kv_len, rows,
                           pos, n, static_cast<const fp8_t*>(c.ref_vals), c.ref_pos, c.ref_norm2, c.ref_count,
                           c.cap_ref, scores, reinterpret_cast<int*>(w + p.off_rescan));
    }
    hipLaunchKernelGGL(search_small_topk_kernel, dim3(small_chunks(p), n, c.B), dim3(256), 0, st, scores, n,
                       c.ref_count, c.cap_ref,
                       p.nsplit, reinterpret_cast<float*>(w + p.off_part_score),
                       reinterpret_cast<int*>(w + p.off_part_slot));
    return hipGetLastError();
}

hipError_t launch_search(const Shape& s, const CacheView& c, const EncodePlan& p, const void* kv, int kv_len,
                         const int* rows, const int* pos, int n, void* ws, hipStream_t st) {
    if (s.f32) return search_impl<float, float, float>(s, c, p, kv, kv_len, rows, pos, n, ws, st);
    if (p.small) return search_small_impl(s, c, p, kv, kv_len, rows, pos, n, ws, st);
    return search_ring_impl(s, c, p, kv, kv_len, rows, pos, n, ws, st);
}

template <typename KvT, typename RefT>
static hipError_t select_impl(const Shape& s, const CacheView& c, const EncodePlan& p, const void* kv, int kv_len,
                              const int* rows, const int* pos, int n, void* ws, hipStream_t st) {
    char* w = static_cast<char*>(ws);
    int* rescan = reinterpret_cast<int*>(w + p.off_rescan);
    KvT* xbar = s.mproj ? nullptr : reinterpret_cast<KvT*>(w + p.off_xbar);
    const int* part_slot = reinterpret_cast<const int*>(w + p.off_part_slot);
    const dim3 grid((n + 3) / 4, c.B);
    hipLaunchKernelGGL((select_kernel<KvT, RefT>), grid, dim3(kThreads), 0, st, static_cast<const KvT*>(kv), kv_len,
                       rows, pos, n, static_cast<const RefT*>(c.ref_vals), c.ref_norm2,
                       reinterpret_cast<const float*>(w + p.off_part_score), part_slot, p.nsplit,
                       p.small ? small_chunks(p) : p.nsplit,
                       (s.f32 || p.small) ? nullptr : reinterpret_cast<const int*>(w + p.off_tile_nblk), p.chunk_slots,
                       s.W2, c.cap_ref, c.cap_tok, s.top_k, c.ref_idx, xbar, rescan, c.err, c.stats);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // queued tokens (usually none): a grid of workgroups walks the queue
    const int chunk_len = p.small ? 0 : p.chunk_slots * (s.f32 ? SC<float>::BM : s2::BM);
    const int grid_r = (int)std::min<long long>(256, (long long)c.B * n * kRqParts);
    hipLaunchKernelGGL((rescan_kernel<KvT, RefT>), dim3(grid_r), dim3(256), 0, st, static_cast<const KvT*>(kv),
                       kv_len, rows, pos, n, static_cast<const RefT*>(c.ref_vals), c.ref_pos, c.ref_count, part_slot,
                       p.nsplit, chunk_len, s.W2, c.cap_ref, c.cap_tok, s.top_k, c.ref_idx, xbar, rescan,
                       reinterpret_cast<uint64_t*>(w + p.off_rescan_part));
    return hipGetLastError();
}

hipError_t launch_select(const Shape& s, const CacheView& c, const EncodePlan& p, const void* kv, int kv_len,
                         const int* rows, const int* pos, int n, void* ws, hipStream_t st) {
    if (s.f32) return select_impl<float, float>(s, c, p, kv, kv_len, rows, pos, n, ws, st);
    return select_impl<bf16_t, fp8_t>(s, c, p, kv, kv_len, rows, pos, n, ws, st);
}

}  // namespace rkv
