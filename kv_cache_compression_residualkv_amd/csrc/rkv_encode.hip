// SwiGLU residual encoder and per-token group quantizer.
//
// ResidualKV review page, section 2.3: f_c(x) = (Swish(x W_c1) * x W_c2) W_c3 and the
// stored residual is z = f_c(kv_i) - f_c(mean_i) (average first, then encode);
// section 2.4: per-token groups of 32 latent coordinates with
// Delta = (max - min)/(2^b - 1), q = round((z - min)/Delta).
//
// Since W_c3 is linear, z = (h(kv_i) - h(mean_i)) W_c3 with h(x) = Swish(x W_c1) * x W_c2.
//   swiglu_kernel       GEMM [kv_i; mean_i] x [W_c1 | W_c2]^T. Rows of a tile alternate
//                       kv_i / mean_i of one token and the B tile interleaves W_c1
//                       and W_c2 columns, so one lane ends with a, g of both rows:
//                       dH = h(kv_i) - h(mean_i) is formed in registers, staged in
//                       LDS and written coalesced. In the bf16 formats dH is written
//                       as three bf16 terms hi + mid + lo (24 significant bits), the
//                       three "planes" of a row of width 3 d_ff.
//   latent_quant_kernel z = dH W_c3 as one bf16 GEMM over K' = 3 d_ff (each plane times
//                       W_c3); the epilogue reduces each group's min/max over the 16
//                       lanes that hold it, stores Delta and min, and packs the codes
//                       through LDS into coalesced record writes.
#include <float.h>

#include <algorithm>

#include "rkv_device.h"
#include "rkv_gemm.h"
#include "rkv_internal.h"
#include "rkv_pipe.h"
#include "rkv_swish.h"

namespace rkv {

namespace {

// ---------------------------------------------------------------- GEMM 1

template <typename T>
struct G1 {
    // bf16: 256 rows (128 tokens) x 128 columns (64 W_c1 + 64 W_c2); fp32: half the rows
    static constexpr int BM = std::is_same<T, float>::value ? 128 : 256;
    static constexpr int BN = 128;
    static constexpr int WM = BM / 2, WN = 64;
    static constexpr int NS = std::is_same<T, float>::value ? 1 : 3;  // dH planes
    static constexpr int P = Pitch<T, kKC>::value;
    static constexpr int kHP = 68;  // fp32 pitch of the dH staging tile
    static constexpr size_t kPipe = (size_t)2 * (BM + BN) * P * sizeof(T);
    static constexpr size_t kEpi = (size_t)(BM / 2) * kHP * sizeof(float);
    static constexpr size_t bytes = kPipe > kEpi ? kPipe : kEpi;
};

template <typename T, int BM>
struct G1LoadA {
    RowTile<T, T, BM> t;
    const T* row[BM / 128];
    __device__ inline void load(int s) { t.load_rows(row, s * kKC); }
    __device__ inline void store(T* lds, int P) const { t.store(lds, P); }
};

template <typename T>
struct G1LoadB {
    RowTile<T, T, 128> t;
    const T* row[1];
    __device__ inline void load(int s) { t.load_rows(row, s * kKC); }
    __device__ inline void store(T* lds, int P) const { t.store(lds, P); }
};

// grid: 8 * per blocks over MT x NT logical tiles (N tiles fastest, so the NT tiles
// that read one A row block run back to back on one XCD).
template <typename T>
__global__ __launch_bounds__(kGemmThreads) void swiglu_kernel(const T* __restrict__ kv, int kv_len,
                                                              const int* __restrict__ rows, int n,
                                                              const T* __restrict__ xbar, const T* __restrict__ w1,
                                                              const T* __restrict__ w2, int W2, int d_ff,
                                                              T* __restrict__ dh, int MT, int NT, int per) {
    typedef G1<T> C;
    extern __shared__ __align__(16) unsigned char smem[];
    T* lds = reinterpret_cast<T*>(smem);
    const int tile = xcd_tile(blockIdx.x, per);
    if (tile >= MT * NT) return;
    const int mt = tile / NT, nt = tile - mt * NT;
    const int b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int tok0 = mt * (C::BM / 2);
    const int j0 = nt * 64;

    G1LoadA<T, C::BM> la;
#pragma unroll
    for (int u = 0; u < C::BM / 128; ++u) {
        const int r = RowTile<T, T, C::BM>::srow(u);
        const int t = tok0 + (r >> 1);
        const T* p = nullptr;
        if (t < n) {
            if (r & 1) {
                p = xbar + ((size_t)b * n + t) * W2;
            } else {
                const int kr = rows[(size_t)b * n + t];
                if (kr >= 0 && kr < kv_len) p = kv + ((size_t)b * kv_len + kr) * W2;
            }
        }
        la.row[u] = p;
    }
    G1LoadB<T> lb;
    {
        // B tile rows: [c1 0..31, c2 0..31, c1 32..63, c2 32..63] so that wave wn's
        // 64 rows are contiguous: its tiles j = 0, 1 are W_c1 and j = 2, 3 are W_c2
        const int r = RowTile<T, T, 128>::srow(0);
        const int half = r >> 6, q = r & 63;
        lb.row[0] = (q < 32) ? w1 + (size_t)(j0 + 32 * half + q) * W2 : w2 + (size_t)(j0 + 32 * half + q - 32) * W2;
    }

    f32x4 acc[C::WM / 16][C::WN / 16];
    mainloop<T, C::BM, C::BN, C::WM, C::WN>(la, lb, W2 / kKC, W2 / kKC, lds, C::WM * wm, 64 * wn, acc,
                                            NoBlockHook{});

    // epilogue: rows 4g+0/4g+1 of a tile are kv/mean of one token, 4g+2/4g+3 of the next
    float* sH = reinterpret_cast<float*>(smem);  // [BM/2 tokens][kHP]
#pragma unroll
    for (int i = 0; i < C::WM / 16; ++i) {
        const int tl = (C::WM / 2) * wm + 8 * i + 2 * (lane >> 4);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const f32x4 a = acc[i][c];
            const f32x4 g = acc[i][c + 2];
            const float h0 = swiglu_h(a[0], g[0]);
            const float h1 = swiglu_h(a[1], g[1]);
            const float h2 = swiglu_h(a[2], g[2]);
            const float h3 = swiglu_h(a[3], g[3]);
            const int cl = 32 * wn + 16 * c + (lane & 15);
            sH[tl * C::kHP + cl] = h0 - h1;
            sH[(tl + 1) * C::kHP + cl] = h2 - h3;
        }
    }
    __syncthreads();
    // coalesced store: each job = 8 consecutive columns of one token, split into planes
    constexpr int kJobs = (C::BM / 2) * 8;
    for (int jb = tid; jb < kJobs; jb += kGemmThreads) {
        const int tl = jb >> 3, ch = jb & 7;
        const int t = tok0 + tl;
        if (t >= n) continue;
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = sH[tl * C::kHP + 8 * ch + e];
        T* dst = dh + ((size_t)b * n + t) * C::NS * d_ff + j0 + 8 * ch;
        if constexpr (C::NS == 1) {
            lds_store8<T>(dst, x);
        } else {
            float r1[8], r2[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float hi = (float)(bf16_t)x[e];
                r1[e] = x[e] - hi;
                const float mi = (float)(bf16_t)r1[e];
                r2[e] = r1[e] - mi;
                x[e] = hi;
                r1[e] = mi;
            }
            lds_store8<T>(dst, x);
            lds_store8<T>(dst + d_ff, r1);
            lds_store8<T>(dst + 2 * d_ff, r2);
        }
    }
}

// bf16 formats: the same GEMM on the direct-to-LDS ring (see rkv_pipe.h), with 8
// wavefronts (two per SIMD, so one wavefront's LDS reads overlap the other's MFMAs)
// on a 256 x 256 tile: 128 tokens (kv and mean rows) x 128 hidden columns (their
// W_c1 and W_c2 rows). Wave w: rows 128 (w / 4) .., B rows 64 (w % 4) ...
namespace g1r {
constexpr int kThreads = 512;
constexpr int BM = 256, BN = 256, NST = 2;
constexpr int kHid = BN / 2;  // hidden columns per tile
// fp32 pitch of the dH staging tile: the epilogue's 4-byte stores (rows tl, tl + 2 in one
// half wavefront) land 24 banks apart and its 16-byte reloads (rows t, t + 1 in one pass)
// an odd number of 16-byte slots apart, so neither has bank conflicts
constexpr int kHP = kHid + 12;
constexpr size_t kRing = (size_t)NST * (BM + BN) * kStageK * 2;
constexpr size_t kEpi = (size_t)(BM / 2) * kHP * sizeof(float);
constexpr size_t bytes = kRing > kEpi ? kRing : kEpi;
static_assert(bytes <= 160 * 1024, "LDS budget");
// mean-projection form: all BM rows are tokens (kv rows only); a table of each token's
// reference count and slots follows the (larger) dH staging tile
constexpr int kTab = 9;  // ints per token: count (-1: no kv row), then up to 8 slots
constexpr size_t kEpiP = (size_t)BM * kHP * sizeof(float);
constexpr size_t kOffTab = kRing > kEpiP ? kRing : kEpiP;
constexpr size_t bytesP = kOffTab + (size_t)BM * kTab * sizeof(int);
static_assert(bytesP <= 160 * 1024, "LDS budget");
}  // namespace g1r

struct G1Frag {
    bf16x8 a[8];
    bf16x8 b[4];
};

// The mean's hidden values of the mean-projection form for one token and hidden column:
// a = (sum over the token's slots, ascending, of [r W_c1, r W_c2]) / k, h = SiLU(a1) a2,
// from the KMAX loaded projections v[q] of its padded slot list (entries q >= k repeat a
// valid slot and are masked out of the sum). k = 0: the zero mean, h = 0.
template <int KMAX>
__device__ inline float mean_h_from(const f32x2 (&v)[KMAX], int k) {
    float a1 = 0.f, a2 = 0.f;
#pragma unroll
    for (int q = 0; q < KMAX; ++q) {
        a1 += q < k ? v[q][0] : 0.f;
        a2 += q < k ? v[q][1] : 0.f;
    }
    if (k > 1) {
        a1 = __fdiv_rn(a1, (float)k);
        a2 = __fdiv_rn(a2, (float)k);
    }
    return swiglu_h(a1, a2);
}

template <int KMAX>
__device__ inline void load_proj(f32x2 (&v)[KMAX], const float* __restrict__ proj_b, const int* tab, int d_ff,
                                 int col) {
#pragma unroll
    for (int q = 0; q < KMAX; ++q)
        v[q] = *reinterpret_cast<const f32x2*>(proj_b + ((size_t)tab[1 + q] * d_ff + col) * 2);
}

// Token table of the mean-projection form: count (-1 when the token has no kv row or its
// position is out of range: dH = 0, the selection kernel has flagged it) and the slots,
// padded to 8 with the first slot (slot 0 for an empty set) so that every load is valid.
__device__ inline void token_entry(int* tab, const int* __restrict__ rows, const int* __restrict__ pos,
                                   const int* __restrict__ ref_idx, int kv_len, int cap_tok, int top_k, int b, int n,
                                   int t) {
    const int kr = rows[(size_t)b * n + t];
    const int p = pos[(size_t)b * n + t];
    int k = -1;
    if (kr >= 0 && kr < kv_len && p >= 0 && p < cap_tok) {
        const int* ri = ref_idx + ((size_t)b * cap_tok + p) * top_k;
        k = 0;
        for (int q = 0; q < top_k; ++q) {
            const int sl = ri[q];
            if (sl >= 0) tab[1 + k++] = sl;
        }
    }
    const int pad = k > 0 ? tab[1] : 0;
    for (int q = max(k, 0); q < 8; ++q) tab[1 + q] = pad;
    tab[0] = k;
}

// kProj = false: A rows alternate kv_i / mean_i of one token (128 tokens per tile).
// kProj = true (mean-projection form): A rows are kv rows only (256 tokens per tile) and
// the mean's hidden values come from the references' projections (proj) in the epilogue.
template <bool kProj, int KMAX>
__global__ __launch_bounds__(g1r::kThreads) void swiglu_ring_kernel(const bf16_t* __restrict__ kv, int kv_len,
                                                                    const int* __restrict__ rows, int n,
                                                                    const bf16_t* __restrict__ xbar,
                                                                    const bf16_t* __restrict__ w1,
                                                                    const bf16_t* __restrict__ w2, int W2, int d_ff,
                                                                    bf16_t* __restrict__ dh, int MT, int NT, int per,
                                                                    const int* __restrict__ pos,
                                                                    const int* __restrict__ ref_idx,
                                                                    const float* __restrict__ proj, int cap_ref,
                                                                    int cap_tok, int top_k) {
    extern __shared__ __align__(16) unsigned char smem_u8[];
    char* smem = reinterpret_cast<char*>(smem_u8);
    const int tile = xcd_tile(blockIdx.x, per);
    if (tile >= MT * NT) return;
    const int mt = tile / NT, nt = tile - mt * NT;
    const int b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    constexpr int kTok = kProj ? g1r::BM : g1r::BM / 2;  // tokens per tile
    const int tok0 = mt * kTok;
    const int j0 = nt * g1r::kHid;

    // Rows past n repeat the last token. A kv row index outside [0, kv_len) reads the
    // token's mean row instead (dH = 0; the selection kernel has flagged the token); in the
    // mean-projection form it reads row 0 and the token's table entry zeroes dH.
    Op16<g1r::BM, 8> la;
    la.init([&](int r) {
        if constexpr (kProj) {
            const int t = min(tok0 + r, n - 1);
            const int kr = rows[(size_t)b * n + t];
            return kv + ((size_t)b * kv_len + ((kr >= 0 && kr < kv_len) ? kr : 0)) * W2;
        } else {
            const int t = min(tok0 + (r >> 1), n - 1);
            const bf16_t* mrow = xbar + ((size_t)b * n + t) * W2;
            if (r & 1) return mrow;
            const int kr = rows[(size_t)b * n + t];
            return (kr >= 0 && kr < kv_len) ? kv + ((size_t)b * kv_len + kr) * W2 : mrow;
        }
    });
    int* sTab = reinterpret_cast<int*>(smem + g1r::kOffTab);
    if constexpr (kProj) {
        // read by the epilogue only, after the barriers of the main loop and its end
        if (tid < kTok && tok0 + tid < n)
            token_entry(sTab + g1r::kTab * tid, rows, pos, ref_idx, kv_len, cap_tok, top_k, b, n, tok0 + tid);
    }
    // B tile rows in groups of 64: [c1 32q .. +32, c2 32q .. +32] for q = 0..3, so that
    // wave wn's 64 rows hold matching W_c1 (tiles j = 0, 1) and W_c2 (j = 2, 3) columns;
    // columns past d_ff repeat the last one (not stored)
    Op16<g1r::BN, 8> lb;
    lb.init([&](int r) {
        const int q = r >> 6, e = r & 63;
        const int col = min(j0 + 32 * q + (e & 31), d_ff - 1);
        return (e < 32) ? w1 + (size_t)col * W2 : w2 + (size_t)col * W2;
    });

    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = zero4();
    auto load = [&](G1Frag& f, const char* sa, const char* sb, int ks) {
#pragma unroll
        for (int j = 0; j < 4; ++j) f.b[j] = Op16<g1r::BN, 8>::template frag<bf16_t>(sb, 4 * wn + j, ks);
#pragma unroll
        for (int i = 0; i < 8; ++i) f.a[i] = Op16<g1r::BM, 8>::template frag<bf16_t>(sa, 8 * wm + i, ks);
    };
    auto mma = [&](const G1Frag& f, f32x4(&c)[8][4]) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) c[i][j] = Mma<bf16_t>::step(c[i][j], f.a[i], f.b[j]);
    };
    const int ns = W2 / kStageK;
    ring_mainloop_lrp<g1r::NST, G1Frag, 12, 32>(la, lb, ns, ns, smem, load, mma, acc,
                                        [](int, f32x4(&)[8][4], bool) {});

    __syncthreads();
    float* sH = reinterpret_cast<float*>(smem);  // [tokens][kHP]
    if constexpr (kProj) {
        // epilogue: row 4 g + e of a tile is one token; its mean's hidden values from the
        // projections of its references
        // (every load of a 16-row block is issued before the sums that use it)
        const float* proj_b = proj + (size_t)b * cap_ref * d_ff * 2;
        int cols[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) cols[c] = min(j0 + 32 * wn + 16 * c + (lane & 15), d_ff - 1);
        constexpr int EB = KMAX > 4 ? 2 : 4;  // rows of a 16-row block per batch of loads
#pragma unroll
        for (int i = 0; i < 8; ++i) {
#pragma unroll
            for (int e0 = 0; e0 < 4; e0 += EB) {
                f32x2 v[EB][2][KMAX];
                int kk[EB];
#pragma unroll
                for (int u = 0; u < EB; ++u) {
                    const int tl = 128 * wm + 16 * i + 4 * (lane >> 4) + e0 + u;
                    const int* tab = sTab + g1r::kTab * (tok0 + tl < n ? tl : 0);
                    kk[u] = tok0 + tl < n ? tab[0] : -1;
#pragma unroll
                    for (int c = 0; c < 2; ++c) load_proj<KMAX>(v[u][c], proj_b, tab, d_ff, cols[c]);
                }
#pragma unroll
                for (int u = 0; u < EB; ++u) {
                    const int tl = 128 * wm + 16 * i + 4 * (lane >> 4) + e0 + u;
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        const float hk = swiglu_h(acc[i][c][e0 + u], acc[i][c + 2][e0 + u]);
                        const float hm = mean_h_from<KMAX>(v[u][c], kk[u]);
                        sH[tl * g1r::kHP + 32 * wn + 16 * c + (lane & 15)] = kk[u] >= 0 ? hk - hm : 0.f;
                    }
                }
            }
        }
    } else {
        // epilogue: rows 4g+0/4g+1 of a tile are kv/mean of one token, 4g+2/4g+3 of the next
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int tl = 64 * wm + 8 * i + 2 * (lane >> 4);
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const f32x4 a = acc[i][c];
                const f32x4 g = acc[i][c + 2];
                const float h0 = swiglu_h(a[0], g[0]);
                const float h1 = swiglu_h(a[1], g[1]);
                const float h2 = swiglu_h(a[2], g[2]);
                const float h3 = swiglu_h(a[3], g[3]);
                const int cl = 32 * wn + 16 * c + (lane & 15);
                sH[tl * g1r::kHP + cl] = h0 - h1;
                sH[(tl + 1) * g1r::kHP + cl] = h2 - h3;
            }
        }
    }
    __syncthreads();
    // coalesced store: each job = 8 consecutive columns of one token, split into the
    // three bf16 planes hi + mid + lo
    constexpr int kCh = g1r::kHid / 8;
    constexpr int kJobs = kTok * kCh;
    for (int jb = tid; jb < kJobs; jb += g1r::kThreads) {
        const int tl = jb / kCh, ch = jb - tl * kCh;
        const int t = tok0 + tl;
        if (t >= n || j0 + 8 * ch >= d_ff) continue;
        float x[8], r1[8], r2[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = sH[tl * g1r::kHP + 8 * ch + e];
        bf16_t* dst = dh + ((size_t)b * n + t) * 3 * d_ff + j0 + 8 * ch;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float hi = (float)(bf16_t)x[e];
            r1[e] = x[e] - hi;
            const float mi = (float)(bf16_t)r1[e];
            r2[e] = r1[e] - mi;
            x[e] = hi;
            r1[e] = mi;
        }
        lds_store8<bf16_t>(dst, x);
        lds_store8<bf16_t>(dst + d_ff, r1);
        lds_store8<bf16_t>(dst + 2 * d_ff, r2);
    }
}

// ---------------------------------------------------------------- GEMM 2 + quantizer

// LDS of the quantizer epilogue (quant_epilogue): per wavefront, CT tokens x (WN + 4) floats,
// where NQ = WN / 32 groups of a wavefront row and CT = min(64 / NQ, WM) tokens make one
// group per lane
constexpr int qe_nq(int WN) { return WN / 32; }
constexpr int qe_ct(int WM, int WN) { return 64 / qe_nq(WN) < WM ? 64 / qe_nq(WN) : WM; }
constexpr int qe_pitch(int WN) { return WN + 4; }
constexpr size_t qe_bytes(int WM, int WN, int nwaves) {
    return (size_t)nwaves * qe_ct(WM, WN) * qe_pitch(WN) * sizeof(float);
}

template <typename T>
struct G2 {
    static constexpr int BM = 128;
    static constexpr int BN = std::is_same<T, float>::value ? 64 : 128;
    static constexpr int WM = BM / 2, WN = BN / 2;
    static constexpr int NS = std::is_same<T, float>::value ? 1 : 3;
    static constexpr int P = Pitch<T, kKC>::value;
    static constexpr size_t kPipe = (size_t)2 * (BM + BN) * P * sizeof(T);
    // epilogue staging: codes (or fp16 latent) per token + step/min per group
    static constexpr size_t kEpi = qe_bytes(WM, WN, kGemmThreads / 64);
    static constexpr size_t bytes = kPipe > kEpi ? kPipe : kEpi;
    static constexpr int kThreads = kGemmThreads;
    static constexpr int kNWN = 2;  // wavefronts along N: wave w owns rows WM (w / kNWN), columns WN (w % kNWN)
};

template <typename T>
struct G2LoadA {
    RowTile<T, T, 128> t;
    const T* row[1];
    __device__ inline void load(int s) { t.load_rows(row, s * kKC); }
    __device__ inline void store(T* lds, int P) const { t.store(lds, P); }
};

// B' stage s holds W_c3 columns k = (s * kKC) mod d_ff: the three planes of dH all
// multiply the same W_c3.
template <typename T, int BN>
struct G2LoadB {
    static constexpr int kUnits = BN >= 128 ? BN / 128 : 1;
    Raw32<T> raw[kUnits];
    const T* row[kUnits];
    int d_ff;
    __device__ inline void load(int s) {
        const int k0 = (s * kKC) % d_ff;
#pragma unroll
        for (int u = 0; u < kUnits; ++u) {
            if (row[u]) raw[u].load(row[u] + k0 + (threadIdx.x & 1) * 32);
            else raw[u].zero();
        }
    }
    __device__ inline void store(T* lds, int P) const {
#pragma unroll
        for (int u = 0; u < kUnits; ++u) {
            const int r = (threadIdx.x >> 1) + 128 * u;
            if (r < BN) stage32<T>(lds + r * P + (threadIdx.x & 1) * 32, raw[u]);
        }
    }
};

template <typename ScT>
__device__ inline float round_scalar(float v);
template <>
__device__ inline float round_scalar<float>(float v) { return v; }
template <>
__device__ inline float round_scalar<f16_t>(float v) { return (float)(f16_t)v; }

// Group quantizer epilogue shared by the GEMM 2 kernels. The lane holds
// z[token WM wm + 16 i + 4 (lane/16) + e][col WN wn + 16 j + lane%16] in acc[i][j][e]. Each
// wavefront transposes its accumulators, a chunk of CT tokens at a time, through a buffer
// of its own in LDS (rows of WN + 4 floats: the 4-byte writes and the 16-byte reads both
// spread over all 64 banks), so that lane l then holds the 32 values of one group
// (token l / NQ of the chunk, group l % NQ of the wavefront's NQ = WN / 32) and does the
// whole group in registers: min and max, one step division, the codes and their packing
// in the record's byte order (dword d of a 4-bit group: columns 8d .. 8d + 7 at bits 4e;
// of a 2-bit group: columns 16d .. 16d + 15 at bits 2e), written with one 16- or 8-byte
// store (fp16 latents: four 16-byte stores). No workgroup barrier: a wavefront's LDS
// operations complete in order.

// Codes of a group: rint((v - zmin) / step) clamped to [0, levels], decided on the IEEE
// fp32 quotient. x r (r = v_rcp_f32(step), 1 ulp) is within 2^-18 of that quotient wherever
// the clamp does not decide (quotients below 16; three roundings of at most one ulp each),
// so both round to the same integer unless x r lies within 2^-14 of a half-integer; when
// any value of the group does, the group's quotients are formed exactly. (Checked on the
// CPU over 2.5e8 random fp16 steps and fp32 values, a tenth of them exact half-integer
// quotients, with r moved one ulp either way.)
template <int BITS>
__device__ inline void group_codes(const float (&x)[32], float zm, float st, float levels, uint32_t (&w)[BITS]) {
    constexpr int PER = 32 / BITS;  // codes per dword
    const float r = __builtin_amdgcn_rcpf(st);
    bool near = false;
#pragma unroll
    for (int d = 0; d < BITS; ++d) {
        uint32_t v = 0;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const float y = (x[PER * d + e] - zm) * r;
            near |= fabsf(y - floorf(y) - 0.5f) < 0x1p-14f;
            v |= (uint32_t)fminf(fmaxf(__builtin_rintf(y), 0.f), levels) << (BITS * e);
        }
        w[d] = v;
    }
    if (near) {
#pragma unroll
        for (int d = 0; d < BITS; ++d) {
            uint32_t v = 0;
#pragma unroll
            for (int e = 0; e < PER; ++e) {
                const float c = __builtin_rintf(__fdiv_rn(x[PER * d + e] - zm, st));
                v |= (uint32_t)fminf(fmaxf(c, 0.f), levels) << (BITS * e);
            }
            w[d] = v;
        }
    }
}

template <class C, typename ScT>
__device__ inline void quant_epilogue(f32x4 (&acc)[C::WM / 16][C::WN / 16], unsigned char* smem, int t0, int c0, int b,
                                      int n, int d_c, int bits, const int* __restrict__ pos, int cap_tok,
                                      uint8_t* __restrict__ codes, size_t code_bytes, ScT* __restrict__ scale,
                                      ScT* __restrict__ zmin) {
    constexpr int NQ = qe_nq(C::WN), CT = qe_ct(C::WM, C::WN), P = qe_pitch(C::WN);
    constexpr int NC = C::WM / CT;  // chunks per wavefront
    static_assert(C::WN % 32 == 0 && CT % 16 == 0 && C::WM % CT == 0, "chunking");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::kNWN, wn = wave % C::kNWN;
    float* sW = reinterpret_cast<float*>(smem) + (size_t)wave * CT * P;
    const int tk = lane / NQ, q = lane % NQ;  // this lane's token within a chunk, group within the wave
    const bool active = tk < CT;
    const int gl = (C::WN * wn) / 32 + q;  // group within the tile row
    const int G = d_c / 32;
    const int g = c0 / 32 + gl;
    const bool gvalid = active && g < G;
    // positions of this lane's tokens (one per chunk), in flight during the arithmetic
    int pch[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int t = t0 + C::WM * wm + CT * c + tk;
        pch[c] = (gvalid && t < n) ? pos[(size_t)b * n + t] : -1;
    }
    const float levels = (float)((1 << (bits == 16 ? 1 : bits)) - 1);
    const float* src = sW + (size_t)(active ? tk : 0) * P + 32 * q;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
        for (int ii = 0; ii < CT / 16; ++ii) {
            const int i = (CT / 16) * c + ii;
#pragma unroll
            for (int j = 0; j < C::WN / 16; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sW[(16 * ii + 4 * (lane >> 4) + e) * P + 16 * j + (lane & 15)] = acc[i][j][e];
        }
        float x[32];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(src + 4 * k);
            x[4 * k] = v[0];
            x[4 * k + 1] = v[1];
            x[4 * k + 2] = v[2];
            x[4 * k + 3] = v[3];
        }
        const int p = pch[c];
        const bool store = p >= 0 && p < cap_tok;
        const size_t rec = (size_t)b * cap_tok + p;
        if (bits == 16) {
            if (store) {
                uint4* dst = reinterpret_cast<uint4*>(codes + rec * code_bytes + (size_t)c0 * 2 + 64 * gl);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    uint32_t h[4];
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const f16_t h0 = (f16_t)x[8 * m + 2 * d], h1 = (f16_t)x[8 * m + 2 * d + 1];
                        h[d] = (uint32_t)__builtin_bit_cast(uint16_t, h0) |
                               ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
                    }
                    dst[m] = make_uint4(h[0], h[1], h[2], h[3]);
                }
            }
            continue;
        }
        float lo = x[0], hi = x[0];
#pragma unroll
        for (int k = 1; k < 32; ++k) {
            lo = fminf(lo, x[k]);
            hi = fmaxf(hi, x[k]);
        }
        const float delta = __fdiv_rn(hi - lo, levels);
        const float st = round_scalar<ScT>(delta);
        const float zm = round_scalar<ScT>(lo);
        if (bits == 4) {
            uint32_t w[4] = {0u, 0u, 0u, 0u};
            if (st != 0.f) group_codes<4>(x, zm, st, levels, w);
            if (store)
                *reinterpret_cast<uint4*>(codes + rec * code_bytes + (size_t)c0 / 2 + 16 * gl) =
                    make_uint4(w[0], w[1], w[2], w[3]);
        } else {
            uint32_t w[2] = {0u, 0u};
            if (st != 0.f) group_codes<2>(x, zm, st, levels, w);
            if (store)
                *reinterpret_cast<uint2*>(codes + rec * code_bytes + (size_t)c0 / 4 + 8 * gl) = make_uint2(w[0], w[1]);
        }
        if (store) {
            scale[rec * G + g] = (ScT)st;
            zmin[rec * G + g] = (ScT)zm;
        }
    }
}

template <typename T, typename ScT>
__global__ __launch_bounds__(kGemmThreads) void latent_quant_kernel(const T* __restrict__ dh, int n,
                                                                    const T* __restrict__ w3, int d_ff, int d_c,
                                                                    int bits, const int* __restrict__ pos,
                                                                    int cap_tok, uint8_t* __restrict__ codes,
                                                                    size_t code_bytes, ScT* __restrict__ scale,
                                                                    ScT* __restrict__ zmin, int MT, int NT, int per) {
    typedef G2<T> C;
    extern __shared__ __align__(16) unsigned char smem[];
    T* lds = reinterpret_cast<T*>(smem);
    const int tile = xcd_tile(blockIdx.x, per);
    if (tile >= MT * NT) return;
    const int mt = tile / NT, nt = tile - mt * NT;
    const int b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int t0 = mt * C::BM;
    const int c0 = nt * C::BN;
    const int Kp = C::NS * d_ff;

    G2LoadA<T> la;
    {
        const int r = RowTile<T, T, 128>::srow(0);
        la.row[0] = (t0 + r < n) ? dh + ((size_t)b * n + t0 + r) * Kp : nullptr;
    }
    G2LoadB<T, C::BN> lb;
    lb.d_ff = d_ff;
#pragma unroll
    for (int u = 0; u < G2LoadB<T, C::BN>::kUnits; ++u) {
        const int r = (tid >> 1) + 128 * u;
        lb.row[u] = (r < C::BN && c0 + r < d_c) ? w3 + (size_t)(c0 + r) * d_ff : nullptr;
    }

    f32x4 acc[C::WM / 16][C::WN / 16];
    // A' rows are [hi | mid | lo] (K' = NS d_ff); stage s of A' pairs with W_c3 stage s mod (d_ff / kKC)
    mainloop<T, C::BM, C::BN, C::WM, C::WN>(la, lb, Kp / kKC, Kp / kKC, lds, C::WM * wm, C::WN * wn, acc,
                                            NoBlockHook{});

    quant_epilogue<C, ScT>(acc, smem, t0, c0, b, n, d_c, bits, pos, cap_tok, codes, code_bytes, scale, zmin);
}

// bf16 formats: W_c3 projection + quantizer on the direct-to-LDS ring: 256 tokens x 256
// latent columns per workgroup of 8 wavefronts (wave w: tokens 128 (w / 4) .., columns
// 64 (w % 4) ..), so each dH row and each W_c3 row is streamed half as often as with
// 128-wide tiles. dH (read once, from HBM) runs on a three-stage ring, W_c3 (the same
// for every workgroup, from L2) on two, which fills the 160 KB of LDS (measured 0.120 ->
// 0.115 ms at 28672 tokens x d_c = 512; the same split slowed the SwiGLU kernel, whose
// W_c1 | W_c2 stream does not stay in L2).
namespace g2r {
constexpr int kThreads = 512;
constexpr int BM = 256, BN = 256, NA = 3, NB = 2;
struct Cfg {
    static constexpr int BM = g2r::BM, BN = g2r::BN, WM = 128, WN = 64;
    static constexpr size_t kEpi = qe_bytes(WM, WN, g2r::kThreads / 64);
    static constexpr int kThreads = g2r::kThreads;
    static constexpr int kNWN = 4;
    static constexpr int NA = g2r::NA, NB = g2r::NB;
};
constexpr size_t kRing = ((size_t)NA * BM + (size_t)NB * BN) * kStageK * 2;
constexpr size_t bytes = kRing > Cfg::kEpi ? kRing : Cfg::kEpi;
static_assert(bytes <= 160 * 1024, "LDS budget");
}  // namespace g2r

// Narrow tiles for a last run of at most 128 latent columns (d_c = 384 after one 256-wide
// tile, or d_c <= 128): 512 tokens x 128 columns, the same 128 x 64 block per wavefront
// (wave w: tokens 128 (w / 2) .., columns 64 (w % 2) ..) and the same MFMA sequence per
// output element, both operands on two-stage rings (160 KB). A 256-wide tile there would
// compute as many padded columns as real ones.
namespace g2n {
constexpr int BM = 512, BN = 128;
struct Cfg {
    static constexpr int BM = g2n::BM, BN = g2n::BN, WM = 128, WN = 64;
    static constexpr size_t kEpi = qe_bytes(WM, WN, g2r::kThreads / 64);
    static constexpr int kThreads = g2r::kThreads;
    static constexpr int kNWN = 2;
    static constexpr int NA = 2, NB = 2;
};
constexpr size_t kRing = (size_t)Cfg::NA * (BM + BN) * kStageK * 2;
constexpr size_t bytes = kRing > Cfg::kEpi ? kRing : Cfg::kEpi;
static_assert(bytes <= 160 * 1024, "LDS budget");
}  // namespace g2n

// W_c3 rows as the B operand: stage s reads K columns ((s mod (d_ff / 64)) * 64), so
// the three planes of dH (K' = 3 d_ff) each meet the same W_c3.
template <int R, int NW>
struct WrapOp16 {
    static constexpr int kLoads = R / (8 * NW);
    static constexpr int kStageBytes = R * kStageK * 2;
    const char* src[kLoads];
    int nkm;  // stages per d_ff
    __device__ inline void issue(int s, char* slot) const {
        const int wave = wave_id();
        const int kc = s % nkm;
#pragma unroll
        for (int u = 0; u < kLoads; ++u) dma16(src[u] + (size_t)kc * (kStageK * 2), slot + 1024 * (wave + NW * u));
    }
};

struct G2Frag {
    bf16x8 a[8];
    bf16x8 b[4];
};

// One tile of the ring quantizer: tokens t0 .. t0 + BM, latent columns c0 .. c0 + BN.
template <class C>
__device__ inline void quant_ring_tile(unsigned char* smem_u8, const bf16_t* __restrict__ dh, int n,
                                       const bf16_t* __restrict__ w3, int d_ff, int d_c, int bits,
                                       const int* __restrict__ pos, int cap_tok, uint8_t* __restrict__ codes,
                                       size_t code_bytes, f16_t* __restrict__ scale, f16_t* __restrict__ zmin, int b,
                                       int t0, int c0) {
    static_assert(C::WM == 128 && C::WN == 64 && C::kThreads / 64 == 8, "one 128 x 64 block per wavefront");
    char* smem = reinterpret_cast<char*>(smem_u8);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::kNWN, wn = wave % C::kNWN;
    const int Kp = 3 * d_ff;

    // rows past n / d_c repeat the last valid row; their results are not stored
    Op16<C::BM, 8> la;
    la.init([&](int r) { return dh + ((size_t)b * n + min(t0 + r, n - 1)) * Kp; });
    WrapOp16<C::BN, 8> lb;
    lb.nkm = d_ff / kStageK;
#pragma unroll
    for (int u = 0; u < WrapOp16<C::BN, 8>::kLoads; ++u) {
        const int blk = wave + 8 * u;
        const int r = 16 * (blk >> 1) + (lane >> 2);
        lb.src[u] = reinterpret_cast<const char*>(w3 + (size_t)min(c0 + r, d_c - 1) * d_ff) + 64 * (blk & 1) +
                    16 * swz(lane >> 2, lane & 3);
    }

    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = zero4();
    auto load = [&](G2Frag& f, const char* sa, const char* sb, int ks) {
#pragma unroll
        for (int j = 0; j < 4; ++j) f.b[j] = Op16<C::BN, 8>::template frag<bf16_t>(sb, 4 * wn + j, ks);
#pragma unroll
        for (int i = 0; i < 8; ++i) f.a[i] = Op16<C::BM, 8>::template frag<bf16_t>(sa, 8 * wm + i, ks);
    };
    auto mma = [&](const G2Frag& f, f32x4(&c)[8][4]) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) c[i][j] = Mma<bf16_t>::step(c[i][j], f.a[i], f.b[j]);
    };
    const int ns = Kp / kStageK;
    if constexpr (C::NA == C::NB + 1)
        ring_mainloop_split<C::NA, C::NB, G2Frag, 12, 32>(la, lb, ns, smem, smem + C::NA * Op16<C::BM, 8>::kStageBytes,
                                                         load, mma, acc);
    else
        ring_mainloop_lrp<C::NA, G2Frag, 12, 32>(la, lb, ns, ns, smem, load, mma, acc,
                                                 [](int, f32x4(&)[8][4], bool) {});
    __syncthreads();
    quant_epilogue<C, f16_t>(acc, smem_u8, t0, c0, b, n, d_c, bits, pos, cap_tok, codes, code_bytes, scale, zmin);
}

// The ring quantizer over all latent columns. Logical tiles come in groups of a 512-token
// block: its 256-wide tiles (nw column tiles for each 256-token half, the last one padded
// when the columns left after them exceed 128) and then, when at most 128 columns are left,
// one narrow tile of the whole block over them. The XCD-grouped order puts a group on one
// XCD at the same time, so the tiles of a token block stream its dH planes together
// through that XCD's L2 (a separate launch of the narrow tiles re-read them from HBM).
__global__ __launch_bounds__(g2r::kThreads) void latent_quant_ring_kernel(
    const bf16_t* __restrict__ dh, int n, const bf16_t* __restrict__ w3, int d_ff, int d_c, int bits,
    const int* __restrict__ pos, int cap_tok, uint8_t* __restrict__ codes, size_t code_bytes, f16_t* __restrict__ scale,
    f16_t* __restrict__ zmin, int ngroups, int nw, int narrow, int per) {
    extern __shared__ __align__(16) unsigned char smem_u8[];
    const int per_group = 2 * nw + narrow;
    const int tile = xcd_tile(blockIdx.x, per);
    if (tile >= ngroups * per_group) return;
    const int g = tile / per_group, k = tile - g * per_group;
    const int b = blockIdx.y;
    if (k < 2 * nw) {
        const int half = k / nw, nt = k - half * nw;
        const int t0 = g * g2n::BM + half * g2r::BM;
        if (t0 >= n) return;
        quant_ring_tile<g2r::Cfg>(smem_u8, dh, n, w3, d_ff, d_c, bits, pos, cap_tok, codes, code_bytes, scale, zmin, b,
                                  t0, nt * g2r::BN);
    } else {
        quant_ring_tile<g2n::Cfg>(smem_u8, dh, n, w3, d_ff, d_c, bits, pos, cap_tok, codes, code_bytes, scale, zmin, b,
                                  g * g2n::BM, nw * g2r::BN);
    }
}

// ---- few tokens per sequence: one-wavefront tiles on deep rings --------------------------
// Every output element goes through the same MFMA sequence as in the tiled kernels above
// (v_mfma_f32_16x16x32_bf16 steps over K in order, starting from zero, the same fragment
// layout) and the same epilogue arithmetic, so a token's hidden values and codes do not
// depend on how many tokens a call carries. A workgroup is one wavefront that keeps up to
// NST small stages in flight.

// s_waitcnt vmcnt(min(ahead, A) * PER) with a compile-time count
template <int PER, int A>
__device__ inline void wait_ahead(int ahead) {
    if constexpr (A == 0) {
        wait_vmcnt<0>();
    } else {
        if (ahead >= A) {
            wait_vmcnt<A * PER>();
            return;
        }
        wait_ahead<PER, A - 1>(ahead);
    }
}

// single-wavefront ring: stage s is multiplied once its own loads have landed (at most NST - 1
// later stages in flight); its slot is refilled with stage s + NST as soon as its fragments
// are in registers, before its MFMAs
template <int NST, class F, class LA, class LB, class Ld, class Mm>
__device__ inline void skinny_ring(const LA& a, const LB& b, int ns, char* lds, Ld&& load, Mm&& mma) {
    constexpr int kSlot = LA::kStageBytes + LB::kStageBytes;
    constexpr int kPer = LA::kLoads + LB::kLoads;
    static_assert((NST - 1) * kPer < 64, "vmcnt range");
#pragma unroll
    for (int p = 0; p < NST; ++p) {
        if (p < ns) {
            a.issue(p, lds + p * kSlot);
            b.issue(p, lds + p * kSlot + LA::kStageBytes);
        }
    }
    int slot = 0;
    for (int s = 0; s < ns; ++s) {
        wait_ahead<kPer, NST - 1>(min(NST - 1, ns - 1 - s));
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        const char* sa = lds + slot * kSlot;
        // both K steps' fragments at once (one LDS latency per stage), the slot refilled as
        // soon as they are in registers, then the MFMAs (K step 0 before K step 1)
        F f0, f1;
        load(f0, sa, sa + LA::kStageBytes, 0);
        load(f1, sa, sa + LA::kStageBytes, 1);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        wait_lgkm0();
        if (s + NST < ns) {
            a.issue(s + NST, lds + slot * kSlot);
            b.issue(s + NST, lds + slot * kSlot + LA::kStageBytes);
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        mma(f0);
        mma(f1);
        slot = slot + 1 == NST ? 0 : slot + 1;
    }
}

namespace sk {
constexpr int NST1 = 10;  // SwiGLU, per wavefront: 32 A rows + 16 B rows per stage (6 KB)
constexpr int NST2 = 11;  // W_c3, per wavefront: 16 A rows + 32 B rows per stage (6 KB); 10 in flight
constexpr size_t ring1 = (size_t)NST1 * (32 + 16) * kStageK * 2;  // one wavefront's ring
constexpr size_t bytes1 = 2 * ring1;
constexpr size_t ring2 = (size_t)NST2 * (16 + 32) * kStageK * 2;  // one wavefront's ring
constexpr size_t bytes2 = 2 * ring2;
struct Q2 {  // quantizer epilogue layout of the W_c3 tile: two wavefronts of 32 columns
    static constexpr int BM = 16, BN = 64, WM = 16, WN = 32;
    static constexpr int kThreads = 128;
    static constexpr int kNWN = 2;
};
static_assert(qe_bytes(Q2::WM, Q2::WN, Q2::kThreads / 64) <= bytes2, "epilogue");
}  // namespace sk

// A 16-bit operand loaded by one wavefront into a ring of its own (every block of a stage);
// with nkm > 0 the K stage index wraps at nkm (W_c3 against the dH planes)
template <int R>
struct SoloOp16 {
    static constexpr int kLoads = R / 8;
    static constexpr int kStageBytes = R * kStageK * 2;
    const char* src[kLoads];
    int nkm = 0;
    template <class RowFn>
    __device__ inline void init(RowFn&& row) {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int u = 0; u < kLoads; ++u)
            src[u] = reinterpret_cast<const char*>(row(16 * (u >> 1) + (lane >> 2))) + 64 * (u & 1) +
                     16 * swz(lane >> 2, lane & 3);
    }
    __device__ inline void issue(int s, char* slot) const {
        const int kc = nkm > 0 ? s % nkm : s;
#pragma unroll
        for (int u = 0; u < kLoads; ++u) dma16(src[u] + (size_t)kc * (kStageK * 2), slot + 1024 * u);
    }
};

struct SkFrag1 {
    bf16x8 a[2];
    bf16x8 b;
};

// SwiGLU for up to 16 tokens of one sequence: grid (d_ff / 16, batch), two wavefronts per
// workgroup, each with its own ring: wavefront 0 multiplies the A rows (kv and mean rows of the
// tokens) by W_c1 rows j0 .. j0 + 16, wavefront 1 by the matching W_c2 rows, and hands its
// accumulators to wavefront 0 through LDS for the epilogue (every output element sees the same
// MFMA sequence as in the tiled kernel).
__global__ __launch_bounds__(128) void swiglu_skinny_kernel(const bf16_t* __restrict__ kv, int kv_len,
                                                            const int* __restrict__ rows, int n,
                                                            const bf16_t* __restrict__ xbar,
                                                            const bf16_t* __restrict__ w1,
                                                            const bf16_t* __restrict__ w2, int W2, int d_ff,
                                                            bf16_t* __restrict__ dh) {
    extern __shared__ __align__(16) unsigned char smem_u8[];
    const int b = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    char* ring = reinterpret_cast<char*>(smem_u8) + wave * sk::ring1;
    const int j0 = 16 * blockIdx.x;
    SoloOp16<32> la;
    la.init([&](int r) {
        const int t = min(r >> 1, n - 1);
        const bf16_t* mrow = xbar + ((size_t)b * n + t) * W2;
        if (r & 1) return mrow;
        const int kr = rows[(size_t)b * n + t];
        return (kr >= 0 && kr < kv_len) ? kv + ((size_t)b * kv_len + kr) * W2 : mrow;
    });
    SoloOp16<16> lb;
    const bf16_t* wsel = wave == 0 ? w1 : w2;
    lb.init([&](int r) { return wsel + (size_t)min(j0 + r, d_ff - 1) * W2; });
    f32x4 acc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) acc[i] = zero4();
    auto load = [&](SkFrag1& f, const char* sa, const char* sb, int ks) {
        f.b = Op16<16, 1>::template frag<bf16_t>(sb, 0, ks);
#pragma unroll
        for (int i = 0; i < 2; ++i) f.a[i] = Op16<32, 1>::template frag<bf16_t>(sa, i, ks);
    };
    auto mma = [&](const SkFrag1& f) {
#pragma unroll
        for (int i = 0; i < 2; ++i) acc[i] = Mma<bf16_t>::step(acc[i], f.a[i], f.b);
    };
    skinny_ring<sk::NST1, SkFrag1>(la, lb, W2 / kStageK, ring, load, mma);
    // wavefront 1's W_c2 accumulators -> LDS (its own ring, which it has finished reading)
    f32x4* xg = reinterpret_cast<f32x4*>(reinterpret_cast<char*>(smem_u8) + sk::ring1);
    if (wave == 1) {
#pragma unroll
        for (int i = 0; i < 2; ++i) xg[64 * i + lane] = acc[i];
    }
    __syncthreads();
    if (wave != 0) return;
    // A rows 2 t, 2 t + 1 are kv and mean of token t; lane: hidden column j0 + lane % 16
    const int col = j0 + (lane & 15);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const f32x4 a = acc[i];
        const f32x4 g = xg[64 * i + lane];
        const float h0 = swiglu_h(a[0], g[0]);
        const float h1 = swiglu_h(a[1], g[1]);
        const float h2 = swiglu_h(a[2], g[2]);
        const float h3 = swiglu_h(a[3], g[3]);
        const int tl = 8 * i + 2 * (lane >> 4);
        const float d[2] = {h0 - h1, h2 - h3};
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int t = tl + u;
            if (t >= n || col >= d_ff) continue;
            const float x = d[u];
            const float hi = (float)(bf16_t)x;
            const float r1 = x - hi;
            const float mi = (float)(bf16_t)r1;
            const float r2 = r1 - mi;
            bf16_t* dst = dh + ((size_t)b * n + t) * 3 * d_ff + col;
            dst[0] = (bf16_t)hi;
            dst[d_ff] = (bf16_t)mi;
            dst[2 * d_ff] = (bf16_t)r2;
        }
    }
}

// Mean-projection form of swiglu_skinny_kernel: A rows are the kv rows of the (up to 16)
// tokens; wavefront 0's epilogue takes each token's mean hidden values from the
// projections of its references.
struct SkFrag1P {
    bf16x8 a;
    bf16x8 b;
};

__global__ __launch_bounds__(128) void swiglu_skinny_proj_kernel(
    const bf16_t* __restrict__ kv, int kv_len, const int* __restrict__ rows, const int* __restrict__ pos, int n,
    const int* __restrict__ ref_idx, const float* __restrict__ proj, int cap_ref, int cap_tok, int top_k,
    const bf16_t* __restrict__ w1, const bf16_t* __restrict__ w2, int W2, int d_ff, bf16_t* __restrict__ dh) {
    extern __shared__ __align__(16) unsigned char smem_u8[];
    const int b = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    char* ring = reinterpret_cast<char*>(smem_u8) + wave * sk::ring1;
    const int j0 = 16 * blockIdx.x;
    SoloOp16<16> la;
    la.init([&](int r) {
        const int t = min(r, n - 1);
        const int kr = rows[(size_t)b * n + t];
        return kv + ((size_t)b * kv_len + ((kr >= 0 && kr < kv_len) ? kr : 0)) * W2;
    });
    SoloOp16<16> lb;
    const bf16_t* wsel = wave == 0 ? w1 : w2;
    lb.init([&](int r) { return wsel + (size_t)min(j0 + r, d_ff - 1) * W2; });
    f32x4 acc = zero4();
    auto load = [&](SkFrag1P& f, const char* sa, const char* sb, int ks) {
        f.b = Op16<16, 1>::template frag<bf16_t>(sb, 0, ks);
        f.a = Op16<16, 1>::template frag<bf16_t>(sa, 0, ks);
    };
    auto mma = [&](const SkFrag1P& f) { acc = Mma<bf16_t>::step(acc, f.a, f.b); };
    skinny_ring<sk::NST1, SkFrag1P>(la, lb, W2 / kStageK, ring, load, mma);
    // wavefront 1's W_c2 accumulators -> LDS (its own ring, which it has finished reading),
    // and the token table after them
    f32x4* xg = reinterpret_cast<f32x4*>(reinterpret_cast<char*>(smem_u8) + sk::ring1);
    int* sTab = reinterpret_cast<int*>(xg + 64);
    if (wave == 1) {
        xg[lane] = acc;
        if (lane < 16 && lane < n) token_entry(sTab + g1r::kTab * lane, rows, pos, ref_idx, kv_len, cap_tok, top_k, b, n, lane);
    }
    __syncthreads();
    if (wave != 0) return;
    // row 4 (lane / 16) + e is token 4 (lane / 16) + e; lane: hidden column j0 + lane % 16
    const int col = j0 + (lane & 15);
    const float* proj_b = proj + (size_t)b * cap_ref * d_ff * 2;
    const f32x4 g = xg[lane];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int t = 4 * (lane >> 4) + e;
        if (t >= n || col >= d_ff) continue;
        const int* tab = sTab + g1r::kTab * t;
        f32x2 v[8];
        load_proj<8>(v, proj_b, tab, d_ff, col);
        const int k = tab[0];
        const float x = k >= 0 ? swiglu_h(acc[e], g[e]) - mean_h_from<8>(v, k) : 0.f;
        const float hi = (float)(bf16_t)x;
        const float r1 = x - hi;
        const float mi = (float)(bf16_t)r1;
        const float r2 = r1 - mi;
        bf16_t* dst = dh + ((size_t)b * n + t) * 3 * d_ff + col;
        dst[0] = (bf16_t)hi;
        dst[d_ff] = (bf16_t)mi;
        dst[2 * d_ff] = (bf16_t)r2;
    }
}

// ---------------------------------------------------------------- reference projections
// Mean-projection form: every stored reference r gets [r W_c1, r W_c2] once (fp32, hidden
// column j at [2 j], [2 j + 1] of its row), so that the encoder can average them instead
// of multiplying every token's mean (the first layer of f_c is linear, section 2.3).
// Tile: 128 pool slots x 128 W rows (64 hidden columns of W_c1 and the same of W_c2),
// four wavefronts of 64 x 64. The FP8 slots go through registers (widened exactly to
// bf16 into the ring layout of rkv_pipe.h); W rows arrive by direct loads. The slots to
// project, [proj_count, ref_count), are known on the device only: workgroups walk the
// slot tiles with a stride of gridDim.y and stop at the first tile past the end.
namespace pj {
constexpr int kThreads = 256;
constexpr int BM = 128, BN = 128;
constexpr int kHid = BN / 2;
constexpr int kMaxMT = 32;
constexpr int kStageA = BM * kStageK * 2;  // bf16
constexpr int kSlot = kStageA + BN * kStageK * 2;
constexpr size_t bytes = 2 * (size_t)kSlot;
}  // namespace pj

__global__ __launch_bounds__(pj::kThreads) void project_refs_kernel(const fp8_t* __restrict__ ref_vals,
                                                                    const int* __restrict__ ref_count,
                                                                    const int* __restrict__ proj_count, int cap_ref,
                                                                    const bf16_t* __restrict__ w1,
                                                                    const bf16_t* __restrict__ w2, int W2, int d_ff,
                                                                    float* __restrict__ proj) {
    extern __shared__ __align__(16) unsigned char smem_u8[];
    char* smem = reinterpret_cast<char*>(smem_u8);
    const int b = blockIdx.z;
    const int hi = min(ref_count[b], cap_ref);
    const int pc = proj_count[b];
    const int lo = (pc >= 0 && pc <= hi) ? pc : 0;
    if (lo + (int)blockIdx.y * pj::BM >= hi) return;
    const int j0 = blockIdx.x * pj::kHid;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    // W rows in groups of 64: [c1 32 q .. + 32, c2 32 q .. + 32]: wave wn's 64 rows hold
    // W_c1 (tiles j = 0, 1) and W_c2 (j = 2, 3) of hidden columns j0 + 32 wn ..
    Op16<pj::BN, 4> lb;
    lb.init([&](int r) {
        const int q = r >> 6, e = r & 63;
        const int col = min(j0 + 32 * q + (e & 31), d_ff - 1);
        return (e < 32) ? w1 + (size_t)col * W2 : w2 + (size_t)col * W2;
    });
    // A: thread -> slot row ar = tid % 128, K half ah = tid / 128 (32 FP8 values of a stage)
    const int ar = tid & (pj::BM - 1), ah = tid >> 7;
    const int ns = W2 / kStageK;
    const fp8_t* pool = ref_vals + (size_t)b * cap_ref * W2;
    float* out_b = proj + (size_t)b * cap_ref * d_ff * 2;
    for (int mt = blockIdx.y;; mt += gridDim.y) {
        const int s0 = lo + mt * pj::BM;
        if (s0 >= hi) break;
        const uint8_t* arow =
            reinterpret_cast<const uint8_t*>(pool + (size_t)min(s0 + ar, hi - 1) * W2) + 32 * ah;
        f32x4 acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = zero4();
        uint4 ra[2];
        auto load_a = [&](int st) {
            const uint4* src = reinterpret_cast<const uint4*>(arow + (size_t)st * kStageK);
            ra[0] = src[0];
            ra[1] = src[1];
        };
        // chunk c = 4 ah + u (8 values) of row ar -> block 2 (ar / 16) + ah, row ar % 16,
        // position swz(ar % 16, u)
        auto store_a = [&](char* slot) {
            char* blk = slot + 1024 * (2 * (ar >> 4) + ah) + 64 * (ar & 15);
            const uint32_t w[8] = {ra[0].x, ra[0].y, ra[0].z, ra[0].w, ra[1].x, ra[1].y, ra[1].z, ra[1].w};
#pragma unroll
            for (int u = 0; u < 4; ++u)
                *reinterpret_cast<bf16x8*>(blk + 16 * swz(ar & 15, u)) = widen8(w[2 * u], w[2 * u + 1]);
        };
        load_a(0);
        lb.issue(0, smem + pj::kStageA);
        for (int st = 0; st < ns; ++st) {
            char* slot = smem + (st & 1) * pj::kSlot;
            store_a(slot);
            wait_vmcnt<0>();
            __syncthreads();
            if (st + 1 < ns) {
                load_a(st + 1);
                lb.issue(st + 1, smem + ((st + 1) & 1) * pj::kSlot + pj::kStageA);
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                bf16x8 fa[4], fb[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) fa[i] = Op16<pj::BM, 4>::template frag<bf16_t>(slot, 4 * wm + i, ks);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    fb[j] = Op16<pj::BN, 4>::template frag<bf16_t>(slot + pj::kStageA, 4 * wn + j, ks);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[i][j] = Mma<bf16_t>::step(acc[i][j], fa[i], fb[j]);
            }
            __syncthreads();
        }
        // row 64 wm + 16 i + 4 (lane / 16) + e is slot s0 + row; tiles j and j + 2 are the
        // W_c1 and W_c2 columns j0 + 32 wn + 16 j + lane % 16
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int slot = s0 + 64 * wm + 16 * i + 4 * (lane >> 4) + e;
                if (slot >= hi) continue;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int col = j0 + 32 * wn + 16 * j + (lane & 15);
                    if (col >= d_ff) continue;
                    f32x2 v;
                    v[0] = acc[i][j][e];
                    v[1] = acc[i][j + 2][e];
                    *reinterpret_cast<f32x2*>(out_b + ((size_t)slot * d_ff + col) * 2) = v;
                }
            }
    }
}

// proj_count = ref_count once the projections of the new slots are written
__global__ void projections_done_kernel(const int* __restrict__ ref_count, int* __restrict__ proj_count, int B,
                                        int cap_ref) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b < B) proj_count[b] = min(ref_count[b], cap_ref);
}

struct SkFrag2 {
    bf16x8 a;
    bf16x8 b[2];
};

// W_c3 projection + quantizer for up to 16 tokens of one sequence: grid (d_c / 64, batch), two
// wavefronts per workgroup, each with its own ring over the 32 W_c3 rows of one quantizer group
// (every output element sees the same MFMA sequence as in the tiled kernel)
__global__ __launch_bounds__(128) void latent_quant_skinny_kernel(
    const bf16_t* __restrict__ dh, int n, const bf16_t* __restrict__ w3, int d_ff, int d_c, int bits,
    const int* __restrict__ pos, int cap_tok, uint8_t* __restrict__ codes, size_t code_bytes, f16_t* __restrict__ scale,
    f16_t* __restrict__ zmin) {
    extern __shared__ __align__(16) unsigned char smem_u8[];
    const int b = blockIdx.y;
    const int wave = threadIdx.x >> 6;
    char* ring = reinterpret_cast<char*>(smem_u8) + wave * sk::ring2;
    const int c0 = 64 * blockIdx.x;       // the workgroup's 64 latent columns
    const int cw = c0 + 32 * wave;        // this wavefront's 32 (one quantizer group)
    const int Kp = 3 * d_ff;
    SoloOp16<16> la;
    la.init([&](int r) { return dh + ((size_t)b * n + min(r, n - 1)) * Kp; });
    SoloOp16<32> lb;
    lb.nkm = d_ff / kStageK;
    lb.init([&](int r) { return w3 + (size_t)min(cw + r, d_c - 1) * d_ff; });
    f32x4 acc[1][2];
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[0][j] = zero4();
    auto load = [&](SkFrag2& f, const char* sa, const char* sb, int ks) {
#pragma unroll
        for (int j = 0; j < 2; ++j) f.b[j] = Op16<32, 1>::template frag<bf16_t>(sb, j, ks);
        f.a = Op16<16, 1>::template frag<bf16_t>(sa, 0, ks);
    };
    auto mma = [&](const SkFrag2& f) {
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[0][j] = Mma<bf16_t>::step(acc[0][j], f.a, f.b[j]);
    };
    skinny_ring<sk::NST2, SkFrag2>(la, lb, Kp / kStageK, ring, load, mma);
    __syncthreads();  // the epilogue's staging overlays the rings of both wavefronts
    quant_epilogue<sk::Q2, f16_t>(acc, smem_u8, 0, c0, b, n, d_c, bits, pos, cap_tok, codes, code_bytes, scale, zmin);
}

}  // namespace

template <typename T>
static hipError_t swiglu_impl(const Shape& s, const CacheView& c, const EncodePlan& p, const void* kv, int kv_len,
                              const int* rows, int n, const void* w1, const void* w2, void* ws, hipStream_t st) {
    typedef G1<T> C;
    const size_t smem = C::bytes;
    auto kern = swiglu_kernel<T>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    char* w = static_cast<char*>(ws);
    const int MT = (2 * n + C::BM - 1) / C::BM;
    const int NT = s.d_ff / 64;
    const int per = xcd_per(MT * NT);
    hipLaunchKernelGGL(kern, dim3(8 * per, c.B), dim3(kGemmThreads), smem, st, static_cast<const T*>(kv), kv_len,
                       rows, n, reinterpret_cast<const T*>(w + p.off_xbar), static_cast<const T*>(w1),
                       static_cast<const T*>(w2), s.W2, s.d_ff, reinterpret_cast<T*>(w + p.off_dh), MT, NT, per);
    return hipGetLastError();
}

static hipError_t swiglu_ring_impl(const Shape& s, const CacheView& c, const EncodePlan& p, const void* kv,
                                   int kv_len, const int* rows, const int* pos, int n, const void* w1, const void* w2,
                                   void* ws, hipStream_t st) {
    const size_t smem = s.mproj ? g1r::bytesP : g1r::bytes;
    auto kern = !s.mproj ? swiglu_ring_kernel<false, 4>
                         : (s.top_k <= 4 ? swiglu_ring_kernel<true, 4> : swiglu_ring_kernel<true, 8>);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    char* w = static_cast<char*>(ws);
    const int MT = ((s.mproj ? n : 2 * n) + g1r::BM - 1) / g1r::BM;
    const int NT = (s.d_ff + g1r::kHid - 1) / g1r::kHid;
    const int per = xcd_per(MT * NT);
    hipLaunchKernelGGL(kern, dim3(8 * per, c.B), dim3(g1r::kThreads), smem, st, static_cast<const bf16_t*>(kv), kv_len,
                       rows, n, s.mproj ? nullptr : reinterpret_cast<const bf16_t*>(w + p.off_xbar),
                       static_cast<const bf16_t*>(w1), static_cast<const bf16_t*>(w2), s.W2, s.d_ff,
                       reinterpret_cast<bf16_t*>(w + p.off_dh), MT, NT, per, pos, c.ref_idx, c.ref_proj, c.cap_ref,
                       c.cap_tok, s.top_k);
    return hipGetLastError();
}

hipError_t launch_project_refs(const Shape& s, const CacheView& c, const void* w1, const void* w2, hipStream_t st) {
    if (s.f32 || !s.mproj) return hipErrorInvalidValue;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(project_refs_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)pj::bytes);
    if (e != hipSuccess) return e;
    const int mt = std::min((c.cap_ref + pj::BM - 1) / pj::BM, pj::kMaxMT);
    hipLaunchKernelGGL(project_refs_kernel, dim3(s.d_ff / pj::kHid, mt, c.B), dim3(pj::kThreads), pj::bytes, st,
                       static_cast<const fp8_t*>(c.ref_vals), c.ref_count, c.proj_count, c.cap_ref,
                       static_cast<const bf16_t*>(w1), static_cast<const bf16_t*>(w2), s.W2, s.d_ff, c.ref_proj);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(projections_done_kernel, dim3((c.B + 63) / 64), dim3(64), 0, st, c.ref_count, c.proj_count,
                       c.B, c.cap_ref);
    return hipGetLastError();
}

// at most this many tokens per sequence take the one-wavefront kernels
constexpr int kSkinnyTokens = 16;

static bool skinny(const Shape& s, int n) {
    return !s.f32 && n <= kSkinnyTokens && s.d_ff % 64 == 0 && s.d_c % 64 == 0;
}

hipError_t launch_swiglu(const Shape& s, const CacheView& c, const EncodePlan& p, const void* kv, int kv_len,
                         const int* rows, const int* pos, int n, const void* w1, const void* w2, void* ws,
                         hipStream_t st) {
    if (s.f32) return swiglu_impl<float>(s, c, p, kv, kv_len, rows, n, w1, w2, ws, st);
    if (skinny(s, n) && s.mproj) {
        char* w = static_cast<char*>(ws);
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(swiglu_skinny_proj_kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)sk::bytes1);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(swiglu_skinny_proj_kernel, dim3(s.d_ff / 16, c.B), dim3(128), sk::bytes1, st,
                           static_cast<const bf16_t*>(kv), kv_len, rows, pos, n, c.ref_idx, c.ref_proj, c.cap_ref,
                           c.cap_tok, s.top_k, static_cast<const bf16_t*>(w1), static_cast<const bf16_t*>(w2), s.W2,
                           s.d_ff, reinterpret_cast<bf16_t*>(w + p.off_dh));
        return hipGetLastError();
    }
    if (skinny(s, n)) {
        char* w = static_cast<char*>(ws);
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(swiglu_skinny_kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)sk::bytes1);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(swiglu_skinny_kernel, dim3(s.d_ff / 16, c.B), dim3(128), sk::bytes1, st,
                           static_cast<const bf16_t*>(kv), kv_len, rows, n,
                           reinterpret_cast<const bf16_t*>(w + p.off_xbar), static_cast<const bf16_t*>(w1),
                           static_cast<const bf16_t*>(w2), s.W2, s.d_ff, reinterpret_cast<bf16_t*>(w + p.off_dh));
        return hipGetLastError();
    }
    return swiglu_ring_impl(s, c, p, kv, kv_len, rows, pos, n, w1, w2, ws, st);
}

template <typename T, typename ScT>
static hipError_t latent_impl(const Shape& s, const CacheView& c, const EncodePlan& p, const int* pos, int n,
                              const void* w3, void* ws, hipStream_t st) {
    typedef G2<T> C;
    const size_t smem = C::bytes;
    auto kern = latent_quant_kernel<T, ScT>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    char* w = static_cast<char*>(ws);
    const int MT = (n + C::BM - 1) / C::BM;
    const int NT = (s.d_c + C::BN - 1) / C::BN;
    const int per = xcd_per(MT * NT);
    hipLaunchKernelGGL(kern, dim3(8 * per, c.B), dim3(kGemmThreads), smem, st,
                       reinterpret_cast<const T*>(w + p.off_dh), n, static_cast<const T*>(w3), s.d_ff, s.d_c, s.bits,
                       pos, c.cap_tok, c.codes, c.code_bytes, static_cast<ScT*>(c.scale), static_cast<ScT*>(c.zmin),
                       MT, NT, per);
    return hipGetLastError();
}

static hipError_t latent_ring_impl(const Shape& s, const CacheView& c, const EncodePlan& p, const int* pos, int n,
                                   const void* w3, void* ws, hipStream_t st) {
    static_assert(g2n::BM == 2 * g2r::BM, "a 512-token group holds two 256-token tiles");
    constexpr size_t smem = g2r::bytes > g2n::bytes ? g2r::bytes : g2n::bytes;
    auto kern = latent_quant_ring_kernel;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    // 256-wide column tiles over whole runs of 256 latent columns; a last run of at most
    // 128 columns goes to the narrow tiles (192 stays on a padded 256-wide tile)
    const int rem = s.d_c % g2r::BN;
    const int narrow = (rem > 0 && rem <= g2n::BN) ? 1 : 0;
    const int nw = narrow ? s.d_c / g2r::BN : (s.d_c + g2r::BN - 1) / g2r::BN;
    const int ngroups = (n + g2n::BM - 1) / g2n::BM;
    const int per = xcd_per(ngroups * (2 * nw + narrow));
    char* w = static_cast<char*>(ws);
    hipLaunchKernelGGL(kern, dim3(8 * per, c.B), dim3(g2r::kThreads), smem, st,
                       reinterpret_cast<const bf16_t*>(w + p.off_dh), n, static_cast<const bf16_t*>(w3), s.d_ff, s.d_c,
                       s.bits, pos, c.cap_tok, c.codes, c.code_bytes, static_cast<f16_t*>(c.scale),
                       static_cast<f16_t*>(c.zmin), ngroups, nw, narrow, per);
    return hipGetLastError();
}

hipError_t launch_latent_quant(const Shape& s, const CacheView& c, const EncodePlan& p, const int* pos, int n,
                               const void* w3, void* ws, hipStream_t st) {
    if (skinny(s, n)) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(latent_quant_skinny_kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)sk::bytes2);
        if (e != hipSuccess) return e;
        char* w = static_cast<char*>(ws);
        hipLaunchKernelGGL(latent_quant_skinny_kernel, dim3(s.d_c / 64, c.B), dim3(128), sk::bytes2, st,
                           reinterpret_cast<const bf16_t*>(w + p.off_dh), n, static_cast<const bf16_t*>(w3), s.d_ff,
                           s.d_c, s.bits, pos, c.cap_tok, c.codes, c.code_bytes, static_cast<f16_t*>(c.scale),
                           static_cast<f16_t*>(c.zmin));
        return hipGetLastError();
    }
    if (s.f32) return latent_impl<float, float>(s, c, p, pos, n, w3, ws, st);
    return latent_ring_impl(s, c, p, pos, n, w3, ws, st);
}

}  // namespace rkv
