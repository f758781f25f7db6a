// Selected-token restore, token-tile form (bf16 formats, INT4 / INT2 codes, groups of 32).
//
// ResidualKV review page, section 2.5 (boxed equation): KV-hat_i = z~_i W_d + mean_i
// with the bias-free linear decoder; section 2.4: z~ = q Delta + z_min per group;
// section 2.7 steps 2-3: only the selected tokens are read and restored; section 2.1
// (last paragraph): the restored pre-RoPE key is rotated at the token's own position.
//
// A workgroup (4 wavefronts, one per SIMD) owns 128 selected tokens and a run of
// 128-column chunks of the output. Wavefront w restores tokens 32 w .. + 32 (two MFMA
// column groups of 16) over all 128 columns of a chunk:
//   * its tokens' latents z~ are dequantized once, into fp16 MFMA fragments that stay
//     in registers for every chunk (fp16: exponent trick and one packed FMA);
//   * W_d (bf16, stored one output column per row) streams through a register ring
//     two stages of 64 latent values ahead, is converted to fp16 once per workgroup
//     and element, and is double-buffered in LDS; out^T = W_d^T z~^T runs on
//     v_mfma_f32_16x16x32_f16 with fp32 accumulation;
//   * the FP8 slices of every token's references for the next chunk are fetched into
//     LDS by direct loads while the current chunk runs (missing references read a
//     zero row); the reference sum is then one more pair of FP8 MFMAs per output tile,
//     against a 0/1 selection matrix, which lands it in the accumulator layout exactly
//     (a sum of at most 8 FP8 values is exact in fp32), and is scaled by 1 / k_i;
//   * RoPE uses per-token cos / sin computed once per workgroup.
// Inside each 8-value fragment both operands hold the latent coordinates in the order
// 0 4 1 5 2 6 3 7, which is what the packed code nibbles give with one mask per pair;
// the contraction does not depend on that order.
#include <math.h>

#include "rkv_device.h"
#include "rkv_internal.h"
#include "rkv_pipe.h"

namespace rkv {

namespace {

namespace dt {
constexpr int kThreads = 256;       // 4 wavefronts
constexpr int TT = 128;             // tokens per workgroup
constexpr int kCols = 128;          // output columns per chunk (reference slices are fetched per chunk)
constexpr int kHalf = 64;           // output columns per pass (4 MFMA tiles of 16)
constexpr int kRefs = 4;            // reference slots per token (k <= 4), all staged in LDS
constexpr int kWP = kStageK + 8;    // fp16 pitch of a staged W_d row (conflict-free fragment reads)
constexpr int kWBuf = kHalf * kWP * 2;       // one W_d stage (64 rows x 64 K fp16)
constexpr int kRefBuf = TT * kRefs * kCols;  // FP8 reference slices of one chunk
constexpr int kOffW = 0;
constexpr int kOffRef = kOffW + 2 * kWBuf;
constexpr int kOffSlot = kOffRef + kRefBuf;            // int [TT][kRefs]; -1: zero row
constexpr int kOffKd = kOffSlot + TT * kRefs * 4;      // int [TT]: divisor of the slot sum (4, or 3)
constexpr int kOffRev = kOffKd + TT * 4;               // double [64]
constexpr int bytes = kOffRev + 64 * 8;
static_assert(bytes <= 160 * 1024, "LDS budget");
}  // namespace dt

// 128 zero bytes: the source of an empty reference slot's slice
__device__ __align__(16) uint8_t g_zero_row[dt::kCols];

// Workgroup barrier for LDS traffic only: a fence would also wait for every
// outstanding global load, including the reference slices fetched for the next chunk.
// The scheduling barriers keep the compiler from moving work across it.
__device__ inline void lds_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_sched_barrier(0);
}

template <typename OutT>
__device__ inline void store_row4(OutT* p, float a, float b, float c, float d);
template <>
__device__ inline void store_row4<float>(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}
template <>
__device__ inline void store_row4<bf16_t>(bf16_t* p, float a, float b, float c, float d) {
    bf16_t t[4] = {(bf16_t)a, (bf16_t)b, (bf16_t)c, (bf16_t)d};
    *reinterpret_cast<uint2*>(p) = *reinterpret_cast<uint2*>(t);
}

// fp16 fragment of 8 codes (latent order 0 4 1 5 2 6 3 7) times the group's step plus
// its minimum. BITS = 4: w holds coordinate c in bits 4c .. 4c + 3; BITS = 2: w holds
// coordinate c in bits 2c, 2c + 1.
template <int BITS>
__device__ inline f16x8 dequant8(uint32_t w, f16x2 sv, f16x2 zv) {
    uint32_t x = w, mask = 0x000F000Fu;
    int sh = 4;
    if constexpr (BITS == 2) {
        x = (w & 0xFFu) | ((w & 0xFF00u) << 8);
        mask = 0x00030003u;
        sh = 2;
    }
    const f16x2 off = {(f16_t)1024.0f, (f16_t)1024.0f};
    f16x8 f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const uint32_t pk = ((x >> (sh * s)) & mask) | 0x64006400u;
        f16x2 v = *reinterpret_cast<const f16x2*>(&pk);
        v = __builtin_elementwise_fma(v - off, sv, zv);
        f[2 * s] = v[0];
        f[2 * s + 1] = v[1];
    }
    return f;
}

// 8 bf16 (latent order 0..7) -> fp16 in the fragment order 0 4 1 5 2 6 3 7
// (exact for every bf16 in the fp16 normal range).
__device__ inline f16x8 w_to_f16(uint4 r) {
    const uint32_t d[4] = {r.x, r.y, r.z, r.w};
    f16x8 h;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const float lo_a = __uint_as_float(d[e] << 16), hi_a = __uint_as_float(d[e] & 0xFFFF0000u);
        const float lo_b = __uint_as_float(d[e + 2] << 16), hi_b = __uint_as_float(d[e + 2] & 0xFFFF0000u);
        const auto p0 = __builtin_amdgcn_cvt_pkrtz(lo_a, lo_b);  // (2e, 2e + 4)
        const auto p1 = __builtin_amdgcn_cvt_pkrtz(hi_a, hi_b);  // (2e + 1, 2e + 5)
        h[4 * e + 0] = p0[0];
        h[4 * e + 1] = p0[1];
        h[4 * e + 2] = p1[0];
        h[4 * e + 3] = p1[1];
    }
    return h;
}

// MFMA column tile (16 output columns) of local tile lt (0..3) in pass h of a 128-column
// chunk. The tiles of a pass hold both halves of their RoPE pairs: with D = 128 the pair
// (j, j + 64) of the chunk's head, with D = 64 the pair (j, j + 32) of one head; local
// tiles (0, 2) and (1, 3) are the pairs.
template <int D>
__device__ constexpr int chunk_tile(int h, int lt) {
    return D == 128 ? 2 * h + (lt & 1) + 4 * (lt >> 1) : 4 * h + lt;
}

// grid: (token tiles, column groups, batch). Each column group is `ncg` chunks of 128
// columns starting at column 128 ncg blockIdx.y. NKS = d_c / 32 latent K-steps (step ks
// covers latent coordinates 32 ks .. +32, i.e. quantizer group ks); D = head dimension;
// BITS = 4 or 2.
template <int NKS, int D, int BITS, typename OutT>
__global__ __launch_bounds__(dt::kThreads) void decode_tiles_kernel(
    const int* __restrict__ idx, int m, int ncg, const fp8_t* __restrict__ ref_vals, const int* __restrict__ self_slot,
    const int* __restrict__ ref_idx, const uint8_t* __restrict__ codes, size_t code_bytes,
    const f16_t* __restrict__ scale, const f16_t* __restrict__ zmin, const bf16_t* __restrict__ wd, int W2, int dk,
    int top_k, int cap_ref, int cap_tok, double theta, OutT* __restrict__ out, int* err) {
    constexpr int d_c = 32 * NKS;
    constexpr int KST = d_c / kStageK;  // W_d stages per pass
    static_assert(KST % 2 == 0 && 2 * KST < 64, "stage shape");
    static_assert(D == 64 || D == 128, "head dimension");
    constexpr int half = D / 2, NJ = D / 8;  // RoPE pairs per head; cos / sin per lane and token
    extern __shared__ __align__(16) unsigned char smem[];
    f16_t* sW = reinterpret_cast<f16_t*>(smem + dt::kOffW);
    unsigned char* sRef = smem + dt::kOffRef;
    int* sSlot = reinterpret_cast<int*>(smem + dt::kOffSlot);
    int* sKd = reinterpret_cast<int*>(smem + dt::kOffKd);
    double* sRev = reinterpret_cast<double*>(smem + dt::kOffRev);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, mrow = lane & 15;
    const int b = blockIdx.z;
    const int tt0 = blockIdx.x * dt::TT;
    const int n0 = blockIdx.y * ncg * dt::kCols;
    const int nchunks = min(ncg, (W2 - n0) / dt::kCols);
    const fp8_t* pool = ref_vals + (size_t)b * cap_ref * W2;

    // ---- W_d register ring. A stage is 64 rows (the pass's output columns) x 64 latent
    // values; thread t holds rows 32 u + t / 8 (u = 0, 1), values 8 (t % 8) .. + 8.
    // Stage x of the run sits in register slot x % 2 and LDS buffer x % 2.
    const int wk8 = tid & 7;
    auto load_w = [&](uint4 (&r)[2], int c, int h, int k) {
        c = min(c, nchunks - 1);  // past the end: any readable stage (never used)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int lr = 32 * u + (tid >> 3);
            const int col = n0 + dt::kCols * c + 16 * chunk_tile<D>(h, lr >> 4) + (lr & 15);
            r[u] = *reinterpret_cast<const uint4*>(wd + (size_t)col * d_c + k * kStageK + 8 * wk8);
        }
    };
    auto store_w = [&](const uint4 (&r)[2], int buf) {
        f16_t* dst = sW + buf * (dt::kWBuf / 2) + (tid >> 3) * dt::kWP + 8 * wk8;
#pragma unroll
        for (int u = 0; u < 2; ++u) *reinterpret_cast<f16x8*>(dst + 32 * u * dt::kWP) = w_to_f16(r[u]);
    };
    // stage (c, h, k) + d of the run, as (c', h', k')
    auto ahead = [](int k, int d, int& du) { du = (k + d) / KST; return (k + d) % KST; };
    uint4 wa[2], wb[2];
    load_w(wa, 0, 0, 0);
    {
        int du;
        const int k1 = ahead(0, 1, du);
        load_w(wb, du >> 1, du & 1, k1);
    }

    // ---- token table: four reference slots per token (-1: zero row) and the divisor
    // of their sum. k_i = 1, 2 or 4 references fill the slots by repetition (slot sum / 4
    // is their mean exactly); k_i = 3 leaves one slot empty and divides by 3. A reference
    // token restores its own stored row (k = 1).
    if (tid < dt::TT) {
        const int t = tt0 + tid;
        int p = -1;
        if (t < m) {
            p = idx[(size_t)b * m + t];
            if (p < 0 || p >= cap_tok) {
                if (blockIdx.y == 0) flag_error(err, DEVERR_IDX_RANGE);
                p = -1;
            }
        }
        const size_t ro = (size_t)b * cap_tok + max(p, 0);
        const int ss = self_slot[ro];
        int r[dt::kRefs];
#pragma unroll
        for (int q = 0; q < dt::kRefs; ++q) r[q] = (q < top_k) ? ref_idx[ro * top_k + q] : -1;
        int sl[dt::kRefs], n = 0;
#pragma unroll
        for (int q = 0; q < dt::kRefs; ++q) sl[q] = -1;
        if (p >= 0) {
            if (ss >= 0) {
                sl[0] = min(ss, cap_ref - 1);
                n = 1;
            } else {
#pragma unroll
                for (int q = 0; q < dt::kRefs; ++q)
                    if (r[q] >= 0) {
                        // compact the valid entries
#pragma unroll
                        for (int u = 0; u < dt::kRefs; ++u)
                            if (u == n) sl[u] = min(r[q], cap_ref - 1);
                        ++n;
                    }
            }
        }
        if (n == 1) sl[1] = sl[2] = sl[3] = sl[0];
        if (n == 2) {
            sl[2] = sl[0];
            sl[3] = sl[1];
        }
#pragma unroll
        for (int q = 0; q < dt::kRefs; ++q) sSlot[tid * dt::kRefs + q] = sl[q];
        sKd[tid] = n == 3 ? 3 : 4;
    }
    // revolutions per position of the RoPE pair frequencies theta^(-2j/D) / (2 pi)
    if (tid < half) sRev[tid] = pow(theta, -2.0 * (double)tid / (double)D) * 0.15915494309189535;

    // ---- this lane's two tokens (MFMA column groups): position, and its latent as
    // fp16 fragments of every K-step (zero for a reference token or an invalid index)
    int tpos[2];
    f16x8 zf[2][NKS];
#pragma unroll
    for (int gr = 0; gr < 2; ++gr) {
        const int t = tt0 + 32 * wave + 16 * gr + mrow;
        int p = t < m ? idx[(size_t)b * m + t] : -1;
        if (p >= cap_tok) p = -1;
        tpos[gr] = p;
        const size_t ro = (size_t)b * cap_tok + max(p, 0);
        const bool enc = p >= 0 && self_slot[ro] < 0;
        const uint8_t* rec = codes + ro * code_bytes;
        uint32_t cw[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            if constexpr (BITS == 4) cw[ks] = *reinterpret_cast<const uint32_t*>(rec + 16 * ks + 4 * g);
            else cw[ks] = *reinterpret_cast<const uint16_t*>(rec + 8 * ks + 2 * g);
        }
        const uint32_t* sp = reinterpret_cast<const uint32_t*>(scale + ro * NKS);
        const uint32_t* zp = reinterpret_cast<const uint32_t*>(zmin + ro * NKS);
        uint32_t st2[NKS / 2], zm2[NKS / 2];
#pragma unroll
        for (int u = 0; u < NKS / 2; ++u) {
            st2[u] = sp[u];
            zm2[u] = zp[u];
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const uint32_t sh = (ks & 1) ? (st2[ks >> 1] >> 16) : (st2[ks >> 1] & 0xFFFFu);
            const uint32_t zh = (ks & 1) ? (zm2[ks >> 1] >> 16) : (zm2[ks >> 1] & 0xFFFFu);
            const uint32_t svp = enc ? (sh | (sh << 16)) : 0u, zvp = enc ? (zh | (zh << 16)) : 0u;
            zf[gr][ks] = dequant8<BITS>(enc ? cw[ks] : 0u, *reinterpret_cast<const f16x2*>(&svp),
                                        *reinterpret_cast<const f16x2*>(&zvp));
        }
    }

    // ---- first W_d stage into LDS buffer 0, the third into the freed registers
    store_w(wa, 0);
    {
        int du;
        const int k2 = ahead(0, 2, du);
        load_w(wa, du >> 1, du & 1, k2);
    }
    __syncthreads();

    // ---- per token: divisor of the slot sum, and cos / sin of the RoPE angles of this
    // lane's pair columns j = 16 jt + 4 g + e of a head's first half; the phase in
    // revolutions is reduced to [-1/2, 1/2] in fp64, then sin / cos in fp32
    float kd[2], rkd[2];
    float rc[2][NJ], rsn[2][NJ];
    bool all4 = true;
#pragma unroll
    for (int gr = 0; gr < 2; ++gr) {
        const int k = sKd[32 * wave + 16 * gr + mrow];
        all4 = all4 && k == 4;
        kd[gr] = (float)k;
        rkd[gr] = __fdiv_rn(1.0f, kd[gr]);
        const double pp = (double)max(tpos[gr], 0);
#pragma unroll
        for (int jt = 0; jt < NJ / 4; ++jt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const double r = pp * sRev[16 * jt + 4 * g + e];
                const float fr = (float)(r - rint(r));
                rc[gr][4 * jt + e] = __builtin_amdgcn_cosf(fr);
                rsn[gr][4 * jt + e] = __builtin_amdgcn_sinf(fr);
            }
    }
    // every token of this wavefront averages its four slots: the 1/4 rides in the
    // selection matrix; otherwise the slot sum is divided exactly per token
    const bool fused_mean = __all(all4);

    // Selection matrix of the reference MFMA (A operand, 16 x 32 FP8): output row r takes
    // K entries (q, r) of the step's two slots q; K entry 8 (lane / 16) + j of this lane
    // is (slot q = lane / 32, column 8 ((lane / 16) % 2) + j). Weight 1/4 (e4m3 0x28) for
    // the fused mean, 1 (0x38) for the exact-division path.
    const bool on = (mrow >> 3) == (g & 1);
    const long sel = on ? (long)((fused_mean ? 0x28ull : 0x38ull) << (8 * (mrow & 7))) : 0l;

    // ---- reference slices of a chunk -> LDS (row p = q * TT + token, 128 bytes; the
    // 16-byte segment s of row p sits at position s ^ (p % 8)). Wave w fetches slot
    // q = w of all 128 tokens, eight rows per load.
    const uint8_t* zero_row = g_zero_row;
    auto issue_refs = [&](int c) {
        const int col = n0 + dt::kCols * c;
        const int wv = wave_id();
        int sl[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) sl[u] = sSlot[(8 * u + (lane >> 3)) * dt::kRefs + wv];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int pr = 128 * wv + 8 * u + (lane >> 3);
            const int seg = (lane & 7) ^ (pr & 7);
            const uint8_t* src =
                sl[u] >= 0 ? reinterpret_cast<const uint8_t*>(pool) + (size_t)sl[u] * W2 + col : zero_row;
            dma16(src + 16 * seg, sRef + 1024 * (16 * wv + u));
        }
        // the reference wait counts the loads issued after these: keep later loads after them
        __builtin_amdgcn_sched_barrier(0);
    };
    issue_refs(0);

    f32x4 acc[2][4];
    for (int c = 0; c < nchunks; ++c) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int gr = 0; gr < 2; ++gr)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[gr][i] = zero4();
#pragma unroll
            for (int k = 0; k < KST; ++k) {
                // stage x: write stage x + 1 to LDS, fetch stage x + 3 into its registers
                int du;
                const int k3 = ahead(k, 3, du);
                const int c3 = c + ((h + du) >> 1), h3 = (h + du) & 1;
                if (k % 2 == 0) {
                    store_w(wb, 1);
                    load_w(wb, c3, h3, k3);
                } else {
                    store_w(wa, 0);
                    load_w(wa, c3, h3, k3);
                }
                const f16_t* W = sW + (k % 2) * (dt::kWBuf / 2);
#pragma unroll
                for (int kh = 0; kh < 2; ++kh) {
                    const int ks = 2 * k + kh;
                    typename Mma<f16_t>::frag fw[4];
#pragma unroll
                    for (int lt = 0; lt < 4; ++lt)
                        fw[lt] = lds_frag<f16_t>(W + (16 * lt + mrow) * dt::kWP + 32 * kh + 8 * g);
#pragma unroll
                    for (int lt = 0; lt < 4; ++lt) {
                        acc[0][lt] = Mma<f16_t>::step(acc[0][lt], fw[lt], zf[0][ks]);
                        acc[1][lt] = Mma<f16_t>::step(acc[1][lt], fw[lt], zf[1][ks]);
                    }
                }
                lds_barrier();
            }

            // ---- pass (c, h) done: reference mean, RoPE, store
            if (h == 0) {
                // this wavefront's reference loads of chunk c have landed once at most the
                // W_d loads of this pass (2 per stage) are still in flight
                wait_vmcnt<2 * KST>();
                lds_barrier();
            }
            const int col0 = n0 + dt::kCols * c;
            const bool rope = col0 < dk;
#pragma unroll
            for (int gr = 0; gr < 2; ++gr) {
                const int tk = 32 * wave + 16 * gr + mrow;
                f32x4 (&a)[4] = acc[gr];
#pragma unroll
                for (int lt = 0; lt < 4; ++lt) {
                    const int ct = chunk_tile<D>(h, lt);
                    long v[2];
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int pr = (2 * hh + (g >> 1)) * dt::TT + tk;
                        v[hh] = *reinterpret_cast<const long*>(sRef + pr * dt::kCols + 16 * (ct ^ (pr & 7)) +
                                                               8 * (g & 1));
                    }
                    if (fused_mean) {
                        a[lt] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(sel, v[0], a[lt], 0, 0, 0);
                        a[lt] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(sel, v[1], a[lt], 0, 0, 0);
                    } else {
                        f32x4 sm = zero4();
                        sm = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(sel, v[0], sm, 0, 0, 0);
                        sm = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(sel, v[1], sm, 0, 0, 0);
#pragma unroll
                        for (int e = 0; e < 4; ++e) a[lt][e] += div_small(sm[e], kd[gr], rkd[gr]);
                    }
                }
                const int p = tpos[gr];
                if (rope) {
#pragma unroll
                    for (int lt = 0; lt < 2; ++lt) {
                        const int jt = D == 128 ? 2 * h + lt : lt;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float cs = rc[gr][4 * jt + e], sn = rsn[gr][4 * jt + e];
                            const float x1 = a[lt][e], x2 = a[lt + 2][e];
                            a[lt][e] = x1 * cs - x2 * sn;
                            a[lt + 2][e] = x2 * cs + x1 * sn;
                        }
                    }
                }
                const int t = tt0 + tk;
                if (t < m) {
                    const bool valid = p >= 0;
                    OutT* o = out + ((size_t)b * m + t) * W2 + col0 + 4 * g;
#pragma unroll
                    for (int lt = 0; lt < 4; ++lt) {
                        OutT* d = o + 16 * chunk_tile<D>(h, lt);
                        if (valid) store_row4<OutT>(d, a[lt][0], a[lt][1], a[lt][2], a[lt][3]);
                        else store_row4<OutT>(d, 0.f, 0.f, 0.f, 0.f);
                    }
                }
            }
            // both passes are done with this chunk's reference slices: fetch the next
            if (h == 1 && c + 1 < nchunks) {
                lds_barrier();
                issue_refs(c + 1);
            }
        }
    }
}

}  // namespace

template <int NKS, int D, int BITS, typename OutT>
static hipError_t tiles_impl(const Shape& s, const CacheView& c, const int* idx, int m, const void* wd, void* out,
                             hipStream_t st) {
    auto kern = decode_tiles_kernel<NKS, D, BITS, OutT>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, dt::bytes);
    if (e != hipSuccess) return e;
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0)
        ncu = 256;
    const int chunks = s.W2 / dt::kCols;
    const long tiles = (long)((m + dt::TT - 1) / dt::TT) * c.B;
    // one workgroup per CU: split the columns into groups so that the rounds of
    // workgroups times the chunks per workgroup (plus about half a chunk of set-up
    // each) is smallest
    int best_ncg = chunks;
    double best = 1e30;
    for (int ncg = chunks; ncg >= 1; --ncg) {
        const long groups = (chunks + ncg - 1) / ncg;
        const long rounds = (tiles * groups + ncu - 1) / ncu;
        const double cost = (double)rounds * (ncg + 0.5);
        if (cost < best - 1e-9) {
            best = cost;
            best_ncg = ncg;
        }
    }
    const int groups = (chunks + best_ncg - 1) / best_ncg;
    const dim3 grid((unsigned)((m + dt::TT - 1) / dt::TT), (unsigned)groups, (unsigned)c.B);
    hipLaunchKernelGGL(kern, grid, dim3(dt::kThreads), dt::bytes, st, idx, m, best_ncg,
                       static_cast<const fp8_t*>(c.ref_vals), c.self_slot, c.ref_idx, c.codes, c.code_bytes,
                       static_cast<const f16_t*>(c.scale), static_cast<const f16_t*>(c.zmin),
                       static_cast<const bf16_t*>(wd), s.W2, s.dk, s.top_k, c.cap_ref, c.cap_tok, s.theta,
                       static_cast<OutT*>(out), c.err);
    return hipGetLastError();
}

template <int D, int BITS, typename OutT>
static hipError_t tiles_dc(const Shape& s, const CacheView& c, const int* idx, int m, const void* wd, void* out,
                           hipStream_t st) {
    switch (s.d_c / 32) {
        case 4: return tiles_impl<4, D, BITS, OutT>(s, c, idx, m, wd, out, st);
        case 8: return tiles_impl<8, D, BITS, OutT>(s, c, idx, m, wd, out, st);
        case 12: return tiles_impl<12, D, BITS, OutT>(s, c, idx, m, wd, out, st);
        case 16: return tiles_impl<16, D, BITS, OutT>(s, c, idx, m, wd, out, st);
        default: return hipErrorInvalidValue;
    }
}

template <typename OutT>
static hipError_t tiles_d(const Shape& s, const CacheView& c, const int* idx, int m, const void* wd, void* out,
                          hipStream_t st) {
    if (s.D == 64) {
        if (s.bits == 4) return tiles_dc<64, 4, OutT>(s, c, idx, m, wd, out, st);
        return tiles_dc<64, 2, OutT>(s, c, idx, m, wd, out, st);
    }
    if (s.bits == 4) return tiles_dc<128, 4, OutT>(s, c, idx, m, wd, out, st);
    return tiles_dc<128, 2, OutT>(s, c, idx, m, wd, out, st);
}

bool decode_tiles_supported(const Shape& s) {
    return !s.f32 && (s.bits == 4 || s.bits == 2) && s.group == 32 && (s.D == 64 || s.D == 128) &&
           s.dk % dt::kCols == 0 &&
           s.W2 % dt::kCols == 0 && s.d_c % 128 == 0 && s.d_c <= 512 && s.top_k <= dt::kRefs;
}

hipError_t launch_decode_tiles(const Shape& s, const CacheView& c, const int* idx, int m, const void* wd, void* out,
                               int out_dtype, hipStream_t st) {
    if (m <= 0) return hipSuccess;
    if (out_dtype == RKV_F32) return tiles_d<float>(s, c, idx, m, wd, out, st);
    return tiles_d<bf16_t>(s, c, idx, m, wd, out, st);
}

}  // namespace rkv
