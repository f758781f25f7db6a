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

#include <type_traits>

#include "rkv_device.h"
#include "rkv_internal.h"
#include "rkv_pipe.h"

namespace rkv {

namespace {

namespace dt {
constexpr int kThreads = 256;       // 4 wavefronts
constexpr int TT = 128;             // tokens per workgroup
constexpr int kCols = 128;          // output columns per chunk
constexpr int kHalf = 64;           // output columns per pass (4 MFMA tiles of 16)
constexpr int kRefs = 4;            // reference slots per token (k <= 4)
constexpr int kRefBuf = TT * kRefs * kHalf;  // FP8 reference slices of one pass
constexpr int kRotBytes = 64 * 8;            // float2 [64]: revolutions per position, split hi + lo
}  // namespace dt

// LDS layout of form 1 (register-staged W_d)
namespace rr {
constexpr int kWP = kStageK + 8;                 // fp16 pitch of a staged W_d row (conflict-free reads)
constexpr int kWBuf = dt::kHalf * kWP * 2;       // one W_d stage (64 rows x 64 K fp16)
constexpr int kWSlots = 3;                       // W_d stages resident in LDS
constexpr int kPieces = dt::kRefBuf / (16 * dt::kThreads);  // 16-byte slices per thread and pass
constexpr int kOffW = 0;
constexpr int kOffRef = kOffW + kWSlots * kWBuf;       // two pass buffers
constexpr int kOffSlot = kOffRef + 2 * dt::kRefBuf;    // int [TT][kRefs]; -1: none
constexpr int kOffKd = kOffSlot + dt::TT * dt::kRefs * 4;  // int [TT]: divisor of the slot sum
constexpr int kOffRot = kOffKd + dt::TT * 4;           // RoPE frequencies (rope_cs)
constexpr int bytes = kOffRot + dt::kRotBytes;
// set-up table that lives in the reference buffers until their first fill
constexpr int kOffPos = kOffRef;                       // int [TT]
static_assert(bytes <= 160 * 1024, "LDS budget");
}  // namespace rr

// LDS layout of form 2 (prepared fp16 W_d by direct loads)
namespace dl {
constexpr int NST = 8;                           // W_d stages in flight
constexpr int kWStage = dt::kHalf * kStageK * 2;  // 8 KB
constexpr int kOffW = 0;
constexpr int kOffRef = kOffW + NST * kWStage;   // two pass buffers (pass h of a chunk: buffer h)
constexpr int kOffSlot = kOffRef + 2 * dt::kRefBuf;
constexpr int kOffKd = kOffSlot + dt::TT * dt::kRefs * 4;
constexpr int kOffRot = kOffKd + dt::TT * 4;
constexpr int kOffPos = kOffRot + dt::kRotBytes;  // int [TT]
constexpr int bytes = kOffPos + dt::TT * 4;
static_assert(bytes <= 160 * 1024, "LDS budget");
}  // namespace dl

// 64 zero bytes: the slices of an empty reference slot
__device__ __align__(16) uint8_t g_zero_slice[64];


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
    const f32x2 lo = {a, b}, hi = {c, d};
    const bf16x2 x = __builtin_convertvector(lo, bf16x2), y = __builtin_convertvector(hi, bf16x2);
    *reinterpret_cast<uint2*>(p) = make_uint2(*reinterpret_cast<const uint32_t*>(&x), *reinterpret_cast<const uint32_t*>(&y));
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

// ---- set-up shared by every restore kernel ------------------------------------------------
// Everything a workgroup needs before its first pass, in two rounds of independent global
// loads: the token indices (round 1), then what hangs off an index, i.e. the self slot,
// the reference slots and the record (round 2). Addresses are clamped to valid memory and
// validity is applied after the loads, so no load waits behind a branch or a wait for an
// earlier one.
//
// Token table (threads 0..TT-1, one token each): four reference slots per token (-1: an
// empty slot, read as zeros) and the divisor of their sum. k_i = 1, 2 or 4 references
// fill the slots by repetition (slot sum / 4 is their mean exactly); k_i = 3 leaves one
// slot empty and divides by 3. A reference token restores its own stored row (k = 1).
// Also the position of every token and, for RoPE, the revolutions per position of the
// pair frequencies theta^(-2j/D) / (2 pi).
//
// Latents: this lane's two tokens (MFMA column groups of token group tg, tokens 32 tg ..
// + 32 of the tile) as fp16 fragments of every K-step in the latent order above (zero for
// a reference token or an invalid index).
template <int NKS, int BITS>
struct TileSetup {
    typedef typename std::conditional<BITS == 16, u32x4, uint32_t>::type Word;
    int tt, tp, tss, tr[dt::kRefs];        // token table: thread tid % TT's token
    int lt[2], lp[2], lss[2];              // the lane's two latent tokens
    Word cw[2][NKS];                       // their code words (BITS 2 / 4) or fp16 values
    uint32_t st[2][NKS / 4], zm[2][NKS / 4];  // their groups' steps and minima (fp16 bits)

    // a loaded value used here on every path: the compiler cannot sink its load into the
    // branch that needs it (with a wait of its own), so a round's loads share one wait
    template <typename T>
    static __device__ inline void pin(const T& v) {
        asm volatile("" ::"v"(v));
    }

    // round 1: the token indices (positions past m read index m - 1 and are dropped later)
    __device__ inline void index(const int* __restrict__ idx, int m, int b, int tt0, int tg) {
        const int tid = threadIdx.x, lane = tid & 63, mrow = lane & 15;
        tt = tt0 + (tid & (dt::TT - 1));
        tp = idx[(size_t)b * m + min(tt, m - 1)];
#pragma unroll
        for (int gr = 0; gr < 2; ++gr) {
            lt[gr] = tt0 + 32 * tg + 16 * gr + mrow;
            lp[gr] = idx[(size_t)b * m + min(lt[gr], m - 1)];
        }
        pin(tp);
        pin(lp[0]);
        pin(lp[1]);
    }

    // round 2: what hangs off an index, at the index clamped into the sequence's records
    __device__ inline void fetch(const int* __restrict__ self_slot, const int* __restrict__ ref_idx, int top_k,
                                 const uint8_t* __restrict__ codes, size_t code_bytes,
                                 const f16_t* __restrict__ scale, const f16_t* __restrict__ zmin, int b,
                                 int cap_tok) {
        const int lane = threadIdx.x & 63, g = lane >> 4;
        {
            const size_t ro = (size_t)b * cap_tok + min(max(tp, 0), cap_tok - 1);
            tss = self_slot[ro];
#pragma unroll
            for (int q = 0; q < dt::kRefs; ++q) tr[q] = ref_idx[ro * top_k + min(q, top_k - 1)];
        }
        constexpr int d_c = 32 * NKS;
#pragma unroll
        for (int gr = 0; gr < 2; ++gr) {
            const size_t ro = (size_t)b * cap_tok + min(max(lp[gr], 0), cap_tok - 1);
            lss[gr] = self_slot[ro];
            const uint8_t* rec = codes + ro * code_bytes;
            if constexpr (BITS == 16) {
                // unquantized record: d_c fp16 values in latent order; K-step ks of lane
                // group g: values d_c / 4 g + 8 ks .. + 8
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    cw[gr][ks] = *reinterpret_cast<const u32x4*>(rec + (d_c / 2) * g + 16 * ks);
            } else {
                if constexpr (BITS == 4) {
                    // 8 codes of K-step ks in one word: the lane's NKS words are contiguous
#pragma unroll
                    for (int j = 0; j < NKS / 4; ++j) {
                        const u32x4 w = *reinterpret_cast<const u32x4*>(rec + (d_c / 8) * g + 16 * j);
#pragma unroll
                        for (int i = 0; i < 4; ++i) cw[gr][4 * j + i] = w[i];
                    }
                } else {
                    // 8 codes of K-step ks in 16 bits
#pragma unroll
                    for (int j = 0; j < NKS / 4; ++j) {
                        const uint2 w = *reinterpret_cast<const uint2*>(rec + (d_c / 16) * g + 8 * j);
                        cw[gr][4 * j + 0] = w.x & 0xFFFFu;
                        cw[gr][4 * j + 1] = w.x >> 16;
                        cw[gr][4 * j + 2] = w.y & 0xFFFFu;
                        cw[gr][4 * j + 3] = w.y >> 16;
                    }
                }
                // the lane's quantizer groups (NKS / 4 g .. + NKS / 4)
                const uint16_t* sp = reinterpret_cast<const uint16_t*>(scale + ro * NKS) + (NKS / 4) * g;
                const uint16_t* zp = reinterpret_cast<const uint16_t*>(zmin + ro * NKS) + (NKS / 4) * g;
#pragma unroll
                for (int j = 0; j < NKS / 4; ++j) {
                    st[gr][j] = sp[j];
                    zm[gr][j] = zp[j];
                }
            }
        }
        pin(tss);
#pragma unroll
        for (int q = 0; q < dt::kRefs; ++q) pin(tr[q]);
#pragma unroll
        for (int gr = 0; gr < 2; ++gr) pin(lss[gr]);
    }

    // the token table (threads 0..TT-1) and the RoPE frequencies; an index outside
    // [0, cap_tok) raises DEVERR_IDX_RANGE (when flag) and restores a zero row
    template <int D>
    __device__ inline void table(int* sSlot, int* sKd, int* sPos, float* sRot, int m, int cap_ref, int cap_tok,
                                 int top_k, bool flag, int* err) const {
        const int tid = threadIdx.x;
        if (tid < dt::TT) {
            const bool in = tt < m;
            const bool bad = in && (tp < 0 || tp >= cap_tok);
            if (bad && flag) flag_error(err, DEVERR_IDX_RANGE);
            const int p = (in && !bad) ? tp : -1;
            int sl[dt::kRefs], n = 0;
#pragma unroll
            for (int q = 0; q < dt::kRefs; ++q) sl[q] = -1;
            if (p >= 0) {
                if (tss >= 0) {
                    sl[0] = min(tss, cap_ref - 1);
                    n = 1;
                } else {
#pragma unroll
                    for (int q = 0; q < dt::kRefs; ++q)
                        if (q < top_k && tr[q] >= 0) {
                            // compact the valid entries
#pragma unroll
                            for (int u = 0; u < dt::kRefs; ++u)
                                if (u == n) sl[u] = min(tr[q], cap_ref - 1);
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
            sPos[tid] = max(p, 0);
        }
        if (tid < D / 2) {
            // revolutions per position of pair j, theta^(-2j/D) / (2 pi), as hi + lo in fp32
            const double r = pow(theta_, -2.0 * (double)tid / (double)D) * 0.15915494309189535;
            const float hi = (float)r;
            sRot[2 * tid] = hi;
            sRot[2 * tid + 1] = (float)(r - (double)hi);
        }
    }

    __device__ inline void latents(f16x8 (&zf)[2][NKS], int m, int cap_tok) const {
#pragma unroll
        for (int gr = 0; gr < 2; ++gr) {
            const bool enc = lt[gr] < m && lp[gr] >= 0 && lp[gr] < cap_tok && lss[gr] < 0;
            if constexpr (BITS == 16) {
                // reordered 0 4 1 5 2 6 3 7 to match the decoder's fragments
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    u32x4 w = cw[gr][ks];
                    if (!enc) w = u32x4{0u, 0u, 0u, 0u};
                    const u32x4 o = {(w[0] & 0xFFFFu) | (w[2] << 16), (w[0] >> 16) | (w[2] & 0xFFFF0000u),
                                     (w[1] & 0xFFFFu) | (w[3] << 16), (w[1] >> 16) | (w[3] & 0xFFFF0000u)};
                    zf[gr][ks] = *reinterpret_cast<const f16x8*>(&o);
                }
            } else {
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    // K-step ks of lane group g lies in the lane's quantizer group ks / 4
                    const uint32_t sh = st[gr][ks >> 2], zh = zm[gr][ks >> 2];
                    const uint32_t svp = enc ? (sh | (sh << 16)) : 0u, zvp = enc ? (zh | (zh << 16)) : 0u;
                    zf[gr][ks] = dequant8<BITS>(enc ? (uint32_t)cw[gr][ks] : 0u, *reinterpret_cast<const f16x2*>(&svp),
                                                *reinterpret_cast<const f16x2*>(&zvp));
                }
            }
        }
    }
    double theta_;
};

// cos and sin of the RoPE angle of one token and pair frequency: pos times the pair's
// revolutions per position rev = hi + lo (fp32 split of the fp64 value), reduced in
// double-float arithmetic: x = pos hi with its rounding error ex from an FMA (exact),
// x minus its nearest integer (exact), plus ex and pos lo; the result, within about
// 2^-24 revolutions of the exact phase in [-1/2, 1/2], goes to the hardware sine and
// cosine of revolutions. pos < 2^24 is exact in fp32. Contraction stays off: fused into
// x - rint(x), the product would enter unrounded and count ex twice.
__device__ inline void rope_cs(float pos, float hi, float lo, float& c, float& s) {
#pragma clang fp contract(off)
    const float x = pos * hi;
    const float ex = fmaf(pos, hi, -x);
    const float f = (x - __builtin_rintf(x)) + fmaf(pos, lo, ex);
    c = __builtin_amdgcn_cosf(f);
    s = __builtin_amdgcn_sinf(f);
}

// Rotation of one RoPE pair (element e of v1, v2) by the angle with cosine c and sine s. Every restore
// path rotates through this one function with contraction off, so all of them round
// alike (the compiler may otherwise fuse either product into the sum differently in
// each context).
__device__ inline void rope_rotate(f32x4& v1, f32x4& v2, int e, float c, float s) {
#pragma clang fp contract(off)
    const float a = v1[e], b = v2[e];
    v1[e] = a * c - b * s;
    v2[e] = b * c + a * s;
}

// A lane's two token positions (MFMA column groups gr of token group tg), from the
// set-up table sPos, as fp32.
__device__ inline void lane_positions(float (&posf)[2], const int* sPos, int tg) {
    const int lane = threadIdx.x & 63, mrow = lane & 15;
#pragma unroll
    for (int gr = 0; gr < 2; ++gr) posf[gr] = (float)sPos[32 * tg + 16 * gr + mrow];
}

// Form of the reference mean of token group tg. When every token averages its four slots the
// 1/4 rides in the selection matrix (fused); otherwise the slot sum is divided exactly per
// token. Selection matrix of the reference MFMA (A operand, 16 x 32 FP8): output row r
// takes K entries (q, r) of the step's two slots q; K entry 8 (lane / 16) + j of this lane
// is (slot q = lane / 32, column 8 ((lane / 16) % 2) + j). Weight 1/4 (e4m3 0x28) for the
// fused mean, 1 (0x38) for the exact division.
struct MeanForm {
    float kd[2], rkd[2];
    long sel;
    bool fused;
};
__device__ inline MeanForm mean_form(const int* sKd, int tg) {
    const int lane = threadIdx.x & 63, g = lane >> 4, mrow = lane & 15;
    MeanForm f;
    bool all4 = true;
#pragma unroll
    for (int gr = 0; gr < 2; ++gr) {
        const int k = sKd[32 * tg + 16 * gr + mrow];
        all4 = all4 && k == 4;
        f.kd[gr] = (float)k;
        f.rkd[gr] = __fdiv_rn(1.0f, f.kd[gr]);
    }
    f.fused = __all(all4);
    const bool on = (mrow >> 3) == (g & 1);
    f.sel = on ? (long)((f.fused ? 0x28ull : 0x38ull) << (8 * (mrow & 7))) : 0l;
    return f;
}

// A pass of a chunk for NT of its four 16-column tiles: local tiles lt(i) = i (NT = 4) or
// ch + 2 i (NT = 2, column half ch), tokens 32 tg .. + 32 of the tile. The lane holds, for
// its token 32 tg + 16 gr + lane % 16, columns 16 chunk_tile(h, lt(i)) + 4 (lane / 16) + e
// of the chunk in acc[gr][i][e]. Every restore path and tile set rounds alike: the
// accumulators start from the reference mean (pass_mean), the W_d product accumulates on
// top, then pass_rope rotates key columns.
template <int NT>
__device__ constexpr int pass_tile(int ch, int i) {
    return NT == 4 ? i : ch + 2 * i;
}

// The reference mean as the accumulators' initial value: two FP8 MFMAs per output tile
// against the slices in R (row r = q * TT + token, 64 bytes, tile t at 16-byte position
// t ^ ((r / 4) % 4)); with the 1/4 in the selection matrix (fused form) that is the mean,
// otherwise the slot sum divided exactly by the token's k. An invalid index has empty
// slots: zero.
template <bool kFused, int NT>
__device__ inline void pass_mean(f32x4 (&acc)[2][NT], const unsigned char* R, const MeanForm& mf, int ch, int tg) {
    static_assert(NT == 2 || NT == 4, "tile set");
    const int lane = threadIdx.x & 63, g = lane >> 4, mrow = lane & 15;
#pragma unroll
    for (int gr = 0; gr < 2; ++gr) {
        const int tk = 32 * tg + 16 * gr + mrow;
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            const int lt = pass_tile<NT>(ch, i);
            long v[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int r = (2 * hh + (g >> 1)) * dt::TT + tk;
                v[hh] = *reinterpret_cast<const long*>(R + r * dt::kHalf + 16 * (lt ^ ((r >> 2) & 3)) + 8 * (g & 1));
            }
            f32x4 sm = zero4();
            sm = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(mf.sel, v[0], sm, 0, 0, 0);
            sm = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(mf.sel, v[1], sm, 0, 0, 0);
            if constexpr (!kFused) {
#pragma unroll
                for (int e = 0; e < 4; ++e) sm[e] = div_small(sm[e], mf.kd[gr], mf.rkd[gr]);
            }
            acc[gr][i] = sm;
        }
    }
}

// RoPE of a key pass: rope_cs at the lane's token positions posf (frequencies in sRot), on
// the pairs of local tiles (lt, lt + 2).
template <int D, int NT>
__device__ inline void pass_rope(f32x4 (&acc)[2][NT], const float* sRot, const float (&posf)[2], int h, int ch) {
    const int lane = threadIdx.x & 63, g = lane >> 4;
#pragma unroll
    for (int gr = 0; gr < 2; ++gr) {
#pragma unroll
        for (int pr = 0; pr < NT / 2; ++pr) {
            const int i0 = NT == 4 ? pr : 0, i1 = NT == 4 ? pr + 2 : 1;
            const int lt = pass_tile<NT>(ch, i0);
            const int jt = D == 128 ? 2 * h + lt : lt;
            const f32x4 r01 = lds_load<f32x4>(sRot + 2 * (16 * jt + 4 * g));
            const f32x4 r23 = lds_load<f32x4>(sRot + 2 * (16 * jt + 4 * g) + 4);
            const float rh[4] = {r01[0], r01[2], r23[0], r23[2]};
            const float rl[4] = {r01[1], r01[3], r23[1], r23[3]};
            float cs[4], sn[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) rope_cs(posf[gr], rh[e], rl[e], cs[e], sn[e]);
#pragma unroll
            for (int e = 0; e < 4; ++e) rope_rotate(acc[gr][i0], acc[gr][i1], e, cs[e], sn[e]);
        }
    }
}

// End of pass h of a chunk starting at column col0: RoPE on key columns, then the rows'
// store.
template <int D, typename OutT, int NT>
__device__ inline void finish_rows(f32x4 (&acc)[2][NT], const float* sRot, const float (&posf)[2], int h, int col0,
                                   bool rope, int tt0, int m, int b, int W2, OutT* __restrict__ out, int ch, int tg) {
    if (rope) pass_rope<D, NT>(acc, sRot, posf, h, ch);
    const int lane = threadIdx.x & 63, g = lane >> 4, mrow = lane & 15;
#pragma unroll
    for (int gr = 0; gr < 2; ++gr) {
        const int t = tt0 + 32 * tg + 16 * gr + mrow;
        if (t < m) {
            OutT* o = out + ((size_t)b * m + t) * W2 + col0 + 4 * g;
#pragma unroll
            for (int i = 0; i < NT; ++i)
                store_row4<OutT>(o + 16 * chunk_tile<D>(h, pass_tile<NT>(ch, i)), acc[gr][i][0], acc[gr][i][1],
                                 acc[gr][i][2], acc[gr][i][3]);
        }
    }
}

// Work of workgroup blockIdx.x: a token tile (of any sequence) and a run of 128-column chunks.
// The first T1 G1 workgroups cover tiles 0 .. T1 - 1 in runs of ncg1 chunks (G1 runs per tile),
// the rest cover the R remaining tiles in runs of ncg2 chunks (G2 runs per tile); within each
// part the run index varies slowest, so workgroups that run together stream the same W_d
// columns. Tile t is tile t % tpb of sequence t / tpb.
struct TileMapArgs {
    int T1, ncg1, R, ncg2, tpb;
};
struct TileMap {
    int b, tt0, n0, nchunks, grp;
};
__device__ inline TileMap tile_map(const TileMapArgs& a, int W2) {
    const int chunks = W2 / dt::kCols;
    const int G1 = (chunks + a.ncg1 - 1) / a.ncg1;
    const int bid = blockIdx.x;
    int t, grp, ncg;
    if (bid < a.T1 * G1) {
        grp = bid / a.T1;
        t = bid - grp * a.T1;
        ncg = a.ncg1;
    } else {
        const int r = bid - a.T1 * G1;
        grp = r / a.R;
        t = a.T1 + (r - grp * a.R);
        ncg = a.ncg2;
    }
    TileMap m;
    m.b = t / a.tpb;
    m.tt0 = (t - m.b * a.tpb) * dt::TT;
    m.n0 = grp * ncg * dt::kCols;
    m.nchunks = min(ncg, (W2 - m.n0) / dt::kCols);
    m.grp = grp;
    return m;
}

// One workgroup per tile_map entry. NKS = d_c / 32 latent K-steps of 32 coordinates; D =
// head dimension; BITS = 4 or 2 (quantized records) or 16 (fp16 latents).
//
// Latent order of the contraction. In K-step ks the MFMA operand positions 8 g .. 8 g + 7
// (lane group g = lane / 16) carry the latent coordinates d_c / 4 g + 8 ks .. + 8, in the
// order 0 4 1 5 2 6 3 7 the nibble masks produce: lane group g walks through its own
// quarter of the latent, so a lane's codes (and its NKS / 4 quantizer groups' steps and
// minima) are contiguous in the record and load as a few wide reads. W_d's operand follows
// the same map (the prepared copy stores it so, form 1 loads it so); the contraction is
// unchanged.

// ---- form 1: W_d as stored (bf16), converted in the workgroup ---------------------------
template <int NKS, int D, int BITS, typename OutT>
__global__ __launch_bounds__(dt::kThreads) void decode_tiles_kernel(
    const int* __restrict__ idx, int m, TileMapArgs ta, const fp8_t* __restrict__ ref_vals, const int* __restrict__ self_slot,
    const int* __restrict__ ref_idx, const uint8_t* __restrict__ codes, size_t code_bytes,
    const f16_t* __restrict__ scale, const f16_t* __restrict__ zmin, const bf16_t* __restrict__ wd, int W2, int dk,
    int top_k, int cap_ref, int cap_tok, double theta, OutT* __restrict__ out, int* err) {
    constexpr int d_c = 32 * NKS;
    constexpr int KST = d_c / kStageK;  // W_d stages per pass
    static_assert(KST % 2 == 0 && 2 * KST < 64, "stage shape");
    static_assert(D == 64 || D == 128, "head dimension");
    extern __shared__ __align__(16) unsigned char smem[];
    f16_t* sW = reinterpret_cast<f16_t*>(smem + rr::kOffW);
    unsigned char* sRef = smem + rr::kOffRef;
    int* sSlot = reinterpret_cast<int*>(smem + rr::kOffSlot);
    int* sKd = reinterpret_cast<int*>(smem + rr::kOffKd);
    float* sRot = reinterpret_cast<float*>(smem + rr::kOffRot);
    int* sPos = reinterpret_cast<int*>(smem + rr::kOffPos);

    const int tid = threadIdx.x, lane = tid & 63;
    const int g = lane >> 4, mrow = lane & 15;
    const TileMap tm = tile_map(ta, W2);
    const int b = tm.b;
    const int tt0 = tm.tt0;
    const int n0 = tm.n0;
    const int nchunks = tm.nchunks;
    const fp8_t* pool = ref_vals + (size_t)b * cap_ref * W2;

    // ---- W_d register ring. A stage is 64 rows (the pass's output columns) x 64 latent
    // values; thread t holds rows 32 u + t / 8 (u = 0, 1), values 8 (t % 8) .. + 8.
    // Stage x of the run is loaded into register slot x % 2 two stages before it is
    // written to LDS slot x % 3, one stage before it is multiplied.
    const int wk8 = tid & 7;
    auto load_w = [&](uint4 (&r)[2], int c, int h, int k) {
        c = min(c, nchunks - 1);  // past the end: any readable stage (never used)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int lr = 32 * u + (tid >> 3);
            const int col = n0 + dt::kCols * c + 16 * chunk_tile<D>(h, lr >> 4) + (lr & 15);
            // LDS position 8 wk8 of stage k is K-step 2 k + wk8 / 4, lane group wk8 % 4
            r[u] = *reinterpret_cast<const uint4*>(wd + (size_t)col * d_c + 8 * (NKS * (wk8 & 3) + 2 * k + (wk8 >> 2)));
        }
    };
    auto store_w = [&](const uint4 (&r)[2], int slot) {
        f16_t* dst = sW + slot * (rr::kWBuf / 2) + (tid >> 3) * rr::kWP + 8 * wk8;
#pragma unroll
        for (int u = 0; u < 2; ++u) *reinterpret_cast<f16x8*>(dst + 32 * u * rr::kWP) = w_to_f16(r[u]);
    };
    // stage (c, h, k) + d of the run as pass offset du and stage k'
    auto ahead = [](int k, int d, int& du) { du = (k + d) / KST; return (k + d) % KST; };
    auto load_ahead = [&](uint4 (&r)[2], int c, int h, int k, int d) {
        int du;
        const int kk = ahead(k, d, du);
        load_w(r, c + ((h + du) >> 1), (h + du) & 1, kk);
    };
    uint4 wa[2], wb[2];
    load_ahead(wa, 0, 0, 0, 0);
    load_ahead(wb, 0, 0, 0, 1);

    f16x8 zf[2][NKS];
    {
        TileSetup<NKS, BITS> su;
        su.theta_ = theta;
        su.index(idx, m, b, tt0, tid >> 6);
        su.fetch(self_slot, ref_idx, top_k, codes, code_bytes, scale, zmin, b, cap_tok);
        su.template table<D>(sSlot, sKd, sPos, sRot, m, cap_ref, cap_tok, top_k, tm.grp == 0, err);
        su.latents(zf, m, cap_tok);
    }

    // ---- stages 0 and 1 into LDS slots 0 and 1, stages 2 and 3 into the registers
    store_w(wa, 0);
    load_ahead(wa, 0, 0, 0, 2);
    store_w(wb, 1);
    load_ahead(wb, 0, 0, 0, 3);
    __syncthreads();
    float posf[2];
    lane_positions(posf, sPos, tid >> 6);
    const MeanForm mf = mean_form(sKd, tid >> 6);

    // ---- reference slices of a pass -> LDS buffer (pass % 2), in the layout pass_mean
    // reads. Thread t moves slices 256 u + t (u = 0..7): row 64 u + t / 4, tile t % 4;
    // they travel through registers, stored one stage after their fetch.
    auto load_ref = [&](int c, int h, int u) -> uint4 {
        c = min(c, nchunks - 1);  // past the end: any readable slice (never used)
        const int r = 64 * u + (tid >> 2), q = r >> 7, tk = r & (dt::TT - 1);
        const int sl = sSlot[tk * dt::kRefs + q];
        const uint4 v = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(pool) +
                                                         (size_t)max(sl, 0) * W2 + dt::kCols * c + n0 +
                                                         16 * chunk_tile<D>(h, tid & 3));
        return sl >= 0 ? v : make_uint4(0u, 0u, 0u, 0u);
    };
    auto store_ref = [&](uint4 v, int buf, int u) {
        const int r = 64 * u + (tid >> 2);
        *reinterpret_cast<uint4*>(sRef + buf * dt::kRefBuf + r * dt::kHalf + 16 * ((tid & 3) ^ ((r >> 2) & 3))) = v;
    };
    // slices of the next pass fetched in stages 0 .. KST - 2 of a pass (all 8 spread over
    // them) and stored one stage later, so a pass's slices are in LDS when it starts
    constexpr int NP = (rr::kPieces + KST - 2) / (KST - 1);
    auto piece_lo = [](int k) { return rr::kPieces * k / (KST - 1); };

    // the set-up tables in the reference buffers are read; pass 0's slices go in directly
    __syncthreads();
    {
        uint4 v[rr::kPieces];
#pragma unroll
        for (int u = 0; u < rr::kPieces; ++u) v[u] = load_ref(0, 0, u);
#pragma unroll
        for (int u = 0; u < rr::kPieces; ++u) store_ref(v[u], 0, u);
    }
    uint4 ra[NP], rb[NP];  // register slots of the slices fetched in even / odd stages

    // W_d fragments of one stage (2 K-steps x 4 tiles), read one stage ahead
    typedef typename Mma<f16_t>::frag Frag;
    auto read_frags = [&](Frag (&f)[2][4], int slot) {
        const f16_t* W = sW + slot * (rr::kWBuf / 2);
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int lt = 0; lt < 4; ++lt) f[kh][lt] = lds_frag<f16_t>(W + (16 * lt + mrow) * rr::kWP + 32 * kh + 8 * g);
    };
    __syncthreads();
    Frag fa[2][4], fb[2][4];
    read_frags(fa, 0);
    int slot = 0;  // LDS slot of the current stage

    f32x4 acc[2][4];
    for (int c = 0; c < nchunks; ++c) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            // pass p = 2 c + h; its slices are in buffer h (stored by the previous pass, the
            // last of them before its final barrier), the next pass's go to 1 - h
            if (mf.fused) pass_mean<true, 4>(acc, sRef + h * dt::kRefBuf, mf, 0, tid >> 6);
            else pass_mean<false, 4>(acc, sRef + h * dt::kRefBuf, mf, 0, tid >> 6);
#pragma unroll
            for (int k = 0; k < KST; ++k) {
                // stage x: fragments of stage x + 1 (resident since the last barrier); stage
                // x + 2 registers -> LDS and stage x + 4 -> those registers; the slices
                // fetched in the stage before -> LDS and the next ones -> the other registers
                Frag (&cur)[2][4] = (k % 2 == 0) ? fa : fb;
                Frag (&nxt)[2][4] = (k % 2 == 0) ? fb : fa;
                uint4 (&rg)[NP] = (k % 2 == 0) ? ra : rb;
                uint4 (&rp)[NP] = (k % 2 == 0) ? rb : ra;
                const int s1 = slot == 2 ? 0 : slot + 1, s2 = slot == 0 ? 2 : slot - 1;
                read_frags(nxt, s1);
                if (k % 2 == 0) {
                    store_w(wa, s2);
                    load_ahead(wa, c, h, k, 4);
                } else {
                    store_w(wb, s2);
                    load_ahead(wb, c, h, k, 4);
                }
                {
                    // the next pass's slices: those fetched in stage k - 1 -> LDS, stage k's
                    // share -> registers (past the last pass: any readable slices, never read)
                    if (k >= 1) {
#pragma unroll
                        for (int u = 0; u < NP; ++u)
                            if (piece_lo(k - 1) + u < piece_lo(k)) store_ref(rp[u], 1 - h, piece_lo(k - 1) + u);
                    }
                    const int cn = c + h, hn = 1 - h;  // the next pass
                    if (k + 1 < KST) {
#pragma unroll
                        for (int u = 0; u < NP; ++u)
                            if (piece_lo(k) + u < piece_lo(k + 1)) rg[u] = load_ref(cn, hn, piece_lo(k) + u);
                    }
                }
#pragma unroll
                for (int kh = 0; kh < 2; ++kh) {
                    const int ks = 2 * k + kh;
#pragma unroll
                    for (int lt = 0; lt < 4; ++lt) {
                        acc[0][lt] = Mma<f16_t>::step(acc[0][lt], cur[kh][lt], zf[0][ks]);
                        acc[1][lt] = Mma<f16_t>::step(acc[1][lt], cur[kh][lt], zf[1][ks]);
                    }
                }
                slot = s1;
                lds_barrier();
            }
            // ---- pass (c, h) done
            const int col0 = n0 + dt::kCols * c;
            finish_rows<D, OutT, 4>(acc, sRot, posf, h, col0, col0 < dk, tt0, m, b, W2, out, 0, tid >> 6);
        }
    }
}

// ---- form 2: W_d prepared as fp16 (rkv_prepare_decoder), fetched by direct loads -------
// The prepared copy and the reference slices go global -> LDS with global_load_lds:
// no registers are staged and no VALU converts, and every wait on those loads is
// counted here. W_d: a ring of NST stages of 64 rows x 64 latent values, each 8 blocks of
// 16 rows x 32 values (1 KB) in the chunk-swizzled layout of rkv_pipe.h; stage x is
// issued NST stages ahead into the slot stage x - NST used. Reference slices: two buffers
// (pass h of a chunk reads buffer h); a pass's slices are fetched at the start of the pass
// before it, so the gather has a whole pass to land.
//
// Eight wavefronts, two per SIMD: wavefront w takes the tile's tokens 32 (w % 4) .. + 32
// (token group tg) and, of a pass's four 16-column tiles, the column half ch = w / 4
// (local tiles ch and ch + 2, one RoPE pair). The two wavefronts of a SIMD hold the same
// latent fragments and different columns, so LDS reads per stage equal a four-wavefront
// layout's, while each SIMD has two independent instruction streams: with one per SIMD
// the fragment reads and the pass epilogue run at their latency, not their throughput.
namespace w8 {
constexpr int kThreads = 2 * dt::kThreads;
}

// L2 warm-up of a run's W_d rows (run_bytes at run): the workgroups of an XCD (the
// hardware places workgroup i on XCD i % 8) take one share each, so every XCD's L2 holds
// the run before its passes ask for it; without it, after other work has cycled the
// caches, each stage's first request goes to HBM, whose latency the W_d ring cannot cover.
// NL loads of 1 KB per wavefront (NW wavefronts) land in the LDS sink, which the caller
// does not read before younger loads overwrite it.
template <int NL, int NW>
__device__ inline void warm_w(const char* run, size_t run_bytes, unsigned char* sink) {
    const int lane = threadIdx.x & 63, wv = wave_id();
    const int J = max(1, (int)((gridDim.x + 7) >> 3));
    const size_t share = (run_bytes + J - 1) / J;
    const size_t first = (size_t)((blockIdx.x >> 3) % J) * share;
#pragma unroll
    for (int u = 0; u < NL; ++u)
        dma16(run + min(first + (size_t)(NW * u + wv) * 1024 + 16 * lane, run_bytes - 16), sink + 1024 * wv);
}
constexpr int kWarm = 8;  // warm-up loads per wavefront of the restore (64 KB per workgroup)
template <int NKS, int D, int BITS, typename OutT>
__global__ __launch_bounds__(w8::kThreads) void decode_tiles_dl_kernel(
    const int* __restrict__ idx, int m, TileMapArgs ta, const fp8_t* __restrict__ ref_vals, const int* __restrict__ self_slot,
    const int* __restrict__ ref_idx, const uint8_t* __restrict__ codes, size_t code_bytes,
    const f16_t* __restrict__ scale, const f16_t* __restrict__ zmin, const f16_t* __restrict__ w16, int W2, int dk,
    int top_k, int cap_ref, int cap_tok, double theta, OutT* __restrict__ out, int* err) {
    constexpr int d_c = 32 * NKS;
    constexpr int KST = d_c / kStageK;  // W_d stages per pass
    constexpr int NST = dl::NST;
    static_assert(KST >= 2 && 2 * KST + 3 < 64 && NST + 6 + kWarm < 64, "stage shape");
    static_assert(D == 64 || D == 128, "head dimension");
    extern __shared__ __align__(16) unsigned char smem[];
    unsigned char* sW = smem + dl::kOffW;
    unsigned char* sRef = smem + dl::kOffRef;
    int* sSlot = reinterpret_cast<int*>(smem + dl::kOffSlot);
    int* sKd = reinterpret_cast<int*>(smem + dl::kOffKd);
    float* sRot = reinterpret_cast<float*>(smem + dl::kOffRot);
    int* sPos = reinterpret_cast<int*>(smem + dl::kOffPos);

    const int tid = threadIdx.x, lane = tid & 63;
    const TileMap tm = tile_map(ta, W2);
    const int b = tm.b;
    const int tt0 = tm.tt0;
    const int n0 = tm.n0;
    const int nchunks = tm.nchunks;
    const fp8_t* pool = ref_vals + (size_t)b * cap_ref * W2;

    const int wv = wave_id(), tg = wv & 3, ch = wv >> 2, lr = lane >> 2;
    // stage (c, h, k) -> slot ((2 c + h) KST + k) % NST. Wave w fills block w = 2 lt + kh
    // (row group lt = local MFMA tile, K half kh); lane l fetches row l / 4, chunk
    // swz(l / 4, l % 4). rowoff[h]: the lane's output column in pass h.
    const int rowoff[2] = {16 * chunk_tile<D>(0, wv >> 1) + lr, 16 * chunk_tile<D>(1, wv >> 1) + lr};
    const f16_t* wbase = w16 + (size_t)n0 * d_c + 8 * swz(lr, lane & 3) + 32 * (wv & 1);
    auto issue_w = [&](int c, int h, int k, int slot) {
        c = min(c, nchunks - 1);  // past the end: any readable stage (never used)
        dma16(wbase + ((size_t)dt::kCols * c + rowoff[h]) * d_c + k * kStageK, sW + slot * dl::kWStage + 1024 * wv);
    };
    // slices of a pass: DMA j (wave w issues 4 w .. + 4) fills rows 16 j .. + 16, i.e. slot
    // q = w / 2 of tokens 16 (j % 8) .. + 16; lane l fills row 16 j + l / 4 at 16-byte
    // position l % 4 with its tile ts = (l % 4) ^ ((row / 4) % 4). The tile's column offset
    // splits into a part of the pass, 16 chunk_tile(h, 0), and a part of the lane; rsrc[u]
    // holds the lane's slot row plus that lane part (null: an empty slot, read from the
    // zero slice), set once the token table is built.
    const int ts_l = (lane & 3) ^ ((lr >> 2) & 3);
    const uint8_t* zsrc = g_zero_slice + 16 * ts_l;
    const uint8_t* rsrc[4];
    auto issue_refs = [&](int c, int h, unsigned char* buf) {
        const size_t off = (size_t)n0 + dt::kCols * c + 16 * chunk_tile<D>(h, 0);
#pragma unroll
        for (int u = 0; u < 4; ++u) dma16(rsrc[u] ? rsrc[u] + off : zsrc, buf + 1024 * (4 * wv + u));
    };
    // stage (c, h, k) + d of the run
    auto ahead = [](int c, int h, int k, int d, int& c2, int& h2) {
        const int du = (k + d) / KST;
        c2 = c + ((h + du) >> 1);
        h2 = (h + du) & 1;
        return (k + d) % KST;
    };

    // W_d stages 0 .. NST - 1 (they do not depend on the tokens)
#pragma unroll
    for (int d = 0; d < NST; ++d) {
        int c2, h2;
        const int k2 = ahead(0, 0, 0, d, c2, h2);
        issue_w(c2, h2, k2, d);
    }
    f16x8 zf[2][NKS];
    TileSetup<NKS, BITS> su;
    su.theta_ = theta;
    su.index(idx, m, b, tt0, tg);
    su.fetch(self_slot, ref_idx, top_k, codes, code_bytes, scale, zmin, b, cap_tok);
    su.template table<D>(sSlot, sKd, sPos, sRot, m, cap_ref, cap_tok, top_k, tm.grp == 0, err);
    // (no workgroup fence here or below: it would wait for every load in flight)
    lds_barrier();
    // slices of the first pass, as soon as the slot table stands (they follow every W_d
    // stage of the prologue; the latents' loads may still be in flight)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int sl = sSlot[(16 * (4 * (wv & 1) + u) + lr) * dt::kRefs + (wv >> 1)];
        const int lane_tile = chunk_tile<D>(0, ts_l) - chunk_tile<D>(0, 0);
        rsrc[u] = sl >= 0 ? reinterpret_cast<const uint8_t*>(pool) + (size_t)sl * W2 + 16 * lane_tile : nullptr;
    }
    issue_refs(0, 0, sRef);
    // the second slice buffer is the warm-up's sink: the slices of pass 1 (younger loads,
    // so they land later) overwrite it before anything reads it
    {
        const char* run = reinterpret_cast<const char*>(w16 + (size_t)n0 * d_c);
        warm_w<kWarm, 8>(run, (size_t)nchunks * dt::kCols * d_c * 2, sRef + dt::kRefBuf);
    }
    su.latents(zf, m, cap_tok);
    float posf[2];
    lane_positions(posf, sPos, tg);
    const MeanForm mf = mean_form(sKd, tg);
    // W_d stages 0 .. NST - 1 and the set-up's loads have landed once at most the first
    // pass's 4 slice loads and the warm-up's are in flight; the barrier makes every
    // wavefront's stages visible
    wait_vmcnt<4 + kWarm>();
    lds_barrier();

    // one K-step of this wavefront's W_d fragments (its 2 tiles)
    typedef typename Mma<f16_t>::frag Frag;
    auto read_frags = [&](Frag (&f)[2], int slot, int kh) {
        const char* sp = reinterpret_cast<const char*>(sW + slot * dl::kWStage);
#pragma unroll
        for (int i = 0; i < 2; ++i) f[i] = Op16<64>::frag<f16_t>(sp, pass_tile<2>(ch, i), kh);
    };
    auto mma = [&](f32x4 (&acc)[2][2], const Frag (&f)[2], int ks) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            acc[0][i] = Mma<f16_t>::step(acc[0][i], f[i], zf[0][ks]);
            acc[1][i] = Mma<f16_t>::step(acc[1][i], f[i], zf[1][ks]);
        }
    };
    // Per pass: wait for its slices (fetched a pass ahead), barrier, the reference mean into
    // the accumulators, then the stages. Per stage x (K-steps 0 and 1, fragments f0, f1):
    //   read f1(x) | MFMA f0(x) | wait stage x + 1, barrier | read f0(x + 1) | MFMA f1(x) |
    //   f0(x + 1) in registers, then refill slot x with stage x + NST (and, in a pass's
    //   first stage, fetch the next pass's reference slices).
    // The direct loads go out right after an explicit wait on the fragment reads: the
    // compiler treats a pending direct load as an access to both LDS and memory and turns
    // its next wait on LDS reads into a full one, so none of its waits may fall behind one.
    Frag f0[2], f1[2];
    read_frags(f0, 0, 0);
    int slot = 0;

    f32x4 acc[2][2];
    for (int c = 0; c < nchunks; ++c) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const bool first = c == 0 && h == 0;
            // this pass's slices: the first pass's came with the set-up (followed by the
            // warm-up's loads); a later pass's were waited for in the previous pass's last
            // stage, whose barrier made them visible
            if (first) {
                wait_vmcnt<kWarm>();
                lds_barrier();
            }
            if (mf.fused) pass_mean<true, 2>(acc, sRef + h * dt::kRefBuf, mf, ch, tg);
            else pass_mean<false, 2>(acc, sRef + h * dt::kRefBuf, mf, ch, tg);
#pragma unroll
            for (int k = 0; k < KST; ++k) {
                read_frags(f1, slot, 1);
                mma(acc, f0, 2 * k);
                // the two fragment reads go out before the four MFMAs that cover them
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
                __builtin_amdgcn_sched_barrier(0);
                // stage x + 1 must have landed. Issued after it (per wavefront): stages x + 2
                // .. x + NST - 1 (1 load each) and, from a pass's second stage on, the 4 slice
                // loads of its first stage; in the first pass also the set-up's slice and
                // warm-up loads (stage x + 1 < NST came with the prologue), so there stage 0
                // counts 4 + kWarm more and stages 1 .. NST - 2 count 8 + kWarm more. A count
                // below the true one only waits longer.
                // The last stage also waits for the next pass's slices (issued in the first
                // stage, followed by the W_d loads of stages 1 .. KST - 2).
                if (k == KST - 1) wait_vmcnt<(KST - 2 < NST - 2 ? KST - 2 : NST - 2)>();
                else if (first && k == 0) wait_vmcnt<NST - 2 + 4 + kWarm>();
                else if (first && k <= NST - 2) wait_vmcnt<NST - 2 + 8 + kWarm>();
                else if (k >= 1 && k <= NST - 1) wait_vmcnt<NST - 2 + 4>();
                else wait_vmcnt<NST - 2>();
                lds_barrier();
                const int next = slot + 1 == NST ? 0 : slot + 1;
                read_frags(f0, next, 0);
                mma(acc, f1, 2 * k + 1);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
                __builtin_amdgcn_sched_barrier(0);
                wait_lgkm0();
                {
                    int c2, h2;
                    const int k2 = ahead(c, h, k, NST, c2, h2);
                    issue_w(c2, h2, k2, slot);
                }
                // the next pass's slices go to the other buffer, last read by the mean at
                // the previous pass's start; past the last pass they reload the last chunk's
                // into a buffer nobody reads, which keeps the counts uniform
                if (k == 0) issue_refs(h == 0 ? c : min(c + 1, nchunks - 1), 1 - h, sRef + (1 - h) * dt::kRefBuf);
                __builtin_amdgcn_sched_barrier(0);
                slot = next;
            }
            // ---- pass (c, h) done: RoPE on key columns, then the rows' store
            const int col0 = n0 + dt::kCols * c;
            finish_rows<D, OutT, 2>(acc, sRot, posf, h, col0, col0 < dk, tt0, m, b, W2, out, ch, tg);
        }
    }
}

// ---- restore fused with the attention of one decoding query per head --------------------
// (review page section 2.7: the layer attends over the restored selected tokens.) A
// workgroup takes a token tile and a run of "units": unit u is the K chunk u (columns
// 128 u ..) and the V chunk u (columns d_k + 128 u ..), i.e. one KV head at D = 128 and
// two at D = 64; the run does K u, V u, K u + 1, V u + 1, ... on the pipeline and with the
// eight wavefronts of decode_tiles_dl_kernel. A pass's restored values (after the
// reference mean and, on keys, RoPE) go to LDS in bf16, the precision the restored rows
// have in the unfused path, instead of to memory:
//   K pass: the keys to LDS [token][column]; the four wavefronts of column half 0 take
//           the scores s[g][t] = q_g . K[t] of their 32 tokens on MFMA (query heads on the
//           16-wide side); when a head's key columns are done, the tile's softmax:
//           m = max_t scale s, p = exp(scale s - m), l = sum_t p (wave reductions, the
//           four token groups through LDS), p to LDS in fp16;
//   V pass: the values to LDS transposed [column][token] in fp16 and o[g][d] =
//           sum_t p[g][t] V[t][d] on MFMA: wavefront w takes 16 columns and half the
//           tokens, the two halves added through LDS.
// Each (tile, KV head, query head) leaves (o, m, l); attend_combine_kernel rescales the
// tiles to the overall maximum and divides by the sum.
namespace fa {
template <int D>
struct L {
    static constexpr int G = kAttendMaxG;  // room for the largest query-head group
    static constexpr int NST = dl::NST;
    static constexpr int kKP = dt::kHalf + 8;    // bf16 pitch of a key row of the pass (144 B)
    static constexpr int kVP = dt::TT + 8;       // f16 pitch of a value column (272 B)
    static constexpr int kQP = D + 8;            // bf16 pitch of a query row
    static constexpr int kPP = dt::TT + 8;       // f16 pitch of a weight row
    static constexpr int kNH = D == 64 ? 2 : 1;  // KV heads of a unit
    static constexpr int kOffW = 0;
    static constexpr int kOffRef = kOffW + NST * dl::kWStage;  // two pass buffers (pass h: buffer h)
    static constexpr int kOffSlot = kOffRef + 2 * dt::kRefBuf;
    static constexpr int kOffKd = kOffSlot + dt::TT * dt::kRefs * 4;
    static constexpr int kOffRot = kOffKd + dt::TT * 4;
    // keys of the pass [TT][kKP] bf16, or values of the pass transposed [64][kVP] f16
    static constexpr int kOffKV = kOffRot + dt::kRotBytes;
    static constexpr int kKVBytes = dt::TT * kKP * 2 > 64 * kVP * 2 ? dt::TT * kKP * 2 : 64 * kVP * 2;
    static constexpr int kOffQ = kOffKV + kKVBytes;                 // bf16 [kNH][G][kQP]
    static constexpr int kOffP = kOffQ + kNH * G * kQP * 2;         // f16 weights [kNH][G][kPP]
    static constexpr int kOffS = kOffP + kNH * G * kPP * 2;         // fp32 partial scores [G][TT]
    static constexpr int kOffRed = kOffS + G * dt::TT * 4;          // fp32 [max, sum][4 waves][8]
    static constexpr int bytes = kOffRed + 2 * 4 * 8 * 4;
    static constexpr int kOffPos = kOffRef;
    static_assert(bytes <= 160 * 1024, "LDS budget");
    // the MFMA operand reads of query / weight rows G .. 15 (unused output columns) stay
    // inside the allocation
    static_assert(kOffRed + 2 * 4 * 8 * 4 >= kOffP + (kNH * G + 8) * kPP * 2, "operand over-read");
};
}  // namespace fa

template <int NKS, int D, int BITS>
__global__ __launch_bounds__(w8::kThreads) void restore_attend_kernel(
    const int* __restrict__ idx, int m, TileMapArgs ta, const fp8_t* __restrict__ ref_vals,
    const int* __restrict__ self_slot, const int* __restrict__ ref_idx, const uint8_t* __restrict__ codes,
    size_t code_bytes, const f16_t* __restrict__ scale, const f16_t* __restrict__ zmin, const f16_t* __restrict__ w16,
    int W2, int dk, int top_k, int cap_ref, int cap_tok, double theta, const bf16_t* __restrict__ q, int G,
    float qscale, float* __restrict__ part_o, float* __restrict__ part_ml, int* err) {
    typedef fa::L<D> Ly;
    constexpr int d_c = 32 * NKS;
    constexpr int KST = d_c / kStageK;
    constexpr int NST = Ly::NST;
    static_assert(KST >= 2 && 2 * KST + 3 < 64 && NST + 6 < 64, "stage shape");
    static_assert(D == 64 || D == 128, "head dimension");
    extern __shared__ __align__(16) unsigned char smem[];
    unsigned char* sW = smem + Ly::kOffW;
    unsigned char* sRef = smem + Ly::kOffRef;
    int* sSlot = reinterpret_cast<int*>(smem + Ly::kOffSlot);
    int* sKd = reinterpret_cast<int*>(smem + Ly::kOffKd);
    float* sRot = reinterpret_cast<float*>(smem + Ly::kOffRot);
    unsigned char* sKV = smem + Ly::kOffKV;
    unsigned char* sQ = smem + Ly::kOffQ;
    unsigned char* sP = smem + Ly::kOffP;
    float* sS = reinterpret_cast<float*>(smem + Ly::kOffS);
    float* sRed = reinterpret_cast<float*>(smem + Ly::kOffRed);
    int* sPos = reinterpret_cast<int*>(smem + Ly::kOffPos);

    const int tid = threadIdx.x, lane = tid & 63;
    const int N = dk / D;
    const int Hq = N * G;
    // units play the part of the restore's chunks in the tile map (dk / 128 of them, as
    // restore_attend_impl built the grid)
    const TileMap tm = tile_map(ta, dk);
    const int b = tm.b, tt0 = tm.tt0, tile = tt0 / dt::TT;
    const int u0 = tm.n0 / dt::kCols;
    const int nchunks = 2 * tm.nchunks;
    const int ntiles = ta.tpb;
    const fp8_t* pool = ref_vals + (size_t)b * cap_ref * W2;
    auto chunk_col = [&](int c) {
        const int u = u0 + (c >> 1);
        return (c & 1) ? dk + dt::kCols * u : dt::kCols * u;
    };

    // the restore's layout and streams as in decode_tiles_dl_kernel: wavefront w takes token
    // group tg = w % 4 and column half ch = w / 4 of each pass, fills W_d block w of every
    // stage and 4 of the 32 slice blocks of every pass
    const int wv = wave_id(), tg = wv & 3, ch = wv >> 2, lr = lane >> 2;
    const int rowoff[2] = {16 * chunk_tile<D>(0, wv >> 1) + lr, 16 * chunk_tile<D>(1, wv >> 1) + lr};
    const f16_t* wswz = w16 + 8 * swz(lr, lane & 3) + 32 * (wv & 1);
    auto issue_w = [&](int c, int h, int k, int slot) {
        c = min(c, nchunks - 1);  // past the end: any readable stage (never used)
        dma16(wswz + ((size_t)chunk_col(c) + rowoff[h]) * d_c + k * kStageK, sW + slot * dl::kWStage + 1024 * wv);
    };
    const int ts_l = (lane & 3) ^ ((lr >> 2) & 3);
    const uint8_t* zsrc = g_zero_slice + 16 * ts_l;
    const uint8_t* rsrc[4];
    auto issue_refs = [&](int c, int h, unsigned char* buf) {
        const size_t off = (size_t)chunk_col(c) + 16 * chunk_tile<D>(h, 0);
#pragma unroll
        for (int u = 0; u < 4; ++u) dma16(rsrc[u] ? rsrc[u] + off : zsrc, buf + 1024 * (4 * wv + u));
    };
    auto ahead = [](int c, int h, int k, int d, int& c2, int& h2) {
        const int du = (k + d) / KST;
        c2 = c + ((h + du) >> 1);
        h2 = (h + du) & 1;
        return (k + d) % KST;
    };

#pragma unroll
    for (int d = 0; d < NST; ++d) {
        int c2, h2;
        const int k2 = ahead(0, 0, 0, d, c2, h2);
        issue_w(c2, h2, k2, d);
    }
    f16x8 zf[2][NKS];
    TileSetup<NKS, BITS> su;
    su.theta_ = theta;
    su.index(idx, m, b, tt0, tg);
    su.fetch(self_slot, ref_idx, top_k, codes, code_bytes, scale, zmin, b, cap_tok);
    su.template table<D>(sSlot, sKd, sPos, sRot, m, cap_ref, cap_tok, top_k, tm.grp == 0, err);
    // (no workgroup fence here or below: it would wait for every load in flight)
    lds_barrier();
    float posf[2];
    lane_positions(posf, sPos, tg);
    const MeanForm mf = mean_form(sKd, tg);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int sl = sSlot[(16 * (4 * (wv & 1) + u) + lr) * dt::kRefs + (wv >> 1)];
        const int lane_tile = chunk_tile<D>(0, ts_l) - chunk_tile<D>(0, 0);
        rsrc[u] = sl >= 0 ? reinterpret_cast<const uint8_t*>(pool) + (size_t)sl * W2 + 16 * lane_tile : nullptr;
    }
    // the token positions live in the first slice buffer: read by all before its fill
    lds_barrier();
    issue_refs(0, 0, sRef);
    su.latents(zf, m, cap_tok);
    // W_d stages 0 .. NST - 1 and the set-up's loads have landed once at most the first
    // pass's 4 slice loads are in flight; the barrier makes every wavefront's stages visible
    wait_vmcnt<4>();
    lds_barrier();

    typedef typename Mma<f16_t>::frag Frag;
    auto read_frags = [&](Frag (&f)[2], int slot, int kh) {
        const char* sp = reinterpret_cast<const char*>(sW + slot * dl::kWStage);
#pragma unroll
        for (int i = 0; i < 2; ++i) f[i] = Op16<64>::frag<f16_t>(sp, pass_tile<2>(ch, i), kh);
    };
    auto mma = [&](f32x4 (&acc)[2][2], const Frag (&f)[2], int ks) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            acc[0][i] = Mma<f16_t>::step(acc[0][i], f[i], zf[0][ks]);
            acc[1][i] = Mma<f16_t>::step(acc[1][i], f[i], zf[1][ks]);
        }
    };

    // queries of a unit, bf16 [kNH][G][kQP] (consecutive query heads share a KV head)
    auto stage_q = [&](int u) {
        for (int e = tid; e < Ly::kNH * G * D; e += w8::kThreads) {
            const int r = e / D, d = e - r * D;  // r = hh G + g
            const int hq = Ly::kNH * u * G + r;
            reinterpret_cast<bf16_t*>(sQ)[r * Ly::kQP + d] = q[((size_t)b * Hq + hq) * D + d];
        }
    };
    stage_q(u0);  // the main loop's barriers order it before the first score pass

    const int g4 = lane >> 4, mrow = lane & 15;
    float* sMax = sRed;
    float* sSum = sRed + 32;

    // The attention part of the end of pass (c, h), on MFMA. Every wavefront stages its own
    // values (its 32 tokens, its 2 column tiles); the wavefronts of column half 0 then take
    // the scores of their 32 tokens (two tiles of 16) and the softmax, and in P V wavefront w
    // takes output columns 16 (w % 4) .. + 16 of the pass over the tokens 64 (w / 4) .. + 64,
    // the two token halves added through the score buffer (free in value passes). The query
    // heads are the 16-wide N side (columns G .. 15 unused).
    auto attend_pass = [&](f32x4(&acc)[2][2], int c, int h) {
        const bool isK = (c & 1) == 0;
        const int u = u0 + (c >> 1);
        const int hh = D == 128 ? 0 : h;  // KV head of the unit in this pass
        const int head = Ly::kNH * u + hh;
        // head dimension of local column block lt (16 columns of the pass)
        auto dim0 = [&](int lt) { return D == 128 ? 16 * chunk_tile<D>(h, lt) : 16 * lt; };
        const unsigned char* qrow = sQ + (hh * G) * Ly::kQP * 2;
        unsigned char* prow = sP + (hh * G) * Ly::kPP * 2;
        const bool gv = mrow < G;
        if (isK) {
            // keys, rounded to bf16 as the restore writes them, to LDS [token][column]
#pragma unroll
            for (int gr = 0; gr < 2; ++gr) {
                unsigned char* row = sKV + (32 * tg + 16 * gr + mrow) * Ly::kKP * 2;
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int lt = pass_tile<2>(ch, i);
                    const f32x2 lo = {acc[gr][i][0], acc[gr][i][1]}, hi = {acc[gr][i][2], acc[gr][i][3]};
                    const bf16x2 x = __builtin_convertvector(lo, bf16x2), y = __builtin_convertvector(hi, bf16x2);
                    *reinterpret_cast<uint2*>(row + 2 * (16 * lt + 4 * g4)) =
                        make_uint2(*reinterpret_cast<const uint32_t*>(&x), *reinterpret_cast<const uint32_t*>(&y));
                }
            }
            lds_barrier();
            const bool first = D == 128 && h == 0;  // the head's first of two key passes
            const bool last = D == 64 || h == 1;    // the head's key columns all in
            // lane: query head mrow, tokens 32 tg + 16 tl + 4 g4 + r
            float* srow = sS + mrow * dt::TT + 32 * tg + 4 * g4;
            f32x4 st[2] = {zero4(), zero4()};
            if (ch == 0) {
                // scores S[t][g] = K[t] . q_g over the pass's 64 columns: 2 K-steps x 2 token tiles
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const int lc = 32 * ks + 8 * g4;  // the lane's 8 columns of the K-step
                    const bf16x8 qb = lds_load<bf16x8>(qrow + mrow * Ly::kQP * 2 + 2 * (dim0(lc >> 4) + (lc & 15)));
#pragma unroll
                    for (int tl = 0; tl < 2; ++tl) {
                        const bf16x8 kb =
                            lds_load<bf16x8>(sKV + (32 * tg + 16 * tl + mrow) * Ly::kKP * 2 + 2 * lc);
                        st[tl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qb, st[tl], 0, 0, 0);
                    }
                }
                if (first && gv) {
#pragma unroll
                    for (int tl = 0; tl < 2; ++tl) *reinterpret_cast<f32x4*>(srow + 16 * tl) = st[tl];
                }
            }
            if (last) {
                // the tile's softmax per query head
                if (ch == 0) {
                    if (D == 128 && gv) {
#pragma unroll
                        for (int tl = 0; tl < 2; ++tl) st[tl] += *reinterpret_cast<const f32x4*>(srow + 16 * tl);
                    }
                    float mxl = -INFINITY;
#pragma unroll
                    for (int tl = 0; tl < 2; ++tl)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const bool ok = gv && tt0 + 32 * tg + 16 * tl + 4 * g4 + r < m;
                            st[tl][r] = ok ? st[tl][r] * qscale : -INFINITY;
                            mxl = fmaxf(mxl, st[tl][r]);
                        }
                    mxl = fmaxf(mxl, __shfl_xor(mxl, 16, 64));
                    mxl = fmaxf(mxl, __shfl_xor(mxl, 32, 64));
                    if (g4 == 0 && gv) sMax[tg * 8 + mrow] = mxl;
                }
                lds_barrier();
                float mx = 0.f;
                if (ch == 0) {
                    mx = gv ? fmaxf(fmaxf(sMax[mrow], sMax[8 + mrow]), fmaxf(sMax[16 + mrow], sMax[24 + mrow])) : 0.f;
                    float sum = 0.f;
                    f16_t pw[2][4];
#pragma unroll
                    for (int tl = 0; tl < 2; ++tl)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float p = st[tl][r] == -INFINITY ? 0.f : expf(st[tl][r] - mx);
                            sum += p;
                            pw[tl][r] = (f16_t)p;
                        }
                    if (gv) {
#pragma unroll
                        for (int tl = 0; tl < 2; ++tl) {
                            const f16x2 a = {pw[tl][0], pw[tl][1]}, bq = {pw[tl][2], pw[tl][3]};
                            *reinterpret_cast<uint2*>(prow + mrow * Ly::kPP * 2 + 2 * (32 * tg + 16 * tl + 4 * g4)) =
                                make_uint2(*reinterpret_cast<const uint32_t*>(&a),
                                           *reinterpret_cast<const uint32_t*>(&bq));
                        }
                    }
                    sum += __shfl_xor(sum, 16, 64);
                    sum += __shfl_xor(sum, 32, 64);
                    if (g4 == 0 && gv) sSum[tg * 8 + mrow] = sum;
                }
                lds_barrier();
                if (wv == 0 && g4 == 0 && gv) {
                    float* ml = part_ml + ((((size_t)b * N + head) * ntiles + tile) * kAttendMaxG + mrow) * 2;
                    ml[0] = mx;
                    ml[1] = (sSum[mrow] + sSum[8 + mrow]) + (sSum[16 + mrow] + sSum[24 + mrow]);
                }
            }
            // the queries of the next unit once this one's last key pass is done (the next
            // score pass is a whole pass of barriers away)
            if (last && (c >> 1) + 1 < tm.nchunks) stage_q(u + 1);
        } else {
            // values to LDS transposed, [column][token] f16 (bf16 first, as the restore writes
            // them; bf16 -> f16 is exact in the normal range)
            f16_t* vt = reinterpret_cast<f16_t*>(sKV);
#pragma unroll
            for (int gr = 0; gr < 2; ++gr) {
                const int tk = 32 * tg + 16 * gr + mrow;
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int lt = pass_tile<2>(ch, i);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        vt[(16 * lt + 4 * g4 + e) * Ly::kVP + tk] = (f16_t)(float)(bf16_t)acc[gr][i][e];
                }
            }
            lds_barrier();
            // out^T[column][g] = sum_t V[t][column] P[g][t] over this wavefront's 2 K-steps of
            // 32 tokens; lane: query head mrow, columns 16 tg + 4 g4 + r of the pass
            f32x4 o = zero4();
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                const int ks = 2 * ch + k2;
                const f16x8 va = lds_load<f16x8>(sKV + ((16 * tg + mrow) * Ly::kVP + 32 * ks + 8 * g4) * 2);
                const f16x8 pb = lds_load<f16x8>(prow + (mrow * Ly::kPP + 32 * ks + 8 * g4) * 2);
                o = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb, o, 0, 0, 0);
            }
            f32x4* red = reinterpret_cast<f32x4*>(sS) + tg * 64 + lane;
            if (ch == 1) *red = o;
            lds_barrier();
            if (ch == 0 && gv) {
                o += *red;
                const int d = dim0(tg) + 4 * g4;
                float* po = part_o + ((((size_t)b * N + head) * ntiles + tile) * kAttendMaxG + mrow) * D + d;
                *reinterpret_cast<f32x4*>(po) = o;
            }
        }
    };

    Frag f0[2], f1[2];
    read_frags(f0, 0, 0);
    int slot = 0;
    f32x4 acc[2][2];
    for (int c = 0; c < nchunks; ++c) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const bool first = c == 0 && h == 0;
            // this pass's slices: the first pass's came with the set-up; a later pass's were
            // waited for in the previous pass's last stage, whose barrier made them visible
            if (first) {
                wait_vmcnt<0>();
                lds_barrier();
            }
            if (mf.fused) pass_mean<true, 2>(acc, sRef + h * dt::kRefBuf, mf, ch, tg);
            else pass_mean<false, 2>(acc, sRef + h * dt::kRefBuf, mf, ch, tg);
#pragma unroll
            for (int k = 0; k < KST; ++k) {
                read_frags(f1, slot, 1);
                mma(acc, f0, 2 * k);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
                __builtin_amdgcn_sched_barrier(0);
                // counts as in decode_tiles_dl_kernel without its warm-up
                if (k == KST - 1) wait_vmcnt<(KST - 2 < NST - 2 ? KST - 2 : NST - 2)>();
                else if (first && k == 0) wait_vmcnt<NST - 2 + 4>();
                else if (first && k <= NST - 2) wait_vmcnt<NST - 2 + 8>();
                else if (k >= 1 && k <= NST - 1) wait_vmcnt<NST - 2 + 4>();
                else wait_vmcnt<NST - 2>();
                lds_barrier();
                const int next = slot + 1 == NST ? 0 : slot + 1;
                read_frags(f0, next, 0);
                mma(acc, f1, 2 * k + 1);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
                __builtin_amdgcn_sched_barrier(0);
                wait_lgkm0();
                {
                    int c2, h2;
                    const int k2 = ahead(c, h, k, NST, c2, h2);
                    issue_w(c2, h2, k2, slot);
                }
                if (k == 0) issue_refs(h == 0 ? c : min(c + 1, nchunks - 1), 1 - h, sRef + (1 - h) * dt::kRefBuf);
                __builtin_amdgcn_sched_barrier(0);
                slot = next;
            }
            const bool isK = (c & 1) == 0;
            if (isK) pass_rope<D, 2>(acc, sRot, posf, h, ch);
            attend_pass(acc, c, h);
            // the staged values are read: the next pass may refill them
            lds_barrier();
        }
    }
}

// rkv_prepare_decoder: W_d bf16 -> fp16 in the restore's latent order: octet 4 ks + g of a
// row (K-step ks, lane group g) holds the row's latent octet NKS g + ks (coordinates d_c / 4
// g + 8 ks .. + 8), its 8 values in the fragment order 0 4 1 5 2 6 3 7 (the conversion form
// 1 applies in LDS, so both forms multiply the same operands in the same order).
__global__ void prepare_decoder_kernel(const uint4* __restrict__ wd, uint4* __restrict__ w16, size_t n8, int nks) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n8) {
        const size_t per_row = 4 * (size_t)nks;  // octets per row (d_c / 8)
        const size_t row = i / per_row;
        const int o = (int)(i - row * per_row);
        const f16x8 h = w_to_f16(wd[row * per_row + (size_t)nks * (o & 3) + (o >> 2)]);
        w16[i] = *reinterpret_cast<const uint4*>(&h);
    }
}

}  // namespace

// Workgroup grid, one workgroup per CU at a time. A run of chunks costs its length plus about
// half a chunk of set-up (token table, latents, RoPE table). Either every tile is cut into runs
// of one length (the length whose rounds of workgroups cost least), or the tiles that fill whole
// rounds of CUs take all chunks in one run and the remaining tiles are cut finer, whichever
// costs less.
static TileMapArgs tiles_grid(const Shape& s, int B, int m, unsigned* nblocks) {
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0)
        ncu = 256;
    const int chunks = s.W2 / dt::kCols;
    const int tpb = (m + dt::TT - 1) / dt::TT;
    const long tiles = (long)tpb * B;
    auto rounds_cost = [&](long ntiles, int ncg) {
        const long groups = (chunks + ncg - 1) / ncg;
        return (double)((ntiles * groups + ncu - 1) / ncu) * (ncg + 0.5);
    };
    TileMapArgs a{(int)tiles, chunks, 0, chunks, tpb};
    double best = 1e30;
    for (int ncg = chunks; ncg >= 1; --ncg) {
        const double c = rounds_cost(tiles, ncg);
        if (c < best - 1e-9) {
            best = c;
            a.ncg1 = ncg;
        }
    }
    const long T1 = tiles / ncu * ncu, R = tiles - T1;
    if (T1 > 0 && R > 0) {
        const double c1 = (double)(T1 / ncu) * (chunks + 0.5);
        for (int ncg = chunks; ncg >= 1; --ncg) {
            const double c = c1 + rounds_cost(R, ncg);
            if (c < best - 1e-9) {
                best = c;
                a = TileMapArgs{(int)T1, chunks, (int)R, ncg, tpb};
            }
        }
    }
    const long g1 = (chunks + a.ncg1 - 1) / a.ncg1, g2 = (chunks + a.ncg2 - 1) / a.ncg2;
    *nblocks = (unsigned)(a.T1 * g1 + a.R * g2);
    return a;
}

template <int NKS, int D, int BITS>
static hipError_t restore_attend_impl(int G, const Shape& s, const CacheView& c, const int* idx, int m,
                                      const void* wd16, const void* q, float qscale, float* part_o, float* part_ml,
                                      hipStream_t st) {
    // the tile map over units (K chunk + V chunk of 128 columns): a run of units costs two
    // chunks per unit
    Shape su = s;
    su.W2 = s.dk;  // units as the map's chunks
    unsigned nblocks = 0;
    const TileMapArgs ta = tiles_grid(su, c.B, m, &nblocks);
    typedef fa::L<D> Ly;
    auto kern = restore_attend_kernel<NKS, D, BITS>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, Ly::bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(nblocks), dim3(w8::kThreads), Ly::bytes, st, idx, m, ta,
                       static_cast<const fp8_t*>(c.ref_vals), c.self_slot, c.ref_idx, c.codes, c.code_bytes,
                       static_cast<const f16_t*>(c.scale), static_cast<const f16_t*>(c.zmin),
                       static_cast<const f16_t*>(wd16), s.W2, s.dk, s.top_k, c.cap_ref, c.cap_tok, s.theta,
                       static_cast<const bf16_t*>(q), G, qscale, part_o, part_ml, c.err);
    return hipGetLastError();
}

template <int D, int BITS>
static hipError_t restore_attend_dc(int G, const Shape& s, const CacheView& c, const int* idx, int m,
                                    const void* wd16, const void* q, float qscale, float* part_o, float* part_ml,
                                    hipStream_t st) {
    switch (s.d_c / 32) {
        case 4: return restore_attend_impl<4, D, BITS>(G, s, c, idx, m, wd16, q, qscale, part_o, part_ml, st);
        case 8: return restore_attend_impl<8, D, BITS>(G, s, c, idx, m, wd16, q, qscale, part_o, part_ml, st);
        case 12: return restore_attend_impl<12, D, BITS>(G, s, c, idx, m, wd16, q, qscale, part_o, part_ml, st);
        case 16: return restore_attend_impl<16, D, BITS>(G, s, c, idx, m, wd16, q, qscale, part_o, part_ml, st);
        default: return hipErrorInvalidValue;
    }
}

template <int NKS, int D, int BITS, typename OutT>
static hipError_t tiles_impl(const Shape& s, const CacheView& c, const int* idx, int m, const void* wd,
                             const void* wd16, void* out, hipStream_t st) {
    unsigned nblocks = 0;
    const TileMapArgs ta = tiles_grid(s, c.B, m, &nblocks);
    const dim3 grid(nblocks);
    if (wd16) {
        auto kern = decode_tiles_dl_kernel<NKS, D, BITS, OutT>;
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, dl::bytes);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, grid, dim3(w8::kThreads), dl::bytes, st, idx, m, ta,
                           static_cast<const fp8_t*>(c.ref_vals), c.self_slot, c.ref_idx, c.codes, c.code_bytes,
                           static_cast<const f16_t*>(c.scale), static_cast<const f16_t*>(c.zmin),
                           static_cast<const f16_t*>(wd16), s.W2, s.dk, s.top_k, c.cap_ref, c.cap_tok, s.theta,
                           static_cast<OutT*>(out), c.err);
    } else {
        auto kern = decode_tiles_kernel<NKS, D, BITS, OutT>;
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, rr::bytes);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, grid, dim3(dt::kThreads), rr::bytes, st, idx, m, ta,
                           static_cast<const fp8_t*>(c.ref_vals), c.self_slot, c.ref_idx, c.codes, c.code_bytes,
                           static_cast<const f16_t*>(c.scale), static_cast<const f16_t*>(c.zmin),
                           static_cast<const bf16_t*>(wd), s.W2, s.dk, s.top_k, c.cap_ref, c.cap_tok, s.theta,
                           static_cast<OutT*>(out), c.err);
    }
    return hipGetLastError();
}

template <int D, int BITS, typename OutT>
static hipError_t tiles_dc(const Shape& s, const CacheView& c, const int* idx, int m, const void* wd,
                           const void* wd16, void* out, hipStream_t st) {
    switch (s.d_c / 32) {
        case 4: return tiles_impl<4, D, BITS, OutT>(s, c, idx, m, wd, wd16, out, st);
        case 8: return tiles_impl<8, D, BITS, OutT>(s, c, idx, m, wd, wd16, out, st);
        case 12: return tiles_impl<12, D, BITS, OutT>(s, c, idx, m, wd, wd16, out, st);
        case 16: return tiles_impl<16, D, BITS, OutT>(s, c, idx, m, wd, wd16, out, st);
        default: return hipErrorInvalidValue;
    }
}

template <typename OutT>
static hipError_t tiles_d(const Shape& s, const CacheView& c, const int* idx, int m, const void* wd,
                          const void* wd16, void* out, hipStream_t st) {
    if (s.D == 64) {
        if (s.bits == 4) return tiles_dc<64, 4, OutT>(s, c, idx, m, wd, wd16, out, st);
        if (s.bits == 16) return tiles_dc<64, 16, OutT>(s, c, idx, m, wd, wd16, out, st);
        return tiles_dc<64, 2, OutT>(s, c, idx, m, wd, wd16, out, st);
    }
    if (s.bits == 4) return tiles_dc<128, 4, OutT>(s, c, idx, m, wd, wd16, out, st);
    if (s.bits == 16) return tiles_dc<128, 16, OutT>(s, c, idx, m, wd, wd16, out, st);
    return tiles_dc<128, 2, OutT>(s, c, idx, m, wd, wd16, out, st);
}

bool decode_tiles_supported(const Shape& s) {
    return !s.f32 && (s.bits == 4 || s.bits == 2 || s.bits == 16) && s.group == 32 && (s.D == 64 || s.D == 128) &&
           s.dk % dt::kCols == 0 && s.W2 % dt::kCols == 0 && s.d_c % 128 == 0 && s.d_c <= 512 &&
           s.top_k <= dt::kRefs;
}

hipError_t launch_decode_tiles(const Shape& s, const CacheView& c, const int* idx, int m, const void* wd,
                               const void* wd16, void* out, int out_dtype, hipStream_t st) {
    if (m <= 0) return hipSuccess;
    if (out_dtype == RKV_F32) return tiles_d<float>(s, c, idx, m, wd, wd16, out, st);
    return tiles_d<bf16_t>(s, c, idx, m, wd, wd16, out, st);
}

hipError_t launch_restore_attend(const Shape& s, const CacheView& c, const int* idx, int m, const void* wd16,
                                 const void* q, int Hq, float qscale, float* part_o, float* part_ml, hipStream_t st) {
    if (m <= 0) return hipSuccess;
    const int G = Hq / s.N;
    if (s.D == 64) {
        if (s.bits == 4) return restore_attend_dc<64, 4>(G, s, c, idx, m, wd16, q, qscale, part_o, part_ml, st);
        if (s.bits == 16) return restore_attend_dc<64, 16>(G, s, c, idx, m, wd16, q, qscale, part_o, part_ml, st);
        return restore_attend_dc<64, 2>(G, s, c, idx, m, wd16, q, qscale, part_o, part_ml, st);
    }
    if (s.bits == 4) return restore_attend_dc<128, 4>(G, s, c, idx, m, wd16, q, qscale, part_o, part_ml, st);
    if (s.bits == 16) return restore_attend_dc<128, 16>(G, s, c, idx, m, wd16, q, qscale, part_o, part_ml, st);
    return restore_attend_dc<128, 2>(G, s, c, idx, m, wd16, q, qscale, part_o, part_ml, st);
}

int restore_attend_tiles(int m) { return (m + dt::TT - 1) / dt::TT; }

hipError_t launch_prepare_decoder(const Shape& s, const void* wd, void* wd16, hipStream_t st) {
    const size_t n8 = (size_t)s.W2 * s.d_c / 8;
    if (n8 == 0) return hipSuccess;
    const unsigned threads = 256;
    const size_t blocks = (n8 + threads - 1) / threads;
    hipLaunchKernelGGL(prepare_decoder_kernel, dim3((unsigned)blocks), dim3(threads), 0, st,
                       static_cast<const uint4*>(wd), static_cast<uint4*>(wd16), n8, s.d_c / 32);
    return hipGetLastError();
}

}  // namespace rkv
