// MFMA mainloop shared by the search and encoder kernels (gfx950).
//
// A workgroup of 256 threads (4 wavefronts) computes a BM x BN tile of
// A[BM x K] * B[BN x K]^T; both operands are K-contiguous rows. K is consumed in
// stages of kKC = 64 elements:
//   * each thread loads its share of the next-but-one stage from global memory
//     into registers while the current stage is multiplied out of LDS;
//   * LDS holds two stages (double buffer), so one barrier per stage suffices;
//   * a stage is converted to the compute type when it is written to LDS.
// Stages are numbered flatly; every `stages_per_block` stages the caller's
// `on_block` hook sees the finished accumulators (used by the search to fold one
// pool block into its running top-k before the next block starts).
//
// Wave layout: wave w owns A rows [a_row0, a_row0 + WM) and B rows
// [b_row0, b_row0 + WN) of the tile; its 16 x 16 MFMA tiles hold
// C[a row 16 i + 4 (lane / 16) + e][b row 16 j + lane % 16] in acc[i][j][e].
#pragma once

#include <type_traits>

#include "rkv_device.h"

namespace rkv {

constexpr int kGemmThreads = 256;
constexpr int kKC = 64;

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

// Write 32 staged elements to LDS in the compute type (a raw copy when the storage
// type is the compute type, a widening/narrowing conversion otherwise).
template <typename T, typename S>
__device__ inline void stage32(T* dst, const Raw32<S>& r) {
    if constexpr (std::is_same<T, S>::value) {
#pragma unroll
        for (int i = 0; i < Raw32<S>::kWords; ++i) reinterpret_cast<uint4*>(dst)[i] = r.w[i];
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float v[8];
            r.get8(j, v);
            lds_store8<T>(dst + 8 * j, v);
        }
    }
}

// FP8 -> bf16 is exact; v_cvt_scalef32_pk_bf16_fp8 (scale 1) widens two bytes per
// call and agrees with the OCP e4m3fn definition on all 256 codes.
template <>
__device__ inline void stage32<bf16_t, fp8_t>(bf16_t* dst, const Raw32<fp8_t>& r) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint4 v = r.w[h];
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
        uint32_t o[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w4[i], 1.0f, false);
            const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w4[i], 1.0f, true);
            o[2 * i] = *reinterpret_cast<const uint32_t*>(&lo);
            o[2 * i + 1] = *reinterpret_cast<const uint32_t*>(&hi);
        }
        reinterpret_cast<uint4*>(dst)[2 * h] = make_uint4(o[0], o[1], o[2], o[3]);
        reinterpret_cast<uint4*>(dst)[2 * h + 1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
}

// A tile operand of R rows (R a multiple of 128): thread t stages row (t >> 1) + 128 u,
// columns [(t & 1) * 32, +32) of the stage, for u < R / 128. The kernel fills row[u]
// (nullptr = zero row) before each load.
template <typename T, typename S, int R>
struct RowTile {
    static constexpr int kUnits = R / 128;
    Raw32<S> raw[kUnits];
    __device__ inline static int srow(int u) { return (threadIdx.x >> 1) + 128 * u; }
    __device__ inline static int scol() { return (threadIdx.x & 1) * 32; }
    __device__ inline void load_rows(const S* const (&row)[kUnits], int k0) {
#pragma unroll
        for (int u = 0; u < kUnits; ++u) {
            if (row[u]) raw[u].load(row[u] + k0 + scol());
            else raw[u].zero();
        }
    }
    __device__ inline void store(T* lds, int P) const {
#pragma unroll
        for (int u = 0; u < kUnits; ++u) stage32<T>(lds + srow(u) * P + scol(), raw[u]);
    }
};

// Double-buffered LDS mainloop (see the header comment). `lds` holds 2 * (BM + BN) * P
// elements of T. la.load(stage) / lb.load(stage) fetch a stage into registers,
// la.store(ptr) / lb.store(ptr) write it to LDS.
template <typename T, int BM, int BN, int WM, int WN, class LA, class LB, class OnBlock>
__device__ inline void mainloop(LA& la, LB& lb, int n_stages, int stages_per_block, T* lds, int a_row0, int b_row0,
                                f32x4 (&acc)[WM / 16][WN / 16], OnBlock&& on_block) {
    constexpr int P = Pitch<T, kKC>::value;
    T* const sA0 = lds;
    T* const sB0 = lds + BM * P;
    T* const sA1 = lds + (BM + BN) * P;
    T* const sB1 = sA1 + BM * P;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < WM / 16; ++i)
#pragma unroll
        for (int j = 0; j < WN / 16; ++j) acc[i][j] = zero4();
    if (n_stages <= 0) return;
    la.load(0);
    lb.load(0);
    la.store(sA0, P);
    lb.store(sB0, P);
    if (n_stages > 1) {
        la.load(1);
        lb.load(1);
    }
    __syncthreads();
    int kin = 0;
    for (int s = 0; s < n_stages; ++s) {
        const T* sA = (s & 1) ? sA1 : sA0;
        const T* sB = (s & 1) ? sB1 : sB0;
#pragma unroll
        for (int ks = 0; ks < kKC / 32; ++ks) {
            const int kof = ks * 32 + 8 * (lane >> 4);
            typename Mma<T>::frag fb[WN / 16];
#pragma unroll
            for (int j = 0; j < WN / 16; ++j) fb[j] = lds_frag<T>(sB + (b_row0 + 16 * j + (lane & 15)) * P + kof);
#pragma unroll
            for (int i = 0; i < WM / 16; ++i) {
                const typename Mma<T>::frag fa = lds_frag<T>(sA + (a_row0 + 16 * i + (lane & 15)) * P + kof);
#pragma unroll
                for (int j = 0; j < WN / 16; ++j) acc[i][j] = Mma<T>::step(acc[i][j], fa, fb[j]);
            }
        }
        if (s + 1 < n_stages) {
            la.store((s & 1) ? sA0 : sA1, P);
            lb.store((s & 1) ? sB0 : sB1, P);
        }
        if (s + 2 < n_stages) {
            la.load(s + 2);
            lb.load(s + 2);
        }
        if (++kin == stages_per_block) {
            kin = 0;
            on_block(s / stages_per_block, acc);
            if (s + 1 < n_stages) {  // the last block's accumulators stay for the caller
#pragma unroll
                for (int i = 0; i < WM / 16; ++i)
#pragma unroll
                    for (int j = 0; j < WN / 16; ++j) acc[i][j] = zero4();
            }
        }
        __syncthreads();
    }
}

struct NoBlockHook {
    template <class A>
    __device__ inline void operator()(int, A&) const {}
};

// The hardware deals workgroups round-robin over the 8 XCDs (each with its own
// L2). Launch 8 * per blocks; this returns the logical tile of a block so that
// each XCD works through a contiguous range of logical tiles, and tiles that
// share an operand (consecutive tiles) share that XCD's L2.
__device__ inline int xcd_tile(int bid, int per) { return (bid & 7) * per + (bid >> 3); }

inline int xcd_per(int ntiles) { return (ntiles + 7) / 8; }

}  // namespace rkv
