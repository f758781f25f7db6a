// Multi-stage MFMA mainloop fed by direct global -> LDS loads (gfx950).
//
// A workgroup of NW wavefronts computes a BM x BN tile of A[BM x K] * B[BN x K]^T;
// both operands are K-contiguous rows read in stages of 64 K values.
//
// LDS layout of one operand stage. Rows are grouped by 16 and K by 32 (64 bytes of
// a 16-bit row): each (row group, K step) is one 1 KB block holding its 16 rows at a
// 64-byte pitch; inside a row, the 16-byte chunk c sits at position c ^ h(r), where
// h depends on the row's quad q = r / 4 only: h = 0, 2, 3, 1 for q = 0 .. 3. One direct
// load of a wavefront (global_load_lds_dwordx4) writes 64 x 16 bytes contiguously, lane
// l at 16 l, so lane l fetches row l / 4, chunk (l % 4) ^ h(l / 4): four consecutive
// lanes read one contiguous 64-byte row segment (the address unit merges them).
//
// Bank conflicts. The LDS has 64 four-byte banks, and a 16-byte read (ds_read_b128) is
// served in four passes of 16 lanes: {0-3, 12-15, 20-23, 24-27}, {4-11, 16-19, 28-31}
// and the same two sets plus 32 (measured with the SQ_LDS_BANK_CONFLICT counter on
// one-dispatch-per-lane-pair patterns). A pass is conflict-free when its 16 lanes hit
// 16 distinct 16-byte bank slots, slot = 4 (r % 4) + position within a block. For the
// v_mfma_f32_16x16x32 fragment (lane l: row l % 16, chunk l / 16, one block) that asks,
// for each r % 4, that h(q0), h(q3), h(q1)^1, h(q2)^1 differ and h(q1), h(q2), h(q0)^1,
// h(q3)^1 differ; for the fragments of the search kernel (lanes 16-31 in the next
// block, one chunk per half wavefront) that h is a permutation over the quads. The
// table above meets both. (A swizzle made for 16 consecutive lanes per pass costs four
// extra cycles on every fragment read here.)
//
// Pipeline (ring_mainloop_lrp): NST stage slots form a ring. In the middle of stage s
// every wavefront waits (s_waitcnt vmcnt) until its own loads of stage s + 1 have
// landed, a barrier makes them visible to all, and stage s + NST is issued into the
// slot stage s used, whose fragments are all in registers by then. Only the raw
// s_barrier is used: a workgroup fence would make the compiler wait for every
// outstanding load, which is exactly what the ring is meant to avoid.
#pragma once

#include "rkv_device.h"

namespace rkv {

#define RKV_LDS __attribute__((address_space(3)))

constexpr int kStageK = 64;

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ inline void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ inline void dma16(const void* g, void* lds_block) {
    __builtin_amdgcn_global_load_lds(g, (RKV_LDS void*)lds_block, 16, 0, 0);
}

// wavefront index as a scalar (the compiler cannot prove threadIdx.x / 64 uniform)
__device__ inline int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// position of chunk c of row r (within its group of 16) inside the row's 64 bytes
__device__ inline int swz(int r, int c) { return c ^ (((r >> 3) & 1) | ((((r >> 2) ^ (r >> 3)) & 1) << 1)); }

// A 16-bit operand of R rows (R a multiple of 8 NW) loaded by NW wavefronts. Each
// wavefront issues R / (8 NW) of the stage's R / 8 block loads: load u of wave w fills
// block (w + NW u) = 2 g + h (row group g, K step h).
template <int R, int NW = 4>
struct Op16 {
    static constexpr int kLoads = R / (8 * NW);
    static constexpr int kStageBytes = R * kStageK * 2;
    static_assert(kLoads * 8 * NW == R, "rows per wavefront");
    const char* src[kLoads];  // per lane: its row's chunk in stage 0
    // row(r) gives the byte address of row r (any row inside the matrix; rows past
    // the valid range must still point at readable memory)
    template <class RowFn>
    __device__ inline void init(RowFn&& row) {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
        for (int u = 0; u < kLoads; ++u) {
            const int blk = wave + NW * u;
            const int g = blk >> 1, h = blk & 1;
            src[u] = reinterpret_cast<const char*>(row(16 * g + (lane >> 2))) + 64 * h + 16 * swz(lane >> 2, lane & 3);
        }
    }
    __device__ inline void issue(int s, char* slot) const {
        const int wave = wave_id();
#pragma unroll
        for (int u = 0; u < kLoads; ++u) dma16(src[u] + (size_t)s * (kStageK * 2), slot + 1024 * (wave + NW * u));
    }
    // fragment of row group g, K step ks
    template <typename T>
    static __device__ inline typename Mma<T>::frag frag(const char* slot, int g, int ks) {
        const int lane = threadIdx.x & 63, r = lane & 15;
        return *reinterpret_cast<const typename Mma<T>::frag*>(slot + 2048 * g + 1024 * ks + 64 * r +
                                                               16 * swz(r, lane >> 4));
    }
};

// Wait until this wavefront's loads of the current stage are done, given that
// `ahead` later stages (each `per_stage` loads) may still be in flight.
template <int NST, int PER_STAGE>
__device__ inline void wait_stage(int ahead) {
    if constexpr (NST >= 4) {
        if (ahead >= 3 && 3 * PER_STAGE < 64) {
            wait_vmcnt<(3 * PER_STAGE < 64 ? 3 * PER_STAGE : 0)>();
            return;
        }
        if (ahead >= 2) {
            wait_vmcnt<2 * PER_STAGE>();
            return;
        }
    }
    if constexpr (NST >= 3) {
        if (ahead >= 1) {
            wait_vmcnt<PER_STAGE>();
            return;
        }
    }
    wait_vmcnt<0>();
}

// s_waitcnt lgkmcnt(0) alone
__device__ inline void wait_lgkm0() { __builtin_amdgcn_s_waitcnt((0xF) | (0x3 << 14) | (0x7 << 4)); }

// Scheduling hint for one half stage: R fragment reads spread over M MFMAs, two MFMAs
// then one read, R times, the remaining MFMAs after. With the reads clustered ahead of
// the MFMAs (the scheduler's own choice) the matrix pipe idles while they issue.
template <int R, int M>
__device__ inline void interleave_reads() {
    static_assert(2 * R <= M, "two MFMAs per read");
#pragma unroll
    for (int i = 0; i < R; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, M - 2 * R, 0);
    __builtin_amdgcn_sched_barrier(0);
}

// Ring mainloop with the LDS fragment reads of one K step overlapped with the MFMAs
// of the other. Per stage s (K steps 0 and 1, fragments f0 and f1):
//   read f1(s) | MFMA f0(s) | wait, barrier | issue stage s + NST | read f0(s + 1) | MFMA f1(s)
// The barrier sits between the two halves: before it, every wavefront has its f1(s)
// fragments in registers (lgkmcnt 0) and its loads of stage s + 1 landed, so the slot
// of stage s can be refilled right after it. Compiler-only fences keep the LDS reads
// on their side of the barrier.
//   load(F&, const char* slot_a, const char* slot_b, int ks)  reads one K step
//   mma(const F&, Acc&)                                       multiplies it
// IL_R / IL_M (when nonzero): fragment reads and MFMAs of one K step, interleaved by
// interleave_reads.
template <int NST, class F, int IL_R = 0, int IL_M = 0, class LA, class LB, class Ld, class Mm, class Acc,
          class OnBlock>
__device__ inline void ring_mainloop_lrp(const LA& a, const LB& b, int n_stages, int stages_per_block, char* lds,
                                         Ld&& load, Mm&& mma, Acc& acc, OnBlock&& on_block) {
    static_assert(NST >= 2 && NST <= 4, "2 to 4 stages");
    constexpr int kSlot = LA::kStageBytes + LB::kStageBytes;
    constexpr int kPer = LA::kLoads + LB::kLoads;
    if (n_stages <= 0) return;
#pragma unroll
    for (int p = 0; p < NST; ++p) {
        if (p < n_stages) {
            a.issue(p, lds + p * kSlot);
            b.issue(p, lds + p * kSlot + LA::kStageBytes);
        }
    }
    wait_stage<NST + 1, kPer>(min(NST - 1, n_stages - 1));
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    F f0, f1;
    load(f0, lds, lds + LA::kStageBytes, 0);
    int kin = 0;
    int slot = 0;
    // every stage but the last: no data-dependent control flow between the two halves
    for (int s = 0; s + 1 < n_stages; ++s) {
        const char* sa = lds + slot * kSlot;
        load(f1, sa, sa + LA::kStageBytes, 1);
        mma(f0, acc);
        if constexpr (IL_R > 0) interleave_reads<IL_R, IL_M>();
        const int next = slot + 1 == NST ? 0 : slot + 1;
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        wait_lgkm0();
        wait_stage<NST, kPer>(min(NST - 2, n_stages - 2 - s));
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (s + NST < n_stages) {
            a.issue(s + NST, lds + slot * kSlot);
            b.issue(s + NST, lds + slot * kSlot + LA::kStageBytes);
        }
        const char* na = lds + next * kSlot;
        load(f0, na, na + LA::kStageBytes, 0);
        mma(f1, acc);
        if constexpr (IL_R > 0) interleave_reads<IL_R, IL_M>();
        slot = next;
        if (++kin == stages_per_block) {
            kin = 0;
            on_block(s / stages_per_block, acc, false);
        }
    }
    {
        const char* sa = lds + slot * kSlot;
        load(f1, sa, sa + LA::kStageBytes, 1);
        mma(f0, acc);
        mma(f1, acc);
        on_block((n_stages - 1) / stages_per_block, acc, true);
    }
}

// ring_mainloop_lrp with a ring per operand: A NA stages deep, B NA - 1. For a product
// whose A rows come from HBM once while every workgroup re-reads the same B (served by
// L2), the extra A stage keeps NA - 1 stages of A in flight against HBM latency within
// the same LDS. Per stage s (slots s mod NA for A, s mod NB for B):
//   read f1(s) | MFMA f0(s) | wait for stage s + 1, barrier |
//   issue B(s + NB), then A(s + NA) | read f0(s + 1) | MFMA f1(s)
// Loads are issued as A(0) B(0) .. A(NB-1) B(NB-1) A(NB), then B(s + NB) A(s + NA) in the
// middle of stage s, so when stage s + 1 is waited for only A(s + NA - 1) may still be in
// flight behind it.
template <int NA, int NB, class F, int IL_R, int IL_M, class LA, class LB, class Ld, class Mm, class Acc>
__device__ inline void ring_mainloop_split(const LA& a, const LB& b, int n_stages, char* lds_a, char* lds_b,
                                           Ld&& load, Mm&& mma, Acc& acc) {
    static_assert(NB >= 2 && NA == NB + 1, "A one stage deeper than B");
    constexpr int kA = LA::kStageBytes, kB = LB::kStageBytes;
    if (n_stages <= 0) return;
#pragma unroll
    for (int p = 0; p < NB; ++p) {
        if (p < n_stages) {
            a.issue(p, lds_a + p * kA);
            b.issue(p, lds_b + p * kB);
        }
    }
    if (NB < n_stages) a.issue(NB, lds_a + NB * kA);
    // stage 0 landed: behind it at most NB - 1 full stages and A(NB)
    if (n_stages > NB)
        wait_vmcnt<(NB - 1) * (LA::kLoads + LB::kLoads) + LA::kLoads>();
    else
        wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    F f0, f1;
    load(f0, lds_a, lds_b, 0);
    int ia = 0, ib = 0;
    for (int s = 0; s + 1 < n_stages; ++s) {
        const char* sa = lds_a + ia * kA;
        const char* sb = lds_b + ib * kB;
        load(f1, sa, sb, 1);
        mma(f0, acc);
        if constexpr (IL_R > 0) interleave_reads<IL_R, IL_M>();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        wait_lgkm0();
        if (s + NA - 1 < n_stages)
            wait_vmcnt<LA::kLoads>();
        else
            wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (s + NB < n_stages) b.issue(s + NB, lds_b + ib * kB);
        if (s + NA < n_stages) a.issue(s + NA, lds_a + ia * kA);
        ia = ia + 1 == NA ? 0 : ia + 1;
        ib = ib + 1 == NB ? 0 : ib + 1;
        load(f0, lds_a + ia * kA, lds_b + ib * kB, 0);
        mma(f1, acc);
        if constexpr (IL_R > 0) interleave_reads<IL_R, IL_M>();
    }
    {
        load(f1, lds_a + ia * kA, lds_b + ib * kB, 1);
        mma(f0, acc);
        mma(f1, acc);
    }
}

}  // namespace rkv
