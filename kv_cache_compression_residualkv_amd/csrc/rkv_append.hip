// Reference append: store tokens directly into the reference pool.
//
// ResidualKV review page, section 2.7 step 4 (a new token goes straight into the
// reference store when the schedule says so) and section 2.4 (references are kept
// in FP8). The squared norm of the stored row is kept beside it for the
// distance search, which scores ||r||^2 - 2 x.r.
#include "rkv_device.h"
#include "rkv_internal.h"

namespace rkv {

namespace {

constexpr int kAppendThreads = 256;

template <typename KvT, typename RefT>
struct StoreRef;

template <>
struct StoreRef<bf16_t, fp8_t> {
    // 8 bf16 -> 8 fp8 codes; returns the sum of squares of the stored values
    static __device__ inline float run(const bf16_t* src, fp8_t* dst) {
        float v[8];
        Load8<bf16_t>::run(src, v);
        uint32_t lo = 0, hi = 0;
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t code = f32_to_fp8(v[i]);
            const float r = fp8_to_f32(code);
            ss = fmaf(r, r, ss);
            if (i < 4) lo |= code << (8 * i);
            else hi |= code << (8 * (i - 4));
        }
        *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
        return ss;
    }
};

template <>
struct StoreRef<float, float> {
    static __device__ inline float run(const float* src, float* dst) {
        const float4 a = *reinterpret_cast<const float4*>(src);
        const float4 b = *reinterpret_cast<const float4*>(src + 4);
        *reinterpret_cast<float4*>(dst) = a;
        *reinterpret_cast<float4*>(dst + 4) = b;
        return a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w + b.x * b.x + b.y * b.y + b.z * b.z + b.w * b.w;
    }
};

template <typename KvT, typename RefT>
__global__ __launch_bounds__(kAppendThreads) void append_ref_kernel(
    const KvT* __restrict__ kv, int kv_len, const int* __restrict__ rows, const int* __restrict__ pos, int n,
    RefT* __restrict__ ref_vals, int* __restrict__ ref_pos, float* __restrict__ ref_norm2,
    const int* __restrict__ ref_count, int* __restrict__ self_slot, int* err, int W2, int cap_ref, int cap_tok) {
    const int r = blockIdx.x;
    const int b = blockIdx.y;
    const int row = rows[(size_t)b * n + r];
    const int p = pos[(size_t)b * n + r];
    const int slot = ref_count[b] + r;
    const bool bad_row = row < 0 || row >= kv_len;
    const bool bad_pos = p < 0 || p >= cap_tok;
    const bool full = slot < 0 || slot >= cap_ref;
    if (bad_row || bad_pos || full) {
        if (threadIdx.x == 0)
            flag_error(err, (bad_row ? DEVERR_ROW_RANGE : 0) | (bad_pos ? DEVERR_POS_RANGE : 0) |
                                (full ? DEVERR_REF_CAPACITY : 0));
        return;
    }
    const KvT* src = kv + ((size_t)b * kv_len + row) * W2;
    RefT* dst = ref_vals + ((size_t)b * cap_ref + slot) * W2;
    float ss = 0.f;
    for (int c = threadIdx.x * 8; c < W2; c += kAppendThreads * 8) ss += StoreRef<KvT, RefT>::run(src + c, dst + c);
    // block reduction in a fixed order
    __shared__ float part[kAppendThreads / 64];
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = 0.f;
        for (int w = 0; w < kAppendThreads / 64; ++w) t += part[w];
        ref_norm2[(size_t)b * cap_ref + slot] = t;
        ref_pos[(size_t)b * cap_ref + slot] = p;
        self_slot[(size_t)b * cap_tok + p] = slot;
    }
}

__global__ void bump_count_kernel(int* ref_count, int B, int n, int cap_ref) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b < B) ref_count[b] = min(cap_ref, ref_count[b] + n);
}

}  // namespace

hipError_t launch_append(const Shape& s, const CacheView& c, const void* kv, int kv_len, const int* rows,
                         const int* pos, int n, hipStream_t st) {
    const dim3 grid(n, c.B);
    if (s.f32) {
        hipLaunchKernelGGL((append_ref_kernel<float, float>), grid, dim3(kAppendThreads), 0, st,
                           static_cast<const float*>(kv), kv_len, rows, pos, n, static_cast<float*>(c.ref_vals),
                           c.ref_pos, c.ref_norm2, c.ref_count, c.self_slot, c.err, s.W2, c.cap_ref, c.cap_tok);
    } else {
        hipLaunchKernelGGL((append_ref_kernel<bf16_t, fp8_t>), grid, dim3(kAppendThreads), 0, st,
                           static_cast<const bf16_t*>(kv), kv_len, rows, pos, n, static_cast<fp8_t*>(c.ref_vals),
                           c.ref_pos, c.ref_norm2, c.ref_count, c.self_slot, c.err, s.W2, c.cap_ref, c.cap_tok);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bump_count_kernel, dim3((c.B + 63) / 64), dim3(64), 0, st, c.ref_count, c.B, n, c.cap_ref);
    return hipGetLastError();
}

}  // namespace rkv
