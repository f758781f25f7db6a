// C ABI of the codec: host-side validation, then asynchronous launches on the
// caller's stream. Nothing here allocates, frees or synchronises.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "rkv.h"
#include "rkv_internal.h"

using namespace rkv;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t dtype_size(int dt) {
    switch (dt) {
        case RKV_F32: return 4;
        case RKV_BF16: return 2;
        case RKV_F16: return 2;
        case RKV_FP8_E4M3: return 1;
        default: return 0;
    }
}

rkv_status check_config(const rkv_config* cfg, Shape* out) {
    if (!cfg) return RKV_ERR_INVALID_ARG;
    if (cfg->n_kv_heads <= 0 || cfg->head_dim <= 0 || cfg->d_ff <= 0 || cfg->d_c <= 0 || cfg->top_k <= 0 ||
        cfg->group <= 0 || !(cfg->rope_theta > 0.0) || (cfg->head_dim & 1))
        return RKV_ERR_INVALID_ARG;
    if (dtype_size(cfg->kv_dtype) == 0 || dtype_size(cfg->ref_dtype) == 0 || dtype_size(cfg->scale_dtype) == 0 ||
        dtype_size(cfg->weight_dtype) == 0)
        return RKV_ERR_INVALID_ARG;
    if (cfg->flags & ~RKV_FLAG_MEAN_PROJECTION) return RKV_ERR_INVALID_ARG;
    if (cfg->bits != 2 && cfg->bits != 4 && cfg->bits != 16) return RKV_ERR_UNSUPPORTED;
    const bool f32 = cfg->kv_dtype == RKV_F32 && cfg->ref_dtype == RKV_F32 && cfg->scale_dtype == RKV_F32 &&
                     cfg->weight_dtype == RKV_F32;
    const bool bf16 = cfg->kv_dtype == RKV_BF16 && cfg->ref_dtype == RKV_FP8_E4M3 && cfg->scale_dtype == RKV_F16 &&
                      cfg->weight_dtype == RKV_BF16;
    if (!f32 && !bf16) return RKV_ERR_UNSUPPORTED;
    const bool mproj = (cfg->flags & RKV_FLAG_MEAN_PROJECTION) != 0;
    if (mproj && f32) return RKV_ERR_UNSUPPORTED;
    const int D = cfg->head_dim;
    if (D != 64 && D != 128) return RKV_ERR_UNSUPPORTED;
    const long dk = (long)cfg->n_kv_heads * D;
    if (dk > (1 << 20)) return RKV_ERR_UNSUPPORTED;
    if (dk % 128 != 0) return RKV_ERR_UNSUPPORTED;
    if (cfg->d_ff % 64 != 0) return RKV_ERR_UNSUPPORTED;
    if (cfg->d_c != 64 && cfg->d_c != 128 && cfg->d_c != 256 && cfg->d_c != 384 && cfg->d_c != 512)
        return RKV_ERR_UNSUPPORTED;
    if (cfg->group != 32) return RKV_ERR_UNSUPPORTED;
    if (cfg->top_k > 8) return RKV_ERR_UNSUPPORTED;
    if (out) {
        out->N = cfg->n_kv_heads;
        out->D = D;
        out->dk = (int)dk;
        out->W2 = (int)(2 * dk);
        out->d_ff = cfg->d_ff;
        out->d_c = cfg->d_c;
        out->top_k = cfg->top_k;
        out->bits = cfg->bits;
        out->group = cfg->group;
        out->G = cfg->d_c / cfg->group;
        out->f32 = f32;
        out->mproj = mproj;
        out->theta = cfg->rope_theta;
    }
    return RKV_OK;
}

size_t code_bytes_of(const Shape& s) { return (size_t)s.d_c * s.bits / 8; }

rkv_status check_cache(const Shape& s, const rkv_cache* c, bool need_records, CacheView* v) {
    if (!c) return RKV_ERR_INVALID_ARG;
    if (c->batch <= 0 || c->cap_ref <= 0 || c->cap_tok <= 0) return RKV_ERR_INVALID_ARG;
    if (!c->ref_vals || !c->ref_pos || !c->ref_norm2 || !c->ref_count || !c->self_slot) return RKV_ERR_INVALID_ARG;
    if (need_records && (!c->codes || !c->ref_idx || (s.bits != 16 && (!c->scale || !c->zmin))))
        return RKV_ERR_INVALID_ARG;
    if (!aligned16(c->ref_vals) || (c->codes && !aligned16(c->codes))) return RKV_ERR_ALIGNMENT;
    if ((c->scale && !aligned16(c->scale)) || (c->zmin && !aligned16(c->zmin))) return RKV_ERR_ALIGNMENT;
    v->B = c->batch;
    v->cap_ref = c->cap_ref;
    v->cap_tok = c->cap_tok;
    v->ref_vals = c->ref_vals;
    v->ref_pos = c->ref_pos;
    v->ref_norm2 = c->ref_norm2;
    v->ref_count = c->ref_count;
    v->codes = c->codes;
    v->scale = c->scale;
    v->zmin = c->zmin;
    v->ref_idx = c->ref_idx;
    v->self_slot = c->self_slot;
    v->err = c->err_word;
    v->stats = c->stats;
    v->ref_proj = c->ref_proj;
    v->proj_count = c->proj_count;
    v->code_bytes = code_bytes_of(s);
    return RKV_OK;
}

rkv_status from_hip(hipError_t e) { return e == hipSuccess ? RKV_OK : RKV_ERR_HIP; }

}  // namespace

extern "C" {

int32_t rkv_abi_version(void) { return RKV_ABI_VERSION; }

const char* rkv_status_string(rkv_status s) {
    switch (s) {
        case RKV_OK: return "ok";
        case RKV_ERR_INVALID_ARG: return "invalid argument";
        case RKV_ERR_UNSUPPORTED: return "unsupported configuration";
        case RKV_ERR_CAPACITY: return "capacity exceeded";
        case RKV_ERR_ALIGNMENT: return "pointer not 16-byte aligned";
        case RKV_ERR_HIP: return "HIP runtime error";
        case RKV_ERR_WORKSPACE: return "workspace missing or too small";
        default: return "unknown status";
    }
}

rkv_status rkv_validate_config(const rkv_config* cfg) { return check_config(cfg, nullptr); }

rkv_status rkv_record_bytes(const rkv_config* cfg, size_t out[6]) {
    Shape s;
    const rkv_status st = check_config(cfg, &s);
    if (st != RKV_OK) return st;
    if (!out) return RKV_ERR_INVALID_ARG;
    const size_t sc = s.bits == 16 ? 0 : dtype_size(cfg->scale_dtype);
    out[0] = code_bytes_of(s);
    out[1] = (size_t)s.G * sc;
    out[2] = (size_t)s.G * sc;
    out[3] = (size_t)s.top_k * sizeof(int32_t);
    out[4] = sizeof(int32_t);
    out[5] = (size_t)s.W2 * dtype_size(cfg->ref_dtype);
    return RKV_OK;
}

size_t rkv_encode_workspace_bytes(const rkv_config* cfg, int32_t batch, int32_t n, int32_t cap_ref) {
    Shape s;
    if (check_config(cfg, &s) != RKV_OK || batch <= 0 || n < 0 || cap_ref <= 0) return 0;
    return plan_encode(s, batch, n, cap_ref).total;
}

rkv_status rkv_reference_schedule(int32_t limit, int32_t s0, int32_t n_sink, int32_t alpha_num, int32_t alpha_den,
                                  int32_t* out, int32_t cap, int32_t* count) {
    if (!count || limit < 0 || s0 < 1 || n_sink < 0 || alpha_num < 0 || alpha_den < 1 || cap < 0 ||
        (cap > 0 && !out))
        return RKV_ERR_INVALID_ARG;
    int64_t n = 0;
    auto put = [&](int64_t p) {
        if (n < cap) out[n] = (int32_t)p;
        ++n;
    };
    for (int64_t p = 0; p < n_sink && p < limit; ++p) put(p);  // sink tokens
    // gap s0 + floor(alpha (p - n_sink)) in integers: alpha_num (p - n_sink) < 2^62
    for (int64_t p = n_sink; p < limit; p += s0 + (int64_t)alpha_num * (p - n_sink) / alpha_den) put(p);
    *count = (int32_t)n;
    return n > cap ? RKV_ERR_CAPACITY : RKV_OK;
}

rkv_status rkv_append_ref(const rkv_config* cfg, rkv_cache* cache, const void* kv, int32_t kv_len,
                          const int32_t* rows, const int32_t* pos, int32_t n, void* stream) {
    Shape s;
    rkv_status st = check_config(cfg, &s);
    if (st != RKV_OK) return st;
    CacheView c;
    st = check_cache(s, cache, false, &c);
    if (st != RKV_OK) return st;
    if (n < 0 || kv_len < 0) return RKV_ERR_INVALID_ARG;
    if (n == 0) return RKV_OK;
    if (!kv || !rows || !pos) return RKV_ERR_INVALID_ARG;
    if (!aligned16(kv)) return RKV_ERR_ALIGNMENT;
    if (n > cache->cap_ref) return RKV_ERR_CAPACITY;
    return from_hip(launch_append(s, c, kv, kv_len, rows, pos, n, static_cast<hipStream_t>(stream)));
}

rkv_status rkv_encode_ex(const rkv_config* cfg, const rkv_weights* w, rkv_cache* cache, const void* kv,
                         int32_t kv_len, const int32_t* rows, const int32_t* pos, int32_t n, void* workspace,
                         size_t workspace_bytes, void* stream, void* const* events) {
    Shape s;
    rkv_status st = check_config(cfg, &s);
    if (st != RKV_OK) return st;
    CacheView c;
    st = check_cache(s, cache, true, &c);
    if (st != RKV_OK) return st;
    if (n < 0 || kv_len < 0) return RKV_ERR_INVALID_ARG;
    if (n == 0) return RKV_OK;
    if (kv_len == 0) return RKV_ERR_INVALID_ARG;  // every token reads a row of kv
    if (!w || !w->w_c1 || !w->w_c2 || !w->w_c3 || !kv || !rows || !pos) return RKV_ERR_INVALID_ARG;
    if (!aligned16(kv) || !aligned16(w->w_c1) || !aligned16(w->w_c2) || !aligned16(w->w_c3))
        return RKV_ERR_ALIGNMENT;
    if (n > cache->cap_tok) return RKV_ERR_CAPACITY;
    if (s.mproj && (!c.ref_proj || !c.proj_count)) return RKV_ERR_INVALID_ARG;
    if (s.mproj && !aligned16(c.ref_proj)) return RKV_ERR_ALIGNMENT;
    const EncodePlan p = plan_encode(s, c.B, n, c.cap_ref);
    if (!workspace || workspace_bytes < p.total) return RKV_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return RKV_ERR_ALIGNMENT;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    auto mark = [&](int i) -> hipError_t {
        return events && events[i] ? hipEventRecord(static_cast<hipEvent_t>(events[i]), hs) : hipSuccess;
    };
    hipError_t e = mark(0);
    if (e == hipSuccess) e = launch_search(s, c, p, kv, kv_len, rows, pos, n, workspace, hs);
    if (e == hipSuccess) e = mark(1);
    if (e == hipSuccess) e = launch_select(s, c, p, kv, kv_len, rows, pos, n, workspace, hs);
    if (e == hipSuccess) e = mark(2);
    if (e == hipSuccess && s.mproj) e = launch_project_refs(s, c, w->w_c1, w->w_c2, hs);
    if (e == hipSuccess) e = launch_swiglu(s, c, p, kv, kv_len, rows, pos, n, w->w_c1, w->w_c2, workspace, hs);
    if (e == hipSuccess) e = mark(3);
    if (e == hipSuccess) e = launch_latent_quant(s, c, p, pos, n, w->w_c3, workspace, hs);
    if (e == hipSuccess) e = mark(4);
    return from_hip(e);
}

rkv_status rkv_encode(const rkv_config* cfg, const rkv_weights* w, rkv_cache* cache, const void* kv,
                      int32_t kv_len, const int32_t* rows, const int32_t* pos, int32_t n, void* workspace,
                      size_t workspace_bytes, void* stream) {
    return rkv_encode_ex(cfg, w, cache, kv, kv_len, rows, pos, n, workspace, workspace_bytes, stream, nullptr);
}

rkv_status rkv_decode_selected(const rkv_config* cfg, const rkv_weights* w, const rkv_cache* cache,
                               const int32_t* idx, int32_t m, void* out, int32_t out_dtype, void* stream) {
    Shape s;
    rkv_status st = check_config(cfg, &s);
    if (st != RKV_OK) return st;
    CacheView c;
    st = check_cache(s, cache, true, &c);
    if (st != RKV_OK) return st;
    if (m < 0) return RKV_ERR_INVALID_ARG;
    if (out_dtype != RKV_F32 && out_dtype != RKV_BF16) return RKV_ERR_UNSUPPORTED;
    if (m == 0) return RKV_OK;
    if (!w || !w->w_d || !idx || !out) return RKV_ERR_INVALID_ARG;
    if (!aligned16(w->w_d) || !aligned16(out)) return RKV_ERR_ALIGNMENT;
    // the prepared fp16 decoder serves the "bf16" formats only
    const void* wd16 = s.f32 ? nullptr : w->w_d_f16;
    if (wd16 && !aligned16(wd16)) return RKV_ERR_ALIGNMENT;
    return from_hip(launch_decode(s, c, idx, m, w->w_d, wd16, out, out_dtype, static_cast<hipStream_t>(stream)));
}

size_t rkv_decode_attend_workspace_bytes(const rkv_config* cfg, int32_t batch, int32_t m, int32_t n_q_heads) {
    Shape s;
    if (check_config(cfg, &s) != RKV_OK || batch <= 0 || m < 0 || !attend_supported(s, n_q_heads)) return 0;
    return attend_workspace_bytes(s, batch, m);
}

rkv_status rkv_decode_attend(const rkv_config* cfg, const rkv_weights* w, const rkv_cache* cache,
                             const int32_t* idx, int32_t m, const void* q, int32_t n_q_heads, float scale,
                             float* out, void* workspace, size_t workspace_bytes, void* stream) {
    Shape s;
    rkv_status st = check_config(cfg, &s);
    if (st != RKV_OK) return st;
    CacheView c;
    st = check_cache(s, cache, true, &c);
    if (st != RKV_OK) return st;
    if (m < 0 || n_q_heads <= 0 || n_q_heads % s.N != 0 || !(scale > 0.f) || !q || !out) return RKV_ERR_INVALID_ARG;
    if (!attend_supported(s, n_q_heads)) return RKV_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(out)) return RKV_ERR_ALIGNMENT;
    if (m > 0) {
        if (!w || !w->w_d || !idx) return RKV_ERR_INVALID_ARG;
        if (!aligned16(w->w_d) || (w->w_d_f16 && !aligned16(w->w_d_f16))) return RKV_ERR_ALIGNMENT;
        if (!workspace || workspace_bytes < attend_workspace_bytes(s, c.B, m)) return RKV_ERR_WORKSPACE;
        if (!aligned16(workspace)) return RKV_ERR_ALIGNMENT;
    }
    return from_hip(launch_attend(s, c, idx, m, m > 0 ? w->w_d : nullptr, m > 0 ? w->w_d_f16 : nullptr, q, n_q_heads,
                                  scale, out, workspace, static_cast<hipStream_t>(stream)));
}

size_t rkv_prepared_decoder_bytes(const rkv_config* cfg) {
    Shape s;
    if (check_config(cfg, &s) != RKV_OK || s.f32) return 0;
    return (size_t)2 * s.W2 * s.d_c;
}

rkv_status rkv_prepare_decoder(const rkv_config* cfg, const rkv_weights* w, void* w_d_f16, void* stream) {
    Shape s;
    rkv_status st = check_config(cfg, &s);
    if (st != RKV_OK) return st;
    if (s.f32) return RKV_ERR_UNSUPPORTED;
    if (!w || !w->w_d || !w_d_f16) return RKV_ERR_INVALID_ARG;
    if (!aligned16(w->w_d) || !aligned16(w_d_f16)) return RKV_ERR_ALIGNMENT;
    return from_hip(launch_prepare_decoder(s, w->w_d, w_d_f16, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
