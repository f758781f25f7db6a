// Internal launch interface between the C ABI layer (rkv_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "rkv.h"

namespace rkv {

// Everything a launcher needs, resolved and validated on the host.
struct Shape {
    int N, D, dk, W2;  // heads, head dim, d_k = N*D, W2 = 2*d_k
    int d_ff, d_c, top_k, bits, group, G;  // G = d_c / group
    bool f32;          // true: "f32" formats, false: "bf16" formats
    bool mproj;        // RKV_FLAG_MEAN_PROJECTION: f_c(mean) from the references' projections
    double theta;
};

struct CacheView {
    int B, cap_ref, cap_tok;
    void* ref_vals;
    int* ref_pos;
    float* ref_norm2;
    int* ref_count;
    uint8_t* codes;
    void* scale;
    void* zmin;
    int* ref_idx;
    int* self_slot;
    int* err;
    int* stats;        // optional encode counters (RKV_STATS_WORDS)
    float* ref_proj;   // [B][cap_ref][d_ff][2] (mean-projection form)
    int* proj_count;   // [B] (mean-projection form)
    size_t code_bytes;  // per token
};

// Search split factor and workspace carve-up of rkv_encode.
struct EncodePlan {
    int nsplit;        // pool chunks searched independently per token tile
    int chunk_slots;   // slots per chunk (multiple of the slot tile)
    bool small;        // few tokens per sequence: pool scan instead of the tiled search
    size_t off_scores; // scan scores [B][n][cap_ref] (small only)
    int cap_q;         // items per queue of the bf16 search's work plan
    size_t off_tile_nblk, off_items, off_ctr;  // work plan: blocks per tile, item queues, counters
    size_t off_part_score, off_part_slot, off_rescan, off_rescan_part, off_xbar, off_dh, total;
};

EncodePlan plan_encode(const Shape& s, int B, int n, int cap_ref);

hipError_t launch_append(const Shape& s, const CacheView& c, const void* kv, int kv_len, const int* rows,
                         const int* pos, int n, hipStream_t st);

hipError_t launch_search(const Shape& s, const CacheView& c, const EncodePlan& p, const void* kv, int kv_len,
                         const int* rows, const int* pos, int n, void* ws, hipStream_t st);

hipError_t launch_select(const Shape& s, const CacheView& c, const EncodePlan& p, const void* kv, int kv_len,
                         const int* rows, const int* pos, int n, void* ws, hipStream_t st);

// kv_len rows of kv; pos [B][n] (the records' positions, read by the mean-projection form)
hipError_t launch_swiglu(const Shape& s, const CacheView& c, const EncodePlan& p, const void* kv, int kv_len,
                         const int* rows, const int* pos, int n, const void* w1, const void* w2, void* ws,
                         hipStream_t st);

// Mean-projection form: project pool slots [proj_count, ref_count) of every sequence into
// ref_proj ([r W_c1, r W_c2] per hidden column, fp32), then set proj_count = ref_count.
hipError_t launch_project_refs(const Shape& s, const CacheView& c, const void* w1, const void* w2, hipStream_t st);

hipError_t launch_latent_quant(const Shape& s, const CacheView& c, const EncodePlan& p, const int* pos, int n,
                               const void* w3, void* ws, hipStream_t st);

// wd16: the prepared fp16 W_d (launch_prepare_decoder) or null
hipError_t launch_decode(const Shape& s, const CacheView& c, const int* idx, int m, const void* wd, const void* wd16,
                         void* out, int out_dtype, hipStream_t st);

// Token-tile restore (bf16 formats with INT4 / INT2 codes).
bool decode_tiles_supported(const Shape& s);
hipError_t launch_decode_tiles(const Shape& s, const CacheView& c, const int* idx, int m, const void* wd,
                               const void* wd16, void* out, int out_dtype, hipStream_t st);
// W_d (bf16, [2 d_k][d_c]) -> the fp16 form the token-tile restore reads by direct loads
hipError_t launch_prepare_decoder(const Shape& s, const void* wd, void* wd16, hipStream_t st);

// Restore fused with the attention (token-tile restore shapes): per (sequence, KV head,
// token tile of restore_attend_tiles(m), query head in the group) the tile's
// unnormalised output part_o [.. D], maximum and weight sum part_ml [.. 2], both strided
// by kAttendMaxG query heads; wd16 = the prepared fp16 W_d.
constexpr int kAttendMaxG = 8;
int restore_attend_tiles(int m);
hipError_t launch_restore_attend(const Shape& s, const CacheView& c, const int* idx, int m, const void* wd16,
                                 const void* q, int Hq, float qscale, float* part_o, float* part_ml, hipStream_t st);

// Attention over the restored selected tokens (bf16 formats): restore into the
// workspace, then split-token softmax attention for Hq query heads.
bool attend_supported(const Shape& s, int Hq);
size_t attend_workspace_bytes(const Shape& s, int B, int m);
hipError_t launch_attend(const Shape& s, const CacheView& c, const int* idx, int m, const void* wd,
                         const void* wd16, const void* q, int Hq, float scale, float* out, void* ws, hipStream_t st);

}  // namespace rkv
