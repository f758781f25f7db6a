/*
 * rkv.h - C ABI of the ResidualKV cache codec for AMD MI355X (gfx950).
 *
 * The codec follows the ResidualKV review page ("ResidualKV: 基于参考向量与残差的
 * KV Cache 压缩", review of arXiv 2602.08005v2):
 *   - a sparse pool of reference tokens stored directly in FP8 (section 2.4,
 *     section 2.6 fixed or dynamic stride, section 2.7 step 4);
 *   - every other token stored as a per-token group-quantized latent residual
 *     z = f_c(kv) - f_c(mean of its k nearest references) (sections 2.2-2.4);
 *   - restore of selected tokens: dequantize, z W_d + mean, split K/V, RoPE at the
 *     token's own position (section 2.5, section 2.1 last paragraph, section 2.7).
 *
 * Conventions shared by every entry point
 *   - All array pointers are DEVICE pointers owned by the caller. The library never
 *     allocates, frees or synchronises; all work is enqueued on `stream` (a
 *     hipStream_t passed as void*, NULL = the default stream) and runs
 *     asynchronously.
 *   - Host-side argument checks run before anything is launched; a failed check
 *     returns a negative rkv_status and launches nothing.
 *   - Conditions only the device can see (an empty reference pool, a position or
 *     index out of range, a full pool) set bits of cache->err_word (RKV_DEVERR_*)
 *     when err_word is not NULL; the offending token is skipped or written with
 *     an empty reference set as documented per call.
 *   - A failed kernel launch returns RKV_ERR_HIP.
 *   - No global mutable state: calls are reentrant; calls that write the same
 *     cache must be ordered by the caller (same stream or events).
 *
 * Layouts (row-major, C order; B = batch of independent sequences)
 *   joint vector width  W2  = 2 * d_k = 2 * n_kv_heads * head_dim, K heads first
 *                         then V heads (section 2.1: kv_i is the K|V concatenation)
 *   kv input             [B, kv_len, W2]        kv_dtype
 *   codec weights        nn.Linear layout [out_features, in_features]:
 *                         w_c1, w_c2 [d_ff, W2]; w_c3 [d_c, d_ff]; w_d [W2, d_c]
 *                         (the pages write x W with W [in, out]; these are W^T)
 *   reference pool       ref_vals  [B, cap_ref, W2]  ref_dtype
 *                         ref_pos   [B, cap_ref] int32 token position of each slot
 *                         ref_norm2 [B, cap_ref] fp32 squared norm of the stored row
 *                         ref_count [B] int32 number of filled slots
 *   per-token records    codes     [B, cap_tok, d_c*bits/8] uint8 (bits = 16: fp16 latent,
 *                                   2*d_c bytes); INT4 low nibble = even coordinate,
 *                                   INT2 bits [2c, 2c+1] = coordinate 4m + c
 *                         scale, zmin [B, cap_tok, d_c/group] scale_dtype: the group's
 *                                   step Delta and minimum (section 2.4)
 *                         ref_idx   [B, cap_tok, top_k] int32 pool slots of the chosen
 *                                   references, ascending, -1 padded
 *                         self_slot [B, cap_tok] int32 pool slot of a reference token,
 *                                   -1 for an encoded token (caller initialises to -1)
 *   decode output        [B, m, W2] = [B, m, 2, n_kv_heads, head_dim], out_dtype
 */
#ifndef RKV_H
#define RKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RKV_ABI_VERSION 4

typedef enum {
    RKV_OK = 0,
    RKV_ERR_INVALID_ARG = -1, /* null pointer, negative size, inconsistent shape      */
    RKV_ERR_UNSUPPORTED = -2, /* valid but not implemented (dtype combo, head_dim..)  */
    RKV_ERR_CAPACITY = -3,    /* n or m larger than the declared capacities          */
    RKV_ERR_ALIGNMENT = -4,   /* a pointer not 16-byte aligned                        */
    RKV_ERR_HIP = -5,         /* a HIP runtime call or kernel launch failed           */
    RKV_ERR_WORKSPACE = -6    /* workspace missing or smaller than required           */
} rkv_status;

typedef enum { RKV_F32 = 0, RKV_BF16 = 1, RKV_F16 = 2, RKV_FP8_E4M3 = 3 } rkv_dtype;

/* Device-side error bits written to rkv_cache.err_word (atomic OR). */
#define RKV_DEVERR_EMPTY_POOL 1   /* a token had no reference with position < its own     */
#define RKV_DEVERR_POS_RANGE 2    /* a position outside [0, cap_tok)                      */
#define RKV_DEVERR_REF_CAPACITY 4 /* append past cap_ref                                  */
#define RKV_DEVERR_IDX_RANGE 8    /* a selected index outside [0, cap_tok)                */
#define RKV_DEVERR_ROW_RANGE 16   /* a kv row index outside [0, kv_len)                   */

/* Static description of one layer's codec. Supported combinations:
 *   "bf16": kv BF16, references FP8_E4M3 (OCP e4m3fn, no scale), weights BF16,
 *           scale/zmin F16                                   (the deployment formats)
 *   "f32" : kv F32, references F32, weights F32, scale/zmin F32      (exact reference runs)
 * Shapes: head_dim in {64, 128}; d_k % 128 == 0; d_ff % 64 == 0;
 * d_c in {64, 128, 256, 384, 512}; group == 32; bits in {2, 4, 16 (= quantization off,
 * fp16 latent)}; 1 <= top_k <= 8. */
typedef struct {
    int32_t n_kv_heads; /* N                                             */
    int32_t head_dim;   /* D                                             */
    int32_t d_ff;       /* compressor hidden width (section 2.3)          */
    int32_t d_c;        /* latent width (section 2.3)                     */
    int32_t top_k;      /* k, references per token (section 2.2)          */
    int32_t bits;       /* residual code width b (section 2.4)            */
    int32_t group;      /* group size g (section 2.4)                     */
    int32_t kv_dtype;     /* rkv_dtype */
    int32_t ref_dtype;    /* rkv_dtype */
    int32_t scale_dtype;  /* rkv_dtype */
    int32_t weight_dtype; /* rkv_dtype */
    int32_t flags;        /* RKV_FLAG_* (0: the default forms)             */
    double rope_theta;  /* RoPE base theta                               */
} rkv_config;

/* rkv_config.flags.
 * RKV_FLAG_MEAN_PROJECTION: the encoder's f_c(mean) takes its first-layer
 *   pre-activations as the average of the chosen references' own. The first layer of f_c
 *   is linear (section 2.3, compressor equation), so mean W = (1/k_i) sum_j r_j W: each
 *   reference is multiplied by [W_c1 | W_c2] once (rkv_cache.ref_proj) instead of every
 *   token's mean, which removes the mean rows from the SwiGLU GEMM. The mean is then never
 *   rounded to kv_dtype (the default form rounds it), so codes can differ from the default
 *   form's within the code-flip allowance. "bf16" formats only (RKV_ERR_UNSUPPORTED
 *   otherwise); the restore is unchanged. Not on the pages: an identity of the method. */
#define RKV_FLAG_MEAN_PROJECTION 1

/* Codec weights of one layer, nn.Linear layout (see above), weight_dtype.
 * w_d_f16 is optional (NULL, or a buffer filled by rkv_prepare_decoder from this w_d):
 * with it, the "bf16" formats' restore fetches the decoder as fp16 directly instead of
 * converting w_d in every call; both give bit-identical output. */
typedef struct {
    const void* w_c1;
    const void* w_c2;
    const void* w_c3;
    const void* w_d;
    const void* w_d_f16;
} rkv_weights;

/* Cache state of one layer for a batch of B sequences; all arrays caller-owned. */
typedef struct {
    int32_t batch;
    int32_t cap_ref;
    int32_t cap_tok;
    int32_t reserved;
    void* ref_vals;
    int32_t* ref_pos;
    float* ref_norm2;
    int32_t* ref_count;
    uint8_t* codes;
    void* scale;
    void* zmin;
    int32_t* ref_idx;
    int32_t* self_slot;
    int32_t* err_word; /* optional (may be NULL) */
    /* optional (may be NULL): device int32[RKV_STATS_WORDS] counters the encode adds to
     * (atomic adds; the caller zeroes them when it wants a fresh count):
     *   [0] tokens whose reference set was decided with exact distances because the
     *       approximate scores at the set boundary lay within their rounding bound;
     *   [1] tokens re-searched with exact distances over whole pool chunks because a
     *       chunk's kept candidates could hide a nearer reference (near-equidistant
     *       references). */
    int32_t* stats;
    /* RKV_FLAG_MEAN_PROJECTION only (NULL otherwise):
     *   ref_proj   [B, cap_ref, d_ff, 2] fp32, 16-byte aligned: per pool slot and hidden
     *              column j, (r W_c1)_j and (r W_c2)_j of the stored reference r;
     *   proj_count [B] int32: slots whose projection is current. The caller zeroes it
     *              whenever it resets ref_count; rkv_encode projects slots
     *              [proj_count, ref_count) and then sets proj_count = ref_count
     *              (a proj_count above ref_count re-projects the whole pool). */
    float* ref_proj;
    int32_t* proj_count;
} rkv_cache;

#define RKV_STATS_WORDS 2

/* Version of this ABI (RKV_ABI_VERSION). */
int32_t rkv_abi_version(void);

/* Human-readable name of a status code (static string, never NULL). */
const char* rkv_status_string(rkv_status status);

/* Host-only check of a configuration (no GPU needed): RKV_OK, RKV_ERR_INVALID_ARG
 * for nonsense values, RKV_ERR_UNSUPPORTED for valid but unimplemented ones. */
rkv_status rkv_validate_config(const rkv_config* cfg);

/* Bytes of one sequence's record arrays, written to out[0..4]:
 * codes, scale, zmin, ref_idx, self_slot (per token), and pool row bytes in out[5].
 * Host-only. Returns RKV_OK or the rkv_validate_config status. */
rkv_status rkv_record_bytes(const rkv_config* cfg, size_t out[6]);

/* Workspace bytes rkv_encode needs for `batch` sequences of `n` tokens with a pool
 * capacity of cap_ref. Host-only; 0 on an invalid configuration. */
size_t rkv_encode_workspace_bytes(const rkv_config* cfg, int32_t batch, int32_t n, int32_t cap_ref);

/* Reference positions of the dynamic stride (ResidualKV review page, section 2.6):
 *   p_0 = n_sink,  p_{m+1} = p_m + s0 + floor(alpha (p_m - n_sink)),  alpha = alpha_num / alpha_den,
 * every p_m < limit, preceded by the sink positions 0 .. n_sink - 1 (below limit),
 * which have no earlier token to be encoded against and so are stored directly.
 * alpha_num = 0 gives the fixed stride s0 from n_sink. alpha is an exact rational
 * so that the floor is exact (0.001 = 1/1000). The pages' Table VI counts at 262K
 * (s0 = 10) are reproduced with n_sink = 0 and limit = 262144 - 256.
 * Host-only. out: host memory for up to `cap` positions (ascending; may be NULL when
 * cap = 0); *count receives the number of positions in the schedule.
 * Returns RKV_ERR_INVALID_ARG for limit < 0, s0 < 1, n_sink < 0, alpha_num < 0,
 * alpha_den < 1, cap < 0, count NULL or out NULL with cap > 0; RKV_ERR_CAPACITY when
 * *count > cap (the first cap positions are written), so a call with cap = 0 asks
 * for the size. The schedule is the caller's: pass the positions to rkv_append_ref
 * and every other position to rkv_encode. */
rkv_status rkv_reference_schedule(int32_t limit, int32_t s0, int32_t n_sink, int32_t alpha_num, int32_t alpha_den,
                                  int32_t* out, int32_t cap, int32_t* count);

/* Store tokens directly as references (section 2.7 step 4; FP8 storage, section 2.4).
 *   kv   [B, kv_len, W2] kv_dtype; rows [B, n] row of kv per token; pos [B, n] positions.
 * Token r of sequence b goes to pool slot ref_count[b] + r, stored in ref_dtype
 * (FP8: round to nearest even, saturating at +-448, sign kept); ref_pos and
 * ref_norm2 of the slot and self_slot[b, pos] are set, then ref_count[b] += n
 * (clamped to cap_ref). Out-of-range rows/positions and slots >= cap_ref are skipped
 * and flagged. Positions must be appended in increasing order for the encode's
 * causal pool (reference position < token position) to be a prefix. */
rkv_status rkv_append_ref(const rkv_config* cfg, rkv_cache* cache, const void* kv, int32_t kv_len,
                          const int32_t* rows, const int32_t* pos, int32_t n, void* stream);

/* Encode tokens into residual records (sections 2.2-2.4).
 *   kv [B, kv_len, W2], rows [B, n], pos [B, n] as for rkv_append_ref.
 * For each token: the k_i = min(top_k, #{slots with ref_pos < pos}) references with
 * the smallest squared L2 distance to kv (ties: lower slot) over the stored
 * reference values; their fp32 mean (ascending-slot sum, one IEEE division), rounded
 * to kv_dtype for the encoder (with RKV_FLAG_MEAN_PROJECTION: f_c(mean)'s
 * pre-activations are the fp32 ascending-slot sum of the references' rows of
 * ref_proj, divided by k_i, after the pool's new slots are projected; ref_proj and
 * proj_count must then be set, RKV_ERR_INVALID_ARG otherwise); z = f_c(kv) - f_c(mean) with
 * f_c(x) = (SiLU(x W_c1) * x W_c2) W_c3; then per group of 32 coordinates:
 * Delta = (max - min)/(2^b - 1), stored Delta and min in scale_dtype,
 * q = clamp(rint((z - min)/Delta), 0, 2^b - 1) (q = 0 when the stored Delta is 0);
 * bits = 16 stores fp16(z) instead. Writes codes/scale/zmin/ref_idx at [b, pos].
 * A token with an empty pool gets ref_idx = -1, a zero mean, and the
 * RKV_DEVERR_EMPTY_POOL bit. workspace: >= rkv_encode_workspace_bytes(cfg, B, n,
 * cap_ref) bytes of device memory, 256-byte aligned, owned by the caller, free to
 * reuse once the stream has passed this call. With n > 0, kv_len must be > 0
 * (RKV_ERR_INVALID_ARG otherwise). */
rkv_status rkv_encode(const rkv_config* cfg, const rkv_weights* w, rkv_cache* cache, const void* kv,
                      int32_t kv_len, const int32_t* rows, const int32_t* pos, int32_t n, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Number of kernels rkv_encode runs, in order: reference search, reference
 * selection + mean, SwiGLU hidden difference, W_c3 projection + group quantizer. */
#define RKV_ENCODE_PHASES 4

/* rkv_encode with optional per-kernel timing, for profiling harnesses. `events` is
 * NULL or points to RKV_ENCODE_PHASES + 1 hipEvent_t handles (created by the caller);
 * events[i] is recorded on `stream` just before kernel i and events[RKV_ENCODE_PHASES]
 * after the last one. A NULL entry is skipped (a recorded timing event leaves the GPU
 * idle for a few microseconds, so a harness may mark only the kernels it times).
 * Everything else is exactly rkv_encode. */
rkv_status rkv_encode_ex(const rkv_config* cfg, const rkv_weights* w, rkv_cache* cache, const void* kv,
                         int32_t kv_len, const int32_t* rows, const int32_t* pos, int32_t n, void* workspace,
                         size_t workspace_bytes, void* stream, void* const* events);

/* Size of the static device scratch of rkv_encode_noalloc (per GPU). */
#define RKV_NOALLOC_SCRATCH_BYTES (16u << 20)

/* rkv_encode for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same call, the
 * same kernels and the same results, with the workspace taken from a static device array
 * of this library (RKV_NOALLOC_SCRATCH_BYTES, one copy per GPU, held until the process
 * ends) instead of a caller buffer. Nothing is allocated or freed; the caller still
 * passes every input and output. The first call on a device looks up that device's copy
 * of the array (hipGetSymbolAddress, with the device current).
 * Returns RKV_ERR_WORKSPACE, launching nothing, when the call needs more than
 * RKV_NOALLOC_SCRATCH_BYTES (rkv_encode_workspace_bytes(cfg, B, n, cap_ref) > the
 * limit: at the Llama-3.1-8B KV shape about 10.5 KB per token, so bulk calls of up to
 * ~1500 tokens and any decode-time call); RKV_ERR_HIP if the array's address cannot be
 * obtained; otherwise what rkv_encode returns. The scratch holds nothing a call needs
 * from an earlier one (every part is written before it is read). All calls on one GPU
 * share the array: calls that overlap on one GPU (different streams, or host threads
 * without ordering) race and must be serialised by the caller. */
rkv_status rkv_encode_noalloc(const rkv_config* cfg, const rkv_weights* w, rkv_cache* cache, const void* kv,
                              int32_t kv_len, const int32_t* rows, const int32_t* pos, int32_t n, void* stream);

/* Bytes of the prepared decoder of a "bf16" configuration: 2 * (2 d_k) * d_c. Host-only;
 * 0 on an invalid or "f32" configuration. */
size_t rkv_prepared_decoder_bytes(const rkv_config* cfg);

/* Prepare the linear decoder W_d (section 2.5, the f_d of the boxed equation) for the
 * restore: w_d_f16 receives w->w_d ([2 d_k, d_c] bf16) as fp16, in a device layout of
 * this library (the runs of 8 latent values of a row permuted, and each reordered, for the
 * restore's MFMA operand).
 * Every bf16 in the fp16 normal range converts exactly; smaller ones round toward zero.
 * w_d_f16: >= rkv_prepared_decoder_bytes(cfg) bytes of device memory, 16-byte aligned,
 * caller-owned; valid for as long as w_d is unchanged. Stream-ordered on `stream`.
 * RKV_ERR_UNSUPPORTED for "f32" configurations. */
rkv_status rkv_prepare_decoder(const rkv_config* cfg, const rkv_weights* w, void* w_d_f16, void* stream);

/* Restore selected tokens (section 2.5 boxed equation, section 2.7 steps 2-3).
 *   idx [B, m] token positions (any order; sorted gives the best locality).
 * out[b, t] = K|V of token idx[b, t]: a reference token yields its stored value;
 * an encoded token yields z~ W_d + mean, z~ = q * Delta + min (or the fp16 latent),
 * mean = fp32 mean of its stored references. The K half is then rotated by RoPE at
 * position idx[b, t]: pair (j, j + D/2) of each head by angle p * theta^(-2j/D).
 * out_dtype: RKV_F32 or RKV_BF16. Indices outside [0, cap_tok) produce zeros and
 * the RKV_DEVERR_IDX_RANGE bit. */
rkv_status rkv_decode_selected(const rkv_config* cfg, const rkv_weights* w, const rkv_cache* cache,
                               const int32_t* idx, int32_t m, void* out, int32_t out_dtype, void* stream);

/* Workspace bytes of rkv_decode_attend for `batch` sequences of m selected tokens.
 * Host-only; 0 on an invalid or unsupported configuration (and for m = 0). */
size_t rkv_decode_attend_workspace_bytes(const rkv_config* cfg, int32_t batch, int32_t m, int32_t n_q_heads);

/* Attend over the selected tokens (section 2.7: the sparse attention method picks I_t,
 * the codec restores those tokens, the layer attends over them). For each sequence b
 * and query head h, with G = n_q_heads / n_kv_heads query heads per KV head
 * (consecutive query heads share KV head h / G):
 *   out[b, h] = sum_t softmax_t(scale * q[b, h] . K[b, t, h / G]) V[b, t, h / G]
 * over the m tokens idx[b, 0..m-1], K|V being exactly what rkv_decode_selected writes
 * in bf16 (keys rotated at their own positions). Where the token-tile restore applies
 * (top_k <= 4, d_c a multiple of 128) the restore and the attention run in one kernel and
 * no restored row is written to memory; other shapes restore into the workspace first.
 * The query must already carry its own rotation.
 *   q   [B, n_q_heads, head_dim] bf16 (device); out [B, n_q_heads, head_dim] fp32;
 *   scale > 0 (usually 1 / sqrt(head_dim)); m = 0 gives zeros.
 * "bf16" configurations, head_dim 64 or 128, G <= 8; RKV_ERR_UNSUPPORTED otherwise.
 * workspace: >= rkv_decode_attend_workspace_bytes(cfg, B, m, n_q_heads) bytes, 16-byte
 * aligned (may be NULL when m = 0): per-tile partial outputs, and room for the fp16
 * decoder when w->w_d_f16 is NULL. The restore's index rules and error bits apply. */
rkv_status rkv_decode_attend(const rkv_config* cfg, const rkv_weights* w, const rkv_cache* cache,
                             const int32_t* idx, int32_t m, const void* q, int32_t n_q_heads, float scale,
                             float* out, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RKV_H */
