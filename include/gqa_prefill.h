/*
 * gqa_prefill.h - causal grouped-query prefill attention for MI355X (gfx950).
 *
 * The operation (as the pages state it; cited by page title and section):
 *   - "DCU使用技术报告（中篇）" §1-§2: one sequence, BF16, 24 query heads over 4 KV
 *     heads (GQA ratio 6), head_dim 256; the prefill kernel computes Q·Kᵀ, the
 *     causal mask, an online softmax and P·V with FP32 accumulation; shapes it
 *     does not support are refused, never run with a wrong mapping (§2, and
 *     "gfx936 DCU上实现INT8 QK MMAC" §7).
 *   - "gfx936 DCU上实现INT8 QK MMAC" §1: score = Q·Kᵀ/sqrt(256); with INT8 keys,
 *     Q ≈ Qq·sQ, K ≈ Kq·sK and score = int32(Qq·Kqᵀ)·sQ·sK/16, restored per score
 *     before the softmax; §3: paged K reached through a block table
 *     (logical token -> physical block -> slot); §4: sQ = max|q|/127,
 *     Qq = round(q/sQ), computed once per query row; §5.2: query head h reads
 *     KV head h/6.
 *   - Chunked prefill with history: the q_len queries are the last q_len
 *     positions of a kv_len-token sequence; query i sits at position
 *     kv_len - q_len + i and attends keys 0 .. kv_len - q_len + i.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller; the library
 *     keeps no reference after the call returns and allocates nothing (its one
 *     piece of device memory is the fixed scratch array of
 *     gqa_attn_prefill_noalloc, reserved with the library's code).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued asynchronously; the library never synchronises.
 *   - Argument errors are detected on the host before anything is enqueued
 *     and returned as a gqa_status; nothing is written in that case.
 *     GQA_ERR_HIP reports a failed launch. A device fault surfaces at the
 *     caller's next synchronisation, as usual for HIP.
 *   - Calls hold no global mutable state and are thread-safe, except
 *     gqa_attn_prefill_noalloc, whose calls on one GPU share that GPU's scratch
 *     array (see there).
 *   - Fixed shape: GQA_NUM_Q_HEADS, GQA_NUM_KV_HEADS, GQA_HEAD_DIM,
 *     GQA_BLOCK_SIZE below. Layouts are row-major and contiguous.
 */
#ifndef GQA_PREFILL_H
#define GQA_PREFILL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GQA_ABI_VERSION 5
#define GQA_NUM_Q_HEADS 24
#define GQA_NUM_KV_HEADS 4
#define GQA_HEAD_DIM 256
#define GQA_BLOCK_SIZE 16
/* largest accepted q_len / kv_len (keeps every device offset inside int64 and
   every grid inside HIP's limits) */
#define GQA_MAX_LEN (1 << 24)
/* longest history gqa_attn_prefill_int8kv accepts: its int32 sums of P and V codes
   (at most 127 * 127 per key) stay below 2^31 */
#define GQA_INT8KV_MAX_KV (1 << 17)
/* bytes of device scratch memory gqa_attn_prefill_noalloc holds per GPU (64 MiB) */
#define GQA_NOALLOC_SCRATCH_BYTES (64u << 20)

typedef enum gqa_status {
  GQA_OK = 0,
  GQA_ERR_NULL_ARG = 1,     /* a required pointer is NULL */
  GQA_ERR_BAD_LENGTH = 2,   /* q_len < 0, kv_len < q_len, a length above GQA_MAX_LEN,
                               rows < 0, or num_blocks too small for kv_len */
  GQA_ERR_MISALIGNED = 3,   /* a tensor pointer is not aligned as documented */
  GQA_ERR_UNSUPPORTED = 4,  /* a combination this build refuses: INT8 values over more than
                               GQA_INT8KV_MAX_KV keys or a paged cache; a comparison build
                               with 32-key tiles also refuses paged INT8 keys and INT8
                               values */
  GQA_ERR_HIP = 5,          /* the HIP launch failed */
  GQA_ERR_WORKSPACE = 6,    /* gqa_attn_prefill_ws: workspace NULL or too small */
  GQA_ERR_SCRATCH = 7       /* gqa_attn_prefill_noalloc: the call's KV segments need more
                               than GQA_NOALLOC_SCRATCH_BYTES */
} gqa_status;

/* Version of this interface; equals GQA_ABI_VERSION of the header the library
   was built with. */
int gqa_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* gqa_status_string(int status);

/*
 * gqa_attn_prefill - causal GQA attention for one prefill chunk.
 *
 *   out[i, h, :] = sum_j softmax_j(score(i, h, j)) * V[j, h/6, :]
 *   over keys j = 0 .. kv_len - q_len + i, with score as described above.
 *
 * q      bf16 [q_len, 24, 256]; 16-byte aligned.
 * k, v   block_table == NULL: contiguous [kv_len, 4, 256];
 *        block_table != NULL: paged caches [num_blocks, 4, 16, 256], logical
 *        key t at cache[block_table[t / 16], :, t % 16, :].
 *        v is always bf16. k is bf16 when k_scale == NULL, and int8 codes when
 *        k_scale != NULL: contiguous [kv_len, 4, 256], or, paged, the split-d
 *        cache of "gfx936 DCU上实现INT8 QK MMAC" §3, [num_blocks, 4, 256/16, 16, 16]
 *        with feature f of logical key t at
 *        [block_table[t / 16], :, f / 16, t % 16, f % 16]. 16-byte aligned.
 * block_table  int32 [ceil(kv_len / 16)] or NULL; 4-byte aligned. Entries
 *        must lie in [0, num_blocks); an entry outside that range is clamped
 *        into it (the output is then wrong but no memory outside the caches is
 *        read).
 * num_blocks   physical blocks in each paged cache; ignored when block_table
 *        is NULL; must be >= ceil(kv_len / 16) when it is not.
 * k_scale  float32 [kv_len, 4] (one scale per key token and KV head) or NULL;
 *        with a block table, float32 [num_blocks, 4, 16], the scale of logical
 *        key t at [block_table[t / 16], :, t % 16]. 4-byte aligned. With INT8 keys each query row (token, head) is
 *        quantised inside the call: sQ = max|q| / 127 in float32,
 *        Qq = round-half-even(q / sQ) (IEEE division), a zero row gives 0.
 * q_len, kv_len  0 <= q_len <= kv_len <= GQA_MAX_LEN. q_len == 0 is a no-op.
 * out    bf16 [q_len, 24, 256]; fully overwritten (round-to-nearest-even);
 *        16-byte aligned; must not overlap q, k, v or the caches.
 * stream hipStream_t or NULL.
 *
 * Returns GQA_OK, GQA_ERR_NULL_ARG, GQA_ERR_BAD_LENGTH, GQA_ERR_MISALIGNED or
 * GQA_ERR_HIP.
 */
int gqa_attn_prefill(const void* q, const void* k, const void* v,
                     const int32_t* block_table, int32_t num_blocks,
                     const float* k_scale, int32_t q_len, int32_t kv_len,
                     void* out, void* stream);

/*
 * gqa_attn_prefill_workspace_size - bytes of device workspace gqa_attn_prefill_ws
 * needs for a call with these lengths; 0 when it runs the history in one piece.
 *
 * Long histories may be cut into KV segments, as the pages do for decode attention
 * and for chunked prefill with history ("gfx936 DCU上实现INT8 QK MMAC" §4): this
 * happens when one workgroup per (KV head, 32 query tokens) would leave compute
 * units idle. With fewer workgroups than CUs every (KV head, token block) is cut the
 * same way; a larger grid whose last round of workgroups would leave CUs idle has only
 * its longest token blocks (the last query tokens) cut, into as many segments as make
 * the work a whole number of rounds. Either choice comes from an estimate of the
 * launch's run time and is taken only for a clear gain. Each segment then
 * writes its unnormalised output, its per-row reference maximum and row sum to the
 * workspace, and a merge step combines them by the log-sum-exp rule into `out`; the
 * rows of token blocks that are not cut are written directly. The workspace holds
 * segments x (rows of the cut token blocks) x 24 x (256 + 2) floats.
 * With INT8 keys every segment quantises its query rows itself (same codes).
 *
 * paged, int8k: 0 or 1 (int8k = 2, INT8 values, gives 0: that call never splits).
 * Pure host function. Returns 0 for arguments gqa_attn_prefill_ws would refuse.
 */
size_t gqa_attn_prefill_workspace_size(int32_t q_len, int32_t kv_len, int paged,
                                       int int8k);

/*
 * gqa_attn_prefill_ws - gqa_attn_prefill with a caller-provided workspace, which
 * lets the call split the history into KV segments (see above). Same arguments,
 * layouts and result as gqa_attn_prefill (up to float rounding), plus:
 *
 * workspace        device memory, 16-byte aligned, owned by the caller; may be
 *                  NULL when gqa_attn_prefill_workspace_size() is 0. Its
 *                  contents on entry are ignored and on return unspecified; it
 *                  must not overlap any other argument, and two calls in flight
 *                  at once must not share it.
 * workspace_bytes  its size in bytes.
 *
 * Returns the codes of gqa_attn_prefill and GQA_ERR_WORKSPACE when the split needs
 * a workspace and it is NULL or smaller than gqa_attn_prefill_workspace_size().
 */
int gqa_attn_prefill_ws(const void* q, const void* k, const void* v,
                        const int32_t* block_table, int32_t num_blocks,
                        const float* k_scale, int32_t q_len, int32_t kv_len,
                        void* out, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * gqa_attn_prefill_noalloc - gqa_attn_prefill_ws for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the KV-segment partials go to scratch memory the library holds,
 * one array of GQA_NOALLOC_SCRATCH_BYTES per GPU, reserved when the library's code is
 * loaded on that GPU and kept until the process ends. The call itself allocates and
 * frees nothing.
 *
 * Arguments, layouts, status codes and result as gqa_attn_prefill_ws, whose launch
 * plan it takes: the output is bit for bit that of gqa_attn_prefill_ws with a workspace
 * of gqa_attn_prefill_workspace_size() bytes. When that size exceeds
 * GQA_NOALLOC_SCRATCH_BYTES the call returns GQA_ERR_SCRATCH before touching any device
 * (gqa_attn_prefill and gqa_attn_prefill_ws still serve such lengths). The scratch array
 * of a GPU is that of the device `stream` belongs to (the current device for NULL); its
 * address is taken on the first call that needs it on that device.
 *
 * Every call on a GPU shares that GPU's array, and nothing in it needs to start at
 * zero: each call writes every partial it later reads. Calls whose work may overlap in
 * time on one GPU (different streams not ordered by events, or different host threads)
 * race on the array and give wrong results; calls in order on one stream are safe.
 */
int gqa_attn_prefill_noalloc(const void* q, const void* k, const void* v,
                             const int32_t* block_table, int32_t num_blocks,
                             const float* k_scale, int32_t q_len, int32_t kv_len,
                             void* out, void* stream);

/*
 * gqa_attn_prefill_qint8 - the INT8-key call with Q quantised beforehand.
 *
 * "gfx936 DCU上实现INT8 QK MMAC" §4 quantises each query row once, before the
 * attention (in the producer that writes Q), so that the KV segments of a long history
 * share one set of codes instead of each reducing and rounding the row again. This
 * entry point takes those codes: with q_codes and q_scale written by
 * gqa_quantize_rows_int8 from a bf16 Q (rows = q_len * 24), the result is bit for bit
 * that of gqa_attn_prefill_ws on that Q with the same keys and values.
 *
 * q_codes  int8 [q_len, 24, 256]: Qq of each query row (token, head); 16-byte aligned.
 * q_scale  float32 [q_len, 24]: sQ of each row, score = int32(Qq·Kqᵀ)·sQ·sK/16;
 *          4-byte aligned. Required.
 * k_scale  required (INT8 keys); k, v, block_table, num_blocks, k_scale, q_len, kv_len,
 *          out, workspace, workspace_bytes and stream as for gqa_attn_prefill_ws, whose
 *          workspace size (int8k = 1) applies.
 *
 * Returns the codes of gqa_attn_prefill_ws; GQA_ERR_NULL_ARG also when q_scale or
 * k_scale is NULL (for q_len > 0).
 */
int gqa_attn_prefill_qint8(const void* q_codes, const float* q_scale, const void* k,
                           const void* v, const int32_t* block_table, int32_t num_blocks,
                           const float* k_scale, int32_t q_len, int32_t kv_len, void* out,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * gqa_attn_prefill_int8kv - attention with INT8 keys, INT8 values and an INT8 P·V product.
 *
 * "gfx936 DCU上实现INT8 QK MMAC" §6 names INT8 PV (V held in INT8) among the pieces of the
 * pages' final submission and defines nothing more. This call takes the reading whose
 * result does not depend on how the work is tiled:
 *   - V codes per (KV head, feature) over the sequence, as gqa_quantize_v_int8 writes
 *     them: sV[g, f] = max_t |V[t, g, f]| / 127 and Vq = round(V / sV), so one scale per
 *     feature factors out of the whole key reduction;
 *   - P codes against each row's exact maximum over its visible keys:
 *     Pq = round(127 * exp(s - max s)) in [0, 127], the scores s as for INT8 keys (§1);
 *   - out = sV * sum_j(Pq_j Vq_j) / sum_j Pq_j, both sums exact in int32, the row sum
 *     from the same codes.
 * The exponential is the GPU's exp2 in float32, so a P code whose 127 exp(s - max s) lies
 * within about 1e-3 of k + 1/2 may round either way.
 * The call first sweeps every visible key for the row maxima, then runs one pass; it
 * never cuts the history into KV segments and has no decode shape.
 *
 * q        bf16 [q_len, 24, 256], quantised per row inside the call as for
 *          gqa_attn_prefill with INT8 keys; or, when q_scale != NULL, the int8 codes
 *          written by gqa_quantize_rows_int8 with q_scale float32 [q_len, 24] (bit for bit
 *          the same result). 16-byte aligned; q_scale 4-byte aligned.
 * k, k_scale  int8 [kv_len, 4, 256] and float32 [kv_len, 4], as for gqa_attn_prefill
 *          (contiguous). 16- and 4-byte aligned.
 * v_codes  int8 [4, 256, v_ld]: code of V[t, g, f] at [g, f, t] (token index fastest);
 *          positions kv_len .. v_ld - 1 of each row are never used. 16-byte aligned.
 * v_scale  float32 [4, 256]; 16-byte aligned.
 * v_ld     tokens per stored row: a multiple of 16, kv_len <= v_ld <= GQA_MAX_LEN.
 * q_len, kv_len  0 <= q_len <= kv_len <= GQA_INT8KV_MAX_KV; q_len == 0 is a no-op.
 * out      bf16 [q_len, 24, 256], fully overwritten; 16-byte aligned; must not overlap
 *          the inputs.
 *
 * Returns GQA_OK, GQA_ERR_NULL_ARG, GQA_ERR_BAD_LENGTH (also for a bad v_ld),
 * GQA_ERR_MISALIGNED, GQA_ERR_UNSUPPORTED (kv_len > GQA_INT8KV_MAX_KV) or GQA_ERR_HIP.
 */
int gqa_attn_prefill_int8kv(const void* q, const float* q_scale, const void* k,
                            const float* k_scale, const void* v_codes, const float* v_scale,
                            int32_t v_ld, int32_t q_len, int32_t kv_len, void* out,
                            void* stream);

/*
 * gqa_quantize_v_int8 - the V producer's quantisation for gqa_attn_prefill_int8kv: the
 * per-row rule of gqa_quantize_rows_int8 applied to each (KV head, feature) column of V
 * along the tokens, written feature-major.
 *
 * v        bf16 [kv_len, 4, 256]; 16-byte aligned (may be NULL when kv_len == 0).
 * v_codes  int8 [4, 256, v_ld] output: the code of v[t, g, f] at [g, f, t]; positions
 *          kv_len .. v_ld - 1 are written as 0. 16-byte aligned.
 * v_scale  float32 [4, 256] output: s = max_t |v[t, g, f]| / 127 (IEEE division);
 *          codes clamp(round-half-even(v / s), -127, 127); a zero column gives s = 0 and
 *          codes 0. 4-byte aligned.
 * kv_len   0 <= kv_len <= GQA_MAX_LEN; v_ld a multiple of 16 with kv_len <= v_ld <=
 *          GQA_MAX_LEN.
 *
 * Returns GQA_OK, GQA_ERR_NULL_ARG, GQA_ERR_BAD_LENGTH, GQA_ERR_MISALIGNED or GQA_ERR_HIP.
 */
int gqa_quantize_v_int8(const void* v, int32_t kv_len, int32_t v_ld, void* v_codes,
                        float* v_scale, void* stream);

/*
 * gqa_quantize_rows_int8 - the per-row INT8 quantiser of "gfx936 DCU上实现INT8 QK
 * MMAC" §1/§4 as a standalone step (the K-cache producer's quantisation; the
 * attention call applies the same rule to Q internally).
 *
 * x      bf16 [rows, 256]; 16-byte aligned.
 * xq     int8 [rows, 256] output; 4-byte aligned.
 * scale  float32 [rows] output: s = max|x| / 127 (float32 IEEE division);
 *        xq = clamp(round-half-even(x / s), -127, 127); a zero row gives s = 0
 *        and xq = 0. 4-byte aligned.
 * rows   >= 0; rows == 0 is a no-op.
 *
 * Returns GQA_OK, GQA_ERR_NULL_ARG, GQA_ERR_BAD_LENGTH, GQA_ERR_MISALIGNED or
 * GQA_ERR_HIP.
 */
int gqa_quantize_rows_int8(const void* x, int64_t rows, void* xq, float* scale,
                           void* stream);

/*
 * gqa_attn_prefill_plan - the launch gqa_attn_prefill_ws would choose for a call
 * with these lengths (variant name, workgroup count, threads per workgroup,
 * bytes of LDS, KV segments, token blocks run whole, workspace bytes), written as
 * text into buf (at most
 * n bytes, NUL-terminated). gqa_attn_prefill makes the same choice with one
 * segment.
 * Pure host function: touches no device. The variant depends on the lengths
 * the same way the pages' dispatch depends on the real q_len and kv_len of a
 * chunk ("DCU使用技术报告（中篇）" §3, §5).
 *
 * paged: 0 or 1; int8k: 0 (bf16 keys), 1 (INT8 keys) or 2 (INT8 keys and values:
 * the launch of gqa_attn_prefill_int8kv, always one segment). Returns the same status
 * codes as the call would for these lengths (argument checks only) and
 * GQA_ERR_NULL_ARG when buf is NULL or n is 0.
 */
int gqa_attn_prefill_plan(int32_t q_len, int32_t kv_len, int paged, int int8k,
                          char* buf, size_t n);

#ifdef __cplusplus
}
#endif

#endif /* GQA_PREFILL_H */
