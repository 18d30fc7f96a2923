/*
 * kvq.h -- C ABI of the rotated INT2 KV-cache library for MI355X (gfx950).
 *
 * The library implements the serving hot path of rotation-based INT2 KV-cache
 * quantisation as described in "Output-Aware Rotation for INT2 KV-Cache
 * Quantization" (Pith review of arXiv 2608.02691; sections "What carries the
 * argument", "Core claim", "If this is right", "Assumptions & free
 * parameters", and the abstract):
 *
 *   append  -- subtract a per-channel key mean, rotate keys and values by a
 *              per-KV-head orthogonal matrix, clip, quantise to 2-bit codes per
 *              group of channels with an fp16 scale and zero, and pack the
 *              codes into a paged cache;
 *   decode  -- single-token attention that reads the paged INT2 cache
 *              directly, with the query rotated by the key rotation, and the
 *              inverse value rotation applied to the output.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument is a DEVICE pointer into memory the caller owns,
 *    except where a comment says "host".  The library allocates nothing,
 *    keeps no global state, never synchronises the device, and launches all
 *    work on the given stream (a hipStream_t passed as void*; NULL = the
 *    default stream).  Calls on different streams may run concurrently as long
 *    as they do not write the same cache pages or workspace.
 *  - Rotations use row vectors: x_rot[j] = sum_i x[i] * R[i][j], R stored
 *    row-major float32 [head_dim][head_dim] per KV head.  The inverse rotation
 *    of the output is o = o_rot * R_V^T.
 *  - head_dim must be 128; group (channels sharing one fp16 scale/zero) is 64
 *    or 128; a block (page) holds 16 tokens.
 *  - Alignment: the cache, window store, k, v, q, out, mu and rotation
 *    pointers must be 16-byte aligned, the int32 arrays (block table, start
 *    positions, context lengths) 4-byte aligned and the workspace 256-byte
 *    aligned; a misaligned pointer is KVQ_ERR_INVALID_ARG (the workspace's,
 *    KVQ_ERR_WORKSPACE).
 *  - Return values are kvq_status codes.  Arguments are validated on the host
 *    before anything is launched; a failing check launches nothing.  A launch
 *    failure reported by the HIP runtime returns KVQ_ERR_HIP.  Values that
 *    live in device memory (block-table entries, start positions, context
 *    lengths) cannot be checked on the host: the kernels never read or write
 *    outside the cache, table and tensors described here, but a block id
 *    outside [0, num_blocks) or a position past the block table gives
 *    unspecified cache contents / outputs for the affected sequence.
 *
 * Cache layout (one buffer per layer; pages are [num_blocks][num_kv_heads]
 * of kvq_page_bytes() bytes each; G = head_dim / group):
 *   byte [0, 512)           K codes, 16 token rows of 32 bytes; channel i of
 *                           token t at byte 32*t + i/4, bits 2*(i%4)
 *   byte [512, 1024)        V codes, 128 little-endian 32-bit words, one per
 *                           channel: channel i at byte 512 + 4*(8*(i%16) +
 *                           i/16); token t at code position u = 3t mod 16,
 *                           bits 2u of the word
 *   byte [1024, 1024+64G)   K (scale, zero) fp16 pairs, [token][group]
 *   byte [.., 1024+128G)    V (scale, zero) fp16 pairs, [token][group]
 * A cached element decodes as x_hat = scale * code + zero (rotated basis).
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_INVALID_ARG = -1, /* null pointer, bad size, bad dtype, bad clip   */
  KVQ_ERR_UNSUPPORTED = -2, /* valid but not implemented (head_dim != 128)   */
  KVQ_ERR_WORKSPACE = -3,   /* workspace pointer null or too small           */
  KVQ_ERR_HIP = -4,         /* the HIP runtime reported a launch error       */
  KVQ_ERR_SCRATCH = -5      /* larger than the static scratch (no-allocation) */
} kvq_status;

typedef enum { KVQ_F32 = 0, KVQ_BF16 = 1 } kvq_dtype;

/* Human-readable text for a kvq_status value (static storage, never NULL). */
const char *kvq_status_string(int status);

/* Bytes of one (block, KV head) page: 1024 + 128 * head_dim / group.
 * Returns 0 for an unsupported (head_dim, group). */
size_t kvq_page_bytes(int32_t head_dim, int32_t group);

/*
 * kvq_append -- encode new key/value tokens into the paged INT2 cache.
 *
 * Defined by the OptR review page, "What carries the argument": keys are
 * centred by a per-channel mean before rotation (attention-equivalent), then
 * rotation, clipping, grouping and rounding; "Core claim": one rotation per
 * KV head and layer; "Assumptions & free parameters": clipping ratios c_K,
 * c_V.  For token tau of sequence b and KV head h:
 *     x = (k - mu[h]) * R_K[h],   y = v * R_V[h]
 * and for every group of `group` rotated channels (separately for x and y):
 *     lo = c*min, hi = c*max, scale = fp16((hi - lo)/3), zero = fp16(lo)
 *     code = clamp(round_half_even((x - zero)/scale), 0, 3)  (0 if scale == 0)
 * fp16 conversion rounds to nearest even and saturates at +-65504.
 *
 *   pages          device  uint8 cache buffer of num_blocks * num_kv_heads
 *                          * kvq_page_bytes(head_dim, group) bytes (written)
 *   block_table    device  int32 [batch][max_blocks_per_seq]: physical block
 *                          of logical block p of sequence b
 *   start_pos      device  int32 [batch]: position of the first new token of
 *                          sequence b; tokens go to positions start_pos[b] ..
 *                          start_pos[b] + num_new - 1 (block pos/16, slot pos%16)
 *   k, v           device  [batch][num_new][num_kv_heads][head_dim] of kv_dtype
 *   mu             device  float32 [num_kv_heads][head_dim] key mean
 *   rot_k, rot_v   device  float32 [num_kv_heads][head_dim][head_dim]; rot_v
 *                          may be NULL: the value rotation is folded into the
 *                          caller's W_V and W_O (the OptR review page, "If this
 *                          is right": value-side rotations are folded into the
 *                          projection weights), so v arrives already rotated and
 *                          is encoded as given (y = v).  rot_k may be NULL: the
 *                          centred key is encoded unrotated (x = k - mu); with
 *                          both NULL the cache is plain per-group INT2, the
 *                          unrotated baseline of the rotation methods
 *   clip_k, clip_v host    clipping ratios in (0, 1]
 * Only the written tokens' codes, scales and zeros change; other tokens in the
 * same pages keep their contents.  Two sequences must not share a physical
 * block that this call writes.  batch == 0 or num_new == 0 is a no-op.
 */
int kvq_append(void *pages, int64_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
               int32_t group, const int32_t *block_table, int32_t max_blocks_per_seq,
               const int32_t *start_pos, int32_t batch, int32_t num_new, const void *k,
               const void *v, int32_t kv_dtype, const float *mu, const float *rot_k,
               const float *rot_v, float clip_k, float clip_v, void *stream);

/*
 * Workspace bytes kvq_decode_attn needs for this shape (host query, no device
 * access).  split_pages as for kvq_decode_attn.  Returns 0 on invalid input.
 */
size_t kvq_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t max_ctx_len, int32_t split_pages);

/*
 * kvq_decode_plan -- how kvq_decode_attn cuts this shape (host query, no
 * device access).  Arguments as for kvq_decode_workspace_bytes; each output
 * pointer may be NULL:
 *   *num_splits        splits (workgroups per query tile of four heads) of the
 *                      longest context; 0 when max_ctx_len is 0
 *   *split_pages_out   pages per split (the automatic choice when split_pages
 *                      is 0)
 *   *operand_in_scan   1 when a call that launches the PREPARE and SPLITS
 *                      stages together (kvq_decode_attn among them) builds the
 *                      query operand inside the split workgroups, in one
 *                      launch, leaving no operand in the workspace; 0 when it
 *                      launches the PREPARE stage's kernel first
 * Returns KVQ_OK, KVQ_ERR_INVALID_ARG or KVQ_ERR_UNSUPPORTED.
 */
int kvq_decode_plan(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t max_ctx_len, int32_t split_pages, int32_t *num_splits,
                    int32_t *split_pages_out, int32_t *operand_in_scan);

/*
 * kvq_decode_attn -- single-token attention over the paged INT2 cache.
 *
 * Defined by the OptR review page ("What carries the argument":
 * dequantisation and inverse rotation after attention over quantised keys and
 * values; the abstract: attention over the quantised cache).  For sequence b
 * and query head hq (KV head h = hq / (num_q_heads / num_kv_heads)):
 *     q_r = q[b][hq] * R_K[h]
 *     p_t = softmax_t( sm_scale * q_r . k_hat_t ),  t < ctx_len[b]
 *     out[b][hq] = ( sum_t p_t v_hat_t ) * R_V[h]^T
 * with k_hat, v_hat the dequantised cache entries.  ctx_len[b] == 0 gives a
 * zero output.  The context is processed in splits with an online softmax and
 * merged by log-sum-exp; the result does not depend on the split size beyond
 * float32 rounding.
 *
 *   pages, block_table     as for kvq_append (pages only read)
 *   ctx_len        device  int32 [batch], each in [0, max_ctx_len]
 *   max_ctx_len    host    upper bound of ctx_len; <= 16 * max_blocks_per_seq
 *   q              device  [batch][num_q_heads][head_dim] of q_dtype
 *   rot_k, rot_v   device  float32 [num_kv_heads][head_dim][head_dim]; rot_v
 *                          may be NULL (value rotation folded into W_V and W_O):
 *                          out is then sum_t p_t v_hat_t, left in the rotated
 *                          value basis for the caller's folded W_O.  rot_k may
 *                          be NULL for a cache whose keys were encoded
 *                          unrotated: q_r = q
 *   sm_scale       host    softmax scale (1/sqrt(head_dim) for standard attention)
 *   out            device  float32 [batch][num_q_heads][head_dim] (written)
 *   workspace      device  at least kvq_decode_workspace_bytes(...) bytes,
 *                          256-byte aligned; contents are scratch
 *   split_pages    host    pages per workgroup split: 0 = automatic, else a
 *                          positive multiple of 8, at most 512.  A context of
 *                          n pages is cut into max(1, round(n / split_pages))
 *                          splits of split_pages pages, the last taking the
 *                          rest.
 * num_q_heads must be a multiple of num_kv_heads.
 */
int kvq_decode_attn(const void *pages, int64_t num_blocks, int32_t num_kv_heads,
                    int32_t head_dim, int32_t group, const int32_t *block_table,
                    int32_t max_blocks_per_seq, const int32_t *ctx_len, int32_t max_ctx_len,
                    int32_t batch, int32_t num_q_heads, const void *q, int32_t q_dtype,
                    const float *rot_k, const float *rot_v, float sm_scale, float *out,
                    void *workspace, size_t workspace_bytes, int32_t split_pages,
                    void *stream);

/*
 * kvq_decode_attn_staged -- the same computation as kvq_decode_attn, run as
 * separately launchable stages (for callers that schedule or time them apart).
 * `stages` is a bit mask of the stages to launch now, in this order:
 */
#define KVQ_STAGE_PREPARE 1 /* rotate q by R_K; write its MFMA operand to workspace */
#define KVQ_STAGE_SPLITS 2  /* stream the cache; write per-split partials           */
#define KVQ_STAGE_MERGE 4   /* log-sum-exp merge, inverse value rotation, write out */
#define KVQ_STAGE_ALL 7
/* A stage reads what the previous stage left in the workspace, so the calls
 * that make up one decode must pass identical arguments and workspace, on one
 * stream (or with the caller ordering them).  When kvq_decode_plan reports
 * operand_in_scan, PREPARE and SPLITS launched together are one launch that
 * leaves only the partials: a later SPLITS-only call then needs a PREPARE of
 * its own.  Every way of splitting the stages gives the same output, bit for
 * bit.  stages outside 1..7 is KVQ_ERR_INVALID_ARG.  kvq_decode_attn(...) ==
 * kvq_decode_attn_staged(..., KVQ_STAGE_ALL, stream). */
int kvq_decode_attn_staged(const void *pages, int64_t num_blocks, int32_t num_kv_heads,
                           int32_t head_dim, int32_t group, const int32_t *block_table,
                           int32_t max_blocks_per_seq, const int32_t *ctx_len,
                           int32_t max_ctx_len, int32_t batch, int32_t num_q_heads,
                           const void *q, int32_t q_dtype, const float *rot_k, const float *rot_v,
                           float sm_scale, float *out, void *workspace, size_t workspace_bytes,
                           int32_t split_pages, int32_t stages, void *stream);

/*
 * kvq_append_decode -- one decode step of one layer: append one new token per
 * sequence, then attend over the cache including it.
 *
 * The same computation as kvq_append with num_new = 1 followed by
 * kvq_decode_attn on the same stream (the two steps of the OptR review page,
 * "What carries the argument": encode the new key and value, then attention
 * over the quantised cache and the inverse value rotation), in fewer
 * launches.  When kvq_decode_plan reports operand_in_scan, num_q_heads is at
 * most 4 * num_kv_heads and max_ctx_len > 0, it is two: the scan's launch also
 * encodes the new tokens (in workgroups dispatched after its splits, which
 * leave the new tokens' slots out) and the merge adds each new token as one
 * more partial.  Otherwise three: the append shares a launch with the query
 * rotation, then the scan and the merge.  The cache bytes written are those
 * of kvq_append either way; the output is that of the two calls bit for bit
 * in the three-launch form, to float32 rounding in the two-launch form (the
 * new token's logit is taken in float32).  Arguments are those of the two
 * calls:
 *   start_pos      device  int32 [batch]: position of the new token
 *   k, v           device  [batch][1][num_kv_heads][head_dim] of kv_dtype
 *   ctx_len        device  int32 [batch]: tokens attended, normally
 *                          start_pos[b] + 1
 *   q              device  [batch][num_q_heads][head_dim] of q_dtype
 *   out, workspace, split_pages, sm_scale, max_ctx_len: as kvq_decode_attn
 * Validation is that of both calls; the workspace size is
 * kvq_decode_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim,
 * max_ctx_len, split_pages).  batch == 0 is a no-op.
 */
int kvq_append_decode(void *pages, int64_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                      int32_t group, const int32_t *block_table, int32_t max_blocks_per_seq,
                      const int32_t *start_pos, const int32_t *ctx_len, int32_t max_ctx_len,
                      int32_t batch, const void *k, const void *v, int32_t kv_dtype,
                      const float *mu, float clip_k, float clip_v, int32_t num_q_heads,
                      const void *q, int32_t q_dtype, const float *rot_k, const float *rot_v,
                      float sm_scale, float *out, void *workspace, size_t workspace_bytes,
                      int32_t split_pages, void *stream);

/*
 * BF16 windows -- the deployed cache of the OptR review page ("Assumptions &
 * free parameters": 64 sink tokens and the 256 most recent tokens kept in
 * BF16 beside the INT2 body).  With windows, a context of n tokens is
 *     sinks  [0, min(64, n))            bfloat16, window store
 *     body   [64, n - 256)  (n > 320)   INT2 pages, as kvq_append writes them
 *     recent [max(64, n - 256), n)      bfloat16, window store
 * and attention is one softmax over all n tokens: window keys score
 * sm_scale * q . (k - mu[h]) (the unrotated query; the same key-mean shift as
 * the centred body keys), window values enter as stored, and the body is
 * attended as in kvq_decode_attn.
 *
 * Window store of one layer: bfloat16 [batch][num_kv_heads][2: K, V][320]
 * [head_dim], caller-owned device memory of kvq_window_bytes() bytes; position
 * p lives in slot p for p < 64, else in ring slot 64 + (p - 64) mod 256.
 * Tokens are stored as given (k not centred, neither rotated), rounded to
 * bfloat16 (round to nearest even).
 */
size_t kvq_window_bytes(int32_t batch, int32_t num_kv_heads, int32_t head_dim);

/*
 * kvq_window_write -- store tokens start_pos[b] .. start_pos[b] + num_new - 1
 * (k, v [batch][num_new][num_kv_heads][head_dim] of kv_dtype) in their window
 * slots; within one call a ring slot keeps the latest of its tokens.  Used to
 * fill the windows of a prompt (whose body goes through kvq_append).
 * batch == 0 or num_new == 0 is a no-op.
 */
int kvq_window_write(void *window, int32_t num_kv_heads, int32_t head_dim, int32_t batch,
                     const int32_t *start_pos, int32_t num_new, const void *k, const void *v,
                     int32_t kv_dtype, void *stream);

/*
 * kvq_decode_attn_window -- kvq_decode_attn over sinks + INT2 body + recent
 * window (see above).  window and mu (float32 [num_kv_heads][head_dim], the
 * key mean the body was encoded with) are device pointers; the other
 * arguments, the workspace size and the errors are those of kvq_decode_attn,
 * except that split_pages 0 may take up to half again the automatic split
 * size, so that the launch's window and split workgroups fit one round of
 * the GPU (it never needs more workspace than kvq_decode_workspace_bytes).
 */
int kvq_decode_attn_window(const void *pages, int64_t num_blocks, int32_t num_kv_heads,
                           int32_t head_dim, int32_t group, const int32_t *block_table,
                           int32_t max_blocks_per_seq, const void *window, const float *mu,
                           const int32_t *ctx_len, int32_t max_ctx_len, int32_t batch,
                           int32_t num_q_heads, const void *q, int32_t q_dtype,
                           const float *rot_k, const float *rot_v, float sm_scale, float *out,
                           void *workspace, size_t workspace_bytes, int32_t split_pages,
                           void *stream);

/*
 * kvq_append_decode_window -- one decode step with windows: the new token of
 * sequence b (position p = start_pos[b], with ctx_len[b] = p + 1) enters the
 * recent window; when p >= 320 the token it displaces, position p - 256, is
 * first encoded from its window copy into the INT2 body (as kvq_append would
 * encode it).  Then kvq_decode_attn_window over ctx_len[b] tokens (its
 * split_pages rule included).  Arguments as kvq_append_decode plus the window
 * store (read and written).
 */
int kvq_append_decode_window(void *pages, int64_t num_blocks, int32_t num_kv_heads,
                             int32_t head_dim, int32_t group, const int32_t *block_table,
                             int32_t max_blocks_per_seq, void *window, const int32_t *start_pos,
                             const int32_t *ctx_len, int32_t max_ctx_len, int32_t batch,
                             const void *k, const void *v, int32_t kv_dtype, const float *mu,
                             float clip_k, float clip_v, int32_t num_q_heads, const void *q,
                             int32_t q_dtype, const float *rot_k, const float *rot_v,
                             float sm_scale, float *out, void *workspace, size_t workspace_bytes,
                             int32_t split_pages, void *stream);

/*
 * kvq_decode_attn_noalloc -- kvq_decode_attn without a workspace argument, for
 * callers that cannot allocate device memory or pass one (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).  It
 * allocates nothing: the workspace is a static device array of
 * KVQ_SCRATCH_BYTES inside the library, one per GPU, held until the process
 * ends (its address is looked up once per device, on the first call there).
 * Arguments, semantics and errors are those of kvq_decode_attn, plus
 * KVQ_ERR_SCRATCH, returned before anything is launched, when the shape needs
 * more than KVQ_SCRATCH_BYTES (kvq_decode_workspace_bytes() tells).  Every
 * call on one GPU uses that GPU's one array: calls that overlap on a GPU
 * (several streams, several host threads) race and must be serialised by the
 * caller.  The array keeps the previous call's contents; nothing in it needs
 * to start at zero.
 */
#define KVQ_SCRATCH_BYTES (32u << 20)
int kvq_decode_attn_noalloc(const void *pages, int64_t num_blocks, int32_t num_kv_heads,
                            int32_t head_dim, int32_t group, const int32_t *block_table,
                            int32_t max_blocks_per_seq, const int32_t *ctx_len,
                            int32_t max_ctx_len, int32_t batch, int32_t num_q_heads,
                            const void *q, int32_t q_dtype, const float *rot_k,
                            const float *rot_v, float sm_scale, float *out, int32_t split_pages,
                            void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
