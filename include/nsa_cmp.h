/*
 * nsa_cmp.h -- C ABI of the MI355X (gfx950) library for the compressed branch
 * of Native Sparse Attention (NSA): compression of K/V, compressed attention,
 * the importance-score remap and the per-(token, KV head) top-k.
 *
 * The operations are the ones two operator pages define:
 *   - "aclnnNsaCompress" (CANN operator page), section "Formula", for
 *     nsa_compress;
 *   - "mindspore.ops.nsa_compress_attention" (MindSpore operator page),
 *     steps 1-7, parameters and returns, for nsa_compress_attention.
 * The call pattern follows the CANN page's two phases: a first call that
 * validates every argument and returns the workspace size (together with a
 * reusable "plan", the executor of that page), and a second call that
 * computes.  Validation failures come back as status codes.
 *
 * Conventions shared by every entry point
 *   - Layout is TND: tokens of all sequences back to back, then heads, then
 *     the head dim (contiguous).  Sequence lengths are passed as host arrays
 *     of prefix sums (cumulative counts, one entry per sequence, the last one
 *     equal to the total), as both pages require.
 *   - Device pointers are caller-owned device memory; the library never
 *     allocates, frees or retains them beyond the call.  Tensors must be
 *     contiguous and 16-byte aligned (topk_indices 4-byte aligned).
 *   - Host arrays are read only during the call that receives them.
 *   - GPU work is enqueued on `stream` (a hipStream_t; NULL is the default
 *     stream) and the library never synchronises: a call returns once its
 *     launches are enqueued.  Launch errors are reported as NSA_ERR_HIP; an
 *     error inside a kernel surfaces at the caller's next synchronisation.
 *   - A status other than NSA_OK means nothing was enqueued.  The reason is
 *     available from nsa_last_error() on the calling thread.
 *   - Results are deterministic: the same inputs give bitwise identical
 *     outputs (no floating-point atomics; every reduction has a fixed order).
 */
#ifndef NSA_CMP_H
#define NSA_CMP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum nsa_status {
    NSA_OK = 0,
    NSA_ERR_NULLPTR = 1,      /* a required pointer is NULL */
    NSA_ERR_DTYPE = 2,        /* dtype code not recognised (Python: TypeError) */
    NSA_ERR_SHAPE = 3,        /* sizes / prefix sums inconsistent (Python: ValueError) */
    NSA_ERR_CONSTRAINT = 4,   /* a documented parameter constraint fails (ValueError) */
    NSA_ERR_WORKSPACE = 5,    /* workspace missing or too small */
    NSA_ERR_UNSUPPORTED = 6,  /* legal on the pages, not built here (never a silent fallback) */
    NSA_ERR_HIP = 7           /* the HIP runtime refused a copy or a launch */
} nsa_status;

/* Element types of q/k/v, of the compression input and weight, and of the
 * outputs that carry them (compressed K/V, attention_out).  The MindSpore
 * page ("mindspore.ops.nsa_compress_attention", Parameters) allows float16
 * and bfloat16 for query, key and value; both are built.  Products run on
 * the 32x32x16 MFMA of that type with float32 accumulation; float32 results
 * are rounded to it once, to nearest even. */
typedef enum nsa_dtype {
    NSA_DTYPE_BF16 = 0,
    NSA_DTYPE_FP16 = 1
} nsa_dtype;

/* Opaque, reusable handle produced by the first phase of the attention
 * operator (the CANN page's "executor").  Never written after it is made,
 * so one plan may serve several streams and threads at once (each with its
 * own workspace).  Free with nsa_plan_destroy. */
typedef struct nsa_plan_s* nsa_plan;

/* Number of compressed entries of a sequence of length seq_len: the window
 * index i runs over 0 .. floor((seq_len - l) / d), so this is
 * floor((seq_len - l) / d) + 1, or 0 when seq_len < l ("aclnnNsaCompress",
 * Formula).  Returns -1 when l < 1, d < 1 or seq_len < 0. */
int64_t nsa_compress_out_len(int64_t seq_len, int64_t compress_block_size,
                             int64_t compress_stride);

/*
 * nsa_compress -- "aclnnNsaCompress", Formula: for every sequence and every
 * window i, output[i, n, :] = sum_{p < l} weight[p, n] * input[i*d + p, n, :]
 * (rows counted from the sequence start; the page's 1-based window
 * k_{id+1 : id+l}), accumulated in float32 in ascending p and rounded once
 * to the output dtype (nearest, ties to even).
 *
 *   input          [total_tokens, num_heads, head_dim], device
 *   weight         [compress_block_size, num_heads], device, same dtype as
 *                  input (one scalar per window position and head, broadcast
 *                  over the head dim)
 *   act_seq_len    host, batch prefix sums of the token counts; non-empty,
 *                  non-decreasing, last entry == total_tokens
 *   output         [output_tokens, num_heads, head_dim], device;
 *                  output_tokens must equal sum_b nsa_compress_out_len(T_b).
 *                  May be NULL only when output_tokens == 0.
 *   stream         hipStream_t
 *
 * Constraints (CANN page, constraints list; its names are garbled in the
 * copy these comments were written from, so the reading is stated):
 * compress_block_size (l) a multiple of 16 in [16, 128]; compress_stride (d)
 * a multiple of 16 with 16 <= d <= l; head_dim a multiple of 16, <= 256;
 * num_heads >= 1.
 * Errors: NSA_ERR_NULLPTR, NSA_ERR_DTYPE (unknown dtype code), NSA_ERR_SHAPE
 * (prefix sums or output_tokens inconsistent), NSA_ERR_CONSTRAINT,
 * NSA_ERR_HIP.
 */
nsa_status nsa_compress(const void* input, const void* weight,
                        const int64_t* act_seq_len, int64_t batch,
                        int64_t total_tokens, int64_t num_heads, int64_t head_dim,
                        int64_t compress_block_size, int64_t compress_stride,
                        nsa_dtype dtype, void* output, int64_t output_tokens,
                        void* stream);

/*
 * nsa_compress_backward -- gradients of nsa_compress (training use; the
 * derivative of the "aclnnNsaCompress" Formula):
 *   d_input[i*d + p, n, :] += weight[p, n] * d_output[i, n, :]
 *   d_weight[p, n] = sum over sequences, windows i and dims e of
 *                    d_output[i, n, e] * input[i*d + p, n, e]
 * (rows counted from each sequence's start; rows in no window get 0).
 *
 *   input, weight     as given to nsa_compress (element type dtype)
 *   d_output          [output_tokens, num_heads, head_dim] float32, device
 *   d_input           [total_tokens, num_heads, head_dim] float32, device, written
 *   d_weight          [compress_block_size, num_heads] float32, device, written
 * When the same weight compresses K and V, add the two calls' d_weight.
 * Results are bitwise repeatable.  Errors: as nsa_compress.
 */
nsa_status nsa_compress_backward(const void* input, const void* weight, const float* d_output,
                                 const int64_t* act_seq_len, int64_t batch,
                                 int64_t total_tokens, int64_t num_heads, int64_t head_dim,
                                 int64_t compress_block_size, int64_t compress_stride,
                                 nsa_dtype dtype, int64_t output_tokens, float* d_input,
                                 float* d_weight, void* stream);

/*
 * nsa_compress_attention_get_workspace -- first phase of
 * "mindspore.ops.nsa_compress_attention".  Host only: validates, derives the
 * per-sequence extents, plans the launches and returns the workspace size
 * and a plan.  Touches no device state.
 *
 *   batch                 number of sequences B >= 1
 *   act_seq_qlen          host [B] prefix sums of the query token counts T_b
 *   act_cmp_seq_kvlen     host [B] prefix sums of the compressed counts;
 *                         entry b must equal floor((T_b - l)/d) + 1 (0 if T_b < l)
 *   act_sel_seq_kvlen     host [B] prefix sums of the select-block counts;
 *                         entry b must equal ceil(T_b / l')
 *   head_num, kv_head_num N1 and N2: N1 >= N2 >= 1, N1 % N2 == 0
 *   d1, d2                q/k and v head dims: multiples of 16, d1 >= d2
 *   scale_value           finite float multiplying q.k^T
 *   compress_block_size   l: multiple of 16 in [16, 128]
 *   compress_stride       d: multiple of 16 in [16, 64], d <= l
 *   select_block_size     l': multiple of 16 in [16, 128], l' >= l, l' % d == 0
 *   select_block_count    k: in [1, 32]
 *   dtype                 element type of q/k/v/out; the second phase must
 *                         be given tensors of this type
 *   workspace_bytes       out: bytes of device workspace the second phase needs:
 *                         the per-sequence table (64 bytes per sequence plus
 *                         one status entry, rounded up to 256), then one
 *                         float32 per (query token, query head) that the
 *                         forward calls fill with the row's base-2
 *                         log-normaliser for the importance pass
 *   plan_out              out: the plan (caller frees it)
 *
 * Errors: NSA_ERR_NULLPTR, NSA_ERR_DTYPE (unknown dtype code), NSA_ERR_SHAPE,
 * NSA_ERR_CONSTRAINT, NSA_ERR_UNSUPPORTED (head dims outside {64,128,192} x {64,128};
 * N1/N2 > 64; more than 1024 select blocks in one sequence).  On error
 * *plan_out is set to NULL.
 */
nsa_status nsa_compress_attention_get_workspace(
    int64_t batch, const int64_t* act_seq_qlen, const int64_t* act_cmp_seq_kvlen,
    const int64_t* act_sel_seq_kvlen, int64_t head_num, int64_t kv_head_num,
    int64_t d1, int64_t d2, float scale_value, int64_t compress_block_size,
    int64_t compress_stride, int64_t select_block_size, int64_t select_block_count,
    nsa_dtype dtype, size_t* workspace_bytes, nsa_plan* plan_out);

/*
 * nsa_compress_attention -- second phase: steps 1-7 of
 * "mindspore.ops.nsa_compress_attention".
 *   1. QK = scale_value * query . key^T, masked: compressed block i is
 *      visible to the query at local position t iff i*d + l - 1 <= t;
 *   2. P_cmp = softmax over the visible blocks (natural base);
 *   3. attention_out = P_cmp . value;
 *   4. P_slc[j] = sum_{m < l'/d} sum_{n < l/d} P_cmp[(l'/d) j - m - n]
 *      (indices outside the sequence's compressed range add 0);
 *   5. P_slc' = sum of P_slc over the N1/N2 query heads of each KV head
 *      (query head h belongs to KV head floor(h / (N1/N2)));
 *   6. top-k mask: select block j is a candidate iff j*l' <= t;
 *   7. topk_indices = the select_block_count candidates with the largest
 *      P_slc' (descending; ties to the lower j), -1 in unused slots.
 *
 *   query          [T1, N1, d1] device
 *   key, value     [T2, N2, d1], [T2, N2, d2] device (T2 = last cmp prefix sum)
 *   attention_out  [T1, N1, d2] device; rows with no visible block are 0
 *   topk_indices   [T1, N2, select_block_count] int32 device
 *   softmax_max    [T1, N1, 8] float32 device: max of the scaled, masked
 *                  scores (all 8 slots equal; -inf when nothing is visible)
 *   softmax_sum    [T1, N1, 8] float32 device: sum of exp(score - max)
 *                  (all 8 slots equal; 0 when nothing is visible)
 *   p_slc_debug    NULL, or [T1, N2, S] float32 device with S the largest
 *                  select-block count of any sequence: P_slc' before the
 *                  top-k mask, 0 beyond the sequence's own count
 *   workspace      device, >= the size phase one returned (may be NULL if 0)
 *   stream         hipStream_t
 *
 * The plan fixes every size; the pointers must describe tensors of those
 * sizes.  Errors: NSA_ERR_NULLPTR, NSA_ERR_WORKSPACE, NSA_ERR_CONSTRAINT
 * (misaligned pointer), NSA_ERR_HIP.
 */
nsa_status nsa_compress_attention(nsa_plan plan, const void* query, const void* key,
                                  const void* value, void* attention_out,
                                  int32_t* topk_indices, float* softmax_max,
                                  float* softmax_sum, float* p_slc_debug,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * nsa_compress_attention_noalloc -- nsa_compress_attention for callers that
 * cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): the same computation,
 * the same kernels and bitwise the same outputs, with no workspace
 * argument.  Its only scratch, the per-sequence table (64 bytes per
 * sequence), lives in a static device array inside the library that holds
 * at most 1024 sequences (64 KiB per GPU, kept until the process ends).
 * The call allocates and frees nothing; it copies the plan's table into
 * that array on `stream` (which must belong to the current device) and
 * launches the two kernels.  Every call on one GPU shares that GPU's array
 * and overwrites it: calls that overlap on one GPU (several streams or
 * threads at once) race and must be serialised by the caller.
 *
 * Arguments and errors as nsa_compress_attention, plus NSA_ERR_UNSUPPORTED
 * when the plan has more than 1024 sequences and NSA_ERR_CONSTRAINT for a
 * device-planned plan.
 */
nsa_status nsa_compress_attention_noalloc(nsa_plan plan, const void* query, const void* key,
                                          const void* value, void* attention_out,
                                          int32_t* topk_indices, float* softmax_max,
                                          float* softmax_sum, float* p_slc_debug, void* stream);

/*
 * The second phase in two stream-ordered halves; nsa_compress_attention is
 * exactly nsa_compress_attention_fwd followed by
 * nsa_compress_attention_select on the same stream.
 *
 * nsa_compress_attention_fwd -- steps 1-3: attention_out, softmax_max and
 * softmax_sum (arguments as for nsa_compress_attention).  It also writes
 * into the workspace, for every query row, max * log2(e) + log2(sum)
 * (+inf where nothing is visible): the row's softmax in base 2, 4 bytes
 * instead of the 64 of the two [.., 8] statistics.
 *
 * nsa_compress_attention_select -- steps 4-7: topk_indices (and p_slc_debug)
 * from query, key and the row statistics of the first half; the recomputed
 * P_cmp = exp(score - max) / sum is the normalised softmax.  The statistics
 * are read from softmax_max / softmax_sum when both are given, or from the
 * per-row array the forward call wrote into this workspace when both are
 * NULL (the same outputs bit for bit; one is NULL and the other not:
 * NSA_ERR_NULLPTR).  nsa_compress_attention takes the second way.  It must
 * run after nsa_compress_attention_fwd of the same inputs (same stream, or
 * an event in between), with the forward's workspace when the statistics
 * are NULL.
 *
 * Both take the plan and a workspace of the size phase one returned, and
 * return the same errors as nsa_compress_attention.
 */
nsa_status nsa_compress_attention_fwd(nsa_plan plan, const void* query, const void* key,
                                      const void* value, void* attention_out, float* softmax_max,
                                      float* softmax_sum, void* workspace, size_t workspace_bytes,
                                      void* stream);

nsa_status nsa_compress_attention_select(nsa_plan plan, const void* query, const void* key,
                                         const float* softmax_max, const float* softmax_sum,
                                         int32_t* topk_indices, float* p_slc_debug,
                                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Explicit masks -- "mindspore.ops.nsa_compress_attention", Parameters: the
 * optional bool atten_mask (rows = query positions, columns = compressed
 * entries) and topk_mask (columns = select blocks), each of shape (S1, S2).
 * The page states no polarity and no varlen layout; the reading taken here:
 *   - one row-major byte matrix shared by every sequence of the batch, row t
 *     for the query at local position t, column i for the sequence's i-th
 *     compressed entry (atten_mask) or select block (topk_mask);
 *   - a non-zero byte masks its pair out (the score becomes -inf before the
 *     softmax, or the block is not a top-k candidate);
 *   - a given mask replaces that step's positional rule (i*d + l - 1 <= t,
 *     resp. j*l' <= t); a NULL mask keeps the rule.
 * The matrices must have at least as many rows as the longest sequence has
 * tokens and at least as many columns as the largest per-sequence count
 * (compressed entries, resp. select blocks); extra rows and columns are not
 * read.  They are device memory owned by the caller, read during the call's
 * stream work only.
 */
typedef struct nsa_masks {
    const void* atten_mask;     /* NULL, or [atten_rows, atten_cols] bytes, device */
    int64_t atten_rows, atten_cols;
    const void* topk_mask;      /* NULL, or [topk_rows, topk_cols] bytes, device */
    int64_t topk_rows, topk_cols;
} nsa_masks;

/*
 * nsa_compress_attention_get_workspace_kv -- as
 * nsa_compress_attention_get_workspace, for chunked prefill: sequence b has
 * Tkv_b = act_seq_kvlen[b] - act_seq_kvlen[b-1] key/value tokens (prefix
 * sums, host) and its Tq_b <= Tkv_b queries are the LAST Tq_b of them (the
 * causal rules of the MindSpore page's steps 3 and 6 aligned to the
 * bottom-right: query i has position Tkv_b - Tq_b + i).  Compressed and
 * select lengths follow the key/value tokens: act_cmp_seq_kvlen must hold
 * floor((Tkv_b - l)/d) + 1 and act_sel_seq_kvlen ceil(Tkv_b / l'); key and
 * value passed to the calls are the compressed key/value tokens.  With
 * Tkv_b = Tq_b for every b the plan equals the plain one.  Every second-phase
 * call takes such a plan: explicit masks keep one row per query (row t for
 * the sequence's t-th query, whatever its position); selected-block
 * attention takes the raw key/value tensors of all Tkv tokens
 * ([sum_b Tkv_b, N2, D]), query t attending to keys at positions
 * <= Tkv_b - Tq_b + t; the backward and the split launch apply the same
 * positions.
 * Errors: those of nsa_compress_attention_get_workspace, plus NSA_ERR_SHAPE
 * when Tkv_b < Tq_b.
 */
nsa_status nsa_compress_attention_get_workspace_kv(
    int64_t batch, const int64_t* act_seq_qlen, const int64_t* act_seq_kvlen,
    const int64_t* act_cmp_seq_kvlen, const int64_t* act_sel_seq_kvlen, int64_t head_num,
    int64_t kv_head_num, int64_t d1, int64_t d2, float scale_value, int64_t l, int64_t d,
    int64_t lsel, int64_t count, nsa_dtype dtype, size_t* workspace_bytes, nsa_plan* plan_out);

/*
 * Split key ranges for nsa_compress_attention_fwd (same outputs, same
 * reading of the MindSpore page's formula steps 1-7 up to P.V; positional
 * causal rule only).  The attention kernel gives each workgroup a block of
 * query rows and walks all the compressed blocks those rows see; when a few
 * row blocks see far more blocks than the rest (short batches, one long
 * sequence), their walk is the critical path of the launch.  Here a row block
 * whose walk is longer than key_tiles_per_piece tiles of 32 compressed
 * blocks is cut into pieces of at most that many tiles; each piece leaves
 * unnormalised partial sums in the workspace, and a second kernel merges the
 * pieces of every row (rescaled to their largest running max and added in
 * piece order, so results are bitwise repeatable) and writes the outputs.
 * The results equal the unsplit call's up to floating-point rounding.
 *
 * nsa_compress_attention_split_workspace -- host only: the workspace the split
 *   call needs for this plan and key_tiles_per_piece (>= workspace_bytes of
 *   the plan).  The work list is built on the device, inside the workspace,
 *   by the split call itself; the plan is not written.
 * nsa_compress_attention_fwd_split -- as nsa_compress_attention_fwd, with
 *   key_tiles_per_piece in [1, 2^20].
 * Errors: those of nsa_compress_attention_fwd, plus NSA_ERR_CONSTRAINT
 * (key_tiles_per_piece out of range) and NSA_ERR_WORKSPACE (workspace below
 * the size returned above).  With a device-planned plan the device checks
 * its work list against the counts of the plan's own lengths and sets the
 * status word (below) when they differ.
 */
nsa_status nsa_compress_attention_split_workspace(nsa_plan plan, int64_t key_tiles_per_piece,
                                                  size_t* workspace_bytes);

nsa_status nsa_compress_attention_fwd_split(nsa_plan plan, const void* query, const void* key,
                                            const void* value, void* attention_out, float* softmax_max,
                                            float* softmax_sum, int64_t key_tiles_per_piece,
                                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * The three second-phase calls with masks (masks may be NULL, and either
 * mask in it may be NULL).  The masks are packed to bits inside the
 * workspace first, so the workspace must hold masked_workspace_bytes (plan
 * info) whenever a mask is given.  nsa_compress_attention_select_masked
 * needs the same atten_mask as the fwd call whose statistics it reads, and
 * takes them from softmax_max / softmax_sum or, when both are NULL, from
 * the workspace as nsa_compress_attention_select does (the fwd calls with
 * and without masks both fill that array).
 * Errors: those of the unmasked calls, plus NSA_ERR_SHAPE (a mask smaller
 * than stated above) and NSA_ERR_WORKSPACE (workspace below
 * masked_workspace_bytes).
 */
nsa_status nsa_compress_attention_masked(nsa_plan plan, const void* query, const void* key,
                                         const void* value, const nsa_masks* masks,
                                         void* attention_out, int32_t* topk_indices,
                                         float* softmax_max, float* softmax_sum,
                                         float* p_slc_debug, void* workspace,
                                         size_t workspace_bytes, void* stream);

nsa_status nsa_compress_attention_fwd_masked(nsa_plan plan, const void* query, const void* key,
                                             const void* value, const nsa_masks* masks,
                                             void* attention_out, float* softmax_max,
                                             float* softmax_sum, void* workspace,
                                             size_t workspace_bytes, void* stream);

nsa_status nsa_compress_attention_select_masked(nsa_plan plan, const void* query, const void* key,
                                                const nsa_masks* masks, const float* softmax_max,
                                                const float* softmax_sum, int32_t* topk_indices,
                                                float* p_slc_debug, void* workspace,
                                                size_t workspace_bytes, void* stream);

/*
 * nsa_select_attention -- the step of Native Sparse Attention that consumes
 * topk_indices.  The pages give it only as an interface
 * ("lite_boost.ops.rain_fusion_attention": per query a -1 padded list of KV
 * blocks to attend to, returning the output and the softmax log-sum-exp);
 * the reading implemented: query token t (local position in its sequence),
 * query head h of KV head g = floor(h / (N1/N2)) attends to the raw keys
 * s <= t of its own sequence whose select block floor(s / l') is listed in
 * topk_indices[t, g, :]; -1, repeated entries and entries at or past the
 * sequence's ceil(T/l') blocks add nothing.
 *
 *   plan           from nsa_compress_attention_get_workspace(_kv) (sequence
 *                  lengths, heads, dims, scale_value, l' = select_block_size,
 *                  select_block_count, dtype); l' must be a multiple of 32.
 *                  With a chunked plan query t of a sequence has position
 *                  Tkv - Tq + t and attends to keys s <= that position.
 *   query          [T1, N1, d1] device
 *   key, value     [Tkv, N2, d1] and [Tkv, N2, d2] device (Tkv = the plan's
 *                  total_kv_tokens, T1 unless chunked): the raw (not
 *                  compressed) keys and values, TND, sequence b at its
 *                  key/value prefix-sum offset
 *   topk_indices   [T1, N2, select_block_count] int32 device (for instance
 *                  the output of nsa_compress_attention)
 *   attention_out  [T1, N1, d2] device; 0 for a query with no key
 *   softmax_lse    [T1, N1] float32 device: natural log of
 *                  sum_s exp(scale * q.k_s) over the attended keys; -inf for
 *                  a query with no key
 *   workspace      device, >= the plan's workspace_bytes
 *
 * Errors: NSA_ERR_NULLPTR, NSA_ERR_WORKSPACE, NSA_ERR_CONSTRAINT (misaligned
 * pointer), NSA_ERR_UNSUPPORTED (l' not a multiple of 32; head dims outside
 * {64,128,192} x {64,128}), NSA_ERR_HIP.
 */
nsa_status nsa_select_attention(nsa_plan plan, const void* query, const void* key,
                                const void* value, const int32_t* topk_indices,
                                void* attention_out, float* softmax_lse, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * nsa_compress_attention_backward -- gradients of steps 1-3 of
 * "mindspore.ops.nsa_compress_attention" for training (the pages keep the
 * softmax max and sum for this use but give no formulas).  With the
 * forward's P = exp(scale * q.k_i - softmax_max) / softmax_sum over the
 * visible blocks and d_attention_out = dout:
 *   d_value[i]  = sum over the rows that see i of P_i * dout
 *   dP_i = dout . value[i],  Delta = dout . attention_out,
 *   dS_i = P_i * (dP_i - Delta)
 *   d_query     = scale * sum_i dS_i * key[i]
 *   d_key[i]    = scale * sum over the rows that see i of dS_i * query
 * (GQA: the heads of a KV group add into its key / value rows).  The top-k
 * indices carry no gradient; softmax_max / softmax_sum are treated as
 * statistics, not outputs with a gradient.
 *
 *   query, key, value   the forward's inputs ([T1,N1,d1], [T2,N2,d1], [T2,N2,d2])
 *   attention_out       the forward's output [T1, N1, d2]
 *   d_attention_out     [T1, N1, d2], the element type of the plan
 *   softmax_max/sum     the forward's [T1, N1, 8] float32 outputs
 *   d_query             [T1, N1, d1] float32, written
 *   d_key, d_value      [T2, N2, d1] / [T2, N2, d2] float32, written (the
 *                       gradients of the compressed key / value; pass them to
 *                       nsa_compress_backward for the raw ones)
 *   workspace           >= backward_workspace_bytes (plan info)
 * Results are bitwise repeatable (fixed summation orders, no atomics).
 * Errors: NSA_ERR_NULLPTR, NSA_ERR_WORKSPACE, NSA_ERR_CONSTRAINT (misaligned
 * pointer), NSA_ERR_UNSUPPORTED (head dims not built), NSA_ERR_HIP.
 */
nsa_status nsa_compress_attention_backward(nsa_plan plan, const void* query, const void* key,
                                          const void* value, const void* attention_out,
                                          const void* d_attention_out, const float* softmax_max,
                                          const float* softmax_sum, float* d_query, float* d_key,
                                          float* d_value, void* workspace, size_t workspace_bytes,
                                          void* stream);

/* Sizes a plan fixed, for callers that allocate outputs from a plan. */
typedef struct nsa_plan_info {
    int64_t batch;
    int64_t total_q_tokens;     /* T1 */
    int64_t total_cmp_tokens;   /* T2 */
    int64_t total_sel_blocks;   /* sum_b ceil(T_b / l') */
    int64_t max_sel_blocks;     /* S of p_slc_debug */
    int64_t head_num, kv_head_num, d1, d2, select_block_count;
    size_t workspace_bytes;
    int64_t dtype;              /* the nsa_dtype the plan was made for */
    size_t masked_workspace_bytes;  /* workspace of the calls given a mask */
    size_t backward_workspace_bytes;  /* workspace of nsa_compress_attention_backward */
    int64_t total_kv_tokens;    /* sum_b Tkv_b (== total_q_tokens unless chunked) */
    int64_t device_metadata;    /* 1 for a plan from nsa_compress_attention_device_plan */
    int64_t status_offset;      /* byte offset of the int32 status word in the workspace */
} nsa_plan_info;

nsa_status nsa_plan_get_info(nsa_plan plan, nsa_plan_info* info);

/* Frees a plan; NULL is ignored. */
void nsa_plan_destroy(nsa_plan plan);

/*
 * Planning on the device -- "QuantLightningIndexerMetadata" (README, 功能说明):
 * a pre-pass on the device derives, from sequence lengths that stay in
 * device memory, each batch's blocks and load, the totals, and each core's
 * start and end points, and hands the main operator that metadata.  Here:
 *
 * nsa_compress_attention_device_plan -- a copy of `plan` whose execute calls
 *   (every second-phase call, the split launch, selected-block attention,
 *   the backward) copy nothing from the host: they read the per-sequence
 *   table that nsa_compress_attention_metadata wrote into their workspace.
 *   Host only.  Free it with nsa_plan_destroy.  Errors: NSA_ERR_NULLPTR.
 *
 * nsa_compress_attention_metadata -- writes that table into `workspace` on
 *   `stream`, derived by one workgroup from the device prefix sums
 *   act_seq_qlen, act_seq_kvlen (NULL: equal to act_seq_qlen),
 *   act_cmp_seq_kvlen and act_sel_seq_kvlen (device int64 [B] each, B the
 *   plan's batch, 8-byte aligned), and an int32 status word at byte
 *   status_offset (nsa_plan_info) of the workspace: 0 when the lengths pass
 *   every check the first phase makes (non-decreasing prefix sums,
 *   Tq_b <= Tkv_b, compressed length floor((Tkv_b - l)/d) + 1, select length
 *   ceil(Tkv_b / l')) and fit the plan: no sequence longer, with more
 *   compressed entries or select blocks than the plan's largest, and the
 *   same totals and launch sizes.  Otherwise the word holds a non-zero code
 *   (bits: 1 prefix sums, 2 fewer key/value tokens than queries, 4
 *   compressed length, 8 select length, 16 exceeds the plan's largest
 *   sequence, 32 totals or launch sizes differ, 64 a work list -- split
 *   attention or key-side backward -- differs from the host's counts)
 *   and every later call on that workspace returns from its kernels without
 *   touching its outputs.  Lengths may differ per sequence from the ones the
 *   plan was made from as long as they pass.  The word is read by the
 *   kernels only; a caller that wants it copies it back after the stream.
 *   The workspace must hold the plan's workspace_bytes; the masked, split
 *   and backward calls need their larger sizes as usual, with the table at
 *   its start.
 *   Errors: NSA_ERR_NULLPTR, NSA_ERR_CONSTRAINT (not a device-planned plan;
 *   misaligned pointers), NSA_ERR_WORKSPACE, NSA_ERR_HIP.
 */
nsa_status nsa_compress_attention_device_plan(nsa_plan plan, nsa_plan* device_plan);

nsa_status nsa_compress_attention_metadata(nsa_plan device_plan, const int64_t* act_seq_qlen,
                                           const int64_t* act_seq_kvlen, const int64_t* act_cmp_seq_kvlen,
                                           const int64_t* act_sel_seq_kvlen, void* workspace,
                                           size_t workspace_bytes, void* stream);

/* Static text naming a status. */
const char* nsa_status_string(nsa_status status);

/* Detail of the last non-OK status returned on the calling thread ("" if
 * none).  Valid until the next call into the library on that thread. */
const char* nsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* NSA_CMP_H */
