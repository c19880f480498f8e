/*
 * sgqa.h -- C ABI of libsgqa.so, the MI355X (gfx950) Sparse GQA full-attention layer.
 *
 * The layer is the full-attention path of StepFun's Step 5 Preview:
 *   - ai.info "StepFun Details Step 5 Preview's 92-Block Agent Design", section
 *     "Sparse GQA targets million-token context": relevant historical blocks are
 *     selected instead of the whole history; tokens are grouped in blocks of 8;
 *     top-k 4096 tokens.
 *   - ai4snews "Step 5 Preview bets on depth over width", Interpretation para. 2:
 *     indexer entries of adjacent history positions are compressed into block
 *     representations of size 8, cutting indexer and top-k cost 8x.
 *   - same ai.info page, section "Why StepFun chose 92 transformer blocks": the
 *     full-attention layers are Gated Grouped-Query Attention.
 *   - phantomic12 "Step 5 Preview" catalogue entry, config.json and ATTENTION
 *     SPLIT parts: 64 query heads, 4 KV heads, head_dim 192, max positions
 *     1048576; sparse_config topk 512 (blocks), proxy_dim 256.
 *
 * Conventions shared by every entry point
 *   - Tensors are dense, row-major, last dimension contiguous.  bf16 values are
 *     passed as raw 16-bit patterns (sgqa_bf16).  Element strides are in
 *     elements, not bytes.
 *   - Device pointers (marked [dev]) must be device memory of the current HIP
 *     device; host pointers (marked [host]) are read during the call only.
 *   - Ownership: the caller owns every buffer, including the workspace.  The
 *     library never allocates, frees or synchronises; all work is enqueued on
 *     `stream` (a hipStream_t; NULL = the default stream).
 *   - Errors: every call validates its arguments in plain host code before any
 *     HIP call and returns a status; SGQA_ERR_HIP reports a failed launch.
 *     Faults inside kernels surface at the caller's next synchronisation.
 *     sgqa_last_error() returns a per-thread description of the last failure.
 *   - Determinism: the same inputs on the same device give bit-identical
 *     outputs (no floating-point atomics).
 *   - Positions are int64.  The query at position t has own block c = t / B.
 *
 * Supported shapes: heads_per_group = Hq / Hkv in 1..16, Hkv in 1..8,
 * head_dim in {64, 128, 192}, proxy_dim a multiple of 32 up to 512,
 * block_size in {1, 2, 4, 8, 16, 32}, 1 <= topk_blocks <= 4096 with
 * topk_blocks * block_size <= 32768, nseq <= 64.  Prefill, sliding-window and backward calls
 * take at most 2^24 query rows (and the backward at most 2^24 cache blocks) per call; larger
 * ones return SGQA_ERR_UNSUPPORTED and are split by the caller into chunks of rows.
 */
#ifndef SGQA_H
#define SGQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t sgqa_bf16; /* raw bf16 bits */

typedef enum {
    SGQA_OK = 0,
    SGQA_ERR_NULL = 1,        /* a required pointer is NULL */
    SGQA_ERR_SHAPE = 2,       /* sizes, strides or positions are inconsistent */
    SGQA_ERR_UNSUPPORTED = 3, /* a valid shape the library does not implement */
    SGQA_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required */
    SGQA_ERR_HIP = 5          /* a HIP launch failed */
} sgqa_status;

/* Layer widths.  num_q_heads = Hq, num_kv_heads = Hkv (the pages' attention
 * groups), head_dim = d, proxy_dim = P, block_size = B, topk_blocks = k
 * (blocks kept per query, the query's own block included). */
typedef struct {
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t proxy_dim;
    int32_t block_size;
    int32_t topk_blocks;
} sgqa_dims;

/* Operation ids for sgqa_workspace_bytes. */
enum { SGQA_OP_INDEXER_TOPK = 1, SGQA_OP_ATTN_DECODE = 2, SGQA_OP_ATTN_PREFILL = 3,
       SGQA_OP_ATTN_BACKWARD = 4 };

/*
 * Block compression (ai4snews Interpretation para. 2; ai.info "Sparse GQA
 * targets million-token context"): for each sequence s and block j in
 * [blk_begin, min(blk_end, ceil(L_s/B))),
 *     kb[s][j][:] = mean of kp[s][jB .. min(jB+B, L_s)-1][:]
 * summed exactly and rounded once to bf16 (nearest, ties to even).  A trailing
 * partial block is the mean of the tokens present.  blk_end < 0 means "to the
 * last block".  Blocks outside the range are not written, so a decode or
 * chunked-prefill loop can refresh only the blocks it touched.
 *   kp        [dev]  [nseq][*][P] bf16, sequence stride kp_seq_stride elements
 *   kb        [dev]  [nseq][*][P] bf16, sequence stride kb_seq_stride elements
 *   seq_lens  [host] [nseq] tokens per sequence (L_s >= 0)
 */
sgqa_status sgqa_index_build(const sgqa_dims *dims, const sgqa_bf16 *kp, int64_t kp_seq_stride,
                             sgqa_bf16 *kb, int64_t kb_seq_stride, const int64_t *seq_lens,
                             int32_t nseq, int64_t blk_begin, int64_t blk_end, void *stream);

/*
 * Index maintenance from the keys (block compression as above, with the proxy
 * key of a token read as the linear projection of its concatenated KV-head
 * keys; phantomic12 config.json, sparse_config, fixes the proxy width).  The
 * projection is linear, so for each sequence s and block j in
 * [blk_begin, min(blk_end, ceil(L_s/B))),
 *     kb[s][j][p] = sum_i w_kt[p][i] * m[i],
 *     m[i] = mean of k_cache[s][jB .. min(jB+B, L_s)-1][i],  i < Hkv*d
 * (i indexes the concatenated key, head g at i = g*d .. g*d+d-1): one
 * projection per block, and no proxy-key tensor.  The mean is formed in fp32
 * and kept to ~2^-17 relative through the bf16 matrix cores (hi + lo split);
 * the result is rounded once to bf16 (nearest, ties to even).  Blocks outside
 * the range are not written, so a decode loop refreshes its trailing block by
 * passing that one block.  Needs proxy_dim in {32, 64, 128, 256, 512}.
 *   k_cache   [dev]  [nseq][*][Hkv][d] bf16, sequence stride cache_seq_stride elements
 *   w_kt      [dev]  [P][Hkv*d] bf16: row p is the projection vector of proxy
 *                    feature p (the projection matrix transposed)
 *   kb        [dev]  [nseq][*][P] bf16, sequence stride kb_seq_stride elements
 *   seq_lens  [host] [nseq] tokens per sequence (L_s >= 0), nseq <= 64
 */
sgqa_status sgqa_index_build_from_keys(const sgqa_dims *dims, const sgqa_bf16 *k_cache,
                                       int64_t cache_seq_stride, const sgqa_bf16 *w_kt,
                                       sgqa_bf16 *kb, int64_t kb_seq_stride,
                                       const int64_t *seq_lens, int32_t nseq, int64_t blk_begin,
                                       int64_t blk_end, void *stream);

/*
 * Indexer scores and causal top-k (phantomic12 sparse_config: topk 512,
 * proxy_dim 256; ai.info "Sparse GQA targets million-token context").  For
 * query i of sequence s at position t = q_start[s] + i, with c = t / B:
 *     score[j] = sum_p qp[s][i][p] * kb[s][j][p]  for every complete past
 *                block j < c (bf16 inputs, fp32 accumulation);
 *     if c <= k-1 the selection is {0..c}; otherwise it is the k-1 highest
 *     scores (ties to the lower block index) plus the own block c.
 * idx[s][i][:] lists the selection in ascending block order, padded with -1
 * to k entries.  sel_scores (optional) holds the fp32 score of each selected
 * block, +inf for the own block and -inf for padding.
 *   qp         [dev]  [nseq][T][P] bf16, sequence stride qp_seq_stride elements
 *   kb         [dev]  [nseq][*][P] bf16 holding at least blocks 0..c-1 of
 *                      every query, sequence stride kb_seq_stride elements
 *   q_start    [host] [nseq] position of each sequence's first query (>= 0)
 *   idx        [dev]  [nseq][T][k] int32
 *   sel_scores [dev]  [nseq][T][k] fp32, may be NULL
 *   workspace  [dev]  scratch of workspace_bytes bytes (at least
 *                      sgqa_workspace_bytes(SGQA_OP_INDEXER_TOPK, ...) with
 *                      T = 1 rounded up; more lets one launch cover more rows)
 * Rows of at most 131072 candidate blocks with k <= 1024 and proxy_dim in
 * {32, 64, 128, 256, 512} are selected without storing their scores: a sampled
 * lower bound of each row's threshold filters the scores as the matrix cores
 * produce them, and only the blocks above it are listed (about 2.5 (k-1) per
 * row) and selected exactly; a row whose bound misses is re-scored in full by
 * one of 64 fallback workgroups.  The result is the same bits either way.  This
 * path needs 256 B + 64 * ceil64(c_max) * 4 B plus, per query row of a pass,
 * 4 ns + 12 + 8 cap bytes (ns, cap = 1024, 2048 up to 32768 candidates, else
 * 4096, 4096); smaller workspaces, longer rows and other shapes store every
 * score row ([rows][ceil64(c_max)] fp32 per pass) and select over it.
 */
sgqa_status sgqa_indexer_topk(const sgqa_dims *dims, const sgqa_bf16 *qp, int64_t qp_seq_stride,
                              const sgqa_bf16 *kb, int64_t kb_seq_stride, const int64_t *q_start,
                              int32_t nseq, int32_t T, int32_t *idx, float *sel_scores,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * Gated sparse GQA attention, prefill (ai.info "Why StepFun chose 92
 * transformer blocks": Gated Grouped-Query Attention; ai4snews Interpretation
 * para. 2: a sparse attention operator over the selected blocks).  For query
 * row i at t = q_start + i and head h, with group g = h / (Hq/Hkv), over the
 * tokens U = { s : s/B in idx[i], s <= t }:
 *     z_s = softmax_scale * q[i][h] . K[s][g];   a = sum_s softmax(z)_s V[s][g]
 *     out[i][h] = a * sigmoid(gate[i][h]);      lse[i][h] = log sum_s exp(z_s)
 * QK^T and PV run on bf16 MFMA with fp32 accumulation; the softmax is fp32
 * online; probabilities are rounded to bf16 for PV; out is rounded to bf16.
 * Only the first min(k, c+1) entries of each idx row are read; entries that
 * are -1 or outside [0, c] are skipped.
 * With a workspace (optional) the selected blocks of each query whose own block
 * c is at least 2k are visited one history range at a time, so that each XCD's
 * L2 holds a smaller working set, with the softmax state carried exactly from
 * range to range.  When the KV groups divide the 8 XCDs, rows whose history spans
 * at most 16 ranges of 5k blocks are attended by one persistent launch whose
 * waves keep their state in registers and step through the ranges together (it
 * uses the first bytes of the workspace for one progress word per wave); the
 * other rows are attended in launches of one 2k-block range each, parking the
 * state in the workspace in row chunks that fit it.  Which ranges a row takes
 * depends only on its own c (and the shape), so every workspace size, and every
 * split of the rows over calls, gives the same bits; a call without a workspace
 * differs from them only in the order of fp32 additions.
 *   q     [dev] [T][Hq][d] bf16        k_cache, v_cache [dev] [L][Hkv][d] bf16
 *   gate  [dev] [T][Hq] bf16 logits    idx [dev] [T][k] int32 (as produced above)
 *   out   [dev] [T][Hq][d] bf16        lse [dev] [T][Hq] fp32, may be NULL
 *   workspace [dev] NULL, or >= sgqa_workspace_bytes(SGQA_OP_ATTN_PREFILL, dims,
 *                   1, 1, L) bytes (one row of parked state, and at least the
 *                   persistent launch's progress words); sgqa_workspace_bytes
 *                   with T rows gives the size for a single row chunk
 *   Calls that overlap on one device must use different workspaces.
 * With a workspace the persistent launch is sized to the workgroups the whole
 * GPU holds at once, and its waves wait (for a bounded time) on each other:
 * kernels running beside it on other streams delay it sharply (a 128K layer
 * with the selections on a second stream: up to ~2.5x), so run it alone.  The
 * same holds for the resident schedules of sgqa_sparse_attn_backward.
 * Requires q_start + T <= L.
 */
sgqa_status sgqa_sparse_attn_prefill(const sgqa_dims *dims, const sgqa_bf16 *q,
                                     const sgqa_bf16 *k_cache, const sgqa_bf16 *v_cache,
                                     const sgqa_bf16 *gate, const int32_t *idx, int64_t q_start,
                                     int32_t T, int64_t L, float softmax_scale, sgqa_bf16 *out,
                                     float *lse, void *workspace, size_t workspace_bytes,
                                     void *stream);

/*
 * Gated sparse GQA attention, decode: one new query per sequence at position
 * t = cache_lens[s] - 1 (its K/V already appended), same arithmetic as the
 * prefill call.  The selected tokens are split across workgroups and the
 * partial softmax states are merged exactly (log-sum-exp) before the gate.
 *   q      [dev]  [nseq][Hq][d] bf16
 *   k_cache, v_cache [dev] [nseq][*][Hkv][d] bf16, sequence stride
 *                  cache_seq_stride elements
 *   gate   [dev]  [nseq][Hq] bf16       idx [dev] [nseq][k] int32
 *   cache_lens [host] [nseq], each >= 1
 *   out    [dev]  [nseq][Hq][d] bf16    lse [dev] [nseq][Hq] fp32, may be NULL
 *   workspace [dev] at least sgqa_workspace_bytes(SGQA_OP_ATTN_DECODE, ...)
 */
sgqa_status sgqa_sparse_attn_decode(const sgqa_dims *dims, const sgqa_bf16 *q,
                                    const sgqa_bf16 *k_cache, const sgqa_bf16 *v_cache,
                                    int64_t cache_seq_stride, const sgqa_bf16 *gate,
                                    const int32_t *idx, const int64_t *cache_lens, int32_t nseq,
                                    float softmax_scale, sgqa_bf16 *out, float *lse,
                                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * sgqa_sparse_attn_decode for callers that cannot allocate device memory (code
 * under stream capture, tight serving loops, harnesses that forbid allocation):
 * the same arguments without the workspace, the same kernels, the same output
 * bits.  The partial softmax states live in a fixed 16 MiB device array that
 * the library holds on every GPU it runs on until the process ends, looked up
 * once per device on the first call there; nothing is allocated or freed.
 * Limit: nseq * parts * Hq * (d + 3) * 4 bytes <= 16 MiB, where parts (the
 * decode workgroups per sequence and KV head) is at most 4; at the real shape
 * (64 heads, d 192, 512 blocks of 8) that is 200 KB per sequence, so every
 * nseq <= 64 fits.  Larger calls return SGQA_ERR_UNSUPPORTED.  Every call on one GPU shares that GPU's array, so calls
 * that overlap on one GPU (other streams, other host threads) race; calls on
 * one stream are ordered.  Nothing in the array needs to start at zero: every
 * call writes each partial state before it reads it.
 */
sgqa_status sgqa_sparse_attn_decode_noalloc(const sgqa_dims *dims, const sgqa_bf16 *q,
                                            const sgqa_bf16 *k_cache, const sgqa_bf16 *v_cache,
                                            int64_t cache_seq_stride, const sgqa_bf16 *gate,
                                            const int32_t *idx, const int64_t *cache_lens,
                                            int32_t nseq, float softmax_scale, sgqa_bf16 *out,
                                            float *lse, void *stream);

/*
 * Gated sliding-window attention, the sibling layer type (ai.info "Why StepFun
 * chose 92 transformer blocks": the efficient layers use Gated Sliding Window
 * Attention; phantomic12 config.json: sliding_window 512).  For query row i at
 * t = q_start + i and head h with group g = h / (Hq/Hkv), over the window
 * U = { s : max(0, t - window + 1) <= s <= t } (the `window` most recent
 * positions, the query's own included), with the same arithmetic as
 * sgqa_sparse_attn_prefill:
 *     out[i][h] = sigmoid(gate[i][h]) * sum_s softmax(z)_s V[s][g],
 *     z_s = softmax_scale * q[i][h] . K[s][g];   lse[i][h] = log sum_s exp(z_s)
 * Only num_q_heads, num_kv_heads and head_dim of dims are read.  Layouts as in
 * sgqa_sparse_attn_prefill (no idx).  Requires window >= 1 and q_start + T <= L.
 */
sgqa_status sgqa_swa_prefill(const sgqa_dims *dims, const sgqa_bf16 *q, const sgqa_bf16 *k_cache,
                             const sgqa_bf16 *v_cache, const sgqa_bf16 *gate, int64_t q_start,
                             int32_t T, int64_t L, int64_t window, float softmax_scale,
                             sgqa_bf16 *out, float *lse, void *stream);

/*
 * Backward of sgqa_sparse_attn_prefill with the selection held fixed (the pages
 * count training at long context among the costs of full attention, ai.info
 * "Sparse GQA targets million-token context"; how the indexer itself is trained
 * is not stated, so idx is an input).  For the loss whose gradient with respect
 * to out is dout, with P_s = exp(z_s - lse) the forward's weights (lse from the
 * forward call) and dP_s = sigmoid(gate) dout . v_s:
 *   D      = sum_s P_s dP_s                per (row, head; = dout . out exactly)
 *   dgate  = D * (1 - sigmoid(gate))
 *   dz_s   = P_s * (dP_s - D)
 *   dq     = softmax_scale * sum_s dz_s k_s
 *   dk_s   = softmax_scale * sum over (row, head of the group) of dz_s q
 *   dv_s   = sum over (row, head of the group) of P_s sigmoid(gate) dout
 * With out NULL, D is formed from the same P and dP the gradients use (a first
 * sweep over the selection), so the dz of a row sum to zero.  EXPERIMENTAL:
 * with out the forward's bf16 output [T][Hq][d] (2-byte aligned), D = dout . out
 * in fp32: one elementwise pass, and dq sweeps the selection once instead of
 * twice; every dz of a row then shares the error of D (from the rounding of
 * out), which grows with the attended keys: on a 128K prefill (4096 keys per
 * row) dq is 0.99 % rel-L2 from the exact gradient with out, at the 1 % bound
 * the default meets with 0.32 %, so rows that attend thousands of keys should
 * pass NULL; dv does not involve D and is the same bits either way.  dk and dv are written for every token
 * of [0, L) (zero where no row attends); every sum runs in a fixed order, so the
 * results are deterministic.  Layouts as sgqa_sparse_attn_prefill; dq
 * [T][Hq][d], dk / dv [L][Hkv][d] and dgate [T][Hq] are fp32.  nseq is 1.
 *   workspace [dev] >= sgqa_workspace_bytes(SGQA_OP_ATTN_BACKWARD, dims, 1, T, L),
 *                   256-byte aligned: dA, D, the row bitmap and the progress words of the
 *                   resident dq and dk / dv schedules (cleared by the call); calls that
 *                   overlap in time need different workspaces
 *   dkdv_row_slice  query rows per dk / dv step: 0 picks it, else a positive multiple of 32
 *                   (anything else is SGQA_ERR_SHAPE).  When the KV heads divide 8, dk / dv
 *                   run as one persistent launch whose waves sweep the query rows in phases
 *                   of this many rows (0: 2048); otherwise as one launch per slice of this
 *                   many rows (0: the rows whose q and dout take about 192 MiB).  Either way
 *                   the rows are added from the last one down and every sum keeps one order,
 *                   so the results do not depend on it or on the schedule.
 */
sgqa_status sgqa_sparse_attn_backward(const sgqa_dims *dims, const sgqa_bf16 *q,
                                      const sgqa_bf16 *k_cache, const sgqa_bf16 *v_cache,
                                      const sgqa_bf16 *gate, const int32_t *idx, int64_t q_start,
                                      int32_t T, int64_t L, float softmax_scale, const float *lse,
                                      const sgqa_bf16 *dout, const sgqa_bf16 *out, float *dq,
                                      float *dk, float *dv, float *dgate, void *workspace,
                                      size_t workspace_bytes, int64_t dkdv_row_slice,
                                      void *stream);

/*
 * FP8 storage for the decode path.  The pages give FP8 (e4m3) only for the
 * released checkpoint (phantomic12 entry: quant_method fp8, e4m3, scaling
 * blocks of 128; ai4snews "Open Weights": FP8 for deployment).  Here a cached
 * row - one token's K or V row of one KV head (d values) or one index row (P
 * values) - is stored as OCP E4M3 codes (sign, 4 exponent bits with bias 7, 3
 * fraction bits; largest finite 448) with one fp32 scale per row, halving the
 * bytes the decode step reads.
 *
 * Row quantisation, every step in fp32: scale[r] = max_i |x[r][i]| / 448 (1 for
 * an all-zero row), codes[r][i] = nearest e4m3 of x[r][i] / scale[r] (ties to
 * even, saturating at +-448).  Dequantised value = e4m3 value * scale[r].
 *   x      [dev] [rows][cols] bf16     codes [dev] [rows][cols] uint8
 *   scales [dev] [rows] fp32;  1 <= cols <= 4096
 * For a [nseq][L][Hkv][d] cache the rows are its nseq*L*Hkv head rows (cols = d).
 */
sgqa_status sgqa_quantize_fp8(const sgqa_bf16 *x, int64_t rows, int32_t cols, uint8_t *codes,
                              float *scales, void *stream);

/*
 * sgqa_indexer_topk for one query per sequence (decode) on an FP8 index: the
 * score of block j is (qp . codes[j]) * scale[j] with the codes read as exact
 * bf16 (fp32 accumulation); selection as sgqa_indexer_topk.  Needs proxy_dim in
 * {64, 128, 256, 512}, k >= 2 and at most 131072 candidate blocks.
 *   qp        [dev]  [nseq][P] bf16, sequence stride qp_seq_stride elements
 *   kb_codes  [dev]  [nseq][kb_seq_stride][P] uint8; kb_scales [dev] [nseq][kb_seq_stride] fp32
 *   q_pos     [host] [nseq] position of each sequence's query
 *   idx       [dev]  [nseq][k]; sel_scores [dev] [nseq][k] or NULL
 *   workspace [dev]  >= sgqa_workspace_bytes(SGQA_OP_INDEXER_TOPK, dims, nseq, 1, Lmax)
 */
sgqa_status sgqa_indexer_topk_fp8(const sgqa_dims *dims, const sgqa_bf16 *qp,
                                  int64_t qp_seq_stride, const uint8_t *kb_codes,
                                  const float *kb_scales, int64_t kb_seq_stride,
                                  const int64_t *q_pos, int32_t nseq, int32_t *idx,
                                  float *sel_scores, void *workspace, size_t workspace_bytes,
                                  void *stream);

/*
 * sgqa_sparse_attn_decode on FP8 caches: logits use (q . codes) * k_scale of the
 * row, and each softmax weight is multiplied by its row's v_scale before the
 * product with the V codes (read as exact bf16); normalisation, merge and gate
 * as sgqa_sparse_attn_decode.
 *   k_codes, v_codes   [dev] [nseq][cache_seq_stride][Hkv][d] uint8
 *   k_scales, v_scales [dev] [nseq][cache_seq_stride][Hkv] fp32
 *   cache_seq_stride: tokens per sequence slot; other arguments as the bf16 call
 */
sgqa_status sgqa_sparse_attn_decode_fp8(const sgqa_dims *dims, const sgqa_bf16 *q,
                                        const uint8_t *k_codes, const uint8_t *v_codes,
                                        const float *k_scales, const float *v_scales,
                                        int64_t cache_seq_stride, const sgqa_bf16 *gate,
                                        const int32_t *idx, const int64_t *cache_lens,
                                        int32_t nseq, float softmax_scale, sgqa_bf16 *out,
                                        float *lse, void *workspace, size_t workspace_bytes,
                                        void *stream);

/*
 * Workspace size in bytes for `op` (SGQA_OP_INDEXER_TOPK, SGQA_OP_ATTN_DECODE or
 * SGQA_OP_ATTN_PREFILL) given nseq sequences of T queries and caches of at
 * most Lmax tokens.  For the indexer this is the size that lets one pass cover
 * all rows, capped at 2 GiB; smaller buffers (down to one 64-row pass) also
 * work.  For the prefill attention it is the parked state of min(T, 32768) rows,
 * and at least 32 KiB (the persistent launch's progress words).
 * Returns 0 for invalid arguments.
 */
size_t sgqa_workspace_bytes(int op, const sgqa_dims *dims, int32_t nseq, int32_t T, int64_t Lmax);

/* Static description of a status code. */
const char *sgqa_status_string(sgqa_status status);

/* Per-thread description of the most recent failure ("" if none). */
const char *sgqa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SGQA_H */
