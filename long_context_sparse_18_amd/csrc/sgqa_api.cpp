// sgqa_api.cpp -- the C ABI of libsgqa.so: argument validation and dispatch.
//
// Every check below is plain host C++ and runs before the first HIP call, so
// each error path can be exercised on a machine without a GPU.  The entry
// points and their arithmetic are specified in include/sgqa.h.
#include "sgqa.h"

#include <stdarg.h>
#include <stdio.h>

#include <cmath>
#include <string>

#include "sgqa_launch.hpp"

namespace {

thread_local std::string g_last_error;

sgqa_status fail(sgqa_status st, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

sgqa_status ok()
{
    g_last_error.clear();
    return SGQA_OK;
}

bool aligned(const void *p, uintptr_t a)
{
    return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

int64_t ceil_div(int64_t a, int64_t b)
{
    return (a + b - 1) / b;
}

int64_t round_up(int64_t a, int64_t b)
{
    return ceil_div(a, b) * b;
}

// Launches sized by query rows (or by cache blocks in the backward) keep their work-item
// counts inside 32 bits up to this many rows per call.
constexpr int64_t kMaxRowsPerCall = (int64_t)1 << 24;

sgqa_status check_rows(int64_t rows, const char *what)
{
    if (rows > kMaxRowsPerCall)
        return fail(SGQA_ERR_UNSUPPORTED, "%s: %lld exceeds %lld per call (split the call)", what,
                    (long long)rows, (long long)kMaxRowsPerCall);
    return SGQA_OK;
}

sgqa_status check_dims(const sgqa_dims *d, bool need_attn, bool need_proxy)
{
    if (!d)
        return fail(SGQA_ERR_NULL, "dims is NULL");
    if (d->block_size <= 0 || d->topk_blocks <= 0)
        return fail(SGQA_ERR_SHAPE, "block_size (%d) and topk_blocks (%d) must be positive",
                    d->block_size, d->topk_blocks);
    const int B = d->block_size;
    if (B != 1 && B != 2 && B != 4 && B != 8 && B != 16 && B != 32)
        return fail(SGQA_ERR_UNSUPPORTED, "block_size %d not in {1,2,4,8,16,32}", B);
    if (d->topk_blocks > 4096 || (int64_t)d->topk_blocks * B > 32768)
        return fail(SGQA_ERR_UNSUPPORTED, "topk_blocks %d x block_size %d exceeds 4096 blocks / 32768 tokens",
                    d->topk_blocks, B);
    if (need_proxy) {
        if (d->proxy_dim <= 0)
            return fail(SGQA_ERR_SHAPE, "proxy_dim %d must be positive", d->proxy_dim);
        if (d->proxy_dim % 32 != 0 || d->proxy_dim > 512)
            return fail(SGQA_ERR_UNSUPPORTED, "proxy_dim %d must be a multiple of 32 up to 512",
                        d->proxy_dim);
    }
    if (need_attn) {
        if (d->num_q_heads <= 0 || d->num_kv_heads <= 0 || d->head_dim <= 0)
            return fail(SGQA_ERR_SHAPE, "head counts and head_dim must be positive");
        if (d->num_q_heads % d->num_kv_heads != 0)
            return fail(SGQA_ERR_SHAPE, "num_q_heads %d is not a multiple of num_kv_heads %d",
                        d->num_q_heads, d->num_kv_heads);
        if (d->num_q_heads / d->num_kv_heads > 16 || d->num_kv_heads > 8)
            return fail(SGQA_ERR_UNSUPPORTED, "need heads per group <= 16 and num_kv_heads <= 8");
        if (d->head_dim != 64 && d->head_dim != 128 && d->head_dim != 192)
            return fail(SGQA_ERR_UNSUPPORTED, "head_dim %d not in {64,128,192}", d->head_dim);
    }
    return SGQA_OK;
}

sgqa_status check_heads(const sgqa_dims *d)
{
    if (!d)
        return fail(SGQA_ERR_NULL, "dims is NULL");
    if (d->num_q_heads <= 0 || d->num_kv_heads <= 0 || d->head_dim <= 0)
        return fail(SGQA_ERR_SHAPE, "head counts and head_dim must be positive");
    if (d->num_q_heads % d->num_kv_heads != 0)
        return fail(SGQA_ERR_SHAPE, "num_q_heads %d is not a multiple of num_kv_heads %d",
                    d->num_q_heads, d->num_kv_heads);
    if (d->num_q_heads / d->num_kv_heads > 16 || d->num_kv_heads > 8)
        return fail(SGQA_ERR_UNSUPPORTED, "need heads per group <= 16 and num_kv_heads <= 8");
    if (d->head_dim != 64 && d->head_dim != 128 && d->head_dim != 192)
        return fail(SGQA_ERR_UNSUPPORTED, "head_dim %d not in {64,128,192}", d->head_dim);
    return SGQA_OK;
}

sgqa_status hip_status(hipError_t e, const char *what)
{
    if (e != hipSuccess)
        return fail(SGQA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

struct TopkPlan {
    int64_t max_cand;  // largest candidate count over all rows
    int64_t ld;        // score row stride (floats)
    int32_t nq;        // queries per sequence per pass
};

TopkPlan topk_plan(const sgqa_dims *d, const int64_t *q_start, int32_t nseq, int32_t T, size_t ws)
{
    TopkPlan p{0, 64, 0};
    int64_t max_pos = 0;
    for (int s = 0; s < nseq; ++s)
        max_pos = q_start[s] + T - 1 > max_pos ? q_start[s] + T - 1 : max_pos;
    p.max_cand = max_pos / d->block_size;
    p.ld = round_up(p.max_cand > 0 ? p.max_cand : 1, 64);
    const int64_t row_bytes = p.ld * (int64_t)sizeof(float) * nseq;
    int64_t nq = (int64_t)(ws / (size_t)row_bytes);
    if (nq >= T)
        nq = T;
    else
        nq = (nq / 64) * 64;
    p.nq = (int32_t)nq;
    return p;
}

constexpr size_t kIndexerWorkspaceCap = size_t(2) << 30;

#ifndef SGQA_SLICE_HALF_K
#define SGQA_SLICE_HALF_K 4
#endif
#ifndef SGQA_LONG_SLICES
#define SGQA_LONG_SLICES 1
#endif
// History ranges of a row whose history is longer than 16 slices of the above.
constexpr int kPrefillLongSlices = SGQA_LONG_SLICES;
// Blocks per history slice of the sliced prefill attention, in units of k/2 (2k: 1024 blocks
// at the real shape).
constexpr int64_t kPrefillSliceHalfK = SGQA_SLICE_HALF_K;
#ifndef SGQA_RESIDENT_HALF_K
#define SGQA_RESIDENT_HALF_K 10
#endif
// Blocks per history range of the resident prefill, in units of k/2 (5k: 2560 blocks at the
// real shape; 0 turns the resident prefill off).
constexpr int64_t kPrefillResidentHalfK = SGQA_RESIDENT_HALF_K;
// The backward's resident dq ranges are wider: 12k blocks (two ranges at 128K) measured
// 647 ms for the whole backward, against 649 / 650 / 655 / 663 ms with 8k / 16k / 5k / 32k
// (one range) and 685 ms with the one-pass dq.
#ifndef SGQA_BWD_RESIDENT_HALF_K
#define SGQA_BWD_RESIDENT_HALF_K 24
#endif
constexpr int64_t kBwdResidentHalfK = SGQA_BWD_RESIDENT_HALF_K;

} // namespace

extern "C" {

const char *sgqa_status_string(sgqa_status st)
{
    switch (st) {
    case SGQA_OK: return "ok";
    case SGQA_ERR_NULL: return "null pointer";
    case SGQA_ERR_SHAPE: return "inconsistent shape";
    case SGQA_ERR_UNSUPPORTED: return "unsupported shape";
    case SGQA_ERR_WORKSPACE: return "workspace too small";
    case SGQA_ERR_HIP: return "HIP error";
    }
    return "unknown status";
}

const char *sgqa_last_error(void)
{
    return g_last_error.c_str();
}

size_t sgqa_workspace_bytes(int op, const sgqa_dims *dims, int32_t nseq, int32_t T, int64_t Lmax)
{
    if (!dims || nseq <= 0 || nseq > sgqa::kMaxSeq || T < 0 || Lmax < 0)
        return 0;
    if (op == SGQA_OP_INDEXER_TOPK) {
        if (check_dims(dims, false, true) != SGQA_OK)
            return 0;
        const int64_t max_cand = Lmax > 0 ? (Lmax - 1) / dims->block_size : 0;
        const int64_t ld = round_up(max_cand > 0 ? max_cand : 1, 64);
        const int64_t per_q = ld * (int64_t)sizeof(float) * nseq;
        const int64_t min_rows = T < 64 ? (T > 0 ? T : 1) : 64;
        int64_t bytes = per_q * (T > 0 ? T : 1);
        if ((size_t)bytes > kIndexerWorkspaceCap)
            bytes = ((int64_t)kIndexerWorkspaceCap / (per_q * 64)) * (per_q * 64);
        if (bytes < per_q * min_rows)
            bytes = per_q * min_rows;
        if (T == 1 && sgqa::decode_topk_supported(max_cand, dims->topk_blocks)) {
            const int64_t dec = (int64_t)sgqa::decode_topk_workspace(nseq, max_cand);
            return (size_t)(dec > bytes ? dec : bytes);
        }
        if (max_cand >= 1 &&
            sgqa::fused_topk_supported(max_cand, dims->topk_blocks, dims->proxy_dim)) {
            const int64_t row = (int64_t)sgqa::fused_topk_row_bytes(max_cand) * nseq;
            const int64_t fixed = (int64_t)sgqa::fused_topk_fixed_bytes(max_cand);
            int64_t rows = T > 0 ? T : 1;
            if (fixed + rows * row > (int64_t)kIndexerWorkspaceCap)
                rows = ((int64_t)kIndexerWorkspaceCap - fixed) / row / 64 * 64;
            if (rows < min_rows)
                rows = min_rows;
            // the path without a score matrix runs whenever its workspace holds one pass
            return (size_t)(fixed + rows * row);
        }
        return (size_t)bytes;
    }
    if (op == SGQA_OP_ATTN_PREFILL) {
        if (check_dims(dims, true, false) != SGQA_OK)
            return 0;
        // the state of min(T, 32768) rows for the sliced launches, and at least the resident
        // prefill's progress words (one per resident wave: at most 8 workgroups of 4 waves per
        // CU on 256 CUs)
        const int64_t rows = T < 1 ? 1 : (T > 32768 ? 32768 : T);
        const size_t state = (size_t)rows * dims->num_kv_heads * 64 *
                             sgqa::prefill_state_stride(dims->head_dim) * sizeof(float);
        return state > sgqa::kResidentProgressBytes ? state : sgqa::kResidentProgressBytes;
    }
    if (op == SGQA_OP_ATTN_BACKWARD) {
        if (check_dims(dims, true, false) != SGQA_OK || nseq != 1)
            return 0;
        return sgqa::attn_backward_workspace(T, dims->num_q_heads, dims->head_dim,
                                             ceil_div(Lmax, dims->block_size));
    }
    if (op == SGQA_OP_ATTN_DECODE) {
        if (check_dims(dims, true, false) != SGQA_OK)
            return 0;
        int nsplit, eps;
        sgqa::decode_split_plan(dims->topk_blocks, dims->block_size, nsplit, eps);
        const size_t slots = (size_t)nseq * nsplit * dims->num_q_heads;
        return slots * dims->head_dim * sizeof(float) + slots * 3 * sizeof(float);
    }
    return 0;
}

sgqa_status sgqa_index_build(const sgqa_dims *dims, const sgqa_bf16 *kp, int64_t kp_seq_stride,
                             sgqa_bf16 *kb, int64_t kb_seq_stride, const int64_t *seq_lens,
                             int32_t nseq, int64_t blk_begin, int64_t blk_end, void *stream)
{
    sgqa_status st = check_dims(dims, false, true);
    if (st != SGQA_OK)
        return st;
    if (nseq < 0 || nseq > sgqa::kMaxSeq)
        return fail(nseq < 0 ? SGQA_ERR_SHAPE : SGQA_ERR_UNSUPPORTED, "nseq %d not in [0, %d]", nseq,
                    sgqa::kMaxSeq);
    if (nseq == 0)
        return ok();
    if (!kp || !kb || !seq_lens)
        return fail(SGQA_ERR_NULL, "kp, kb and seq_lens must be non-NULL");
    if (!aligned(kp, 16) || !aligned(kb, 16))
        return fail(SGQA_ERR_SHAPE, "kp and kb must be 16-byte aligned");
    if (blk_begin < 0)
        return fail(SGQA_ERR_SHAPE, "blk_begin %lld is negative", (long long)blk_begin);
    const int P = dims->proxy_dim, B = dims->block_size;
    int64_t max_len = 0;
    for (int s = 0; s < nseq; ++s) {
        if (seq_lens[s] < 0)
            return fail(SGQA_ERR_SHAPE, "seq_lens[%d] = %lld is negative", s, (long long)seq_lens[s]);
        max_len = seq_lens[s] > max_len ? seq_lens[s] : max_len;
    }
    if (nseq > 1) {
        if (kp_seq_stride < max_len * P || kp_seq_stride % 8 != 0)
            return fail(SGQA_ERR_SHAPE, "kp_seq_stride %lld must be >= %lld and a multiple of 8",
                        (long long)kp_seq_stride, (long long)(max_len * P));
        if (kb_seq_stride < ceil_div(max_len, B) * P || kb_seq_stride % 8 != 0)
            return fail(SGQA_ERR_SHAPE, "kb_seq_stride %lld must be >= %lld and a multiple of 8",
                        (long long)kb_seq_stride, (long long)(ceil_div(max_len, B) * P));
    }
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    for (int s = 0; s < nseq; ++s) {
        const int64_t nblk = ceil_div(seq_lens[s], B);
        const int64_t j0 = blk_begin < nblk ? blk_begin : nblk;
        const int64_t j1 = (blk_end < 0 || blk_end > nblk) ? nblk : blk_end;
        if (j1 <= j0)
            continue;
        hipError_t e = sgqa::launch_index_build(kp + (int64_t)s * kp_seq_stride,
                                                kb + (int64_t)s * kb_seq_stride, seq_lens[s], P, B,
                                                j0, j1, hs);
        if (e != hipSuccess)
            return hip_status(e, "index_build launch");
    }
    return ok();
}

sgqa_status sgqa_index_build_from_keys(const sgqa_dims *dims, const sgqa_bf16 *k_cache,
                                       int64_t cache_seq_stride, const sgqa_bf16 *w_kt,
                                       sgqa_bf16 *kb, int64_t kb_seq_stride,
                                       const int64_t *seq_lens, int32_t nseq, int64_t blk_begin,
                                       int64_t blk_end, void *stream)
{
    sgqa_status st = check_dims(dims, false, true);
    if (st != SGQA_OK)
        return st;
    st = check_heads(dims);
    if (st != SGQA_OK)
        return st;
    const int P = dims->proxy_dim, B = dims->block_size;
    if (P != 32 && P != 64 && P != 128 && P != 256 && P != 512)
        return fail(SGQA_ERR_UNSUPPORTED, "proxy_dim %d not in {32,64,128,256,512}", P);
    if (nseq < 0 || nseq > sgqa::kMaxSeq)
        return fail(nseq < 0 ? SGQA_ERR_SHAPE : SGQA_ERR_UNSUPPORTED, "nseq %d not in [0, %d]", nseq,
                    sgqa::kMaxSeq);
    if (nseq == 0)
        return ok();
    if (!k_cache || !w_kt || !kb || !seq_lens)
        return fail(SGQA_ERR_NULL, "k_cache, w_kt, kb and seq_lens must be non-NULL");
    if (!aligned(k_cache, 16) || !aligned(w_kt, 16) || !aligned(kb, 2))
        return fail(SGQA_ERR_SHAPE, "k_cache and w_kt must be 16-byte aligned");
    if (blk_begin < 0)
        return fail(SGQA_ERR_SHAPE, "blk_begin %lld is negative", (long long)blk_begin);
    const int64_t width = (int64_t)dims->num_kv_heads * dims->head_dim;
    int64_t max_len = 0;
    for (int s = 0; s < nseq; ++s) {
        if (seq_lens[s] < 0)
            return fail(SGQA_ERR_SHAPE, "seq_lens[%d] = %lld is negative", s, (long long)seq_lens[s]);
        max_len = seq_lens[s] > max_len ? seq_lens[s] : max_len;
    }
    if (nseq > 1) {
        if (cache_seq_stride < max_len * width || cache_seq_stride % 8 != 0)
            return fail(SGQA_ERR_SHAPE, "cache_seq_stride %lld must be >= %lld and a multiple of 8",
                        (long long)cache_seq_stride, (long long)(max_len * width));
        if (kb_seq_stride < ceil_div(max_len, B) * P)
            return fail(SGQA_ERR_SHAPE, "kb_seq_stride %lld must be >= %lld",
                        (long long)kb_seq_stride, (long long)(ceil_div(max_len, B) * P));
    }
    sgqa::IndexKeysArgs a{};
    a.k = k_cache;
    a.cache_seq_stride = cache_seq_stride;
    a.wt = w_kt;
    a.kb = kb;
    a.kb_seq_stride = kb_seq_stride;
    a.width = (int)width;
    a.P = P;
    a.B = B;
    a.nseq = nseq;
    int64_t max_blocks = 0;
    for (int s = 0; s < nseq; ++s) {
        const int64_t nblk = ceil_div(seq_lens[s], B);
        const int64_t j0 = blk_begin < nblk ? blk_begin : nblk;
        const int64_t j1 = (blk_end < 0 || blk_end > nblk) ? nblk : (blk_end > j0 ? blk_end : j0);
        a.len.v[s] = seq_lens[s];
        a.j0.v[s] = j0;
        a.j1.v[s] = j1;
        max_blocks = j1 - j0 > max_blocks ? j1 - j0 : max_blocks;
    }
    return hip_status(sgqa::launch_index_from_keys(a, max_blocks, reinterpret_cast<hipStream_t>(stream)),
                      "index_build_from_keys launch");
}

sgqa_status sgqa_indexer_topk(const sgqa_dims *dims, const sgqa_bf16 *qp, int64_t qp_seq_stride,
                              const sgqa_bf16 *kb, int64_t kb_seq_stride, const int64_t *q_start,
                              int32_t nseq, int32_t T, int32_t *idx, float *sel_scores,
                              void *workspace, size_t workspace_bytes, void *stream)
{
    sgqa_status st = check_dims(dims, false, true);
    if (st != SGQA_OK)
        return st;
    if (nseq < 0 || T < 0)
        return fail(SGQA_ERR_SHAPE, "nseq %d and T %d must be non-negative", nseq, T);
    if (nseq > sgqa::kMaxSeq)
        return fail(SGQA_ERR_UNSUPPORTED, "nseq %d exceeds %d", nseq, sgqa::kMaxSeq);
    if (nseq == 0 || T == 0)
        return ok();
    if (!qp || !kb || !q_start || !idx)
        return fail(SGQA_ERR_NULL, "qp, kb, q_start and idx must be non-NULL");
    if (!aligned(qp, 16) || !aligned(kb, 16) || !aligned(idx, 4) || !aligned(sel_scores, 4))
        return fail(SGQA_ERR_SHAPE, "qp and kb must be 16-byte aligned");
    const int P = dims->proxy_dim;
    for (int s = 0; s < nseq; ++s)
        if (q_start[s] < 0)
            return fail(SGQA_ERR_SHAPE, "q_start[%d] = %lld is negative", s, (long long)q_start[s]);
    if (nseq > 1 && (qp_seq_stride < (int64_t)T * P || qp_seq_stride % 8 != 0))
        return fail(SGQA_ERR_SHAPE, "qp_seq_stride %lld must be >= T*P and a multiple of 8",
                    (long long)qp_seq_stride);
    if (nseq > 1 && kb_seq_stride % 8 != 0)
        return fail(SGQA_ERR_SHAPE, "kb_seq_stride must be a multiple of 8");
    const TopkPlan plan = topk_plan(dims, q_start, nseq, T, workspace ? workspace_bytes : 0);
    if (!workspace)
        return fail(SGQA_ERR_WORKSPACE, "workspace is NULL");
    if (!aligned(workspace, 16))
        return fail(SGQA_ERR_SHAPE, "workspace must be 16-byte aligned");

    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);

    // One query per sequence: score keys with a top-bit histogram, then one select per sequence.
    const bool p_ok = P == 32 || P == 64 || P == 128 || P == 256;
    if (T == 1 && p_ok && sgqa::decode_topk_supported(plan.max_cand, dims->topk_blocks) &&
        workspace_bytes >= sgqa::decode_topk_workspace(nseq, plan.max_cand)) {
        sgqa::DecodeTopkArgs da{};
        da.qp = qp;
        da.qp_seq_stride = qp_seq_stride;
        da.kb = kb;
        da.kb_seq_stride = kb_seq_stride;
        for (int s = 0; s < nseq; ++s)
            da.pos.v[s] = q_start[s];
        da.nseq = nseq;
        da.P = P;
        da.B = dims->block_size;
        da.k = dims->topk_blocks;
        da.keys = static_cast<uint32_t *>(workspace);
        da.keys_ld = sgqa::decode_keys_ld(plan.max_cand);
        da.umax = da.keys + (size_t)nseq * da.keys_ld;
        da.units_ld = sgqa::decode_units_ld(plan.max_cand);
        da.idx = idx;
        da.sel_scores = sel_scores;
        return hip_status(sgqa::launch_decode_topk(da, hs), "decode top-k launch");
    }

    // Rows of at most 131072 candidates: scores are filtered against a sampled threshold as
    // they are computed, so no score matrix is stored (k_fused_*).
    const int k = dims->topk_blocks;
    if (plan.max_cand >= 1 && sgqa::fused_topk_supported(plan.max_cand, k, P)) {
        const size_t fixed = sgqa::fused_topk_fixed_bytes(plan.max_cand);
        const size_t row = sgqa::fused_topk_row_bytes(plan.max_cand) * (size_t)nseq;
        int64_t nq = workspace_bytes > fixed ? (int64_t)((workspace_bytes - fixed) / row) : 0;
        if (nq >= T)
            nq = T;
        else
            nq = nq / 64 * 64;
        if (nq > 0) {
            sgqa::FusedTopkArgs fa{};
            fa.qp = qp;
            fa.qp_seq_stride = qp_seq_stride;
            fa.kb = kb;
            fa.kb_seq_stride = kb_seq_stride;
            for (int s = 0; s < nseq; ++s)
                fa.q_start.v[s] = q_start[s];
            fa.nseq = nseq;
            fa.T = T;
            fa.P = P;
            fa.B = dims->block_size;
            fa.k = k;
            sgqa::fused_topk_geometry(plan.max_cand, fa.ns, fa.cap);
            fa.fb_ld = round_up(plan.max_cand, 64);
            char *w = static_cast<char *>(workspace);
            fa.queue_ctr = reinterpret_cast<uint32_t *>(w);
            fa.fb_scores = reinterpret_cast<float *>(w + 256);
            char *rows0 = w + fixed;
            const int64_t nrows = nq * nseq;
            fa.cand = reinterpret_cast<uint2 *>(rows0);
            fa.samp = reinterpret_cast<uint32_t *>(rows0 + (size_t)nrows * fa.cap * 8);
            fa.thr = fa.samp + (size_t)nrows * fa.ns;
            fa.cnt = fa.thr + nrows;
            fa.queue = fa.cnt + nrows;
            fa.idx = idx;
            fa.sel_scores = sel_scores;
            for (int32_t t0 = 0; t0 < T; t0 += (int32_t)nq) {
                const int32_t n = (T - t0) < nq ? (T - t0) : (int32_t)nq;
                int64_t max_pos = 0;
                for (int s = 0; s < nseq; ++s)
                    max_pos = q_start[s] + t0 + n - 1 > max_pos ? q_start[s] + t0 + n - 1 : max_pos;
                fa.t0 = t0;
                fa.nq = n;
                fa.max_cand = max_pos / dims->block_size;
                if (fa.max_cand < 1)
                    fa.max_cand = 1;
                hipError_t e = sgqa::launch_fused_topk(fa, hs);
                if (e != hipSuccess)
                    return hip_status(e, "fused top-k launch");
            }
            return ok();
        }
    }

    if (plan.nq <= 0)
        return fail(SGQA_ERR_WORKSPACE,
                    "workspace of %zu bytes cannot hold one pass (need >= %lld bytes)",
                    workspace_bytes, (long long)(plan.ld * 4 * nseq * (T < 64 ? T : 64)));
    sgqa::ScoreArgs sa{};
    sa.qp = qp;
    sa.qp_seq_stride = qp_seq_stride;
    sa.kb = kb;
    sa.kb_seq_stride = kb_seq_stride;
    sa.nseq = nseq;
    sa.P = P;
    sa.B = dims->block_size;
    sa.ws = static_cast<float *>(workspace);
    sa.ld = plan.ld;
    sgqa::SelectArgs se{};
    se.ws = sa.ws;
    se.ld = plan.ld;
    se.nseq = nseq;
    se.T = T;
    se.B = dims->block_size;
    se.k = dims->topk_blocks;
    se.idx = idx;
    se.sel_scores = sel_scores;
    for (int s = 0; s < nseq; ++s)
        sa.q_start.v[s] = se.q_start.v[s] = q_start[s];
    for (int32_t t0 = 0; t0 < T; t0 += plan.nq) {
        const int32_t nq = (T - t0) < plan.nq ? (T - t0) : plan.nq;
        int64_t max_pos = 0;
        for (int s = 0; s < nseq; ++s)
            max_pos = q_start[s] + t0 + nq - 1 > max_pos ? q_start[s] + t0 + nq - 1 : max_pos;
        sa.t0 = se.t0 = t0;
        sa.nq = se.nq = nq;
        sa.max_cand = se.max_cand = max_pos / dims->block_size;
        hipError_t e = sgqa::launch_scores(sa, hs);
        if (e != hipSuccess)
            return hip_status(e, "indexer scores launch");
        e = sgqa::launch_select(se, hs);
        if (e != hipSuccess)
            return hip_status(e, "top-k select launch");
    }
    return ok();
}

sgqa_status sgqa_sparse_attn_prefill(const sgqa_dims *dims, const sgqa_bf16 *q,
                                     const sgqa_bf16 *k_cache, const sgqa_bf16 *v_cache,
                                     const sgqa_bf16 *gate, const int32_t *idx, int64_t q_start,
                                     int32_t T, int64_t L, float softmax_scale, sgqa_bf16 *out,
                                     float *lse, void *workspace, size_t workspace_bytes,
                                     void *stream)
{
    sgqa_status st = check_dims(dims, true, false);
    if (st != SGQA_OK)
        return st;
    if (T < 0 || q_start < 0 || L < 0)
        return fail(SGQA_ERR_SHAPE, "T, q_start and L must be non-negative");
    if (q_start + T > L)
        return fail(SGQA_ERR_SHAPE, "q_start + T = %lld exceeds L = %lld", (long long)(q_start + T),
                    (long long)L);
    if (!std::isfinite(softmax_scale))
        return fail(SGQA_ERR_SHAPE, "softmax_scale must be finite");
    if ((st = check_rows(T, "query rows")) != SGQA_OK)
        return st;
    if (T == 0)
        return ok();
    if (!q || !k_cache || !v_cache || !gate || !idx || !out)
        return fail(SGQA_ERR_NULL, "q, k_cache, v_cache, gate, idx and out must be non-NULL");
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 8) ||
        !aligned(idx, 4) || !aligned(lse, 4) || !aligned(gate, 2))
        return fail(SGQA_ERR_SHAPE, "q, k_cache, v_cache must be 16-byte and out 8-byte aligned");
    sgqa::AttnArgs a{};
    a.q = q;
    a.kc = k_cache;
    a.vc = v_cache;
    a.gate = gate;
    a.idx = idx;
    a.q_start = q_start;
    a.rows = T;
    a.Hq = dims->num_q_heads;
    a.Hkv = dims->num_kv_heads;
    a.d = dims->head_dim;
    a.B = dims->block_size;
    a.k = dims->topk_blocks;
    a.scale_log2 = softmax_scale * 1.4426950408889634f;
    a.out = out;
    a.lse = lse;
    a.slice_blocks = 0;
    const size_t row_state = sgqa_workspace_bytes(SGQA_OP_ATTN_PREFILL, dims, 1, 1, L);
    if (workspace) {
        if (!aligned(workspace, 16))
            return fail(SGQA_ERR_SHAPE, "workspace must be 16-byte aligned");
        if (workspace_bytes < row_state)
            return fail(SGQA_ERR_WORKSPACE, "prefill workspace needs >= %zu bytes, got %zu",
                        row_state, workspace_bytes);
        // With a workspace, rows whose histories span at most 16 resident ranges are attended by
        // the resident prefill (one launch; each XCD's waves take a batch of rows through the
        // ranges together, so the L2 holds one range at a time, and keep their state in
        // registers: 111 against 121 ms for the 128K prefill), the other rows by the sliced
        // launches.
        // History slices of W = kPrefillSliceHalfK * k / 2 blocks: each launch's rows gather from
        // one such range of the cache, which each XCD's L2 holds for its KV group, while every
        // slice boundary a row crosses parks ~13 KB of state per group.  Short histories gain
        // nothing and stay in one pass (row by row: the kernel attends rows with c < 2k in one
        // pass even in a sliced launch), and so do histories longer than 16 ranges (chunked
        // prefill at 1M tokens: ~4 entries per range, 13.9 ms unsliced against 14.0/14.5/15.2 ms
        // with 4/8/16 ranges of the row's own length).
        const int64_t max_cand = (q_start + T - 1) / dims->block_size;
        const int64_t W = (kPrefillSliceHalfK * dims->topk_blocks + 1) / 2;
        a.slice_blocks = max_cand >= 2 * (int64_t)dims->topk_blocks ? W : 0;
        a.long_slices = kPrefillLongSlices;
        // the resident prefill (one launch, the state in registers across the ranges) takes
        // the rows whose histories span at most 16 of its ranges
        a.resident_blocks = (kPrefillResidentHalfK * dims->topk_blocks + 1) / 2;
        a.state = static_cast<float *>(workspace);
        a.state_bytes = (int64_t)workspace_bytes;
        a.state_stride = sgqa::prefill_state_stride(a.d);
    }
    return hip_status(sgqa::launch_attn_prefill(a, reinterpret_cast<hipStream_t>(stream)),
                      "sparse_attn_prefill launch");
}

sgqa_status sgqa_swa_prefill(const sgqa_dims *dims, const sgqa_bf16 *q, const sgqa_bf16 *k_cache,
                             const sgqa_bf16 *v_cache, const sgqa_bf16 *gate, int64_t q_start,
                             int32_t T, int64_t L, int64_t window, float softmax_scale,
                             sgqa_bf16 *out, float *lse, void *stream)
{
    sgqa_status st = check_heads(dims);
    if (st != SGQA_OK)
        return st;
    if (T < 0 || q_start < 0 || L < 0)
        return fail(SGQA_ERR_SHAPE, "T, q_start and L must be non-negative");
    if (q_start + T > L)
        return fail(SGQA_ERR_SHAPE, "q_start + T = %lld exceeds L = %lld", (long long)(q_start + T),
                    (long long)L);
    if (window < 1)
        return fail(SGQA_ERR_SHAPE, "window %lld must be >= 1", (long long)window);
    if (!std::isfinite(softmax_scale))
        return fail(SGQA_ERR_SHAPE, "softmax_scale must be finite");
    if ((st = check_rows(T, "query rows")) != SGQA_OK)
        return st;
    if (T == 0)
        return ok();
    if (!q || !k_cache || !v_cache || !gate || !out)
        return fail(SGQA_ERR_NULL, "q, k_cache, v_cache, gate and out must be non-NULL");
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 8) ||
        !aligned(lse, 4) || !aligned(gate, 2))
        return fail(SGQA_ERR_SHAPE, "q, k_cache, v_cache must be 16-byte and out 8-byte aligned");
    sgqa::AttnArgs a{};
    a.q = q;
    a.kc = k_cache;
    a.vc = v_cache;
    a.gate = gate;
    a.q_start = q_start;
    a.rows = T;
    a.Hq = dims->num_q_heads;
    a.Hkv = dims->num_kv_heads;
    a.d = dims->head_dim;
    a.window = window;
    a.scale_log2 = softmax_scale * 1.4426950408889634f;
    a.out = out;
    a.lse = lse;
    return hip_status(sgqa::launch_swa(a, reinterpret_cast<hipStream_t>(stream)),
                      "swa_prefill launch");
}

// Validation and launch shared by sgqa_sparse_attn_decode (caller's workspace, partial
// states laid out by split) and sgqa_sparse_attn_decode_noalloc (the library's fixed scratch,
// partial states laid out by workgroup part, which is all the kernels write).
static sgqa_status attn_decode_impl(const sgqa_dims *dims, const sgqa_bf16 *q,
                                    const sgqa_bf16 *k_cache, const sgqa_bf16 *v_cache,
                                    int64_t cache_seq_stride, const sgqa_bf16 *gate,
                                    const int32_t *idx, const int64_t *cache_lens, int32_t nseq,
                                    float softmax_scale, sgqa_bf16 *out, float *lse,
                                    void *workspace, size_t workspace_bytes, bool fixed_scratch,
                                    void *stream)
{
    sgqa_status st = check_dims(dims, true, false);
    if (st != SGQA_OK)
        return st;
    if (nseq < 0)
        return fail(SGQA_ERR_SHAPE, "nseq %d is negative", nseq);
    if (nseq > sgqa::kMaxSeq)
        return fail(SGQA_ERR_UNSUPPORTED, "nseq %d exceeds %d", nseq, sgqa::kMaxSeq);
    if (!std::isfinite(softmax_scale))
        return fail(SGQA_ERR_SHAPE, "softmax_scale must be finite");
    if (nseq == 0)
        return ok();
    if (!q || !k_cache || !v_cache || !gate || !idx || !out || !cache_lens)
        return fail(SGQA_ERR_NULL, "q, caches, gate, idx, cache_lens and out must be non-NULL");
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 2) ||
        !aligned(idx, 4) || !aligned(lse, 4) || !aligned(gate, 2))
        return fail(SGQA_ERR_SHAPE, "q and caches must be 16-byte aligned");
    const int64_t row = (int64_t)dims->num_kv_heads * dims->head_dim;
    int64_t max_len = 0;
    for (int s = 0; s < nseq; ++s) {
        if (cache_lens[s] < 1)
            return fail(SGQA_ERR_SHAPE, "cache_lens[%d] = %lld must be >= 1", s,
                        (long long)cache_lens[s]);
        max_len = cache_lens[s] > max_len ? cache_lens[s] : max_len;
    }
    if (nseq > 1 && (cache_seq_stride < max_len * row || cache_seq_stride % 8 != 0))
        return fail(SGQA_ERR_SHAPE, "cache_seq_stride %lld must be >= %lld and a multiple of 8",
                    (long long)cache_seq_stride, (long long)(max_len * row));
    sgqa::AttnArgs a{};
    sgqa::decode_split_plan(dims->topk_blocks, dims->block_size, a.nsplit, a.entries_per_split);
    size_t slots = 0;
    if (fixed_scratch) {
        slots = (size_t)nseq * sgqa::decode_parts(a.nsplit) * dims->num_q_heads;
        const size_t need = slots * ((size_t)dims->head_dim + 3) * sizeof(float);
        if (need > sgqa::kScratchBytes)
            return fail(SGQA_ERR_UNSUPPORTED,
                        "decode without allocation needs %zu bytes of partial states, more than "
                        "the library's fixed %zu-byte scratch (fewer sequences per call)",
                        need, sgqa::kScratchBytes);
        size_t have = 0;
        hipError_t e = sgqa::scratch_region(&workspace, &have);
        if (e != hipSuccess)
            return hip_status(e, "scratch address lookup");
    } else {
        slots = (size_t)nseq * a.nsplit * dims->num_q_heads;
        const size_t need = sgqa_workspace_bytes(SGQA_OP_ATTN_DECODE, dims, nseq, 1, max_len);
        if (!workspace || workspace_bytes < need)
            return fail(SGQA_ERR_WORKSPACE, "decode workspace needs %zu bytes, got %zu", need,
                        workspace ? workspace_bytes : (size_t)0);
        if (!aligned(workspace, 16))
            return fail(SGQA_ERR_SHAPE, "workspace must be 16-byte aligned");
    }
    a.q = q;
    a.kc = k_cache;
    a.vc = v_cache;
    a.cache_seq_stride = cache_seq_stride;
    a.gate = gate;
    a.idx = idx;
    for (int s = 0; s < nseq; ++s)
        a.qpos.v[s] = cache_lens[s] - 1;
    a.rows = nseq;
    a.Hq = dims->num_q_heads;
    a.Hkv = dims->num_kv_heads;
    a.d = dims->head_dim;
    a.B = dims->block_size;
    a.k = dims->topk_blocks;
    a.scale_log2 = softmax_scale * 1.4426950408889634f;
    a.out = out;
    a.lse = lse;
    a.part_o = static_cast<float *>(workspace);
    a.part_ml = a.part_o + slots * a.d;
    return hip_status(sgqa::launch_attn_decode(a, reinterpret_cast<hipStream_t>(stream)),
                      "sparse_attn_decode launch");
}

sgqa_status sgqa_sparse_attn_decode(const sgqa_dims *dims, const sgqa_bf16 *q,
                                    const sgqa_bf16 *k_cache, const sgqa_bf16 *v_cache,
                                    int64_t cache_seq_stride, const sgqa_bf16 *gate,
                                    const int32_t *idx, const int64_t *cache_lens, int32_t nseq,
                                    float softmax_scale, sgqa_bf16 *out, float *lse,
                                    void *workspace, size_t workspace_bytes, void *stream)
{
    return attn_decode_impl(dims, q, k_cache, v_cache, cache_seq_stride, gate, idx, cache_lens,
                            nseq, softmax_scale, out, lse, workspace, workspace_bytes, false,
                            stream);
}

sgqa_status sgqa_sparse_attn_decode_noalloc(const sgqa_dims *dims, const sgqa_bf16 *q,
                                            const sgqa_bf16 *k_cache, const sgqa_bf16 *v_cache,
                                            int64_t cache_seq_stride, const sgqa_bf16 *gate,
                                            const int32_t *idx, const int64_t *cache_lens,
                                            int32_t nseq, float softmax_scale, sgqa_bf16 *out,
                                            float *lse, void *stream)
{
    return attn_decode_impl(dims, q, k_cache, v_cache, cache_seq_stride, gate, idx, cache_lens,
                            nseq, softmax_scale, out, lse, nullptr, 0, true, stream);
}

} // extern "C"

// ---------------------------------------------------------------------------------- FP8 decode
sgqa_status sgqa_quantize_fp8(const sgqa_bf16 *x, int64_t rows, int32_t cols, uint8_t *codes,
                              float *scales, void *stream)
{
    if (rows < 0 || cols <= 0 || cols > 4096)
        return fail(rows < 0 || cols <= 0 ? SGQA_ERR_SHAPE : SGQA_ERR_UNSUPPORTED,
                    "rows %lld must be >= 0 and cols %d in [1, 4096]", (long long)rows, cols);
    if (rows == 0)
        return ok();
    if (!x || !codes || !scales)
        return fail(SGQA_ERR_NULL, "x, codes and scales must be non-NULL");
    if (!aligned(x, 2) || !aligned(scales, 4))
        return fail(SGQA_ERR_SHAPE, "x must be 2-byte and scales 4-byte aligned");
    return hip_status(sgqa::launch_quantize_rows(x, rows, cols, codes, scales,
                                                 reinterpret_cast<hipStream_t>(stream)),
                      "quantize_fp8 launch");
}

sgqa_status sgqa_indexer_topk_fp8(const sgqa_dims *dims, const sgqa_bf16 *qp,
                                  int64_t qp_seq_stride, const uint8_t *kb_codes,
                                  const float *kb_scales, int64_t kb_seq_stride,
                                  const int64_t *q_pos, int32_t nseq, int32_t *idx,
                                  float *sel_scores, void *workspace, size_t workspace_bytes,
                                  void *stream)
{
    sgqa_status st = check_dims(dims, false, true);
    if (st != SGQA_OK)
        return st;
    const int P = dims->proxy_dim;
    if (P != 64 && P != 128 && P != 256 && P != 512)
        return fail(SGQA_ERR_UNSUPPORTED, "FP8 index needs proxy_dim in {64,128,256,512}, got %d", P);
    if (nseq < 0)
        return fail(SGQA_ERR_SHAPE, "nseq %d is negative", nseq);
    if (nseq > sgqa::kMaxSeq)
        return fail(SGQA_ERR_UNSUPPORTED, "nseq %d exceeds %d", nseq, sgqa::kMaxSeq);
    if (nseq == 0)
        return ok();
    if (!qp || !kb_codes || !kb_scales || !q_pos || !idx)
        return fail(SGQA_ERR_NULL, "qp, kb_codes, kb_scales, q_pos and idx must be non-NULL");
    if (!aligned(qp, 16) || !aligned(kb_codes, 16) || !aligned(kb_scales, 4) ||
        !aligned(idx, 4) || !aligned(sel_scores, 4))
        return fail(SGQA_ERR_SHAPE, "qp and kb_codes must be 16-byte aligned");
    int64_t max_pos = 0;
    for (int s = 0; s < nseq; ++s) {
        if (q_pos[s] < 0)
            return fail(SGQA_ERR_SHAPE, "q_pos[%d] = %lld is negative", s, (long long)q_pos[s]);
        max_pos = q_pos[s] > max_pos ? q_pos[s] : max_pos;
    }
    const int64_t max_cand = max_pos / dims->block_size;
    if (nseq > 1 && (qp_seq_stride < P || qp_seq_stride % 8 != 0))
        return fail(SGQA_ERR_SHAPE, "qp_seq_stride %lld must be >= P and a multiple of 8",
                    (long long)qp_seq_stride);
    if (nseq > 1 && kb_seq_stride < max_cand)
        return fail(SGQA_ERR_SHAPE, "kb_seq_stride %lld must cover %lld blocks",
                    (long long)kb_seq_stride, (long long)max_cand);
    if (max_cand > 0 && !sgqa::decode_topk_supported(max_cand, dims->topk_blocks))
        return fail(SGQA_ERR_UNSUPPORTED, "FP8 decode top-k needs 2 <= k and <= %lld candidate blocks",
                    (long long)sgqa::kDecodeMaxCand);
    const size_t need = max_cand > 0 ? sgqa::decode_topk_workspace(nseq, max_cand) : 0;
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(SGQA_ERR_WORKSPACE, "FP8 decode top-k needs %zu bytes of workspace, got %zu",
                    need, workspace ? workspace_bytes : (size_t)0);
    if (workspace && !aligned(workspace, 16))
        return fail(SGQA_ERR_SHAPE, "workspace must be 16-byte aligned");
    sgqa::DecodeTopkArgs da{};
    da.qp = qp;
    da.qp_seq_stride = qp_seq_stride;
    da.kbq = kb_codes;
    da.kbs = kb_scales;
    da.kbs_seq_stride = kb_seq_stride;
    for (int s = 0; s < nseq; ++s)
        da.pos.v[s] = q_pos[s];
    da.nseq = nseq;
    da.P = P;
    da.B = dims->block_size;
    da.k = dims->topk_blocks;
    const int64_t mc = max_cand > 0 ? max_cand : 1;
    da.keys = static_cast<uint32_t *>(workspace);
    da.keys_ld = sgqa::decode_keys_ld(mc);
    da.umax = da.keys ? da.keys + (size_t)nseq * da.keys_ld : nullptr;
    da.units_ld = sgqa::decode_units_ld(mc);
    da.idx = idx;
    da.sel_scores = sel_scores;
    return hip_status(sgqa::launch_decode_topk(da, reinterpret_cast<hipStream_t>(stream)),
                      "FP8 decode top-k launch");
}

sgqa_status sgqa_sparse_attn_decode_fp8(const sgqa_dims *dims, const sgqa_bf16 *q,
                                        const uint8_t *k_codes, const uint8_t *v_codes,
                                        const float *k_scales, const float *v_scales,
                                        int64_t cache_seq_stride, const sgqa_bf16 *gate,
                                        const int32_t *idx, const int64_t *cache_lens,
                                        int32_t nseq, float softmax_scale, sgqa_bf16 *out,
                                        float *lse, void *workspace, size_t workspace_bytes,
                                        void *stream)
{
    sgqa_status st = check_dims(dims, true, false);
    if (st != SGQA_OK)
        return st;
    if (nseq < 0)
        return fail(SGQA_ERR_SHAPE, "nseq %d is negative", nseq);
    if (nseq > sgqa::kMaxSeq)
        return fail(SGQA_ERR_UNSUPPORTED, "nseq %d exceeds %d", nseq, sgqa::kMaxSeq);
    if (!std::isfinite(softmax_scale))
        return fail(SGQA_ERR_SHAPE, "softmax_scale must be finite");
    if (nseq == 0)
        return ok();
    if (!q || !k_codes || !v_codes || !k_scales || !v_scales || !gate || !idx || !out ||
        !cache_lens)
        return fail(SGQA_ERR_NULL, "q, codes, scales, gate, idx, cache_lens and out must be non-NULL");
    if (!aligned(q, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) ||
        !aligned(k_scales, 4) || !aligned(v_scales, 4) || !aligned(out, 2) || !aligned(idx, 4) ||
        !aligned(lse, 4) || !aligned(gate, 2))
        return fail(SGQA_ERR_SHAPE, "q and code arrays must be 16-byte aligned");
    int64_t max_len = 0;
    for (int s = 0; s < nseq; ++s) {
        if (cache_lens[s] < 1)
            return fail(SGQA_ERR_SHAPE, "cache_lens[%d] = %lld must be >= 1", s,
                        (long long)cache_lens[s]);
        max_len = cache_lens[s] > max_len ? cache_lens[s] : max_len;
    }
    if (nseq > 1 && cache_seq_stride < max_len)
        return fail(SGQA_ERR_SHAPE, "cache_seq_stride %lld (tokens) must be >= %lld",
                    (long long)cache_seq_stride, (long long)max_len);
    const size_t need = sgqa_workspace_bytes(SGQA_OP_ATTN_DECODE, dims, nseq, 1, max_len);
    if (!workspace || workspace_bytes < need)
        return fail(SGQA_ERR_WORKSPACE, "decode workspace needs %zu bytes, got %zu", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 16))
        return fail(SGQA_ERR_SHAPE, "workspace must be 16-byte aligned");
    const int64_t row = (int64_t)dims->num_kv_heads * dims->head_dim;
    sgqa::AttnArgs a{};
    a.q = q;
    a.kq = k_codes;
    a.vq = v_codes;
    a.ksc = k_scales;
    a.vsc = v_scales;
    a.scale_seq_stride = cache_seq_stride;
    a.cache_seq_stride = cache_seq_stride * row;  // elements (= bytes) of codes
    a.gate = gate;
    a.idx = idx;
    for (int s = 0; s < nseq; ++s)
        a.qpos.v[s] = cache_lens[s] - 1;
    a.rows = nseq;
    a.Hq = dims->num_q_heads;
    a.Hkv = dims->num_kv_heads;
    a.d = dims->head_dim;
    a.B = dims->block_size;
    a.k = dims->topk_blocks;
    a.scale_log2 = softmax_scale * 1.4426950408889634f;
    a.out = out;
    a.lse = lse;
    sgqa::decode_split_plan(a.k, a.B, a.nsplit, a.entries_per_split);
    const size_t slots = (size_t)nseq * a.nsplit * a.Hq;
    a.part_o = static_cast<float *>(workspace);
    a.part_ml = a.part_o + slots * a.d;
    return hip_status(sgqa::launch_attn_decode(a, reinterpret_cast<hipStream_t>(stream)),
                      "FP8 sparse_attn_decode launch");
}

// ------------------------------------------------------------------------------ backward
sgqa_status sgqa_sparse_attn_backward(const sgqa_dims *dims, const sgqa_bf16 *q,
                                      const sgqa_bf16 *k_cache, const sgqa_bf16 *v_cache,
                                      const sgqa_bf16 *gate, const int32_t *idx, int64_t q_start,
                                      int32_t T, int64_t L, float softmax_scale, const float *lse,
                                      const sgqa_bf16 *dout, const sgqa_bf16 *out, float *dq,
                                      float *dk, float *dv, float *dgate, void *workspace,
                                      size_t workspace_bytes, int64_t dkdv_row_slice,
                                      void *stream)
{
    sgqa_status st = check_dims(dims, true, false);
    if (st != SGQA_OK)
        return st;
    if (T < 0 || q_start < 0 || L < 0)
        return fail(SGQA_ERR_SHAPE, "T %d, q_start %lld and L %lld must be non-negative", T,
                    (long long)q_start, (long long)L);
    if (q_start + T > L)
        return fail(SGQA_ERR_SHAPE, "queries [q_start, q_start+T) must lie inside the cache of %lld",
                    (long long)L);
    if (!std::isfinite(softmax_scale))
        return fail(SGQA_ERR_SHAPE, "softmax_scale must be finite");
    if (dkdv_row_slice < 0 || dkdv_row_slice % 32 != 0)
        return fail(SGQA_ERR_SHAPE, "dkdv_row_slice %lld must be 0 or a positive multiple of 32",
                    (long long)dkdv_row_slice);
    if ((st = check_rows(T, "query rows")) != SGQA_OK ||
        (st = check_rows(ceil_div(L, dims->block_size), "cache blocks")) != SGQA_OK)
        return st;
    if (T == 0 || L == 0)
        return ok();
    if (!q || !k_cache || !v_cache || !gate || !idx || !lse || !dout || !dq || !dk || !dv ||
        !dgate)
        return fail(SGQA_ERR_NULL, "every tensor argument must be non-NULL");
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(dq, 16) ||
        !aligned(dout, 2) || !aligned(out, 2) || !aligned(gate, 2) || !aligned(idx, 4) ||
        !aligned(lse, 4) || !aligned(dk, 4) || !aligned(dv, 4) || !aligned(dgate, 4))
        return fail(SGQA_ERR_SHAPE, "q, caches and dq must be 16-byte aligned");
    const size_t need = sgqa_workspace_bytes(SGQA_OP_ATTN_BACKWARD, dims, 1, T, L);
    if (!workspace || workspace_bytes < need)
        return fail(SGQA_ERR_WORKSPACE, "backward workspace needs %zu bytes, got %zu", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 256))
        return fail(SGQA_ERR_SHAPE, "workspace must be 256-byte aligned");
    sgqa::BwdArgs a{};
    a.q = q;
    a.kc = k_cache;
    a.vc = v_cache;
    a.gate = gate;
    a.dout = dout;
    a.out = out;
    a.lse = lse;
    a.idx = idx;
    a.q_start = q_start;
    a.rows = T;
    a.L = L;
    a.Hq = dims->num_q_heads;
    a.Hkv = dims->num_kv_heads;
    a.d = dims->head_dim;
    a.B = dims->block_size;
    a.k = dims->topk_blocks;
    a.scale = softmax_scale;
    a.scale_log2 = softmax_scale * 1.4426950408889634f;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.dgate = dgate;
    a.row_slice = dkdv_row_slice;
    a.nblk = ceil_div(L, dims->block_size);
    a.bits_ld = ((((int64_t)T + 31) / 32) + 3) / 4 * 4;
    char *w = static_cast<char *>(workspace);
    const size_t da_bytes = ((size_t)T * a.Hq * a.d * 2 + 255) / 256 * 256;
    const size_t ds_bytes = ((size_t)T * a.Hq * 4 + 255) / 256 * 256;
    const size_t bits_bytes = ((size_t)a.nblk * a.bits_ld * 4 + 255) / 256 * 256;
    a.da = reinterpret_cast<uint16_t *>(w);
    a.dsum = reinterpret_cast<float *>(w + da_bytes);
    a.bits = reinterpret_cast<uint32_t *>(w + da_bytes + ds_bytes);
    a.prog = reinterpret_cast<uint32_t *>(w + da_bytes + ds_bytes + bits_bytes);
    a.res_w = (kBwdResidentHalfK * (int64_t)a.k + 1) / 2;
    return hip_status(sgqa::launch_attn_backward(a, reinterpret_cast<hipStream_t>(stream)),
                      "sparse_attn_backward launch");
}
