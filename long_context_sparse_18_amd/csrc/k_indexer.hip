// k_indexer.hip -- indexer scores (bf16 MFMA) and causal top-k selection (gfx950).
//
// phantomic12 "Step 5 Preview" catalogue entry, ATTENTION SPLIT part:
// sparse_config turns on an indexer with topk 512 and proxy_dim 256 for the
// full-attention layers.  ai.info "Sparse GQA targets million-token context":
// it selects relevant historical blocks of 8 tokens.  ai4snews Interpretation
// para. 2: the block compression cuts indexer and top-k selection cost 8x.
//
// Scores: one workgroup computes a 64-query x 64-block tile of qp . kb^T with
// v_mfma_f32_16x16x32_bf16.  The kb tile is staged once in LDS and read by all
// four waves; each wave owns 16 queries.  Tiles entirely past the causal limit
// exit at once, and only complete past blocks (j < t/B) are written.
//
// Selection: one workgroup per query row runs an exact radix select on
// order-preserving u32 keys (digits of 12, 12 and 8 bits, histograms in LDS),
// then emits the chosen block ids in ascending order with a workgroup scan.
// Ties at the threshold go to the lowest block indices, so the result is the
// unique set "k-1 best by (score desc, index asc)" plus the own block.
#include <hip/hip_runtime.h>

#include "sgqa_device.hpp"
#include "sgqa_launch.hpp"

namespace sgqa {

constexpr int kTileQ = 64;
constexpr int kTileB = 64;

__global__ __launch_bounds__(256) void k_scores(ScoreArgs a)
{
    extern __shared__ __align__(16) uint16_t kb_tile[];  // [kTileB][P + 8]
    const int s = blockIdx.z;
    const int i0 = blockIdx.y * kTileQ;
    const int64_t j0 = (int64_t)blockIdx.x * kTileB;
    const int64_t pos0 = a.q_start.v[s] + a.t0;
    const int i_last = min(i0 + kTileQ, a.nq) - 1;
    const int64_t c_last = (pos0 + i_last) / a.B;
    if (j0 >= c_last)
        return;

    const int P = a.P;
    const int ldt = P + 8;
    const int tid = threadIdx.x;
    const uint16_t *kb = a.kb + (int64_t)s * a.kb_seq_stride;

    // Stage kb rows j0 .. j0+63 (rows at or past c_last are zero).
    const int chunks = P >> 3;
    for (int e = tid; e < kTileB * chunks; e += 256) {
        const int r = e / chunks, cc = e - r * chunks;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (j0 + r < c_last)
            v = load16(kb + (j0 + r) * P + cc * 8);
        *reinterpret_cast<u32x4 *>(kb_tile + r * ldt + cc * 8) = v;
    }
    __syncthreads();

    const int wave = tid >> 6, lane = tid & 63;
    const int col = lane & 15, q4 = lane >> 4;
    const int qrow = i0 + wave * 16 + col;  // A-operand row of this lane
    if (i0 + wave * 16 >= a.nq)
        return;
    const uint16_t *qp = a.qp + (int64_t)s * a.qp_seq_stride + (int64_t)(a.t0 + qrow) * P;

    f32x4 acc[4];
#pragma unroll
    for (int n = 0; n < 4; ++n)
        acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kk = 0; kk < P; kk += 32) {
        u32x4 av = {0u, 0u, 0u, 0u};
        if (qrow < a.nq)
            av = load16(qp + kk + q4 * 8);
        const bf16x8 af = as_bf16x8(av);
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const u32x4 bv =
                *reinterpret_cast<const u32x4 *>(kb_tile + (n * 16 + col) * ldt + kk + q4 * 8);
            acc[n] = mfma_16x16x32(af, as_bf16x8(bv), acc[n]);
        }
    }

    // Lane holds D[row 4*q4 + r][block col] of each 16x16 sub-tile.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int i = i0 + wave * 16 + q4 * 4 + r;
        if (i >= a.nq)
            continue;
        const int64_t c = (pos0 + i) / a.B;
        float *dst = a.ws + ((int64_t)s * a.nq + i) * a.ld;
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const int64_t j = j0 + n * 16 + col;
            if (j < c)
                dst[j] = acc[n][r];
        }
    }
}

hipError_t launch_scores(const ScoreArgs &a, hipStream_t stream)
{
    if (a.max_cand <= 0)
        return hipSuccess;
    const dim3 grid((unsigned)((a.max_cand + kTileB - 1) / kTileB),
                    (unsigned)((a.nq + kTileQ - 1) / kTileQ), (unsigned)a.nseq);
    const size_t lds = (size_t)kTileB * (a.P + 8) * sizeof(uint16_t);
    hipLaunchKernelGGL(k_scores, grid, dim3(256), lds, stream, a);
    return hipGetLastError();
}

// --------------------------------------------------------------------------------------------
template <int NT>
__global__ __launch_bounds__(NT) void k_select(SelectArgs a)
{
    constexpr int kItems = 4;
    __shared__ uint32_t hist[4096];
    __shared__ int scan_buf[NT / 64];
    __shared__ uint32_t sh_digit;
    __shared__ int sh_need;

    const int tid = threadIdx.x;
    const int row = blockIdx.x;
    const int s = row / a.nq;
    const int i = row - s * a.nq;
    const int64_t t = a.q_start.v[s] + a.t0 + i;
    const int64_t c = t / a.B;
    const int k = a.k;
    const float *srow = a.ws + (int64_t)row * a.ld;
    int32_t *out = a.idx + ((int64_t)s * a.T + a.t0 + i) * k;
    float *osc = a.sel_scores ? a.sel_scores + ((int64_t)s * a.T + a.t0 + i) * k : nullptr;

    if (c <= (int64_t)k - 1) {
        // Every past block and the own block are kept.
        for (int e = tid; e < k; e += NT) {
            const bool live = e <= c;
            out[e] = live ? e : -1;
            if (osc)
                osc[e] = (e < c) ? srow[e] : (e == c ? __builtin_inff() : -__builtin_inff());
        }
        return;
    }

    if (k == 1) {
        // Only the own block is kept.
        if (tid == 0) {
            out[0] = (int32_t)c;
            if (osc)
                osc[0] = __builtin_inff();
        }
        return;
    }

    // ---- radix select of the (k-1)-th largest key
    int need = k - 1;
    uint32_t prefix = 0, pmask = 0;
    const int cn = (int)c;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 20 : (pass == 1 ? 8 : 0);
        const int nb = pass == 2 ? 256 : 4096;
        for (int b = tid; b < nb; b += NT)
            hist[b] = 0;
        __syncthreads();
        for (int j = tid; j < cn; j += NT) {
            const uint32_t key = score_key(srow[j]);
            if ((key & pmask) == prefix)
                atomicAdd(&hist[(key >> shift) & (nb - 1)], 1u);
        }
        __syncthreads();
        const int per = nb >= NT ? nb / NT : 1;
        const int lo = tid * per;
        int local = 0;
        if (lo < nb)
            for (int b = lo; b < lo + per; ++b)
                local += (int)hist[b];
        int total;
        const int below = block_exclusive_scan<NT>(local, scan_buf, total);
        const int above = total - below - local;
        if (lo < nb && above < need && need <= above + local) {
            int acc = above;
            for (int b = lo + per - 1; b >= lo; --b) {
                const int h = (int)hist[b];
                if (acc + h >= need) {
                    sh_digit = (uint32_t)b;
                    sh_need = need - acc;
                    break;
                }
                acc += h;
            }
        }
        __syncthreads();
        need = sh_need;
        prefix |= sh_digit << shift;
        pmask |= (uint32_t)(nb - 1) << shift;
        __syncthreads();
    }
    const uint32_t kth = prefix;  // exact key of the (k-1)-th largest score

    // ---- emit in ascending block order
    int run_sel = 0, run_eq = 0;
#pragma unroll 1
    for (int base = 0; base < cn; base += NT * kItems) {
        uint32_t keys[kItems];
        int n_eq = 0;
#pragma unroll
        for (int e = 0; e < kItems; ++e) {
            const int j = base + tid * kItems + e;
            keys[e] = j < cn ? score_key(srow[j]) : 0u;
            n_eq += (j < cn && keys[e] == kth) ? 1 : 0;
        }
        int eq_total;
        int eq_before = block_exclusive_scan<NT>(n_eq, scan_buf, eq_total) + run_eq;
        bool take[kItems];
        int n_take = 0;
#pragma unroll
        for (int e = 0; e < kItems; ++e) {
            const int j = base + tid * kItems + e;
            bool tk = false;
            if (j < cn) {
                if (keys[e] > kth)
                    tk = true;
                else if (keys[e] == kth) {
                    tk = eq_before < need;
                    ++eq_before;
                }
            }
            take[e] = tk;
            n_take += tk ? 1 : 0;
        }
        int sel_total;
        int pos = block_exclusive_scan<NT>(n_take, scan_buf, sel_total) + run_sel;
#pragma unroll
        for (int e = 0; e < kItems; ++e) {
            if (take[e] && pos < k - 1) {
                const int j = base + tid * kItems + e;
                out[pos] = j;
                if (osc)
                    osc[pos] = key_score(keys[e]);
                ++pos;
            }
        }
        run_eq += eq_total;
        run_sel += sel_total;
    }
    if (tid == 0) {
        out[k - 1] = (int32_t)c;
        if (osc)
            osc[k - 1] = __builtin_inff();
    }
}

hipError_t launch_select(const SelectArgs &a, hipStream_t stream)
{
    const unsigned rows = (unsigned)(a.nseq * a.nq);
    if (rows == 0)
        return hipSuccess;
    if (a.max_cand > 32768 && rows <= 256)
        hipLaunchKernelGGL(k_select<1024>, dim3(rows), dim3(1024), 0, stream, a);
    else
        hipLaunchKernelGGL(k_select<256>, dim3(rows), dim3(256), 0, stream, a);
    return hipGetLastError();
}

} // namespace sgqa
