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
// Exact radix select, shared by every selection kernel.  `key_at(j)` yields the
// order-preserving key of element j in [0, n).  Returns the key of the need-th
// largest element and how many elements equal to it are kept (the lowest positions).
struct KthKey {
    uint32_t key;
    int take_eq;
};

struct SelectShared {
    uint32_t hist[4096];
    int scan[16];
    uint32_t digit;
    int need;
};

// Radix select over the bits top..0 of keys that all share `prefix` on the bits in `pmask`.
template <int NT, typename KeyAt>
__device__ KthKey radix_select_bits(KeyAt key_at, int n, int need, SelectShared &sh, int top,
                                    uint32_t prefix, uint32_t pmask)
{
    const int tid = threadIdx.x;
#pragma unroll 1
    while (top >= 0) {
        const int width = top + 1 < 12 ? top + 1 : 12;
        const int shift = top + 1 - width;
        const int nb = 1 << width;
        for (int b = tid; b < nb; b += NT)
            sh.hist[b] = 0;
        __syncthreads();
        for (int j = tid; j < n; j += NT) {
            const uint32_t key = key_at(j);
            if ((key & pmask) == prefix)
                atomicAdd(&sh.hist[(key >> shift) & (nb - 1)], 1u);
        }
        __syncthreads();
        const int per = nb >= NT ? nb / NT : 1;
        const int lo = tid * per;
        int local = 0;
        if (lo < nb)
            for (int b = lo; b < lo + per; ++b)
                local += (int)sh.hist[b];
        int total;
        const int below = block_exclusive_scan<NT>(local, sh.scan, total);
        const int above = total - below - local;
        if (lo < nb && above < need && need <= above + local) {
            int acc = above;
            for (int b = lo + per - 1; b >= lo; --b) {
                const int h = (int)sh.hist[b];
                if (acc + h >= need) {
                    sh.digit = (uint32_t)b;
                    sh.need = need - acc;
                    break;
                }
                acc += h;
            }
        }
        __syncthreads();
        need = sh.need;
        prefix |= sh.digit << shift;
        pmask |= (uint32_t)(nb - 1) << shift;
        top = shift - 1;
        __syncthreads();
    }
    return KthKey{prefix, need};
}

template <int NT, typename KeyAt>
__device__ KthKey radix_select(KeyAt key_at, int n, int need, SelectShared &sh)
{
    return radix_select_bits<NT>(key_at, n, need, sh, 31, 0u, 0u);
}

// Ordered compaction of the selected elements: emit(pos, j, key) for every element
// with key > kth, and for the first th.take_eq elements equal to kth, in increasing j;
// positions count from 0 and stop at `limit`.
template <int NT, typename KeyAt, typename Emit>
__device__ void emit_selected(KeyAt key_at, int n, KthKey th, int limit, SelectShared &sh,
                              Emit emit)
{
    constexpr int kItems = 4;
    const int tid = threadIdx.x;
    int run_sel = 0, run_eq = 0;
#pragma unroll 1
    for (int base = 0; base < n; base += NT * kItems) {
        uint32_t keys[kItems];
        int n_eq = 0;
#pragma unroll
        for (int e = 0; e < kItems; ++e) {
            const int j = base + tid * kItems + e;
            keys[e] = j < n ? key_at(j) : 0u;
            n_eq += (j < n && keys[e] == th.key) ? 1 : 0;
        }
        int eq_total;
        int eq_before = block_exclusive_scan<NT>(n_eq, sh.scan, eq_total) + run_eq;
        bool take[kItems];
        int n_take = 0;
#pragma unroll
        for (int e = 0; e < kItems; ++e) {
            const int j = base + tid * kItems + e;
            bool tk = false;
            if (j < n) {
                if (keys[e] > th.key)
                    tk = true;
                else if (keys[e] == th.key) {
                    tk = eq_before < th.take_eq;
                    ++eq_before;
                }
            }
            take[e] = tk;
            n_take += tk ? 1 : 0;
        }
        int sel_total;
        int pos = block_exclusive_scan<NT>(n_take, sh.scan, sel_total) + run_sel;
#pragma unroll
        for (int e = 0; e < kItems; ++e) {
            if (take[e] && pos < limit) {
                emit(pos, base + tid * kItems + e, keys[e]);
                ++pos;
            }
        }
        run_eq += eq_total;
        run_sel += sel_total;
    }
}

// One workgroup per query row of a score pass (rows of any length).
template <int NT>
__global__ __launch_bounds__(NT) void k_select(SelectArgs a)
{
    __shared__ SelectShared sh;
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
            out[e] = e <= c ? e : -1;
            if (osc)
                osc[e] = (e < c) ? srow[e] : (e == c ? __builtin_inff() : -__builtin_inff());
        }
        return;
    }
    if (k > 1) {
        auto key_at = [&](int j) { return score_key(srow[j]); };
        const KthKey th = radix_select<NT>(key_at, (int)c, k - 1, sh);
        emit_selected<NT>(key_at, (int)c, th, k - 1, sh, [&](int pos, int j, uint32_t key) {
            out[pos] = j;
            if (osc)
                osc[pos] = key_score(key);
        });
    }
    if (tid == 0) {
        out[k - 1] = (int32_t)c;
        if (osc)
            osc[k - 1] = __builtin_inff();
    }
}

// --------------------------------------------------------------------------------------------
// Decode: one query per sequence against the whole index.
//  1. k_decode_keys streams kb at HBM rate (one workgroup per 1024 blocks): the MFMA A
//     operand is the query proxy broadcast to all 16 rows, so row 0 of each 16x16 result
//     holds 16 block scores; they are stored as order-preserving keys, and the largest
//     key of every "unit" of 64 consecutive blocks is stored too.
//  2. k_decode_select (one workgroup per sequence): K* = the (k-1)-th largest unit maximum
//     is an exact lower bound for the selection (the k-1 best unit maxima are themselves
//     blocks at or above K*, so the (k-1)-th best block is too), and every selected block
//     lies in a unit whose maximum is >= K*.  Only those units' keys are read; the blocks
//     at or above K* among them are selected exactly (ties to the lowest block) and written
//     in ascending order through an LDS bitmap.  If too many units qualify (heavy ties) it
//     selects exactly over all keys instead.
constexpr int kKeysPerWG = 1024;
constexpr int kUnitBlocks = 64;        // consecutive blocks per unit
constexpr int kUnitsPerWG = kKeysPerWG / kUnitBlocks;
constexpr int kMaxUnits = 8192;        // LDS words of the select (unit maxima, then bitmap)
constexpr int kUnitListCap = 4096;
constexpr int kCandCap = 2048;

template <int P>
__global__ __launch_bounds__(256) void k_decode_keys(DecodeTopkArgs a)
{
    constexpr int U = 4;  // 16-block groups in flight per wave
    const int s = blockIdx.y;
    const int64_t t = a.pos.v[s];
    const int64_t c = t / a.B;
    const int64_t j0 = (int64_t)blockIdx.x * kKeysPerWG;
    if (j0 >= c)
        return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 15, q4 = lane >> 4;
    const uint16_t *kb = a.kb + (int64_t)s * a.kb_seq_stride;
    const uint16_t *qp = a.qp + (int64_t)s * a.qp_seq_stride;
    uint32_t *keys = a.keys + (int64_t)s * a.keys_ld;

    bf16x8 af[P / 32];
#pragma unroll
    for (int kk = 0; kk < P / 32; ++kk)
        af[kk] = as_bf16x8(load16(qp + kk * 32 + q4 * 8));

    // waves interleave over the workgroup's 64 groups (adjacent waves read adjacent rows)
    __shared__ uint32_t kl[kKeysPerWG];
    constexpr int NG = kKeysPerWG / 16;
#pragma unroll 1
    for (int g0 = wave; g0 < NG; g0 += 4 * U) {
        u32x4 bv[U][P / 32];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int64_t jb = j0 + (int64_t)(g0 + 4 * u) * 16 + col;
            if (jb >= c)
                jb = j0;  // a valid row; its score is discarded
#pragma unroll
            for (int kk = 0; kk < P / 32; ++kk)
                bv[u][kk] = load16(kb + jb * P + kk * 32 + q4 * 8);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < P / 32; ++kk)
                acc = mfma_16x16x32(af[kk], as_bf16x8(bv[u][kk]), acc);
            const int jl = (g0 + 4 * u) * 16 + col;
            if (q4 == 0) {
                const uint32_t key = j0 + jl < c ? score_key(acc[0]) : 0u;
                kl[jl] = key;
                if (j0 + jl < c)
                    keys[j0 + jl] = key;
            }
        }
    }
    __syncthreads();
    // unit maxima: 16 threads per unit, 4 consecutive keys each, then a 16-lane max
    uint32_t m4 = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t v = kl[tid * 4 + e];
        m4 = v > m4 ? v : m4;
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) {
        const uint32_t v = (uint32_t)__shfl_xor((int)m4, o);
        m4 = v > m4 ? v : m4;
    }
    if ((tid & 15) == 0)
        a.umax[(int64_t)s * a.units_ld + (int64_t)blockIdx.x * kUnitsPerWG + (tid >> 4)] = m4;
}

template <int NT>
__global__ __launch_bounds__(NT) void k_decode_select(DecodeTopkArgs a)
{
    __shared__ SelectShared sh;
    __shared__ uint32_t big[kMaxUnits];          // unit maxima, then candidate keys + blocks
    __shared__ uint16_t units[kUnitListCap];
    __shared__ int n_cand;
    uint32_t *cand_key = big;
    int32_t *cand_idx = reinterpret_cast<int32_t *>(big + kCandCap);
    uint32_t *bitmap = big + 2 * kCandCap;       // one bit per block, after the candidates
    const int s = blockIdx.x, tid = threadIdx.x;
    const int64_t t = a.pos.v[s];
    const int64_t c = t / a.B;
    const int k = a.k, keep = k - 1;
    const uint32_t *keys = a.keys + (int64_t)s * a.keys_ld;
    int32_t *out = a.idx + (int64_t)s * k;
    float *osc = a.sel_scores ? a.sel_scores + (int64_t)s * k : nullptr;

    if (c <= (int64_t)keep) {
        for (int e = tid; e < k; e += NT) {
            out[e] = e <= c ? e : -1;
            if (osc)
                osc[e] = e < c ? key_score(keys[e]) : (e == c ? __builtin_inff() : -__builtin_inff());
        }
        return;
    }
    if (tid == 0) {
        out[keep] = (int32_t)c;
        if (osc)
            osc[keep] = __builtin_inff();
    }
    if (keep == 0)
        return;
    const int cn = (int)c;
    auto emit = [&](int pos, int j, uint32_t key) {
        out[pos] = j;
        if (osc)
            osc[pos] = key_score(key);
    };

    // 1) K* = the keep-th largest unit maximum
    const int nunits = (int)((c + kUnitBlocks - 1) / kUnitBlocks);
    const uint32_t *um = a.umax + (int64_t)s * a.units_ld;
    for (int u = tid; u < nunits; u += NT)
        big[u] = um[u];
    __syncthreads();
    auto umax_at = [&](int u) { return big[u]; };
    // with no more units than blocks to keep, every unit qualifies
    const uint32_t kstar = nunits <= keep ? 0u : radix_select<NT>(umax_at, nunits, keep, sh).key;

    // 2) units whose maximum reaches K*, in order
    int flag = 0;
    const int per = (nunits + NT - 1) / NT;
    for (int u = tid * per; u < tid * per + per && u < nunits; ++u)
        flag += big[u] >= kstar ? 1 : 0;
    int nu;
    int pos = block_exclusive_scan<NT>(flag, sh.scan, nu);
    if (nu <= kUnitListCap) {
        for (int u = tid * per; u < tid * per + per && u < nunits; ++u)
            if (big[u] >= kstar)
                units[pos++] = (uint16_t)u;
    }
    if (tid == 0)
        n_cand = 0;
    __syncthreads();

    if (nu <= kUnitListCap) {
        // 3) the blocks of those units that reach K* (16 independent loads per unit)
        const int nwords = (cn + 31) >> 5;
        for (int w = tid; w < nwords; w += NT)
            bitmap[w] = 0u;
        bool overflow = false;
        constexpr int kG = 8;  // loads in flight per thread; a unit is 256 contiguous bytes
        for (int e0 = 0; e0 < nu * kUnitBlocks; e0 += NT * kG) {
            uint32_t kv[kG];
            int64_t jv[kG];
#pragma unroll
            for (int b = 0; b < kG; ++b) {
                const int e = e0 + b * NT + tid;
                jv[b] = e < nu * kUnitBlocks
                            ? (int64_t)units[e / kUnitBlocks] * kUnitBlocks + (e % kUnitBlocks)
                            : (int64_t)cn;
            }
#pragma unroll
            for (int b = 0; b < kG; ++b)
                kv[b] = jv[b] < cn ? keys[jv[b]] : 0u;
#pragma unroll
            for (int b = 0; b < kG; ++b) {
                if (jv[b] < cn && kv[b] >= kstar) {
                    const int slot = atomicAdd(&n_cand, 1);
                    if (slot < kCandCap) {
                        cand_key[slot] = kv[b];
                        cand_idx[slot] = (int32_t)jv[b];
                    }
                }
            }
        }
        __syncthreads();
        const int m = n_cand;
        overflow = m > kCandCap;
        if (!overflow) {
            // 4) exact selection among the candidates, ties to the lowest block
            auto cand_at = [&](int e) { return cand_key[e]; };
            const KthKey th = radix_select<NT>(cand_at, m, keep, sh);
            // keys equal to the threshold: all of them are kept unless there are more than
            // needed (exact float ties), then the lowest blocks win
            int n_eq_local = 0;
            for (int e = tid; e < m; e += NT)
                n_eq_local += cand_key[e] == th.key ? 1 : 0;
            int n_eq;
            block_exclusive_scan<NT>(n_eq_local, sh.scan, n_eq);
            for (int e = tid; e < m; e += NT) {
                const uint32_t key = cand_key[e];
                const int32_t j = cand_idx[e];
                bool take = key > th.key;
                if (key == th.key) {
                    if (n_eq == th.take_eq) {
                        take = true;
                    } else {
                        int rank = 0;  // equal keys with a lower block index
                        for (int f = 0; f < m; ++f)
                            rank += (cand_key[f] == key && cand_idx[f] < j) ? 1 : 0;
                        take = rank < th.take_eq;
                    }
                }
                if (take)
                    atomicOr(&bitmap[j >> 5], 1u << (j & 31));
            }
            __syncthreads();
            // 5) ascending compaction of the bitmap
            const int per_w = (nwords + NT - 1) / NT;
            const int w0 = tid * per_w;
            int local = 0;
            for (int w = w0; w < w0 + per_w && w < nwords; ++w)
                local += __popc(bitmap[w]);
            int total;
            int p = block_exclusive_scan<NT>(local, sh.scan, total);
            for (int w = w0; w < w0 + per_w && w < nwords; ++w) {
                uint32_t bits = bitmap[w];
                while (bits && p < keep) {
                    const int j = (w << 5) + __builtin_ctz(bits);
                    bits &= bits - 1;
                    emit(p, j, keys[j]);
                    ++p;
                }
            }
            return;
        }
    }
    // heavy ties: exact selection over every key
    auto key_at = [&](int j) { return keys[j]; };
    const KthKey th = radix_select<NT>(key_at, cn, keep, sh);
    emit_selected<NT>(key_at, cn, th, keep, sh, emit);
}

bool decode_topk_supported(int64_t max_cand, int k)
{
    // the unit maxima of one sequence and the bitmap of its blocks fit in the select's LDS
    return k >= 2 && max_cand > 0 && max_cand <= kDecodeMaxCand &&
           (max_cand + kUnitBlocks - 1) / kUnitBlocks <= kMaxUnits &&
           (max_cand + 31) / 32 <= kMaxUnits - 2 * kCandCap;
}

int64_t decode_keys_ld(int64_t max_cand)
{
    return ((max_cand + kKeysPerWG - 1) / kKeysPerWG) * kKeysPerWG;
}

int64_t decode_units_ld(int64_t max_cand)
{
    return decode_keys_ld(max_cand) / kKeysPerWG * kUnitsPerWG;
}

size_t decode_topk_workspace(int nseq, int64_t max_cand)
{
    return (size_t)nseq * (decode_keys_ld(max_cand) + decode_units_ld(max_cand)) * 4;
}

template <int P>
static void launch_decode_keys_p(const DecodeTopkArgs &a, hipStream_t stream)
{
    const unsigned nwg = (unsigned)(a.keys_ld / kKeysPerWG);
    hipLaunchKernelGGL(k_decode_keys<P>, dim3(nwg, (unsigned)a.nseq), dim3(256), 0, stream, a);
}

hipError_t launch_decode_topk(const DecodeTopkArgs &a, hipStream_t stream)
{
    switch (a.P) {
    case 32: launch_decode_keys_p<32>(a, stream); break;
    case 64: launch_decode_keys_p<64>(a, stream); break;
    case 128: launch_decode_keys_p<128>(a, stream); break;
    case 256: launch_decode_keys_p<256>(a, stream); break;
    default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(k_decode_select<1024>, dim3((unsigned)a.nseq), dim3(1024), 0, stream, a);
    return hipGetLastError();
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
