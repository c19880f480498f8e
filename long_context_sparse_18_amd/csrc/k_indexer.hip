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
// Prefill selection without a score matrix (k_fused_*, the default for rows of up to
// 131072 candidates): a sampled lower bound of each row's threshold filters the scores
// as the matrix cores produce them; the listed blocks are selected exactly, one wave per
// row, with ballot counts.  Otherwise the scores are stored and one workgroup per query
// row runs an exact radix select on order-preserving u32 keys (digits of 12, 12 and
// 8 bits, histograms in LDS), then emits the chosen block ids in ascending order with a
// workgroup scan.  Ties at the threshold go to the lowest block indices, so the result
// is the unique set "k-1 best by (score desc, index asc)" plus the own block.
#include <hip/hip_runtime.h>
#include <algorithm>
#include <type_traits>

#include "sgqa_device.hpp"
#include "sgqa_launch.hpp"

namespace sgqa {

constexpr int kTileQ = 64;
constexpr int kTileB = 64;

template <int P>
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

    constexpr int ldt = P + 8;
    const int tid = threadIdx.x;
    const uint16_t *kb = a.kb + (int64_t)s * a.kb_seq_stride;

    // Stage kb rows j0 .. j0+63 (rows at or past c_last are zero); every load of the tile is
    // issued before the first store
    constexpr int chunks = P / 8;
    constexpr int kPer = (kTileB * chunks + 255) / 256;
    u32x4 tv[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {  // unconditional loads (row j0 is always valid)
        const int e = u * 256 + tid;
        const int r = e / chunks, cc = e - r * chunks;
        const int64_t row = j0 + r < c_last && e < kTileB * chunks ? j0 + r : j0;
        tv[u] = load16(kb + row * P + cc * 8);
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int e = u * 256 + tid;
        if (j0 + e / chunks >= c_last)
            tv[u] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int e = u * 256 + tid;
        const int r = e / chunks, cc = e - r * chunks;
        if (e < kTileB * chunks)
            *reinterpret_cast<u32x4 *>(kb_tile + r * ldt + cc * 8) = tv[u];
    }
    __syncthreads();

    const int wave = tid >> 6, lane = tid & 63;
    const int col = lane & 15, q4 = lane >> 4;
    const int qrow = i0 + wave * 16 + col;  // A-operand row of this lane
    if (i0 + wave * 16 >= a.nq)
        return;
    const uint16_t *qp = a.qp + (int64_t)s * a.qp_seq_stride + (int64_t)(a.t0 + qrow) * P;

    // the query proxies of this lane's row, every slice loaded together
    // (rows past nq read row i0 + 16 wave, which exists, and are never stored)
    const uint16_t *qpr = qrow < a.nq ? qp : qp - (int64_t)col * P;
    u32x4 av[P / 32];
#pragma unroll
    for (int kk = 0; kk < P / 32; ++kk)
        av[kk] = load16(qpr + kk * 32 + q4 * 8);
    f32x4 acc[4];
#pragma unroll
    for (int n = 0; n < 4; ++n)
        acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < P / 32; ++kk) {
        const bf16x8 af = as_bf16x8(av[kk]);
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const u32x4 bv = *reinterpret_cast<const u32x4 *>(kb_tile + (n * 16 + col) * ldt +
                                                              kk * 32 + q4 * 8);
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
    switch (a.P) {
    case 32: hipLaunchKernelGGL(k_scores<32>, grid, dim3(256), lds, stream, a); break;
    case 64: hipLaunchKernelGGL(k_scores<64>, grid, dim3(256), lds, stream, a); break;
    case 96: hipLaunchKernelGGL(k_scores<96>, grid, dim3(256), lds, stream, a); break;
    case 128: hipLaunchKernelGGL(k_scores<128>, grid, dim3(256), lds, stream, a); break;
    case 160: hipLaunchKernelGGL(k_scores<160>, grid, dim3(256), lds, stream, a); break;
    case 192: hipLaunchKernelGGL(k_scores<192>, grid, dim3(256), lds, stream, a); break;
    case 224: hipLaunchKernelGGL(k_scores<224>, grid, dim3(256), lds, stream, a); break;
    case 256: hipLaunchKernelGGL(k_scores<256>, grid, dim3(256), lds, stream, a); break;
    case 288: hipLaunchKernelGGL(k_scores<288>, grid, dim3(256), lds, stream, a); break;
    case 320: hipLaunchKernelGGL(k_scores<320>, grid, dim3(256), lds, stream, a); break;
    case 352: hipLaunchKernelGGL(k_scores<352>, grid, dim3(256), lds, stream, a); break;
    case 384: hipLaunchKernelGGL(k_scores<384>, grid, dim3(256), lds, stream, a); break;
    case 416: hipLaunchKernelGGL(k_scores<416>, grid, dim3(256), lds, stream, a); break;
    case 448: hipLaunchKernelGGL(k_scores<448>, grid, dim3(256), lds, stream, a); break;
    case 480: hipLaunchKernelGGL(k_scores<480>, grid, dim3(256), lds, stream, a); break;
    case 512: hipLaunchKernelGGL(k_scores<512>, grid, dim3(256), lds, stream, a); break;
    default: return hipErrorInvalidValue;
    }
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
//  1. k_decode_keys streams kb at HBM rate in 1024-block items: every block's score is
//     stored as an order-preserving key, and the largest key of each "unit" of 16
//     consecutive blocks (the unit maximum) is stored too.
//  2. k_decode_select (one workgroup per sequence): K* = the (k-1)-th largest unit maximum
//     is a lower bound for the selection (the k-1 best unit maxima are themselves blocks
//     at or above K*, so the (k-1)-th best block is too), and so is any K' <= K*; every
//     selected block lies in a unit whose maximum is >= K'.  K' is the lower edge of the
//     histogram bin that holds K* (one pass, the digit taken just below the bits all maxima
//     share).  Only the qualifying units' keys are read; the blocks at or above K' among
//     them are selected exactly (ties to the lowest block) and written in ascending order
//     from per-word prefix counts of an LDS bitmap.  If too many units or candidates
//     qualify (heavy ties) it selects exactly over all keys instead.
constexpr int kKeysPerWG = 1024;
constexpr int kUnitBlocks = 16;        // consecutive blocks per unit (one MFMA result row)
constexpr int kUnitsPerWG = kKeysPerWG / kUnitBlocks;
constexpr int kMaxUnits = 8192;        // unit maxima one select workgroup holds
constexpr int kBitmapWords = 4096;     // one bit per candidate block
constexpr int kUnitListCap = 4096;
constexpr int kCandCap = 2048;

// Sums over the `L` consecutive lanes of each lane group (L = 4 .. 32, a power of two) of N
// values at once, left in every lane of the group: pair and quad sums by quad permutes, 8 and
// 16 by rotating each 16-lane row by 4 and then 8 (each lane adds the quads before it, so
// after both every lane holds its row's total), 32 by the gfx950 row swap.  Each step is
// applied to all N values before the next, so no permute waits for the add just before it.
// A fixed order: the same values always round the same way.
template <int L, int N>
__device__ __forceinline__ void group_sums(float (&x)[N])
{
    static_assert(L >= 4 && L <= 32 && (L & (L - 1)) == 0, "lane groups of 4 to 32");
    auto dpp = [](float v, auto ctrl) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v),
                                                          decltype(ctrl)::value, 0xf, 0xf, false));
    };
#pragma unroll
    for (int n = 0; n < N; ++n)
        x[n] += dpp(x[n], std::integral_constant<int, 0xb1>{});  // quad_perm [1,0,3,2]
#pragma unroll
    for (int n = 0; n < N; ++n)
        x[n] += dpp(x[n], std::integral_constant<int, 0x4e>{});  // quad_perm [2,3,0,1]
    if constexpr (L == 8) {
#pragma unroll
        for (int n = 0; n < N; ++n)
            x[n] += __shfl_xor(x[n], 4);
    }
    if constexpr (L >= 16) {
#pragma unroll
        for (int n = 0; n < N; ++n)
            x[n] += dpp(x[n], std::integral_constant<int, 0x124>{});  // row_ror:4
#pragma unroll
        for (int n = 0; n < N; ++n)
            x[n] += dpp(x[n], std::integral_constant<int, 0x128>{});  // row_ror:8
    }
    if constexpr (L == 32) {
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const uint32_t u = __float_as_uint(x[n]);
            const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
            x[n] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
        }
    }
}

// Largest uint32 over the wave, in every lane (the rotations of group_sums, then both swaps).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x)
{
    auto dpp = [](uint32_t v, auto ctrl) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, decltype(ctrl)::value, 0xf, 0xf,
                                                     false);
    };
    auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
    x = mx(x, dpp(x, std::integral_constant<int, 0xb1>{}));
    x = mx(x, dpp(x, std::integral_constant<int, 0x4e>{}));
    x = mx(x, dpp(x, std::integral_constant<int, 0x124>{}));
    x = mx(x, dpp(x, std::integral_constant<int, 0x128>{}));
    const auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = mx((uint32_t)p[0], (uint32_t)p[1]);
    const auto q = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return mx((uint32_t)q[0], (uint32_t)q[1]);
}

// The bf16 index scan reads kb as a stream: every wave load covers 1 KB of consecutive rows
// (lane l takes 16 bytes, 8 dims of one row), which the memory system serves faster than 16
// rows x 64 bytes per load in the matrix-core operand layout (a 1 GiB read of this pattern
// measured 7.0 against 6.05 TB/s).  So the dot products are vector code: 8 products per lane
// in four bf16 dot instructions, then a fixed-order sum over the row's P / 8 lanes.  A grid of
// one workgroup per CU strides over the (sequence, 1024-block chunk) items (more, smaller
// workgroups read slower: a decode step of 16 x 1M measured 230.5 / 233 / 232 us with 1 / 2 / 3
// per CU; the FP8 scan, with more conversion work per byte, is fastest with 3: 140.6 against
// 147.5 and 142 us with 2 and 4).  Within an item a wave takes the 16-block units w, w + 4,
// ...; lane (row group g, lane-in-group i) keeps the key of the unit's row i * R + g (R = rows
// per load), so 16 lanes store a unit's 16 keys together and a wave maximum gives the unit
// maximum.  Only an item that reaches past the sequence's last candidate clamps its
// rows (to a valid one; those scores are discarded).
constexpr int kScanWGsPerCU = 1;
constexpr int kScanFp8WGsPerCU = 3;

template <int P>
__global__ __launch_bounds__(256) void k_decode_keys(DecodeTopkArgs a)
{
    constexpr int LPR = P / 8;             // lanes per row
    constexpr int RPI = 64 / LPR;          // rows per wave load
    constexpr int NI = kUnitBlocks / RPI;  // loads per unit
    static_assert(LPR >= 4 && LPR <= 32 && NI <= LPR, "P from 32 to 256");
    static_assert(kUnitsPerWG == 64, "a wave takes units w + 4 u, u < 16, in four halves of 2");
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2v;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int grp = lane / LPR, sub = lane % LPR;
    const int nwg = (int)(a.keys_ld / kKeysPerWG);
    const int nitems = nwg * a.nseq;
#pragma unroll 1
    for (int it = blockIdx.x; it < nitems; it += gridDim.x) {
        const int s = it / nwg, x = it - s * nwg;
        const int64_t c = a.pos.v[s] / a.B;
        const int64_t j0 = (int64_t)x * kKeysPerWG;
        if (j0 >= c)
            continue;
        // rows of this item are j0 + r, r < nrow (uniform); lane offset within a unit
        const int nrow = c - j0 < kKeysPerWG ? (int)(c - j0) : kKeysPerWG;
        const char *kbi =
            reinterpret_cast<const char *>(a.kb + (int64_t)s * a.kb_seq_stride + j0 * P);
        const u32x4 qv = load16(a.qp + (int64_t)s * a.qp_seq_stride + sub * 8);
        uint32_t *keys = a.keys + (int64_t)s * a.keys_ld + j0;
        uint32_t *umax = a.umax + (int64_t)s * a.units_ld + (int64_t)x * kUnitsPerWG;
        // two units per half, two halves in flight: a half's rows are requested before the
        // other half is computed (4.5 us less per 16 x 1M decode step than loading four units,
        // then computing them)
        auto load_units = [&](u32x4 (&v)[2][NI], int gb) {
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    int r = (gb + 4 * u) * kUnitBlocks + i * RPI + grp;
                    r = r < nrow ? r : nrow - 1;
                    v[u][i] = load16_stream(kbi + ((uint32_t)r * (uint32_t)(P * 2) + sub * 16));
                }
        };
        auto compute_units = [&](const u32x4 (&v)[2][NI], int gb) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int ru = (gb + 4 * u) * kUnitBlocks;
                float sc[NI];
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    float part = 0.f;
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        // copies first: a bit_cast of an indexed vector element read element 0
                        const uint32_t kw = v[u][i][w], qw = qv[w];
                        part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, kw),
                                                               __builtin_bit_cast(bf16x2v, qw),
                                                               part, false);
                    }
                    sc[i] = part;
                }
                group_sums<LPR, NI>(sc);
                float pick = sc[0];
#pragma unroll
                for (int i = 1; i < NI; ++i)
                    pick = sub == i ? sc[i] : pick;
                const int r = ru + sub * RPI + grp;
                const uint32_t kreg = r < nrow ? score_key(pick) : 0u;
                if (sub < NI && r < nrow)
                    keys[r] = kreg;
                const uint32_t m = wave_max_u32(kreg);
                if (lane == 0)
                    umax[gb + 4 * u] = m;
            }
        };
        u32x4 va[2][NI], vb[2][NI];
        load_units(va, wave);
        load_units(vb, wave + 8);
        int g0 = wave;
#pragma unroll 1
        for (; g0 + 16 < kUnitsPerWG; g0 += 16) {  // the last iteration, peeled, loads nothing
            compute_units(va, g0);
            load_units(va, g0 + 16);
            compute_units(vb, g0 + 8);
            load_units(vb, g0 + 24);
        }
        compute_units(va, g0);
        compute_units(vb, g0 + 8);
    }
}

// FP8 index variant of k_decode_keys: rows of P e4m3 codes with one fp32 scale each, read
// the same way (1 KB of consecutive rows per wave load; a lane takes 16 codes of one row,
// converted exactly to bf16 and dotted with the query proxy's 16 dims in eight bf16 dot
// instructions); the row's scale multiplies its summed product.
template <int P>
__global__ __launch_bounds__(256) void k_decode_keys_fp8(DecodeTopkArgs a)
{
    constexpr int LPR = P / 16;            // lanes per row
    constexpr int RPI = 64 / LPR;          // rows per wave load
    constexpr int NI = kUnitBlocks / RPI;  // loads per unit
    constexpr int U = 4;                   // units in flight per wave
    static_assert(LPR >= 4 && LPR <= 32 && NI <= LPR, "P from 64 to 512");
    static_assert((kUnitsPerWG / 4) % U == 0, "whole iterations over an item's units");
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2v;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int grp = lane / LPR, sub = lane % LPR;
    const int nwg = (int)(a.keys_ld / kKeysPerWG);
    const int nitems = nwg * a.nseq;
#pragma unroll 1
    for (int it = blockIdx.x; it < nitems; it += gridDim.x) {
        const int s = it / nwg, x = it - s * nwg;
        const int64_t c = a.pos.v[s] / a.B;
        const int64_t j0 = (int64_t)x * kKeysPerWG;
        if (j0 >= c)
            continue;
        const int nrow = c - j0 < kKeysPerWG ? (int)(c - j0) : kKeysPerWG;
        const char *kqi = reinterpret_cast<const char *>(a.kbq + ((int64_t)s * a.kbs_seq_stride + j0) * P);
        const float *ksc = a.kbs + (int64_t)s * a.kbs_seq_stride + j0;
        const uint16_t *qp = a.qp + (int64_t)s * a.qp_seq_stride + sub * 16;
        const u32x4 q0 = load16(qp), q1 = load16(qp + 8);
        const uint32_t qw[8] = {q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]};
        uint32_t *keys = a.keys + (int64_t)s * a.keys_ld + j0;
        uint32_t *umax = a.umax + (int64_t)s * a.units_ld + (int64_t)x * kUnitsPerWG;
#pragma unroll 1
        for (int g0 = wave; g0 < kUnitsPerWG; g0 += 4 * U) {
            u32x4 v[U][NI];
            float rs[U][NI];
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    int r = (g0 + 4 * u) * kUnitBlocks + i * RPI + grp;
                    r = r < nrow ? r : nrow - 1;
                    v[u][i] = load16_stream(kqi + ((uint32_t)r * (uint32_t)P + sub * 16));
                    rs[u][i] = ksc[r];
                }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int ru = (g0 + 4 * u) * kUnitBlocks;
                float sc[NI];
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    uint32_t w[8];
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        const uint32_t code = v[u][i][h];  // a copy: see k_decode_keys
                        e4m3x4_to_bf16(code, w[2 * h], w[2 * h + 1]);
                    }
                    float part = 0.f;
#pragma unroll
                    for (int m = 0; m < 8; ++m) {
                        const uint32_t kw = w[m], q = qw[m];
                        part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, kw),
                                                               __builtin_bit_cast(bf16x2v, q),
                                                               part, false);
                    }
                    sc[i] = part;
                }
                group_sums<LPR, NI>(sc);
                float pick = sc[0] * rs[u][0];
#pragma unroll
                for (int i = 1; i < NI; ++i)
                    pick = sub == i ? sc[i] * rs[u][i] : pick;
                const int r = ru + sub * RPI + grp;
                const uint32_t kreg = r < nrow ? score_key(pick) : 0u;
                if (sub < NI && r < nrow)
                    keys[r] = kreg;
                const uint32_t m = wave_max_u32(kreg);
                if (lane == 0)
                    umax[g0 + 4 * u] = m;
            }
        }
    }
}

// Bitwise OR and AND over the workgroup (every thread calls; `red` holds 2 * NT/64 words).
template <int NT>
__device__ __forceinline__ void block_or_and(uint32_t &vor, uint32_t &vand, uint32_t *red)
{
    constexpr int NW = NT / 64;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        vor |= (uint32_t)__shfl_xor((int)vor, o);
        vand &= (uint32_t)__shfl_xor((int)vand, o);
    }
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) {
        red[w] = vor;
        red[NW + w] = vand;
    }
    __syncthreads();
    vor = 0u;
    vand = ~0u;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        vor |= red[i];
        vand &= red[NW + i];
    }
}

// Reserve `cnt` consecutive slots per lane behind the counter; returns this lane's first.
__device__ __forceinline__ int wave_append(int cnt, int *counter)
{
    const int inc = wave_inclusive_scan(cnt);
    const int tot = __shfl(inc, 63);
    int base = 0;
    if ((threadIdx.x & 63) == 63 && tot > 0)
        base = atomicAdd(counter, tot);
    return __shfl(base, 63) + inc - cnt;
}

// The bin of a 4096-bin histogram that holds the need-th largest counted element:
// thread t owns bins [4t, 4t + 4).  Results are valid for every thread on return.
struct BinFind {
    uint32_t digit;
    int need;  // rank of the element inside its bin (1 = the bin's largest)
    int cnt;   // elements in the bin
    int ge;    // elements in this bin and above
};

template <int NT>
__device__ __forceinline__ BinFind find_bin(const uint32_t *hist, int need, int *scan,
                                            BinFind &res)
{
    static_assert(NT * 4 == 4096, "four bins per thread");
    const int tid = threadIdx.x;
    const u32x4 h = *reinterpret_cast<const u32x4 *>(hist + 4 * tid);
    const int local = (int)(h[0] + h[1] + h[2] + h[3]);
    int total;
    const int below = block_exclusive_scan<NT>(local, scan, total);
    const int above = total - below - local;
    if (above < need && need <= above + local) {
        int acc = above;
#pragma unroll
        for (int b = 3; b >= 0; --b) {
            const int hb = (int)h[b];
            if (acc < need && need <= acc + hb) {
                res.digit = (uint32_t)(4 * tid + b);
                res.need = need - acc;
                res.cnt = hb;
                res.ge = acc + hb;
            }
            acc += hb;
        }
    }
    __syncthreads();
    return res;
}

template <int NT>
__global__ __launch_bounds__(NT) void k_decode_select(DecodeTopkArgs a)
{
    constexpr int kPer = kMaxUnits / NT;       // unit maxima per thread
    constexpr int kCandPer = kCandCap / NT;    // candidates per thread
    static_assert(kPer * NT == kMaxUnits && kCandPer * NT == kCandCap, "");
    __shared__ __align__(16) SelectShared sh;  // histogram A (+ scan scratch)
    __shared__ __align__(16) uint32_t hist_b[4096];
    __shared__ __align__(16) uint32_t bitmap[kBitmapWords];
    __shared__ uint32_t cand_key[kCandCap];
    __shared__ int32_t cand_idx[kCandCap];
    __shared__ uint16_t units[kUnitListCap];
    __shared__ uint32_t red[4 * (NT / 64)];  // two OR/AND reductions
    __shared__ int unit_overflow, n_cand;
    __shared__ BinFind bf;
    uint32_t *hist_a = sh.hist;
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
    const int nunits = (cn + kUnitBlocks - 1) / kUnitBlocks;

#pragma unroll
    for (int i = 0; i < 4096 / NT; ++i) {
        hist_a[i * NT + tid] = 0u;
        hist_b[i * NT + tid] = 0u;
    }
    for (int w = tid; w < kBitmapWords; w += NT)
        bitmap[w] = 0u;
    if (tid == 0) {
        unit_overflow = 0;
        n_cand = 0;
    }

    // 1) K' <= K*: the unit maxima (thread tid holds units b * NT + tid), their common
    //    leading bits, and one 12-bit histogram below them
    const uint32_t *um = a.umax + (int64_t)s * a.units_ld;
    uint32_t mx[kPer];
    uint32_t vor = 0u, vand = ~0u;
#pragma unroll
    for (int b = 0; b < kPer; ++b) {
        const int u = b * NT + tid;
        mx[b] = u < nunits ? um[u] : 0u;
    }
#pragma unroll
    for (int b = 0; b < kPer; ++b)
        if (b * NT + tid < nunits) {
            vor |= mx[b];
            vand &= mx[b];
        }
    block_or_and<NT>(vor, vand, red);
    uint32_t kp = 0u;  // with no more units than blocks to keep, every unit qualifies
    int nu = nunits;
    if (nunits > keep) {
        const uint32_t diff = vor ^ vand;
        if (diff == 0u) {
            kp = vand;  // all maxima equal
        } else {
            const int top = 31 - __builtin_clz(diff);
            const int width = top + 1 < 12 ? top + 1 : 12;
            const int shift = top + 1 - width;
            const uint32_t dmask = (1u << width) - 1u;
#pragma unroll
            for (int b = 0; b < kPer; ++b)
                if (b * NT + tid < nunits)
                    atomicAdd(&hist_a[(mx[b] >> shift) & dmask], 1u);
            __syncthreads();
            const BinFind r = find_bin<NT>(hist_a, keep, sh.scan, bf);
            kp = (vand & ~((2u << top) - 1u)) | (r.digit << shift);
            nu = r.ge;
#pragma unroll
            for (int i = 0; i < 4096 / NT; ++i)
                hist_a[i * NT + tid] = 0u;  // for the third candidate pass
        }
    }

    bool exact_done = false;
    if (nu <= kUnitListCap) {
        // 2) each wave lists its own qualifying units in its share of `units` (only the wave
        //    reads its list, so no workgroup barrier) and 3) reads their keys, keeping those at
        //    or above K' (16 bytes = 4 blocks per load).  A wave with more qualifying units
        //    than its share (heavy ties) flags the exact selection over every key instead.
        constexpr int kWaveUnits = kUnitListCap / (NT / 64);
        const int lane = tid & 63;
        uint16_t *wunits = units + (tid >> 6) * kWaveUnits;
        int q = 0;
#pragma unroll
        for (int b = 0; b < kPer; ++b)
            q += (b * NT + tid < nunits && mx[b] >= kp) ? 1 : 0;
        const int q_inc = wave_inclusive_scan(q);
        const int wq = __shfl(q_inc, 63);
        if (wq > kWaveUnits) {
            if (lane == 0)
                unit_overflow = 1;  // no exact result from the candidates
        } else {
            int pos = q_inc - q;
#pragma unroll
            for (int b = 0; b < kPer; ++b)
                if (b * NT + tid < nunits && mx[b] >= kp)
                    wunits[pos++] = (uint16_t)(b * NT + tid);
            wave_lds_handoff();
            const int nchunks = wq * (kUnitBlocks / 4);
            for (int e0 = 0; e0 < nchunks; e0 += 4 * 64) {
                u32x4 kv[4];
                int jc[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int e = e0 + r * 64 + lane;
                    jc[r] = e < nchunks ? (int)wunits[e / (kUnitBlocks / 4)] * kUnitBlocks +
                                              (e % (kUnitBlocks / 4)) * 4
                                        : -1;
                }
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    kv[r] = jc[r] >= 0 ? *reinterpret_cast<const u32x4 *>(keys + jc[r])
                                       : u32x4{0u, 0u, 0u, 0u};
                int cnt = 0;
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        cnt += (jc[r] >= 0 && jc[r] + i < cn && kv[r][i] >= kp) ? 1 : 0;
                int slot = wave_append(cnt, &n_cand);
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (jc[r] >= 0 && jc[r] + i < cn && kv[r][i] >= kp) {
                            if (slot < kCandCap) {
                                cand_key[slot] = kv[r][i];
                                cand_idx[slot] = jc[r] + i;
                            }
                            ++slot;
                        }
            }
        }
        __syncthreads();
        const int m = unit_overflow == 0 ? n_cand : kCandCap + 1;
        if (m <= kCandCap) {
            // 4) exact selection of `keep` candidates: radix passes below their common bits,
            //    stopping once the threshold bin is taken whole
            uint32_t ck[kCandPer];
            int32_t cj[kCandPer];
            vor = 0u;
            vand = ~0u;
#pragma unroll
            for (int r = 0; r < kCandPer; ++r) {
                const int e = r * NT + tid;
                ck[r] = e < m ? cand_key[e] : 0u;
                cj[r] = e < m ? cand_idx[e] : -1;
                if (e < m) {
                    vor |= ck[r];
                    vand &= ck[r];
                }
            }
            block_or_and<NT>(vor, vand, red + NT / 32);
            uint32_t P = vand, pmask = ~0u;
            int need = keep, cnt = m;
            const uint32_t diff = vor ^ vand;
            if (diff != 0u) {
                int top = 31 - __builtin_clz(diff);
                pmask = ~((2u << top) - 1u);
                P = vand & pmask;
#pragma unroll 1
                for (int pass = 0;; ++pass) {
                    const int width = top + 1 < 12 ? top + 1 : 12;
                    const int shift = top + 1 - width;
                    const uint32_t dmask = (1u << width) - 1u;
                    uint32_t *H = (pass & 1) ? hist_a : hist_b;
#pragma unroll
                    for (int r = 0; r < kCandPer; ++r)
                        if (cj[r] >= 0 && (ck[r] & pmask) == P)
                            atomicAdd(&H[(ck[r] >> shift) & dmask], 1u);
                    __syncthreads();
                    const BinFind rb = find_bin<NT>(H, need, sh.scan, bf);
#pragma unroll
                    for (int i = 0; i < 4096 / NT; ++i)
                        H[i * NT + tid] = 0u;  // for the pass after next
                    P |= rb.digit << shift;
                    pmask |= dmask << shift;
                    need = rb.need;
                    cnt = rb.cnt;
                    if (need == cnt || shift == 0)
                        break;
                    top = shift - 1;
                }
            }
            // take: every key above the prefix P; at P, all of them when the count matches,
            // else (exact ties of the full key) the `need` lowest blocks
            bool take[kCandPer];
#pragma unroll
            for (int r = 0; r < kCandPer; ++r) {
                take[r] = false;
                if (cj[r] < 0)
                    continue;
                const uint32_t km = ck[r] & pmask;
                if (km != P) {
                    take[r] = km > P;
                } else if (need == cnt) {
                    take[r] = true;
                } else {
                    int rank = 0;
                    for (int f = 0; f < m; ++f)
                        rank += (cand_key[f] == ck[r] && cand_idx[f] < cj[r]) ? 1 : 0;
                    take[r] = rank < need;
                }
                if (take[r])
                    atomicOr(&bitmap[cj[r] >> 5], 1u << (cj[r] & 31));
            }
            __syncthreads();
            // 5) output positions: exclusive prefix of the bitmap popcounts per word
            uint32_t *wpre = hist_a;
            static_assert(kBitmapWords == 4 * NT, "four bitmap words per thread");
            const u32x4 bw = *reinterpret_cast<const u32x4 *>(bitmap + 4 * tid);
            const int p0 = __popc(bw[0]), p1 = __popc(bw[1]), p2 = __popc(bw[2]);
            int total;
            const int before = block_exclusive_scan<NT>(p0 + p1 + p2 + __popc(bw[3]), sh.scan,
                                                        total);
            *reinterpret_cast<u32x4 *>(wpre + 4 * tid) =
                u32x4{(uint32_t)before, (uint32_t)(before + p0), (uint32_t)(before + p0 + p1),
                      (uint32_t)(before + p0 + p1 + p2)};
            __syncthreads();
#pragma unroll
            for (int r = 0; r < kCandPer; ++r)
                if (take[r]) {
                    const int j = cj[r], w = j >> 5;
                    const int p = (int)wpre[w] + __popc(bitmap[w] & ((1u << (j & 31)) - 1u));
                    if (p < keep) {  // exactly `keep` bits are set
                        out[p] = j;
                        if (osc)
                            osc[p] = key_score(ck[r]);
                    }
                }
            exact_done = true;
        }
    }
    if (exact_done)
        return;
    // heavy ties: exact selection over every key
    auto emit = [&](int p, int j, uint32_t key) {
        out[p] = j;
        if (osc)
            osc[p] = key_score(key);
    };
    auto key_at = [&](int j) { return keys[j]; };
    const KthKey th = radix_select<NT>(key_at, cn, keep, sh);
    emit_selected<NT>(key_at, cn, th, keep, sh, emit);
}

// ---- prefill rows of at most kSel2MaxCand candidates, without a histogram of the whole row ----
// Normally distributed scores put nearly all keys into a few dozen bins of a 12-bit histogram,
// so a full-row histogram serialises on LDS atomics.  Instead: (1) a sample of at most
// kSel2Samp keys (every stride-th block) gives T0, its q-th largest key, with q about twice
// the sample's expected share of the kept blocks; (2) one read of the row lists every block
// whose key is >= T0 (about twice `keep` of them); (3) the `keep` largest of the listed keys are
// found exactly (radix passes over the list in LDS, exact ties of the full key to the lowest
// block) and marked in an LDS bitmap, which (4) gives every selected block its output
// position in block order.  The result does not depend on the sample: when fewer than `keep`
// or more than kSel2Cap blocks reach T0, the four-read selection over the whole row runs.
constexpr int kSel2MaxCand = 16384;
constexpr int kSel2Words = kSel2MaxCand / 32;
constexpr int kSel2Cap = 2048;
constexpr int kSel2Samp = 1024;

// find_bin for any NT dividing 4096: thread t owns bins [t * 4096/NT, (t+1) * 4096/NT).
template <int NT>
__device__ __forceinline__ BinFind find_bin_n(const uint32_t *hist, int need, int *scan,
                                              BinFind &res)
{
    constexpr int kPer = 4096 / NT;
    const int tid = threadIdx.x;
    int local = 0;
#pragma unroll
    for (int b = 0; b < kPer; ++b)
        local += (int)hist[tid * kPer + b];
    int total;
    const int below = block_exclusive_scan<NT>(local, scan, total);
    const int above = total - below - local;
    if (above < need && need <= above + local) {
        int acc = above;
#pragma unroll
        for (int b = kPer - 1; b >= 0; --b) {
            const int hb = (int)hist[tid * kPer + b];
            if (acc < need && need <= acc + hb) {
                res.digit = (uint32_t)(tid * kPer + b);
                res.need = need - acc;
                res.cnt = hb;
                res.ge = acc + hb;
            }
            acc += hb;
        }
    }
    __syncthreads();
    return res;
}

template <int NT>
__global__ __launch_bounds__(NT) void k_select2(SelectArgs a)
{
    static_assert(kSel2Words % NT == 0, "");
    __shared__ __align__(16) SelectShared sh;
    __shared__ uint32_t bitmap[kSel2Words];
    __shared__ uint32_t samp[kSel2Samp];
    __shared__ uint32_t cand_key[kSel2Cap];
    __shared__ int32_t cand_idx[kSel2Cap];
    __shared__ int n_cand;
    __shared__ BinFind bf;
    const int tid = threadIdx.x;
    const int row = blockIdx.x;
    const int s = row / a.nq;
    const int i = row - s * a.nq;
    const int64_t t = a.q_start.v[s] + a.t0 + i;
    const int64_t c = t / a.B;
    const int k = a.k, keep = k - 1;
    const float *srow = a.ws + (int64_t)row * a.ld;
    int32_t *out = a.idx + ((int64_t)s * a.T + a.t0 + i) * k;
    float *osc = a.sel_scores ? a.sel_scores + ((int64_t)s * a.T + a.t0 + i) * k : nullptr;

    if (c <= (int64_t)keep) {
        for (int e = tid; e < k; e += NT) {
            out[e] = e <= c ? e : -1;
            if (osc)
                osc[e] = (e < c) ? srow[e] : (e == c ? __builtin_inff() : -__builtin_inff());
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
    const int n = (int)c;
    uint32_t *hist = sh.hist;
    auto emit = [&](int pos, int j, uint32_t key) {
        out[pos] = j;
        if (osc)
            osc[pos] = key_score(key);
    };

    // (1) T0 from the sample
    const int stride = (n + kSel2Samp - 1) / kSel2Samp;
    const int ns = (n + stride - 1) / stride;
    {
        constexpr int kSp = kSel2Samp / NT;  // samples per thread, loaded together
        float sv[kSp];
#pragma unroll
        for (int u = 0; u < kSp; ++u) {
            const int e = u * NT + tid;
            sv[u] = srow[(int64_t)(e < ns ? e : 0) * stride];
        }
#pragma unroll
        for (int u = 0; u < kSp; ++u)
            if (u * NT + tid < ns)
                samp[u * NT + tid] = score_key(sv[u]);
    }
    // The whole row, 16 keys per thread and group (at most kIt groups per thread), is requested
    // now: its loads are in flight while T0 is selected from the sample.  Rows start 256-byte
    // aligned and hold at least round_up(n, 64) floats, so a group that starts inside the row
    // reads inside it; groups past the row re-read group 0 and are skipped.
    constexpr int kIt = kSel2MaxCand / (16 * NT);
    const u32x4 *row4 = reinterpret_cast<const u32x4 *>(srow);
    u32x4 v[kIt][4];
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
        const int g = it * NT + tid;
#pragma unroll
        for (int u = 0; u < 4; ++u)
            v[it][u] = row4[(g * 16 < n ? g : 0) * 4 + u];
    }
    const int64_t share = ((int64_t)keep * ns + n - 1) / n;  // expected kept samples, rounded up
    const int q = (int)(2 * share + 16 < ns ? 2 * share + 16 : ns);
    __syncthreads();
    const KthKey tq = radix_select<NT>([&](int e) { return samp[e]; }, ns, q, sh);
    const uint32_t t0key = tq.key;

    // (2) the blocks whose key reaches T0
    if (tid == 0)
        n_cand = 0;
    __syncthreads();
    // 16 keys per thread and group (the whole row, requested above)
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
        if (it * NT * 16 >= n)
            break;  // uniform: every thread leaves together
        const int g = it * NT + tid;
        uint32_t kk[16];
        int cnt = 0;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int j = g * 16 + e;
            kk[e] = score_key(__uint_as_float(v[it][e >> 2][e & 3]));
            cnt += (j < n && kk[e] >= t0key) ? 1 : 0;
        }
        int slot = wave_append(cnt, &n_cand);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int j = g * 16 + e;
            if (j < n && kk[e] >= t0key) {
                if (slot < kSel2Cap) {
                    cand_key[slot] = kk[e];
                    cand_idx[slot] = j;
                }
                ++slot;
            }
        }
    }
    __syncthreads();
    const int m = n_cand;
    if (m < keep || m > kSel2Cap) {
        auto key_at = [&](int j) { return score_key(srow[j]); };
        const KthKey th = radix_select<NT>(key_at, n, keep, sh);
        emit_selected<NT>(key_at, n, th, keep, sh, emit);
        return;
    }

    // (3) exact selection of `keep` of the m listed keys
    int need = keep, cnt = m;
    uint32_t P = 0u, pmask = 0u;
    const int shifts[3] = {20, 8, 0};
    const uint32_t dmasks[3] = {0xfffu, 0xfffu, 0xffu};
#pragma unroll 1
    for (int pass = 0; pass < 3 && need != cnt; ++pass) {
        const int shift = shifts[pass];
        const uint32_t dmask = dmasks[pass];
        for (int b = tid; b < 4096; b += NT)
            hist[b] = 0u;
        __syncthreads();
        for (int e = tid; e < m; e += NT)
            if ((cand_key[e] & pmask) == P)
                atomicAdd(&hist[(cand_key[e] >> shift) & dmask], 1u);
        __syncthreads();
        const BinFind rb = find_bin_n<NT>(hist, need, sh.scan, bf);
        P |= rb.digit << shift;
        pmask |= dmask << shift;
        need = rb.need;
        cnt = rb.cnt;
    }
    const int nwords = (n + 31) / 32;
    for (int w = tid; w < nwords; w += NT)
        bitmap[w] = 0u;
    __syncthreads();
    // take: keys above the prefix P; at P all of them when the count matches, else (exact
    // ties of the full key) the `need` lowest blocks
    for (int e = tid; e < m; e += NT) {
        const uint32_t key = cand_key[e];
        const int j = cand_idx[e];
        const uint32_t km = key & pmask;
        bool take = km > P;
        if (km == P) {
            if (need == cnt) {
                take = true;
            } else {
                int rank = 0;
                for (int f = 0; f < m; ++f)
                    rank += (cand_key[f] == key && cand_idx[f] < j) ? 1 : 0;
                take = rank < need;
            }
        }
        if (take)
            atomicOr(&bitmap[j >> 5], 1u << (j & 31));
    }
    __syncthreads();

    // (4) output positions: exclusive prefix of the bitmap popcounts
    constexpr int kWpt = kSel2Words / NT;  // bitmap words per thread
    uint32_t wv[kWpt];
    int cntw = 0;
#pragma unroll
    for (int qq = 0; qq < kWpt; ++qq) {
        const int w = tid * kWpt + qq;
        wv[qq] = w < nwords ? bitmap[w] : 0u;
        cntw += __popc(wv[qq]);
    }
    int total;
    int pos = block_exclusive_scan<NT>(cntw, sh.scan, total);
#pragma unroll
    for (int qq = 0; qq < kWpt; ++qq) {
        uint32_t bits = wv[qq];
        while (bits) {
            const int b = __builtin_ctz(bits);
            bits &= bits - 1u;
            const int j = (tid * kWpt + qq) * 32 + b;
            if (pos < keep)  // exactly `keep` bits are set
                emit(pos, j, score_key(srow[j]));
            ++pos;
        }
    }
}

// ---- prefill top-k without the score matrix -------------------------------------------------
// For rows of at most kFusedMaxCand candidate blocks (and k <= kFusedMaxK) no score row is
// stored.  One pass over a block of query rows runs:
//  1. k_fused_sample<P>: the scores of a strided sample of each row's blocks (ns per row; the
//     stride is set per 64-row tile from the tile's first row), as order-preserving keys;
//  2. k_fused_threshold: one wave per row takes T0 = the q-th largest sample key, found bit by
//     bit from the top with the wave counting the keys at or above each candidate value
//     (q is about twice the sample's expected share of the kept blocks, plus 16);
//  3. k_fused_filter<P>: the scores of every candidate block, 64 queries x 64 blocks per
//     workgroup on the matrix cores as in k_scores; each key >= T0 of a row is appended as
//     (key, block) to that row's list (the 16 lanes holding a row's keys of a tile reserve their
//     slots with one atomic add; the count keeps counting past the list's capacity);
//  4. k_fused_select_wave (rows of up to 32768 candidates; one wave per row, bit by bit with
//     ballot counts) or k_fused_select<NT> (longer rows; one workgroup per row, radix passes
//     over the list in LDS) selects the k-1 largest listed keys exactly (exact ties of the
//     full key go to the lowest block) and writes them in block order from per-word prefix
//     counts of an LDS bitmap.  A row whose list holds fewer than k-1 keys (T0 above the
//     row's threshold) or overflowed is queued instead;
//  5. k_fused_fallback<NT>: a few persistent workgroups take the queued rows one at a time,
//     score every candidate block of the row into their own scratch row with the same
//     matrix-core arithmetic (so the same fp32 scores), and select exactly over it.
// The listed keys are a superset of the selection whenever step 4 accepts a row, so the result
// never depends on the sample, and it equals what the score-matrix path selects.
constexpr int64_t kFusedMaxCand = 131072;       // bitmap words of the select's LDS, times 32
constexpr int kFusedMaxK = 1024;
constexpr int kFusedBitmapWords = (int)(kFusedMaxCand / 32);
constexpr int kFusedFallbackWGs = 64;

// sample size, list capacity and stride rule shared by the host and the kernels
__host__ __device__ __forceinline__ int fused_ns(int64_t max_cand)
{
    return max_cand <= 32768 ? 1024 : 4096;
}
__host__ __device__ __forceinline__ int fused_cap(int64_t max_cand)
{
    return max_cand <= 32768 ? 2048 : 4096;
}
__device__ __forceinline__ int64_t fused_stride(int64_t c_first, int ns)
{
    const int64_t s = (c_first + ns - 1) / ns;
    return s > 1 ? s : 1;
}

// Row r = s * nq + i of a pass; its position and own block.
__device__ __forceinline__ int64_t fused_c(const FusedTopkArgs &a, int s, int i)
{
    return (a.q_start.v[s] + a.t0 + i) / a.B;
}

template <int P>
__global__ __launch_bounds__(256) void k_fused_sample(FusedTopkArgs a)
{
    extern __shared__ __align__(16) uint16_t kb_tile[];  // [kTileB][P + 8]
    const int s = blockIdx.z;
    const int i0 = blockIdx.y * kTileQ;
    const int m0 = blockIdx.x * kTileB;  // first sample of this tile
    const int64_t stride = fused_stride(fused_c(a, s, i0), a.ns);
    const int i_last = min(i0 + kTileQ, a.nq) - 1;
    const int64_t c_last = fused_c(a, s, i_last);
    constexpr int ldt = P + 8;
    const int tid = threadIdx.x;
    const uint16_t *kb = a.kb + (int64_t)s * a.kb_seq_stride;
    constexpr int chunks = P / 8;
    constexpr int kPer = (kTileB * chunks + 255) / 256;
    u32x4 tv[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {  // rows past the tile's last candidate load block 0
        const int e = u * 256 + tid;
        const int r = e / chunks, cc = e - r * chunks;
        const int64_t j = (int64_t)(m0 + r) * stride;
        const int64_t row = j < c_last && e < kTileB * chunks ? j : 0;
        tv[u] = load16(kb + row * P + cc * 8);
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int e = u * 256 + tid;
        const int r = e / chunks, cc = e - r * chunks;
        if (e < kTileB * chunks)
            *reinterpret_cast<u32x4 *>(kb_tile + r * ldt + cc * 8) = tv[u];
    }
    __syncthreads();
    const int wave = tid >> 6, lane = tid & 63;
    const int col = lane & 15, q4 = lane >> 4;
    if (i0 + wave * 16 >= a.nq)
        return;
    const int qrow = i0 + wave * 16 + col;
    const uint16_t *qp = a.qp + (int64_t)s * a.qp_seq_stride + (int64_t)(a.t0 + qrow) * P;
    const uint16_t *qpr = qrow < a.nq ? qp : qp - (int64_t)col * P;
    u32x4 av[P / 32];
#pragma unroll
    for (int kk = 0; kk < P / 32; ++kk)
        av[kk] = load16(qpr + kk * 32 + q4 * 8);
    f32x4 acc[4];
#pragma unroll
    for (int n = 0; n < 4; ++n)
        acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < P / 32; ++kk) {
        const bf16x8 af = as_bf16x8(av[kk]);
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const u32x4 bv = *reinterpret_cast<const u32x4 *>(kb_tile + (n * 16 + col) * ldt +
                                                              kk * 32 + q4 * 8);
            acc[n] = mfma_16x16x32(af, as_bf16x8(bv), acc[n]);
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int i = i0 + wave * 16 + q4 * 4 + r;
        if (i >= a.nq)
            continue;
        const int64_t c = fused_c(a, s, i);
        uint32_t *dst = a.samp + ((int64_t)s * a.nq + i) * a.ns;
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const int m = m0 + n * 16 + col;
            const int64_t j = (int64_t)m * stride;
            if (m < a.ns)
                dst[m] = j < c ? score_key(acc[n][r]) : 0u;  // 0: below every real key
        }
    }
}

// Number of sample keys of a row and the rank q whose key becomes T0.
__device__ __forceinline__ void fused_rank(const FusedTopkArgs &a, int64_t c, int64_t stride,
                                           int &ns_row, int &q)
{
    const int64_t n = (c + stride - 1) / stride;
    ns_row = (int)(n < a.ns ? n : a.ns);
    const int keep = a.k - 1;
    if (stride == 1 && ns_row == c) {  // the sample is the whole row: T0 is the exact threshold
        q = keep;
        return;
    }
    const int64_t share = ((int64_t)keep * ns_row + c - 1) / c;  // expected kept samples, up
    const int64_t qq = 2 * share + 16;
    q = (int)(qq < ns_row ? qq : ns_row);
}

template <int KPL>  // sample keys per lane: ns / 64
__global__ __launch_bounds__(256) void k_fused_threshold(FusedTopkArgs a)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= (int64_t)a.nseq * a.nq)
        return;
    const int s = (int)(row / a.nq), i = (int)(row - (int64_t)s * a.nq);
    const int64_t c = fused_c(a, s, i);
    if (c <= a.k - 1) {  // every past block is kept: list them all
        if (lane == 0)
            a.thr[row] = 0u;
        return;
    }
    const int64_t stride = fused_stride(fused_c(a, s, i & ~(kTileQ - 1)), a.ns);
    int ns_row, q;
    fused_rank(a, c, stride, ns_row, q);
    const uint32_t *src = a.samp + row * a.ns;
    uint32_t key[KPL];
#pragma unroll
    for (int e = 0; e < KPL; ++e)
        key[e] = src[e * 64 + lane];  // invalid samples hold 0 and never count
    // the largest T with #{keys >= T} >= q, decided from the top bit down (the wave counts
    // with one ballot per key slot)
    uint32_t t = 0u;
#pragma unroll 1
    for (int b = 31; b >= 0; --b) {
        const uint32_t cand = t | (1u << b);
        int n = 0;
#pragma unroll
        for (int e = 0; e < KPL; ++e)
            n += __popcll(__ballot(key[e] >= cand));
        if (n >= q)
            t = cand;
    }
    if (lane == 0)
        a.thr[row] = t;
}

// A filter workgroup takes kFilterWaves * 16 queries x kFilterTiles tiles of 64 blocks.  The
// keys a row keeps are staged in LDS, and each row then reserves its slots in the global list
// with one atomic add per workgroup; a tile's keys that no longer fit a row's stage (rows that
// keep most of their blocks) reserve and write their slots in the global list at once.  A
// row's stage and its count are only touched by the 16 lanes that hold the row's keys.
#ifndef SGQA_FILTER_WAVES
#define SGQA_FILTER_WAVES 4
#endif
#ifndef SGQA_FILTER_TILES
#define SGQA_FILTER_TILES 8
#endif
#ifndef SGQA_FILTER_STAGE
#define SGQA_FILTER_STAGE 32
#endif
constexpr int kFilterWaves = SGQA_FILTER_WAVES;
constexpr int kFilterTiles = SGQA_FILTER_TILES;
#ifndef SGQA_FILTER_TILES_LONG
#define SGQA_FILTER_TILES_LONG 32
#endif
constexpr int kFilterTilesLong = SGQA_FILTER_TILES_LONG;  // passes of > 32768 candidates
constexpr int kStage = SGQA_FILTER_STAGE;
constexpr int kFilterQ = 16 * kFilterWaves;  // query rows per workgroup
constexpr int kFilterNT = 64 * kFilterWaves;

// Occupancy: a workgroup holds its kb tile (~34 KB at P = 256) and the row stages (16 KB), and
// for P <= 256 the second launch bound keeps the kernel within 168 VGPRs (it took 232 at
// P = 256), so three workgroups (12 waves) share a CU instead of two: 128K top-k 3.13-3.20 ->
// 2.88 ms, chunked prefill 1.75 -> 1.46 ms, the same selections (stages of 32 entries with two
// workgroups per CU: no gain).  At P = 512 the kb tile alone is 66 KB, so the bound stays loose.
template <int P>
constexpr int filter_min_waves()
{
    return P <= 256 ? 3 : 1;
}

template <int P, int FT>
__global__ __launch_bounds__(kFilterNT, filter_min_waves<P>()) void k_fused_filter(FusedTopkArgs a)
{
    extern __shared__ __align__(16) uint16_t kb_tile[];  // [kTileB][P + 8], then the stage
    constexpr int ldt = P + 8;
    uint2 *stage = reinterpret_cast<uint2 *>(kb_tile + kTileB * ldt);  // [kFilterQ][kStage]
    // [kFilterQ * kStage] row stages, then one trash entry per thread
    const int trash = kFilterQ * kStage + (int)threadIdx.x;
    uint32_t *lcnt = reinterpret_cast<uint32_t *>(stage + kFilterQ * kStage + kFilterNT);
    uint32_t *gbase = lcnt + kFilterQ;  // [kFilterQ]
    const int s = blockIdx.z;
    const int i0 = blockIdx.x * kFilterQ;  // query tiles vary fastest: neighbouring workgroups
                                           // share their kb tiles in L2, their counters differ
    const int i_last = min(i0 + kFilterQ, a.nq) - 1;
    const int64_t c_last = fused_c(a, s, i_last);
    const int64_t jt0 = (int64_t)blockIdx.y * FT * kTileB;
    if (jt0 >= c_last)
        return;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int col = lane & 15, q4 = lane >> 4;
    const uint16_t *kb = a.kb + (int64_t)s * a.kb_seq_stride;
    if (tid < kFilterQ)
        lcnt[tid] = 0u;
    const bool wave_live = i0 + wave * 16 < a.nq;
    const int qrow = i0 + wave * 16 + col;
    const uint16_t *qp = a.qp + (int64_t)s * a.qp_seq_stride + (int64_t)(a.t0 + qrow) * P;
    const uint16_t *qpr = qrow < a.nq ? qp : qp - (int64_t)(qrow - i0) * P;  // row i0 exists
    u32x4 av[P / 32];
#pragma unroll
    for (int kk = 0; kk < P / 32; ++kk)
        av[kk] = load16(qpr + kk * 32 + q4 * 8);
    // this lane's query (col of the wave's 16): its threshold, candidate count and row
    const int rl = wave * 16 + col;  // row within the workgroup
    const uint32_t thr_row = a.thr[(int64_t)s * a.nq + (qrow < a.nq ? qrow : i0)];
    const int64_t c_row = qrow < a.nq ? fused_c(a, s, qrow) : 0;
    constexpr int chunks = P / 8;
    constexpr int kPer = (kTileB * chunks + kFilterNT - 1) / kFilterNT;
    // a tile's kb rows are requested while the previous tile is computed
    u32x4 tv[kPer];
    auto load_tile = [&](int64_t j0) {
#pragma unroll
        for (int u = 0; u < kPer; ++u) {  // unconditional loads (row j0 is always valid)
            const int e = u * kFilterNT + tid;
            const int r = e / chunks, cc = e - r * chunks;
            const int64_t row = j0 + r < c_last && e < kTileB * chunks ? j0 + r : j0;
            tv[u] = load16(kb + row * P + cc * 8);
        }
    };
    load_tile(jt0);
#pragma unroll 1
    for (int tl = 0; tl < FT; ++tl) {
        const int64_t j0 = jt0 + (int64_t)tl * kTileB;
        if (j0 >= c_last)
            break;  // uniform over the workgroup
        __syncthreads();  // the previous tile's operand reads are done
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int e = u * kFilterNT + tid;
            const int r = e / chunks, cc = e - r * chunks;
            if (e < kTileB * chunks)
                *reinterpret_cast<u32x4 *>(kb_tile + r * ldt + cc * 8) = tv[u];
        }
        __syncthreads();
        if (tl + 1 < FT && j0 + kTileB < c_last)
            load_tile(j0 + kTileB);
        if (!wave_live)
            continue;
        // Sᵀ: the tile's blocks as the MFMA rows, the wave's 16 queries as its columns, so lane
        // (col, q4) holds the keys of query col at blocks j0 + 16 n + 4 q4 + r (each output is
        // the same sum of the same 32-element products as in the score kernel)
        f32x4 acc[4];
#pragma unroll
        for (int n = 0; n < 4; ++n)
            acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < P / 32; ++kk) {
            const bf16x8 qf = as_bf16x8(av[kk]);
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                const u32x4 bv = *reinterpret_cast<const u32x4 *>(
                    kb_tile + (n * 16 + col) * ldt + kk * 32 + q4 * 8);
                acc[n] = mfma_16x16x32(as_bf16x8(bv), qf, acc[n]);
            }
        }
        // the query's keys >= its threshold among its candidate blocks (block < c): j0 + 16 n +
        // 4 q4 + r < c, i.e. 16 n + r < lim
        const int lim = (int)(c_row - j0) - 4 * q4;
        uint32_t key[4][4];
        int cnt = 0;
#pragma unroll
        for (int n = 0; n < 4; ++n)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                key[n][r] = score_key(acc[n][r]);
                cnt += (16 * n + r < lim && key[n][r] >= thr_row) ? 1 : 0;
            }
        // the query's 4 lanes (q4 = 0..3): exclusive prefix of their counts and the total
        const int c1 = __shfl_xor(cnt, 16);
        const int pair = cnt + c1;
        const int c2 = __shfl_xor(pair, 32);
        const int tot = pair + c2;
        if (tot != 0) {  // (the same for the query's 4 lanes)
            const int excl = ((q4 & 1) ? c1 : 0) + ((q4 & 2) ? c2 : 0);
            const int local = (int)lcnt[rl];
            const bool spill = local + tot > kStage;
            int base = 0;
            if (spill && q4 == 0)
                base = (int)atomicAdd(&a.cnt[(int64_t)s * a.nq + i0 + rl], (uint32_t)tot);
            base = spill ? __shfl(base, col) : local;
            int slot = base + excl;
            if (!spill) {
                // every key is written, the ones not kept to this lane's own trash entry, so
                // the writes need no branches
#pragma unroll
                for (int n = 0; n < 4; ++n)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const bool keep = 16 * n + r < lim && key[n][r] >= thr_row;
                        const uint32_t j = (uint32_t)j0 + (uint32_t)(16 * n + 4 * q4 + r);
                        stage[keep ? rl * kStage + slot : trash] = uint2{key[n][r], j};
                        slot += keep ? 1 : 0;
                    }
                if (q4 == 3)
                    lcnt[rl] = (uint32_t)(local + tot);
            } else {
                uint2 *list = a.cand + ((int64_t)s * a.nq + i0 + rl) * a.cap;
#pragma unroll
                for (int n = 0; n < 4; ++n)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if (16 * n + r < lim && key[n][r] >= thr_row) {
                            const uint32_t j = (uint32_t)j0 + (uint32_t)(16 * n + 4 * q4 + r);
                            if (slot < a.cap)
                                list[slot] = uint2{key[n][r], j};
                            ++slot;
                        }
                    }
            }
        }
    }
    __syncthreads();
    // one reservation per row for its staged keys
    if (tid < kFilterQ) {
        const uint32_t n = lcnt[tid];
        uint32_t b = 0u;
        if (n > 0u && i0 + tid < a.nq)
            b = atomicAdd(&a.cnt[(int64_t)s * a.nq + i0 + tid], n);
        gbase[tid] = b;
    }
    __syncthreads();
    for (int e = tid; e < kFilterQ * kStage; e += kFilterNT) {
        const int rl = e / kStage, f = e - rl * kStage;
        const uint32_t n = lcnt[rl];
        if ((uint32_t)f < n && i0 + rl < a.nq) {
            const uint32_t slot = gbase[rl] + (uint32_t)f;
            if (slot < (uint32_t)a.cap)
                a.cand[((int64_t)s * a.nq + i0 + rl) * a.cap + slot] = stage[e];
        }
    }
}

// Clear the pass's counters (a fill kernel, so a captured pass records no memset).
__global__ __launch_bounds__(256) void k_fused_clear(FusedTopkArgs a)
{
    const int64_t n = (int64_t)a.nseq * a.nq;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256)
        a.cnt[e] = 0u;
    if (blockIdx.x == 0 && threadIdx.x < 2)
        a.queue_ctr[threadIdx.x] = 0u;
}

template <int NT>
__global__ __launch_bounds__(NT) void k_fused_select(FusedTopkArgs a)
{
    __shared__ __align__(16) SelectShared sh;
    __shared__ __align__(16) uint32_t bitmap[kFusedBitmapWords];
    __shared__ uint32_t cand_key[4096];
    __shared__ int32_t cand_idx[4096];
    __shared__ BinFind bf;
    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    const int s = (int)(row / a.nq), i = (int)(row - (int64_t)s * a.nq);
    const int64_t c = fused_c(a, s, i);
    const int k = a.k, keep = k - 1;
    int32_t *out = a.idx + ((int64_t)s * a.T + a.t0 + i) * k;
    float *osc = a.sel_scores ? a.sel_scores + ((int64_t)s * a.T + a.t0 + i) * k : nullptr;
    const int m = (int)a.cnt[row];
    const uint2 *list = a.cand + row * a.cap;

    if (c <= (int64_t)keep) {
        // every past block and the own block are kept; the list holds all c past blocks
        for (int e = tid; e < k; e += NT) {
            out[e] = e <= c ? e : -1;
            if (osc && e >= c)
                osc[e] = e == c ? __builtin_inff() : -__builtin_inff();
        }
        if (osc)
            for (int e = tid; e < m && e < a.cap; e += NT) {
                const uint2 v = list[e];
                osc[v.y] = key_score(v.x);
            }
        return;
    }
    if (m < keep || m > a.cap) {  // T0 missed: the fallback selects over every block
        if (tid == 0)
            a.queue[atomicAdd(&a.queue_ctr[0], 1u)] = (uint32_t)row;
        return;
    }
    if (tid == 0) {
        out[keep] = (int32_t)c;
        if (osc)
            osc[keep] = __builtin_inff();
    }
    for (int e = tid; e < m; e += NT) {
        const uint2 v = list[e];
        cand_key[e] = v.x;
        cand_idx[e] = (int32_t)v.y;
    }
    const int nwords = (int)((c + 31) / 32);
    for (int w = tid; w < nwords; w += NT)
        bitmap[w] = 0u;
    __syncthreads();
    // exact selection of `keep` of the m listed keys: radix passes below the bits all taken
    int need = keep, cnt = m;
    uint32_t Pf = 0u, pmask = 0u;
    uint32_t *hist = sh.hist;
    const int shifts[3] = {20, 8, 0};
    const uint32_t dmasks[3] = {0xfffu, 0xfffu, 0xffu};
#pragma unroll 1
    for (int pass = 0; pass < 3 && need != cnt; ++pass) {
        const int shift = shifts[pass];
        const uint32_t dmask = dmasks[pass];
        for (int b = tid; b < 4096; b += NT)
            hist[b] = 0u;
        __syncthreads();
        for (int e = tid; e < m; e += NT)
            if ((cand_key[e] & pmask) == Pf)
                atomicAdd(&hist[(cand_key[e] >> shift) & dmask], 1u);
        __syncthreads();
        const BinFind rb = find_bin_n<NT>(hist, need, sh.scan, bf);
        Pf |= rb.digit << shift;
        pmask |= dmask << shift;
        need = rb.need;
        cnt = rb.cnt;
    }
    // take: keys above the prefix; at the prefix all of them when the count matches, else
    // (exact ties of the full key) the `need` lowest blocks.  The flags are kept in registers
    // until every thread has ranked its ties against the unmodified list.
    constexpr int kPerThread = 4096 / NT;
    bool taken[kPerThread];
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
        const int e = tid + u * NT;
        taken[u] = false;
        if (e >= m)
            continue;
        const uint32_t key = cand_key[e];
        const int j = cand_idx[e];
        const uint32_t km = key & pmask;
        bool take = km > Pf;
        if (km == Pf) {
            if (need == cnt) {
                take = true;
            } else {
                int rank = 0;
                for (int f = 0; f < m; ++f)
                    rank += (cand_key[f] == key && cand_idx[f] < j) ? 1 : 0;
                take = rank < need;
            }
        }
        if (take)
            atomicOr(&bitmap[j >> 5], 1u << (j & 31));
        taken[u] = take;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
        const int e = tid + u * NT;
        if (e < m && !taken[u])
            cand_idx[e] = -1;
    }
    // output positions: exclusive prefix of the bitmap popcounts per word, then each taken
    // candidate writes itself at its rank among the set bits
    uint32_t *wpre = hist;  // kFusedBitmapWords == 4096 words
    constexpr int kWpt = kFusedBitmapWords / NT;
    int cntw = 0;
#pragma unroll
    for (int qq = 0; qq < kWpt; ++qq) {
        const int w = tid * kWpt + qq;
        cntw += w < nwords ? __popc(bitmap[w]) : 0;
    }
    int total;
    int before = block_exclusive_scan<NT>(cntw, sh.scan, total);
#pragma unroll
    for (int qq = 0; qq < kWpt; ++qq) {
        const int w = tid * kWpt + qq;
        wpre[w] = (uint32_t)before;
        before += w < nwords ? __popc(bitmap[w]) : 0;
    }
    __syncthreads();
    for (int e = tid; e < m; e += NT) {
        const int j = cand_idx[e];
        if (j >= 0) {
            const int w = j >> 5;
            const int p = (int)wpre[w] + __popc(bitmap[w] & ((1u << (j & 31)) - 1u));
            if (p < keep) {  // exactly `keep` bits are set
                out[p] = j;
                if (osc)
                    osc[p] = key_score(cand_key[e]);
            }
        }
    }
}

// The selection of a pass, one wave per row and no workgroup barriers: CAP listed keys per row
// at most (CAP / 64 per lane in registers), candidates below WORDS * 32, NW rows (waves) per
// workgroup.  The (k-1)-th largest listed key K is found bit by bit from the top, counting the
// keys at or above each candidate value with ballots; if fewer keys equal K are taken than are
// listed, the taken ones are those up to the right block, found the same way over the blocks of
// the tied keys.  The taken blocks are marked in the wave's LDS bitmap, whose per-word prefix
// counts (a wave scan) give every taken block its output position.
template <int CAP, int WORDS, int NW>
__global__ __launch_bounds__(64 * NW) void k_fused_select_wave(FusedTopkArgs a)
{
    __shared__ uint32_t bitmap_all[NW][WORDS];
    __shared__ uint32_t wpre_all[NW][WORDS];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * NW + wave;
    if (row >= (int64_t)a.nseq * a.nq)
        return;  // waves never synchronise with each other
    const int s = (int)(row / a.nq), i = (int)(row - (int64_t)s * a.nq);
    const int64_t c = fused_c(a, s, i);
    const int k = a.k, keep = k - 1;
    int32_t *out = a.idx + ((int64_t)s * a.T + a.t0 + i) * k;
    float *osc = a.sel_scores ? a.sel_scores + ((int64_t)s * a.T + a.t0 + i) * k : nullptr;
    const int m = (int)a.cnt[row];
    const uint2 *list = a.cand + row * a.cap;

    if (c <= (int64_t)keep) {
        // every past block and the own block are kept; the list holds all c past blocks
        for (int e = lane; e < k; e += 64) {
            out[e] = e <= c ? e : -1;
            if (osc && e >= c)
                osc[e] = e == c ? __builtin_inff() : -__builtin_inff();
        }
        if (osc)
            for (int e = lane; e < m && e < a.cap; e += 64) {
                const uint2 v = list[e];
                osc[v.y] = key_score(v.x);
            }
        return;
    }
    if (m < keep || m > a.cap) {  // T0 missed: the fallback selects over every block
        if (lane == 0)
            a.queue[atomicAdd(&a.queue_ctr[0], 1u)] = (uint32_t)row;
        return;
    }
    constexpr int U = CAP / 64;
    uint32_t kr[U];
    int32_t jr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int e = lane + 64 * u;
        const uint2 v = list[e < m ? e : 0];
        kr[u] = e < m ? v.x : 0u;  // 0 lies below every listed key
        jr[u] = e < m ? (int32_t)v.y : -1;
    }
    // K: the largest value with at least `keep` listed keys at or above it
    uint32_t K = 0u;
#pragma unroll 1
    for (int b = 31; b >= 0; --b) {
        const uint32_t cand = K | (1u << b);
        int n = 0;
#pragma unroll
        for (int u = 0; u < U; ++u)
            n += __popcll(__ballot(kr[u] >= cand));
        if (n >= keep)
            K = cand;
    }
    int n_gt = 0, n_eq = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        n_gt += __popcll(__ballot(kr[u] > K));
        n_eq += __popcll(__ballot(kr[u] == K));
    }
    const int take_eq = keep - n_gt;  // 1 .. n_eq
    int32_t jmax = 0x7fffffff;         // tied keys are taken up to this block
    if (take_eq < n_eq) {
        // the largest J with fewer than take_eq tied keys at blocks below J is the block of
        // the take_eq-th tied key in block order
        int32_t J = 0;
#pragma unroll 1
        for (int b = 17; b >= 0; --b) {
            const int32_t cand = J | (1 << b);
            int n = 0;
#pragma unroll
            for (int u = 0; u < U; ++u)
                n += __popcll(__ballot(kr[u] == K && jr[u] < cand));
            if (n < take_eq)
                J = cand;
        }
        jmax = J;
    }
    uint32_t *bitmap = bitmap_all[wave];
    uint32_t *wpre = wpre_all[wave];
    const int nwords = (int)((c + 31) / 32);
    for (int w = lane; w < nwords; w += 64)
        bitmap[w] = 0u;
    wave_lds_handoff();
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const bool take = kr[u] > K || (kr[u] == K && jr[u] <= jmax);
        if (take)
            atomicOr(&bitmap[jr[u] >> 5], 1u << (jr[u] & 31));
    }
    wave_lds_handoff();
    constexpr int kWpl = WORDS / 64;  // bitmap words per lane
    int cntw = 0;
    for (int q = 0; q < kWpl; ++q) {
        const int w = lane * kWpl + q;
        cntw += w < nwords ? __popc(bitmap[w]) : 0;
    }
    int before = wave_inclusive_scan(cntw) - cntw;
    for (int q = 0; q < kWpl; ++q) {
        const int w = lane * kWpl + q;
        wpre[w] = (uint32_t)before;
        before += w < nwords ? __popc(bitmap[w]) : 0;
    }
    wave_lds_handoff();
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const bool take = kr[u] > K || (kr[u] == K && jr[u] <= jmax);
        if (take) {
            const int j = jr[u], w = j >> 5;
            const int p = (int)wpre[w] + __popc(bitmap[w] & ((1u << (j & 31)) - 1u));
            if (p < keep) {  // exactly `keep` bits are set
                out[p] = j;
                if (osc)
                    osc[p] = key_score(kr[u]);
            }
        }
    }
    if (lane == 0) {
        out[keep] = (int32_t)c;
        if (osc)
            osc[keep] = __builtin_inff();
    }
}

// The queued rows: each workgroup scores one row's blocks into its scratch row with the
// filter's matrix-core arithmetic (the query proxy broadcast to all 16 A rows, so one
// product gives 16 blocks), then selects exactly over the row.  Workgroups loop until the
// queue, complete before this launch, is empty.
template <int P, int NT>
__global__ __launch_bounds__(NT) void k_fused_fallback(FusedTopkArgs a)
{
    __shared__ SelectShared sh;
    __shared__ int cur;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 15, q4 = lane >> 4;
    float *sc = a.fb_scores + (int64_t)blockIdx.x * a.fb_ld;
    const int nq_total = (int)a.queue_ctr[0];
#pragma unroll 1
    for (;;) {
        if (tid == 0)
            cur = (int)atomicAdd(&a.queue_ctr[1], 1u);
        __syncthreads();
        const int qi = cur;
        __syncthreads();
        if (qi >= nq_total)
            break;
        const int64_t row = a.queue[qi];
        const int s = (int)(row / a.nq), i = (int)(row - (int64_t)s * a.nq);
        const int64_t c = fused_c(a, s, i);
        const int k = a.k, keep = k - 1;
        const uint16_t *qp = a.qp + (int64_t)s * a.qp_seq_stride + (int64_t)(a.t0 + i) * P;
        const uint16_t *kb = a.kb + (int64_t)s * a.kb_seq_stride;
        bf16x8 af[P / 32];
#pragma unroll
        for (int kk = 0; kk < P / 32; ++kk)
            af[kk] = as_bf16x8(load16(qp + kk * 32 + q4 * 8));
        for (int64_t jb = (int64_t)wave * 16; jb < c; jb += (NT / 64) * 16) {
            const int64_t j = jb + col < c ? jb + col : jb;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < P / 32; ++kk)
                acc = mfma_16x16x32(af[kk], as_bf16x8(load16(kb + j * P + kk * 32 + q4 * 8)),
                                    acc);
            if (q4 == 0 && jb + col < c)
                sc[jb + col] = acc[0];
        }
        __syncthreads();
        int32_t *out = a.idx + ((int64_t)s * a.T + a.t0 + i) * k;
        float *osc = a.sel_scores ? a.sel_scores + ((int64_t)s * a.T + a.t0 + i) * k : nullptr;
        auto key_at = [&](int j) { return score_key(sc[j]); };
        const KthKey th = radix_select<NT>(key_at, (int)c, keep, sh);
        emit_selected<NT>(key_at, (int)c, th, keep, sh, [&](int pos, int j, uint32_t key) {
            out[pos] = j;
            if (osc)
                osc[pos] = key_score(key);
        });
        if (tid == 0) {
            out[keep] = (int32_t)c;
            if (osc)
                osc[keep] = __builtin_inff();
        }
        __syncthreads();
    }
}

bool fused_topk_supported(int64_t max_cand, int k, int P)
{
    return max_cand <= kFusedMaxCand && k >= 2 && k <= kFusedMaxK &&
           (P == 32 || P == 64 || P == 128 || P == 256 || P == 512);
}

void fused_topk_geometry(int64_t max_cand, int &ns, int &cap)
{
    ns = fused_ns(max_cand);
    cap = fused_cap(max_cand);
}

size_t fused_topk_row_bytes(int64_t max_cand)
{
    // sample keys, threshold, count, queue slot, candidate list
    return (size_t)fused_ns(max_cand) * 4 + 12 + (size_t)fused_cap(max_cand) * 8;
}

size_t fused_topk_fixed_bytes(int64_t max_cand)
{
    const int64_t ld = (max_cand + 63) / 64 * 64;
    return 256 + (size_t)kFusedFallbackWGs * ld * 4;
}

template <int P>
static void launch_fused_p(const FusedTopkArgs &a, hipStream_t stream)
{
    const unsigned qt = (unsigned)((a.nq + kTileQ - 1) / kTileQ);
    const size_t lds = (size_t)kTileB * (P + 8) * sizeof(uint16_t);
    const int64_t rows = (int64_t)a.nseq * a.nq;
    hipLaunchKernelGGL(k_fused_clear, dim3((unsigned)((rows + 255) / 256 < 1024 ? (rows + 255) / 256 : 1024)),
                       dim3(256), 0, stream, a);
    hipLaunchKernelGGL(k_fused_sample<P>, dim3((unsigned)(a.ns / kTileB), qt, (unsigned)a.nseq),
                       dim3(256), lds, stream, a);
    if (a.ns == 1024)
        hipLaunchKernelGGL(k_fused_threshold<16>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0,
                           stream, a);
    else
        hipLaunchKernelGGL(k_fused_threshold<64>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0,
                           stream, a);
    const size_t lds_f = lds + (size_t)(kFilterQ * kStage + kFilterNT) * 8 + 2 * kFilterQ * 4;
    const unsigned fq = (unsigned)((a.nq + kFilterQ - 1) / kFilterQ);
    if (a.cap > 2048) {  // long rows keep few keys per block: longer spans per workgroup
        const int64_t span = (int64_t)kFilterTilesLong * kTileB;
        hipLaunchKernelGGL((k_fused_filter<P, kFilterTilesLong>),
                           dim3(fq, (unsigned)((a.max_cand + span - 1) / span), (unsigned)a.nseq),
                           dim3(kFilterNT), lds_f, stream, a);
    } else {
        const int64_t span = (int64_t)kFilterTiles * kTileB;
        hipLaunchKernelGGL((k_fused_filter<P, kFilterTiles>),
                           dim3(fq, (unsigned)((a.max_cand + span - 1) / span), (unsigned)a.nseq),
                           dim3(kFilterNT), lds_f, stream, a);
    }
    // one wave per row for lists of 2048 keys with bitmaps for 32768 candidates, four rows per
    // workgroup; longer rows take a 512-thread workgroup each (one wave per row with 4096-key
    // lists holds 256 registers and 32 KB of LDS: 2.75 against 2.45 ms for the chunked prefill)
    if (a.cap <= 2048 && a.max_cand <= 32768)
        hipLaunchKernelGGL((k_fused_select_wave<2048, 1024, 4>),
                           dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(k_fused_select<512>, dim3((unsigned)rows), dim3(512), 0, stream, a);
    const unsigned nfb = (unsigned)(rows < kFusedFallbackWGs ? rows : kFusedFallbackWGs);
    hipLaunchKernelGGL((k_fused_fallback<P, 512>), dim3(nfb), dim3(512), 0, stream, a);
}

hipError_t launch_fused_topk(const FusedTopkArgs &a, hipStream_t stream)
{
    if ((int64_t)a.nseq * a.nq == 0)
        return hipSuccess;
    if (a.max_cand > kFusedMaxCand || a.fb_ld < a.max_cand)
        return hipErrorInvalidValue;  // the select's bitmap and the scratch rows hold max_cand
    switch (a.P) {
    case 32: launch_fused_p<32>(a, stream); break;
    case 64: launch_fused_p<64>(a, stream); break;
    case 128: launch_fused_p<128>(a, stream); break;
    case 256: launch_fused_p<256>(a, stream); break;
    case 512: launch_fused_p<512>(a, stream); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

bool decode_topk_supported(int64_t max_cand, int k)
{
    // the unit maxima of one sequence and the bitmap of its blocks fit in the select's LDS
    return k >= 2 && max_cand > 0 && max_cand <= kDecodeMaxCand &&
           (max_cand + kUnitBlocks - 1) / kUnitBlocks <= kMaxUnits &&
           (max_cand + 31) / 32 <= kBitmapWords;
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

// Workgroups of a decode scan: kScanWGsPerCU (bf16) or kScanFp8WGsPerCU per CU, at most one
// per item.
static int64_t scan_grid(const DecodeTopkArgs &a)
{
    const int per_cu = a.kbq ? kScanFp8WGsPerCU : kScanWGsPerCU;
    const int64_t nitems = a.keys_ld / kKeysPerWG * a.nseq;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
    return std::min<int64_t>(nitems, (int64_t)per_cu * cus);
}

template <int P>
static void launch_decode_keys_p(const DecodeTopkArgs &a, hipStream_t stream)
{
    hipLaunchKernelGGL(k_decode_keys<P>, dim3((unsigned)scan_grid(a)), dim3(256), 0, stream, a);
}

template <int P>
static void launch_decode_keys_fp8_p(const DecodeTopkArgs &a, hipStream_t stream)
{
    hipLaunchKernelGGL(k_decode_keys_fp8<P>, dim3((unsigned)scan_grid(a)), dim3(256), 0, stream, a);
}

hipError_t launch_decode_topk(const DecodeTopkArgs &a, hipStream_t stream)
{
    if (a.kbq) {
        switch (a.P) {
        case 64: launch_decode_keys_fp8_p<64>(a, stream); break;
        case 128: launch_decode_keys_fp8_p<128>(a, stream); break;
        case 256: launch_decode_keys_fp8_p<256>(a, stream); break;
        case 512: launch_decode_keys_fp8_p<512>(a, stream); break;
        default: return hipErrorInvalidValue;
        }
    } else {
        switch (a.P) {
        case 32: launch_decode_keys_p<32>(a, stream); break;
        case 64: launch_decode_keys_p<64>(a, stream); break;
        case 128: launch_decode_keys_p<128>(a, stream); break;
        case 256: launch_decode_keys_p<256>(a, stream); break;
        default: return hipErrorInvalidValue;
        }
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
    if (a.max_cand <= kSel2MaxCand) {
        // 512 threads per row: 4.99 ms for the 128K prefill's rows against 5.24 ms with 256
        // and 7.04 ms with 128 (same selections); 512 is the most the bitmap split allows
        hipLaunchKernelGGL(k_select2<512>, dim3(rows), dim3(512), 0, stream, a);
        return hipGetLastError();
    }
    if (a.max_cand > 32768 && rows <= 256)
        hipLaunchKernelGGL(k_select<1024>, dim3(rows), dim3(1024), 0, stream, a);
    else
        hipLaunchKernelGGL(k_select<256>, dim3(rows), dim3(256), 0, stream, a);
    return hipGetLastError();
}

} // namespace sgqa
