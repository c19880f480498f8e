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
//  1. k_decode_keys streams kb at HBM rate (one workgroup per 1024 blocks): the MFMA A
//     operand is the query proxy broadcast to all 16 rows, so row 0 of each 16x16 result
//     holds the scores of 16 consecutive blocks; they are stored as order-preserving keys,
//     and their largest key (the maximum of that "unit" of 16 blocks) is stored too.
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

    // waves interleave over the workgroup's 64 units (adjacent waves read adjacent rows)
    uint32_t *umax = a.umax + (int64_t)s * a.units_ld + (int64_t)blockIdx.x * kUnitsPerWG;
    constexpr int NG = kKeysPerWG / kUnitBlocks;
#pragma unroll 1
    for (int g0 = wave; g0 < NG; g0 += 4 * U) {
        u32x4 bv[U][P / 32];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int64_t jb = j0 + (int64_t)(g0 + 4 * u) * kUnitBlocks + col;
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
            const int64_t j = j0 + (int64_t)(g0 + 4 * u) * kUnitBlocks + col;
            const uint32_t key = j < c ? score_key(acc[0]) : 0u;
            // unit maximum over the 16 lanes of this lane's row group (xor stays inside it)
            uint32_t m = key;
#pragma unroll
            for (int o = 8; o > 0; o >>= 1) {
                const uint32_t v = (uint32_t)__shfl_xor((int)m, o);
                m = v > m ? v : m;
            }
            if (q4 == 0) {
                if (j < c)
                    keys[j] = key;
                if (col == 0)
                    umax[g0 + 4 * u] = m;
            }
        }
    }
}

// FP8 index variant of k_decode_keys: rows of P e4m3 codes with one fp32 scale each.  A lane
// loads 16 codes (dims [64 k2 + 16 q4, +16)) per 64-dim step and converts them exactly to two
// bf16 fragments for two MFMA steps; the query proxy is loaded in the same permuted order, so
// the contraction is unchanged.  The row's scale multiplies the product afterwards.
template <int P>
__global__ __launch_bounds__(256) void k_decode_keys_fp8(DecodeTopkArgs a)
{
    // 16-block groups in flight per wave (16 B per row and step): 4 keeps the wave under 128
    // registers (4 waves per SIMD); measured 124 us per 16 x 1M batch vs 131 us with 8
    constexpr int U = 4;
    const int s = blockIdx.y;
    const int64_t t = a.pos.v[s];
    const int64_t c = t / a.B;
    const int64_t j0 = (int64_t)blockIdx.x * kKeysPerWG;
    if (j0 >= c)
        return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 15, q4 = lane >> 4;
    const uint8_t *kq = a.kbq + (int64_t)s * a.kbs_seq_stride * P;
    const float *ksc = a.kbs + (int64_t)s * a.kbs_seq_stride;
    const uint16_t *qp = a.qp + (int64_t)s * a.qp_seq_stride;
    uint32_t *keys = a.keys + (int64_t)s * a.keys_ld;

    bf16x8 af[P / 32];  // af[2 k2 + h] = qp[64 k2 + 16 q4 + 8 h, +8)
#pragma unroll
    for (int k2 = 0; k2 < P / 64; ++k2) {
        af[2 * k2] = as_bf16x8(load16(qp + k2 * 64 + q4 * 16));
        af[2 * k2 + 1] = as_bf16x8(load16(qp + k2 * 64 + q4 * 16 + 8));
    }

    uint32_t *umax = a.umax + (int64_t)s * a.units_ld + (int64_t)blockIdx.x * kUnitsPerWG;
    constexpr int NG = kKeysPerWG / kUnitBlocks;
#pragma unroll 1
    for (int g0 = wave; g0 < NG; g0 += 4 * U) {
        u32x4 bv[U][P / 64];
        float sc[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int64_t jb = j0 + (int64_t)(g0 + 4 * u) * kUnitBlocks + col;
            if (jb >= c)
                jb = j0;  // a valid row; its score is discarded
#pragma unroll
            for (int k2 = 0; k2 < P / 64; ++k2)
                bv[u][k2] = load16(kq + jb * P + k2 * 64 + q4 * 16);
            sc[u] = ksc[jb];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k2 = 0; k2 < P / 64; ++k2) {
                bf16x8 lo, hi;
                e4m3x16_to_bf16x8x2(bv[u][k2], lo, hi);
                acc = mfma_16x16x32(af[2 * k2], lo, acc);
                acc = mfma_16x16x32(af[2 * k2 + 1], hi, acc);
            }
            const int64_t j = j0 + (int64_t)(g0 + 4 * u) * kUnitBlocks + col;
            const uint32_t key = j < c ? score_key(acc[0] * sc[u]) : 0u;
            uint32_t m = key;
#pragma unroll
            for (int o = 8; o > 0; o >>= 1) {
                const uint32_t v = (uint32_t)__shfl_xor((int)m, o);
                m = v > m ? v : m;
            }
            if (q4 == 0) {
                if (j < c)
                    keys[j] = key;
                if (col == 0)
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
    __shared__ int n_units, n_cand;
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
        n_units = 0;
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
        // 2) the qualifying units, in any order
        int q = 0;
#pragma unroll
        for (int b = 0; b < kPer; ++b)
            q += (b * NT + tid < nunits && mx[b] >= kp) ? 1 : 0;
        int pos = wave_append(q, &n_units);
#pragma unroll
        for (int b = 0; b < kPer; ++b)
            if (b * NT + tid < nunits && mx[b] >= kp)
                units[pos++] = (uint16_t)(b * NT + tid);
        __syncthreads();
        nu = n_units;

        // 3) their keys at or above K' (16 bytes = 4 blocks per load)
        const int nchunks = nu * (kUnitBlocks / 4);
        for (int e0 = 0; e0 < nchunks; e0 += 4 * NT) {
            u32x4 kv[4];
            int jc[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int e = e0 + r * NT + tid;
                jc[r] = e < nchunks ? (int)units[e / (kUnitBlocks / 4)] * kUnitBlocks +
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
        __syncthreads();
        const int m = n_cand;
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

template <int P>
static void launch_decode_keys_p(const DecodeTopkArgs &a, hipStream_t stream)
{
    const unsigned nwg = (unsigned)(a.keys_ld / kKeysPerWG);
    hipLaunchKernelGGL(k_decode_keys<P>, dim3(nwg, (unsigned)a.nseq), dim3(256), 0, stream, a);
}

template <int P>
static void launch_decode_keys_fp8_p(const DecodeTopkArgs &a, hipStream_t stream)
{
    const unsigned nwg = (unsigned)(a.keys_ld / kKeysPerWG);
    hipLaunchKernelGGL(k_decode_keys_fp8<P>, dim3(nwg, (unsigned)a.nseq), dim3(256), 0, stream, a);
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
