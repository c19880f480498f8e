// k_index.hip -- block compression of the indexer's proxy keys (gfx950).
//
// ai4snews "Step 5 Preview bets on depth over width", Interpretation para. 2,
// and ai.info "Sparse GQA targets million-token context": the proxy keys of
// adjacent history positions are compressed into one representation per block
// of 8 tokens.  Here the representation is the mean over the tokens present.
//
// Pure HBM streaming: each thread owns 8 consecutive proxy features (16 B) of
// one block, issues all B row loads at once, sums exactly in fp64 and writes
// one 16 B chunk of correctly rounded bf16 means.  The proxy keys are read once,
// by non-temporal loads (128K: 14.6-14.9 -> 12.7-12.9 us; 16 x 1M tokens:
// 1.89 -> 1.71 ms); the means stay cacheable for the scoring that follows.  A wave covers 64 x 16 B = 1 KiB of contiguous output, and its
// loads for row r of the blocks it covers are contiguous 512 B runs.
#include <hip/hip_runtime.h>

#include "sgqa_device.hpp"
#include "sgqa_launch.hpp"

namespace sgqa {

template <int B>
__global__ __launch_bounds__(256) void k_index_build(const uint16_t *__restrict__ kp,
                                                     uint16_t *__restrict__ kb, int64_t L, int P,
                                                     int64_t j0, int64_t nj)
{
    const int chunks = P >> 3;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t jr = gid / chunks;
    if (jr >= nj)
        return;
    const int c = (int)(gid - jr * chunks);
    const int64_t j = j0 + jr;
    const int64_t first = j * B;
    const int64_t n = (L - first < B) ? (L - first) : B;
    const uint16_t *src = kp + first * P + c * 8;

    // fp64 sums of bf16 inputs are exact (8-bit significands, 53-bit accumulator), so the
    // mean below is the correctly rounded fp64 quotient; it is then rounded once more to
    // bf16, through a round-to-odd fp32 step that keeps the final rounding exact.
    double acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        acc[e] = 0.0;

    if (n == B) {
        u32x4 v[B];
#pragma unroll
        for (int r = 0; r < B; ++r)
            v[r] = load16_stream(src + (int64_t)r * P);
#pragma unroll
        for (int r = 0; r < B; ++r) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                acc[2 * w] += (double)bf16_bits_to_f32(v[r][w] & 0xffffu);
                acc[2 * w + 1] += (double)bf16_bits_to_f32(v[r][w] >> 16);
            }
        }
    } else {
        for (int64_t r = 0; r < n; ++r) {
            u32x4 v = load16_stream(src + r * P);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                acc[2 * w] += (double)bf16_bits_to_f32(v[w] & 0xffffu);
                acc[2 * w + 1] += (double)bf16_bits_to_f32(v[w] >> 16);
            }
        }
    }
    const double dn = (double)n;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        acc[e] = acc[e] / dn;
    u32x4 o;
#pragma unroll
    for (int w = 0; w < 4; ++w)
        o[w] = f64_to_bf16_bits(acc[2 * w]) | (f64_to_bf16_bits(acc[2 * w + 1]) << 16);
    *reinterpret_cast<u32x4 *>(kb + j * P + c * 8) = o;
}

hipError_t launch_index_build(const uint16_t *kp, uint16_t *kb, int64_t L, int P, int B,
                              int64_t j0, int64_t j1, hipStream_t stream)
{
    const int64_t nj = j1 - j0;
    if (nj <= 0)
        return hipSuccess;
    const int64_t threads = nj * (P / 8);
    const int nt = 256;
    const dim3 grid((unsigned)((threads + nt - 1) / nt));
    switch (B) {
    case 1: hipLaunchKernelGGL(k_index_build<1>, grid, dim3(nt), 0, stream, kp, kb, L, P, j0, nj); break;
    case 2: hipLaunchKernelGGL(k_index_build<2>, grid, dim3(nt), 0, stream, kp, kb, L, P, j0, nj); break;
    case 4: hipLaunchKernelGGL(k_index_build<4>, grid, dim3(nt), 0, stream, kp, kb, L, P, j0, nj); break;
    case 8: hipLaunchKernelGGL(k_index_build<8>, grid, dim3(nt), 0, stream, kp, kb, L, P, j0, nj); break;
    case 16: hipLaunchKernelGGL(k_index_build<16>, grid, dim3(nt), 0, stream, kp, kb, L, P, j0, nj); break;
    case 32: hipLaunchKernelGGL(k_index_build<32>, grid, dim3(nt), 0, stream, kp, kb, L, P, j0, nj); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// --------------------------------------------------------------------------------------------
// Index maintenance straight from the keys.  The pages fix the proxy width (phantomic12
// config.json, sparse_config: proxy_dim 256) and the block size; with the proxy key of a
// token read as a linear projection of its concatenated KV-head keys, the block mean of the
// proxy keys is the projection of the block's mean key:
//   kb[j] = ((1/n_j) sum_{s in block j} K[s]) . W,
// so the projection runs once per block instead of once per token and no proxy-key tensor is
// kept.  One workgroup of 8 waves owns 64 consecutive blocks (4 row tiles of
// v_mfma_f32_16x16x32_bf16) and walks the key width in steps of 128 columns:
//  1. each thread sums 8 token rows of two (block, 16-byte column chunk) pairs in fp32
//     (consecutive threads on consecutive chunks: 256-byte runs of one token row per 16
//     lanes), divides by the block's token count and stores the mean to LDS split into
//     bf16 hi + lo (hi = RNE(m), lo = RNE(m - hi); |m - hi - lo| <= 2^-17 |m|);
//  2. wave w multiplies the step's means by its P/8 output columns of W^T: two MFMAs (hi, lo)
//     per 16x16 tile and 32-column slice, so the product keeps fp32 accuracy; one rounding
//     to bf16 at the end.
// The steps are software-pipelined: the W^T fragments of step i and then the keys of step
// i + 1 are requested before the MFMAs of step i, which therefore run while the next keys
// stream in (the LDS means are double-buffered).  A W^T fragment feeds 4 row tiles, so W^T
// (P * width * 2 bytes, resident in L2) is read once per 64 blocks; with 16 blocks per
// workgroup those L2 reads, not HBM, had set the kernel's pace.  The keys stream from HBM
// once (width * 2 bytes per token).
constexpr int kFkM = 64;              // blocks per workgroup
constexpr int kFkKC = 128;            // key columns per step (a last step may hold 64)
constexpr int kFkLd = kFkKC + 8;      // LDS row stride of the staged means (elements)
constexpr int kFkThreads = 512;
constexpr int kFkPairs = kFkM * (kFkKC / 8) / kFkThreads;  // (block, chunk) pairs per thread
static_assert(kFkPairs * kFkThreads == kFkM * (kFkKC / 8), "");

static size_t index_from_keys_lds()
{
    return (size_t)2 * 2 * kFkM * kFkLd * sizeof(uint16_t);  // [buffer][hi, lo][block][column]
}

// NRG = ceil(B / 8) groups of 8 token rows per step, fixed at compile time so that the
// compiler sees every load consumed before its registers are reloaded (and puts no wait
// for the next step's keys into this step)
template <int NP, int NRG>
__global__ __launch_bounds__(kFkThreads) void k_index_from_keys(IndexKeysArgs a)
{
    extern __shared__ __align__(16) uint16_t am[];
    const int s = blockIdx.y;
    const int64_t jw = a.j0.v[s] + (int64_t)blockIdx.x * kFkM;
    const int64_t j_end = a.j1.v[s];
    if (jw >= j_end)
        return;  // the whole workgroup: no barrier is skipped by part of it
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, q4 = lane >> 4;
    const int width = a.width, B = a.B;
    const int64_t L = a.len.v[s];
    const uint16_t *kseq = a.k + (int64_t)s * a.cache_seq_stride;
    const int nch = (width + kFkKC - 1) / kFkKC;

    // this thread's (block, 16-byte chunk) pairs: pair u is f = tid + u * 512, block f / 16,
    // chunk f % 16 of the step's 128 columns.  Addresses are 32-bit byte offsets from the
    // first token of the workgroup's first block (its 64 blocks span < 2^32 bytes).
    const uint16_t *kwg = kseq + (jw * B) * (int64_t)width;
    int nb[kFkPairs], pblk[kFkPairs], pck[kFkPairs];
    uint32_t poff[kFkPairs];
#pragma unroll
    for (int u = 0; u < kFkPairs; ++u) {
        const int f = tid + u * kFkThreads;
        pblk[u] = f >> 4;
        pck[u] = f & 15;
        const int64_t jj = jw + pblk[u];
        const int64_t left = jj < j_end ? L - jj * B : 0;
        nb[u] = left <= 0 ? 0 : (left < B ? (int)left : B);
        poff[u] = (uint32_t)(((int64_t)pblk[u] * B * width + pck[u] * 8) * 2);
    }
    // row i of group rg of pair u in step ch: in the cache when the row exists and the column
    // chunk lies inside the key width; otherwise the load reads the workgroup's first key row
    // (always in bounds) and the value is discarded
    auto row_ok = [&](int u, int ch, int rg, int i) {
        return rg * 8 + i < nb[u] && ch * kFkKC + pck[u] * 8 < width;
    };
    const uint32_t row_bytes = (uint32_t)width * 2;
    u32x4 raw[kFkPairs][8];
    auto issue = [&](int ch, int rg) {
#pragma unroll
        for (int u = 0; u < kFkPairs; ++u)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t off = row_ok(u, ch, rg, i)
                                         ? poff[u] + (uint32_t)(rg * 8 + i) * row_bytes +
                                               (uint32_t)(ch * kFkKC * 2)
                                         : 0u;
                raw[u][i] = load16(reinterpret_cast<const char *>(kwg) + off);
            }
    };

    // output tiles of this wave: columns [16 n0, 16 (n0 + NPW)) of P, all 4 row tiles
    constexpr int NPW = (NP + 7) / 8;
    const int n0 = wave * NPW;
    f32x4 acc[4][NPW];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int n = 0; n < NPW; ++n)
            acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    // byte offset of this lane's W^T fragment of output tile n (clamped into the matrix;
    // unused beyond NP); W^T is P * width * 2 < 2^32 bytes
    uint32_t woff[NPW];
#pragma unroll
    for (int n = 0; n < NPW; ++n)
        woff[n] = (uint32_t)(((n0 + n < NP ? n0 + n : NP - 1) * 16 + col) * width + q4 * 8) * 2;

    issue(0, 0);
#pragma unroll 1
    for (int ch = 0; ch < nch; ++ch) {
        uint16_t *hi = am + (ch & 1) * 2 * kFkM * kFkLd;
        uint16_t *lo = hi + kFkM * kFkLd;
        float sum[kFkPairs][8];
#pragma unroll
        for (int u = 0; u < kFkPairs; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                sum[u][e] = 0.f;
#pragma unroll 1
        for (int rg = 0; rg < NRG; ++rg) {
#pragma unroll
            for (int u = 0; u < kFkPairs; ++u)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const u32x4 v = row_ok(u, ch, rg, i) ? raw[u][i] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        sum[u][2 * w] += bf16_bits_to_f32(v[w] & 0xffffu);
                        sum[u][2 * w + 1] += bf16_bits_to_f32(v[w] >> 16);
                    }
                }
            if (rg + 1 < NRG)
                issue(ch, rg + 1);
        }
        // means -> LDS (hi, lo); chunks outside the key width are not read back
#pragma unroll
        for (int u = 0; u < kFkPairs; ++u) {
            const int n = nb[u];
            const bool pow2 = (n & (n - 1)) == 0;  // then the product by 1/n is exact
            const float inv_n = n > 0 ? 1.0f / (float)n : 0.0f;
            u32x4 hw, lw;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                float m0 = 0.f, m1 = 0.f;
                if (n > 0) {
                    m0 = pow2 ? sum[u][2 * w] * inv_n : sum[u][2 * w] / (float)n;
                    m1 = pow2 ? sum[u][2 * w + 1] * inv_n : sum[u][2 * w + 1] / (float)n;
                }
                const uint32_t h0 = f32_to_bf16_bits(m0), h1 = f32_to_bf16_bits(m1);
                hw[w] = h0 | (h1 << 16);
                lw[w] = f32_to_bf16_bits(m0 - bf16_bits_to_f32(h0)) |
                        (f32_to_bf16_bits(m1 - bf16_bits_to_f32(h1)) << 16);
            }
            *reinterpret_cast<u32x4 *>(hi + pblk[u] * kFkLd + pck[u] * 8) = hw;
            *reinterpret_cast<u32x4 *>(lo + pblk[u] * kFkLd + pck[u] * 8) = lw;
        }
        // this step's W^T fragments, then the next step's keys: the MFMAs below wait for the
        // former only, the latter stay in flight.  After the last step the "next" keys are
        // all out of range and read the first key row: issuing them unconditionally keeps
        // the number of loads in flight the same on every path, so the MFMAs' waits do not
        // count the keys
        const int nsl = (width - ch * kFkKC < kFkKC ? width - ch * kFkKC : kFkKC) / 32;
        u32x4 wf[kFkKC / 32][NPW];
#pragma unroll
        for (int c = 0; c < kFkKC / 32; ++c)
#pragma unroll
            for (int n = 0; n < NPW; ++n)
                wf[c][n] = load16(reinterpret_cast<const char *>(a.wt) + woff[n] +
                                  (uint32_t)((ch * kFkKC + (c < nsl ? c : 0) * 32) * 2));
        issue(ch + 1, 0);
        __syncthreads();  // the step's means are in LDS
        if (n0 < NP) {
#pragma unroll
            for (int c = 0; c < kFkKC / 32; ++c) {
                if (c >= nsl)
                    break;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const bf16x8 ah = as_bf16x8(
                        *reinterpret_cast<const u32x4 *>(hi + (m * 16 + col) * kFkLd + c * 32 + q4 * 8));
                    const bf16x8 al = as_bf16x8(
                        *reinterpret_cast<const u32x4 *>(lo + (m * 16 + col) * kFkLd + c * 32 + q4 * 8));
#pragma unroll
                    for (int n = 0; n < NPW; ++n) {
                        acc[m][n] = mfma_16x16x32(ah, as_bf16x8(wf[c][n]), acc[m][n]);
                        acc[m][n] = mfma_16x16x32(al, as_bf16x8(wf[c][n]), acc[m][n]);
                    }
                }
            }
        }
    }

    // lane holds kb[jw + 16 m + 4 q4 + i][16 (n0 + n) + col]
    if (n0 < NP) {
        uint16_t *kb = a.kb + (int64_t)s * a.kb_seq_stride;
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t jo = jw + m * 16 + 4 * q4 + i;
                if (jo < j_end) {
#pragma unroll
                    for (int n = 0; n < NPW; ++n)
                        if (n0 + n < NP)
                            kb[jo * NP * 16 + (n0 + n) * 16 + col] =
                                (uint16_t)f32_to_bf16_bits(acc[m][n][i]);
                }
            }
    }
}

hipError_t launch_index_from_keys(const IndexKeysArgs &a, int64_t max_blocks, hipStream_t stream)
{
    if (max_blocks <= 0 || a.nseq <= 0)
        return hipSuccess;
    if (a.width % 32 != 0 || a.width < 32)
        return hipErrorInvalidValue;  // the steps are whole 32-column MFMA slices
    const dim3 grid((unsigned)((max_blocks + kFkM - 1) / kFkM), (unsigned)a.nseq);
    const size_t lds = index_from_keys_lds();
    const int nrg = (a.B + 7) / 8;
    if (nrg != 1 && nrg != 2 && nrg != 4)
        return hipErrorInvalidValue;
#define SGQA_FK_LAUNCH(NP)                                                                      \
    do {                                                                                       \
        if (nrg == 1)                                                                          \
            hipLaunchKernelGGL((k_index_from_keys<NP, 1>), grid, dim3(kFkThreads), lds, stream, a); \
        else if (nrg == 2)                                                                     \
            hipLaunchKernelGGL((k_index_from_keys<NP, 2>), grid, dim3(kFkThreads), lds, stream, a); \
        else                                                                                   \
            hipLaunchKernelGGL((k_index_from_keys<NP, 4>), grid, dim3(kFkThreads), lds, stream, a); \
    } while (0)
    switch (a.P) {
    case 32: SGQA_FK_LAUNCH(2); break;
    case 64: SGQA_FK_LAUNCH(4); break;
    case 128: SGQA_FK_LAUNCH(8); break;
    case 256: SGQA_FK_LAUNCH(16); break;
    case 512: SGQA_FK_LAUNCH(32); break;
    default: return hipErrorInvalidValue;
    }
#undef SGQA_FK_LAUNCH
    return hipGetLastError();
}

// --------------------------------------------------------------------------------------------
// FP8 storage of cached rows for the decode path (the released checkpoint is e4m3 with
// scaling blocks; here one fp32 scale per cached row).  One wave per row: the row's largest
// magnitude by a wave reduction, scale = amax / 448 (1 for a zero row), then each element's
// e4m3 code of x / scale; every step in fp32, rounding to nearest even.
__global__ __launch_bounds__(256) void k_quantize_rows(const uint16_t *__restrict__ x, int64_t rows,
                                                       int cols, uint8_t *__restrict__ codes,
                                                       float *__restrict__ scales)
{
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= rows)
        return;
    const int lane = threadIdx.x & 63;
    const uint16_t *xr = x + r * cols;
    float amax = 0.0f;
    for (int e = lane; e < cols; e += 64)
        amax = fmaxf(amax, fabsf(bf16_bits_to_f32(xr[e])));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        amax = fmaxf(amax, __shfl_xor(amax, o));
    float scale = amax / 448.0f;
    if (!(scale > 0.0f))
        scale = 1.0f;
    uint8_t *cr = codes + r * cols;
    for (int e = lane; e < cols; e += 64)
        cr[e] = (uint8_t)e4m3_encode(bf16_bits_to_f32(xr[e]) / scale);
    if (lane == 0)
        scales[r] = scale;
}

hipError_t launch_quantize_rows(const uint16_t *x, int64_t rows, int cols, uint8_t *codes,
                                float *scales, hipStream_t stream)
{
    // a dispatch counts its work-items in 32 bits: launch at most 2^24 rows (2^30 items) at once
    constexpr int64_t kChunk = (int64_t)1 << 24;
    for (int64_t r0 = 0; r0 < rows; r0 += kChunk) {
        const int64_t n = rows - r0 < kChunk ? rows - r0 : kChunk;
        hipLaunchKernelGGL(k_quantize_rows, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, stream,
                           x + r0 * cols, n, cols, codes + r0 * cols, scales + r0);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

} // namespace sgqa
