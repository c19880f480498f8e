// k_index.hip -- block compression of the indexer's proxy keys (gfx950).
//
// ai4snews "Step 5 Preview bets on depth over width", Interpretation para. 2,
// and ai.info "Sparse GQA targets million-token context": the proxy keys of
// adjacent history positions are compressed into one representation per block
// of 8 tokens.  Here the representation is the mean over the tokens present.
//
// Pure HBM streaming: each thread owns 8 consecutive proxy features (16 B) of
// one block, issues all B row loads at once, sums exactly in fp64 and writes
// one 16 B chunk of correctly rounded bf16 means.  A wave covers 64 x 16 B = 1 KiB of contiguous output, and its
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
            v[r] = load16(src + (int64_t)r * P);
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
            u32x4 v = load16(src + r * P);
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
// kept.  One workgroup owns 16 consecutive blocks (the M rows of v_mfma_f32_16x16x32_bf16):
//  1. the block means, formed in fp32 by threads that each own (block, 16-byte chunk of the
//     concatenated key) pairs, consecutive threads on consecutive chunks (coalesced 1 KiB
//     loads), are written to LDS split into bf16 hi + lo (hi = RNE(m), lo = RNE(m - hi);
//     |m - hi - lo| <= 2^-17 |m|);
//  2. wave w computes a quarter of the P output columns over every slice: two MFMAs (hi, lo)
//     per 16-column tile of W^T, so the product keeps fp32 accuracy; one rounding to bf16.
// The keys stream from HBM once (width * 2 bytes per token); W^T (P * width * 2 bytes) stays
// in L2.
constexpr int kFkPairs = 2;  // (block, 16-byte chunk) pairs per thread whose loads are in flight

template <int NP>
__global__ __launch_bounds__(256) void k_index_from_keys(IndexKeysArgs a)
{
    extern __shared__ __align__(16) uint16_t am[];  // [2][16][width + 8]: hi, lo means
    const int s = blockIdx.y;
    const int64_t jw = a.j0.v[s] + (int64_t)blockIdx.x * 16;
    const int64_t j_end = a.j1.v[s];
    if (jw >= j_end)
        return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, q4 = lane >> 4;
    const int width = a.width, B = a.B, nsl = width / 32;
    const int ld = width + 8;
    const int64_t L = a.len.v[s];
    const uint16_t *kseq = a.k + (int64_t)s * a.cache_seq_stride;

    // 1) block means -> LDS (hi, lo).  Pair f = (block f / nck, 16-byte chunk f % nck of the
    //    token row): consecutive threads take consecutive chunks, so each load instruction
    //    reads 1 KiB of contiguous keys; kFkPairs pairs (8 token rows each) are in flight.
    const int nck = width / 8;
    const int total = 16 * nck;
    const int tid = threadIdx.x;
#pragma unroll 1
    for (int f0 = 0; f0 < total; f0 += 256 * kFkPairs) {
        int blk[kFkPairs], ck[kFkPairs], nb[kFkPairs];
        const uint16_t *src[kFkPairs];
#pragma unroll
        for (int b = 0; b < kFkPairs; ++b) {
            const int f = f0 + b * 256 + tid;
            blk[b] = f < total ? f / nck : 0;
            ck[b] = f < total ? f - blk[b] * nck : 0;
            const int64_t jj = jw + blk[b];
            nb[b] = 0;
            if (f < total && jj < j_end) {
                const int64_t left = L - jj * B;
                nb[b] = left < B ? (int)left : B;
            }
            src[b] = kseq + (jj * B) * (int64_t)width + ck[b] * 8;
        }
        float sum[kFkPairs][8];
#pragma unroll
        for (int b = 0; b < kFkPairs; ++b)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                sum[b][e] = 0.f;
#pragma unroll 1
        for (int r0 = 0; r0 < B; r0 += 8) {
            u32x4 v[kFkPairs][8];
#pragma unroll
            for (int b = 0; b < kFkPairs; ++b)
#pragma unroll
                for (int r = 0; r < 8; ++r)
                    v[b][r] = r0 + r < nb[b] ? load16(src[b] + (int64_t)(r0 + r) * width)
                                             : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int b = 0; b < kFkPairs; ++b)
#pragma unroll
                for (int r = 0; r < 8; ++r)
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        sum[b][2 * w] += bf16_bits_to_f32(v[b][r][w] & 0xffffu);
                        sum[b][2 * w + 1] += bf16_bits_to_f32(v[b][r][w] >> 16);
                    }
        }
#pragma unroll
        for (int b = 0; b < kFkPairs; ++b) {
            if (f0 + b * 256 + tid >= total)
                continue;
            const int n = nb[b];
            const bool pow2 = (n & (n - 1)) == 0;  // then the product by 1/n is exact
            const float inv_n = n > 0 ? 1.0f / (float)n : 0.0f;
            u32x4 hw, lw;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                float m0 = 0.f, m1 = 0.f;
                if (n > 0) {
                    m0 = pow2 ? sum[b][2 * w] * inv_n : sum[b][2 * w] / (float)n;
                    m1 = pow2 ? sum[b][2 * w + 1] * inv_n : sum[b][2 * w + 1] / (float)n;
                }
                const uint32_t h0 = f32_to_bf16_bits(m0), h1 = f32_to_bf16_bits(m1);
                hw[w] = h0 | (h1 << 16);
                lw[w] = f32_to_bf16_bits(m0 - bf16_bits_to_f32(h0)) |
                        (f32_to_bf16_bits(m1 - bf16_bits_to_f32(h1)) << 16);
            }
            *reinterpret_cast<u32x4 *>(am + blk[b] * ld + ck[b] * 8) = hw;
            *reinterpret_cast<u32x4 *>(am + (16 + blk[b]) * ld + ck[b] * 8) = lw;
        }
    }
    __syncthreads();

    // 2) this wave's output tiles [t0, t0 + TPW) over every slice; the W^T fragments of
    //    kWB slices are loaded together (32 loads per lane), then their MFMAs run
    constexpr int TPW = (NP + 3) / 4;
    constexpr int kWB = TPW >= 32 ? 1 : 32 / TPW;
    const int t0 = wave * TPW;
    f32x4 acc[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
        acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (t0 < NP) {
        const uint16_t *wr = a.wt + (int64_t)(t0 * 16 + col) * width + q4 * 8;
#pragma unroll 1
        for (int c0 = 0; c0 < nsl; c0 += kWB) {
            u32x4 wb[kWB][TPW];
#pragma unroll
            for (int b = 0; b < kWB; ++b)
#pragma unroll
                for (int t = 0; t < TPW; ++t)
                    wb[b][t] = (c0 + b < nsl && t0 + t < NP)
                                   ? load16(wr + (int64_t)t * 16 * width + (c0 + b) * 32)
                                   : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int b = 0; b < kWB; ++b) {
                if (c0 + b >= nsl)
                    break;
                const int c = c0 + b;
                const bf16x8 ah =
                    as_bf16x8(*reinterpret_cast<const u32x4 *>(am + col * ld + c * 32 + q4 * 8));
                const bf16x8 al = as_bf16x8(
                    *reinterpret_cast<const u32x4 *>(am + (16 + col) * ld + c * 32 + q4 * 8));
#pragma unroll
                for (int t = 0; t < TPW; ++t) {
                    acc[t] = mfma_16x16x32(ah, as_bf16x8(wb[b][t]), acc[t]);
                    acc[t] = mfma_16x16x32(al, as_bf16x8(wb[b][t]), acc[t]);
                }
            }
        }
    }

    // lane holds kb[jw + 4 q4 + i][16 (t0 + t) + col]
    uint16_t *kb = a.kb + (int64_t)s * a.kb_seq_stride;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t jo = jw + 4 * q4 + i;
        if (jo < j_end) {
#pragma unroll
            for (int t = 0; t < TPW; ++t)
                if (t0 + t < NP)
                    kb[jo * NP * 16 + (t0 + t) * 16 + col] = (uint16_t)f32_to_bf16_bits(acc[t][i]);
        }
    }
}

hipError_t launch_index_from_keys(const IndexKeysArgs &a, int64_t max_blocks, hipStream_t stream)
{
    if (max_blocks <= 0 || a.nseq <= 0)
        return hipSuccess;
    const dim3 grid((unsigned)((max_blocks + 15) / 16), (unsigned)a.nseq);
    const size_t lds = (size_t)2 * 16 * (a.width + 8) * sizeof(uint16_t);
    switch (a.P) {
    case 32: hipLaunchKernelGGL(k_index_from_keys<2>, grid, dim3(256), lds, stream, a); break;
    case 64: hipLaunchKernelGGL(k_index_from_keys<4>, grid, dim3(256), lds, stream, a); break;
    case 128: hipLaunchKernelGGL(k_index_from_keys<8>, grid, dim3(256), lds, stream, a); break;
    case 256: hipLaunchKernelGGL(k_index_from_keys<16>, grid, dim3(256), lds, stream, a); break;
    case 512: hipLaunchKernelGGL(k_index_from_keys<32>, grid, dim3(256), lds, stream, a); break;
    default: return hipErrorInvalidValue;
    }
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
