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

} // namespace sgqa
