// k_probe.hip -- machine-peak probes for the rooflines of the measurement: a dense bf16 MFMA
// loop and a streaming read.  Both produce results with a closed form, so a run that was
// optimised away or read the wrong bytes is caught.
#include "sgqa_device.hpp"
#include "probe_launch.hpp"

namespace sgqa {

// Each wave runs `iters` rounds of 8 independent v_mfma_f32_32x32x16_bf16 chains (32 768 flop
// each; measured the fastest shape for a peak loop: 16x16x32 chains need twice as many
// independent accumulators to hide their latency) on operands whose every element is `one`
// (1.0 from the host, so nothing can be folded at compile time).  Every accumulator element
// ends at 16 * iters; lane 0 of wave w writes the sum of its 128 accumulator values,
// 2048 * iters, to sink[w] (exact in fp32 for iters <= 8192).
typedef __attribute__((ext_vector_type(16))) float f32x16;

__global__ __launch_bounds__(256) void k_probe_mfma(int iters, float one, float *sink, int waves)
{
    const int wave = (int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
    const uint32_t h = f32_to_bf16_bits(one);
    const uint32_t w2 = h | (h << 16);
    const bf16x8 a = as_bf16x8(u32x4{w2, w2, w2, w2});
    f32x16 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            acc[j][e] = 0.f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, acc[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            s += acc[j][e];
    if ((threadIdx.x & 63) == 0 && wave < waves)
        sink[wave] = s;
}

// Streaming read of n16 16-byte words: each workgroup writes the sum (mod 2^32) of the uint32
// words it read to sink[blockIdx.x]; the partial sums add up to the buffer's word sum.
__global__ __launch_bounds__(256) void k_probe_read(const u32x4 *__restrict__ p, int64_t n16,
                                                    uint32_t *sink)
{
    __shared__ uint32_t part[4];
    const int64_t stride = (int64_t)gridDim.x * 256;
    uint32_t x = 0;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {  // four loads in flight per thread
        const u32x4 v0 = p[i], v1 = p[i + stride], v2 = p[i + 2 * stride], v3 = p[i + 3 * stride];
        x += (v0[0] + v0[1] + v0[2] + v0[3]) + (v1[0] + v1[1] + v1[2] + v1[3]) +
             (v2[0] + v2[1] + v2[2] + v2[3]) + (v3[0] + v3[1] + v3[2] + v3[3]);
    }
    for (; i < n16; i += stride) {
        const u32x4 v = p[i];
        x += v[0] + v[1] + v[2] + v[3];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        x += (uint32_t)__shfl_xor((int)x, o);
    if ((threadIdx.x & 63) == 0)
        part[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0)
        sink[blockIdx.x] = part[0] + part[1] + part[2] + part[3];
}

// Random-row gather: for i < n, the row16 16-byte words of row idx[i] of the table, the
// workgroups striding over the n * row16 words one word per lane; sink[b] is the sum
// (mod 2^32) of the uint32 words workgroup b read.  The access pattern of the sparse
// attention's K/V gathers without the arithmetic.
__global__ __launch_bounds__(256) void k_probe_gather(const u32x4 *__restrict__ table,
                                                      int row16, const int32_t *__restrict__ idx,
                                                      int64_t n, uint32_t *sink)
{
    __shared__ uint32_t part[4];
    // word w = i * row16 + k; the stride is split once into rows and words, so the walk
    // needs no division
    const int64_t stride = (int64_t)gridDim.x * 256;
    const int64_t sq = stride / row16;
    const int sr = (int)(stride - sq * row16);
    const int64_t w0 = (int64_t)blockIdx.x * 256 + threadIdx.x;
    int64_t i = w0 / row16;
    int k = (int)(w0 - i * row16);
    auto step = [&](int64_t &ii, int &kk) {
        ii += sq;
        kk += sr;
        if (kk >= row16) {
            kk -= row16;
            ++ii;
        }
    };
    uint32_t x = 0;
    while (true) {  // four rows' words in flight per thread
        int64_t iu[4];
        int ku[4];
        iu[0] = i;
        ku[0] = k;
#pragma unroll
        for (int u = 1; u < 4; ++u) {
            iu[u] = iu[u - 1];
            ku[u] = ku[u - 1];
            step(iu[u], ku[u]);
        }
        if (iu[3] >= n)
            break;
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            v[u] = table[(int64_t)idx[iu[u]] * row16 + ku[u]];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            x += v[u][0] + v[u][1] + v[u][2] + v[u][3];
        i = iu[3];
        k = ku[3];
        step(i, k);
    }
    for (; i < n; step(i, k)) {
        const u32x4 v = table[(int64_t)idx[i] * row16 + k];
        x += v[0] + v[1] + v[2] + v[3];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        x += (uint32_t)__shfl_xor((int)x, o);
    if ((threadIdx.x & 63) == 0)
        part[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0)
        sink[blockIdx.x] = part[0] + part[1] + part[2] + part[3];
}

hipError_t launch_probe_gather(const void *table, int row16, const int32_t *idx, int64_t n,
                               uint32_t *sink, int blocks, hipStream_t stream)
{
    hipLaunchKernelGGL(k_probe_gather, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const u32x4 *>(table), row16, idx, n, sink);
    return hipGetLastError();
}

hipError_t launch_probe_mfma(int waves, int iters, float *sink, hipStream_t stream)
{
    const int blocks = (waves + 3) / 4;
    hipLaunchKernelGGL(k_probe_mfma, dim3((unsigned)blocks), dim3(256), 0, stream, iters, 1.0f,
                       sink, waves);
    return hipGetLastError();
}

hipError_t launch_probe_read(const void *buf, int64_t bytes, uint32_t *sink, int blocks,
                             hipStream_t stream)
{
    hipLaunchKernelGGL(k_probe_read, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const u32x4 *>(buf), bytes / 16, sink);
    return hipGetLastError();
}

} // namespace sgqa
