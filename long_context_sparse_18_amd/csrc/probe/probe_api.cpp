// probe_api.cpp -- C ABI of libsgqa_probe.so: argument checks and launches of the machine-peak
// probes (include/sgqa_probe.h).
#include "sgqa_probe.h"

#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "probe_launch.hpp"

namespace {

thread_local char g_probe_error[256] = "";

sgqa_status fail(sgqa_status st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_probe_error, sizeof(g_probe_error), fmt, ap);
    va_end(ap);
    return st;
}

sgqa_status hip_status(hipError_t e, const char *what)
{
    if (e == hipSuccess) {
        g_probe_error[0] = '\0';
        return SGQA_OK;
    }
    return fail(SGQA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void *p, uintptr_t a)
{
    return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

} // namespace

extern "C" {

sgqa_status sgqa_probe_mfma_bf16(int32_t waves, int32_t iters, float *sink, void *stream)
{
    if (waves < 1 || waves > (1 << 20) || iters < 1 || iters > 8192)
        return fail(SGQA_ERR_SHAPE, "probe needs 1 <= waves <= 2^20 and 1 <= iters <= 8192");
    if (!sink)
        return fail(SGQA_ERR_NULL, "sink is NULL");
    if (!aligned(sink, 4))
        return fail(SGQA_ERR_SHAPE, "sink must be 4-byte aligned");
    return hip_status(sgqa::launch_probe_mfma(waves, iters, sink,
                                              reinterpret_cast<hipStream_t>(stream)),
                      "probe_mfma launch");
}

sgqa_status sgqa_probe_read(const void *buf, size_t bytes, uint32_t *sink, int32_t blocks,
                            void *stream)
{
    if (bytes == 0 || bytes % 16 != 0 || blocks < 1 || blocks > 65536)
        return fail(SGQA_ERR_SHAPE, "probe needs bytes a positive multiple of 16 and 1..65536 "
                                    "workgroups");
    if (!buf || !sink)
        return fail(SGQA_ERR_NULL, "buf and sink must be non-NULL");
    if (!aligned(buf, 16) || !aligned(sink, 4))
        return fail(SGQA_ERR_SHAPE, "buf must be 16-byte and sink 4-byte aligned");
    return hip_status(sgqa::launch_probe_read(buf, (int64_t)bytes, sink, blocks,
                                              reinterpret_cast<hipStream_t>(stream)),
                      "probe_read launch");
}

sgqa_status sgqa_probe_gather(const void *table, int64_t table_rows, int32_t row_bytes,
                              const int32_t *idx, int64_t n, uint32_t *sink, int32_t blocks,
                              void *stream)
{
    if (table_rows < 1 || row_bytes < 16 || row_bytes > 65536 || row_bytes % 16 != 0 || n < 1 ||
        blocks < 1 || blocks > 65536)
        return fail(SGQA_ERR_SHAPE, "probe needs table_rows >= 1, row_bytes a multiple of 16 in "
                                    "[16, 65536], n >= 1 and 1..65536 workgroups");
    if (!table || !idx || !sink)
        return fail(SGQA_ERR_NULL, "table, idx and sink must be non-NULL");
    if (!aligned(table, 16) || !aligned(idx, 4) || !aligned(sink, 4))
        return fail(SGQA_ERR_SHAPE, "table must be 16-byte, idx and sink 4-byte aligned");
    return hip_status(sgqa::launch_probe_gather(table, row_bytes / 16, idx, n, sink, blocks,
                                                reinterpret_cast<hipStream_t>(stream)),
                      "probe_gather launch");
}

const char *sgqa_probe_last_error(void)
{
    return g_probe_error;
}

} // extern "C"
