// Read-only gather of whole pool records at given slot ids: the memory access
// pattern of the INT2 history stream (page_size 1, one record per token) with
// no arithmetic and nothing written but one word per thread.  A measurement
// reference for the decode kernel's read rate, not a step of the method.
#include "common.h"
#include "internal.h"

namespace oscar {
namespace {

constexpr int kGatherThreads = 256;
constexpr int kGatherUnroll = 4;

// Thread t of the grid reads 16-byte unit e % UNITS of record idx[e / UNITS]
// for e = t, t + T, t + 2T, ... (T threads in the grid): consecutive lanes read
// consecutive units of one record, so each record is read as whole lines.
// Indices outside 0 .. num_rows - 1 read the last row.
template <int UNITS>
__global__ __launch_bounds__(kGatherThreads) void gather_read_kernel(const uint8_t *rows, const int32_t *idx,
                                                                     int64_t n, uint32_t last_row, uint32_t *sink) {
    // n * UNITS < 2^32 (checked on the host): 32-bit element indices
    const uint32_t total = uint32_t(n) * UNITS;
    const uint32_t stride = gridDim.x * kGatherThreads;
    uint32_t acc = 0;
    for (uint32_t e0 = blockIdx.x * kGatherThreads + threadIdx.x; e0 < total; e0 += kGatherUnroll * stride) {
        u32x4 v[kGatherUnroll];
#pragma unroll
        for (int k = 0; k < kGatherUnroll; ++k) {
            const uint32_t e = e0 + k * stride;
            v[k] = u32x4{0, 0, 0, 0};
            if (e < total) {
                const uint32_t r = e / UNITS;
                const uint32_t u = e - r * UNITS;
                const uint32_t row = min(uint32_t(idx[r]), last_row);
                const u32x4 *p = reinterpret_cast<const u32x4 *>(rows + int64_t(row) * (16 * UNITS)) + u;
                v[k] = __builtin_nontemporal_load(p);
            }
        }
#pragma unroll
        for (int k = 0; k < kGatherUnroll; ++k) acc ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
    }
    sink[int64_t(blockIdx.x) * kGatherThreads + threadIdx.x] = acc;
}

}  // namespace
}  // namespace oscar

using namespace oscar;

extern "C" oscar_status oscar_gather_read_reference(hipStream_t stream, const void *rows, int64_t row_bytes,
                                                    int64_t num_rows, const int32_t *idx, int64_t n,
                                                    uint32_t *sink, int64_t sink_words) {
    if (!rows || !idx || !sink) return fail(OSCAR_ERR_INVALID_ARG, "a required pointer is null");
    if (row_bytes != 768) return fail(OSCAR_ERR_UNSUPPORTED, "row_bytes must be 768 (8 KV heads of 96-byte head records)");
    if (n < 0 || n >= (int64_t(1) << 32) / 48 - 2048 * 256 * 4 || num_rows <= 0 || num_rows > (int64_t(1) << 31))
        return fail(OSCAR_ERR_INVALID_ARG, "n must be in 0 .. 89 M and num_rows in 1 .. 2^31");
    if (reinterpret_cast<uintptr_t>(rows) % 16 != 0) return fail(OSCAR_ERR_INVALID_ARG, "rows must be 16-byte aligned");
    if (sink_words < int64_t(OSCAR_GATHER_REF_SINK_WORDS))
        return fail(OSCAR_ERR_INVALID_ARG, "sink must hold OSCAR_GATHER_REF_SINK_WORDS words");
    if (n == 0) return OSCAR_OK;
    constexpr int blocks = OSCAR_GATHER_REF_SINK_WORDS / kGatherThreads;
    hipLaunchKernelGGL((gather_read_kernel<48>), dim3(blocks), dim3(kGatherThreads), 0, stream,
                       static_cast<const uint8_t *>(rows), idx, n, uint32_t(num_rows - 1), sink);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(OSCAR_ERR_HIP, std::string("gather reference launch: ") + hipGetErrorString(e));
    return OSCAR_OK;
}
