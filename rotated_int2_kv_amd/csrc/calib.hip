// Calibration statistics: Gram sums of captured activations per KV head.
//
// The OSCAR page ("What OSCAR does differently") builds the key basis from
// the query covariance C_Q = (1/N) sum q^T q and the value basis from
// C_S = (1/N) V^T S^T S V, which is (1/N) sum o^T o over the attention
// outputs o = S V of the same query rows.  Both are the Gram matrix of a set
// of 128-wide rows, pooled over the g query heads that share a KV head.  This
// file accumulates those sums on the matrix cores:
//   * gram_partial_kernel: one workgroup per (row slab, KV head) stages 32
//     rows at a time in LDS as fp32 and accumulates X^T X with
//     v_mfma_f32_16x16x4_f32 (exact fp32 products); wave w owns the 64 x 64
//     quadrant (w / 2, w % 2) of the 128 x 128 result;
//   * gram_reduce_kernel: adds the slabs' partial sums in fp64 into the
//     caller's accumulator (one thread per element: deterministic).
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <algorithm>
#include <string>

#include "common.h"
#include "internal.h"

namespace oscar {
namespace {

constexpr int kStageRows = 32;
constexpr int kXsStride = kHeadDim + 4;     // floats per staged row (bank offset 4 per row)
constexpr int kMaxSlabs = 64;               // partial sums per KV head
constexpr int kMinSlabRows = 512;

struct GramArgs {
    const void *x;          // [n_rows][Hq][128]
    float *part;            // [Hkv][slabs][128][128]
    double *acc;            // [Hkv][128][128]
    int64_t n_rows;
    int64_t slab_rows;      // pooled rows per slab
    int32_t dtype;
    int32_t hq;
    int32_t g;
    int32_t hkv;
    int32_t slabs;
};

__device__ __forceinline__ float load_x(const void *p, int dtype, size_t idx) {
    if (dtype == OSCAR_F32) return static_cast<const float *>(p)[idx];
    const uint16_t u = static_cast<const uint16_t *>(p)[idx];
    if (dtype == OSCAR_BF16) return bf16_bits_to_f32(u);
    return __half2float(__ushort_as_half(u));
}

__global__ __launch_bounds__(256) void gram_partial_kernel(GramArgs a) {
    __shared__ __attribute__((aligned(16))) float xs[kStageRows][kXsStride];
    const int slab = blockIdx.x;
    const int hk = blockIdx.y;
    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63;
    const int col = lane & 15, kk = lane >> 4;
    const int I = 64 * (w >> 1), J = 64 * (w & 1);
    const int64_t total = a.n_rows * a.g;                   // pooled rows of this KV head
    const int64_t r0 = int64_t(slab) * a.slab_rows;
    const int64_t r1 = min(total, r0 + a.slab_rows);

    f32x4 c[4][4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
        for (int tj = 0; tj < 4; ++tj) c[ti][tj] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // staging: thread (row sr, channels 16 sc .. +15)
    const int sr = tid >> 3, sc = tid & 7;
    for (int64_t rb = r0; rb < r1; rb += kStageRows) {
        __syncthreads();                                    // previous stage consumed
        const int64_t r = rb + sr;
        float v[16];
        if (r < r1) {
            const int64_t n = r / a.g;
            const int hh = int(r - n * a.g);
            const size_t base = (size_t(n) * a.hq + size_t(hk) * a.g + hh) * kHeadDim + 16 * sc;
#pragma unroll
            for (int e = 0; e < 16; ++e) v[e] = load_x(a.x, a.dtype, base + e);
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) v[e] = 0.0f;       // rows past the slab add nothing
        }
#pragma unroll
        for (int e = 0; e < 16; e += 4)
            *reinterpret_cast<f32x4 *>(&xs[sr][16 * sc + e]) = f32x4{v[e], v[e + 1], v[e + 2], v[e + 3]};
        __syncthreads();
        // C[i][j] += sum_k X[k][I + i] X[k][J + j]: A = X^T (lane: i = col, k = kk), B = X
#pragma unroll 2
        for (int k0 = 0; k0 < kStageRows; k0 += 4) {
            float av[4], bv[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                av[t] = xs[k0 + kk][I + 16 * t + col];
                bv[t] = xs[k0 + kk][J + 16 * t + col];
            }
#pragma unroll
            for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                for (int tj = 0; tj < 4; ++tj)
                    c[ti][tj] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[ti], bv[tj], c[ti][tj], 0, 0, 0);
        }
    }
    // lane holds C rows I + 16 ti + 4 kk + e, column J + 16 tj + col
    float *out = a.part + (size_t(hk) * a.slabs + slab) * kHeadDim * kHeadDim;
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
        for (int tj = 0; tj < 4; ++tj)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                out[size_t(I + 16 * ti + 4 * kk + e) * kHeadDim + J + 16 * tj + col] = c[ti][tj][e];
}

__global__ __launch_bounds__(256) void gram_reduce_kernel(GramArgs a) {
    const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;    // over Hkv x 128 x 128
    if (idx >= int64_t(a.hkv) * kHeadDim * kHeadDim) return;
    const int hk = int(idx / (kHeadDim * kHeadDim));
    const int e = int(idx - int64_t(hk) * kHeadDim * kHeadDim);
    double s = 0.0;
    for (int b = 0; b < a.slabs; ++b) s += double(a.part[(size_t(hk) * a.slabs + b) * kHeadDim * kHeadDim + e]);
    a.acc[idx] += s;
}

void gram_plan(const oscar_layout &lay, int64_t n_rows, int32_t *slabs, int64_t *slab_rows) {
    const int64_t total = n_rows * (lay.num_q_heads / lay.num_kv_heads);
    int64_t s = (total + kMinSlabRows - 1) / kMinSlabRows;
    s = std::max<int64_t>(1, std::min<int64_t>(kMaxSlabs, s));
    int64_t rows = (total + s - 1) / s;
    rows = (rows + kStageRows - 1) / kStageRows * kStageRows;
    *slabs = int32_t(s);
    *slab_rows = std::max<int64_t>(kStageRows, rows);
}

}  // namespace
}  // namespace oscar

using namespace oscar;

extern "C" oscar_status oscar_covariance_workspace_size(const oscar_layout *layout, int64_t n_rows, size_t *bytes) {
    oscar_status st = check_layout(layout);
    if (st != OSCAR_OK) return st;
    if (!bytes) return fail(OSCAR_ERR_INVALID_ARG, "bytes is null");
    if (n_rows < 0) return fail(OSCAR_ERR_INVALID_ARG, "n_rows must be >= 0");
    int32_t slabs = 0;
    int64_t slab_rows = 0;
    gram_plan(*layout, n_rows, &slabs, &slab_rows);
    *bytes = size_t(layout->num_kv_heads) * slabs * kHeadDim * kHeadDim * sizeof(float);
    return OSCAR_OK;
}

extern "C" oscar_status oscar_covariance_accumulate(hipStream_t stream, const oscar_layout *layout, const void *x,
                                                    oscar_dtype dtype, int64_t n_rows, double *acc,
                                                    void *workspace, size_t workspace_bytes) {
    oscar_status st = check_layout(layout);
    if (st != OSCAR_OK) return st;
    if (n_rows < 0) return fail(OSCAR_ERR_INVALID_ARG, "n_rows must be >= 0");
    if (n_rows == 0) return OSCAR_OK;
    if (!x || !acc) return fail(OSCAR_ERR_INVALID_ARG, "a required pointer is null");
    if (dtype != OSCAR_F32 && dtype != OSCAR_BF16 && dtype != OSCAR_F16)
        return fail(OSCAR_ERR_INVALID_ARG, "dtype must be F32, BF16 or F16");
    if (n_rows > int64_t(1) << 40) return fail(OSCAR_ERR_UNSUPPORTED, "n_rows is too large");
    GramArgs a;
    a.x = x;
    a.acc = acc;
    a.n_rows = n_rows;
    a.dtype = dtype;
    a.hq = layout->num_q_heads;
    a.hkv = layout->num_kv_heads;
    a.g = layout->num_q_heads / layout->num_kv_heads;
    gram_plan(*layout, n_rows, &a.slabs, &a.slab_rows);
    const size_t need = size_t(a.hkv) * a.slabs * kHeadDim * kHeadDim * sizeof(float);
    if (!workspace || workspace_bytes < need)
        return fail(OSCAR_ERR_WORKSPACE, "workspace is smaller than the size the library reported");
    if (reinterpret_cast<uintptr_t>(workspace) % 256)
        return fail(OSCAR_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    a.part = static_cast<float *>(workspace);
    hipLaunchKernelGGL(gram_partial_kernel, dim3(a.slabs, a.hkv), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(OSCAR_ERR_HIP, std::string("gram launch: ") + hipGetErrorString(e));
    const int64_t elems = int64_t(a.hkv) * kHeadDim * kHeadDim;
    hipLaunchKernelGGL(gram_reduce_kernel, dim3(unsigned((elems + 255) / 256)), dim3(256), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(OSCAR_ERR_HIP, std::string("gram reduce launch: ") + hipGetErrorString(e));
    return OSCAR_OK;
}
