// BF16 paged KV cache: append and split-K decode attention.
//
// This is the comparison point of the OSCAR announcement's "Results" section
// (decode speed-up at 100K context and job throughput at batch 32 are both
// quoted against a BF16 KV cache): the same page_size-1 pool of token slots,
// holding every token's K and V in BF16, unrotated.  The decode reads each
// token's 512 bytes per KV head once; the INT2 path reads 96.
//
// Pool layout: [num_slots][Hkv][2][128] bf16 (K then V of each KV head), so
// one token's rows for all heads are one contiguous 4 KB record at 8 heads.
//
// Decode: one wave per (request, work item, KV head), four KV heads per
// workgroup.  A work item is a chunk of the request's positions; each wave
// walks its chunk in steps of 32 tokens:
//   * slot ids of the next step are fetched one step ahead;
//   * QK on the matrix cores: A = the g query rows of the KV head (scaled by
//     sm_scale log2 e, split into bf16 hi + lo parts), B = the K rows as
//     loaded (lane l holds 16 bytes of token l % 16), 16 MFMAs per step;
//   * online softmax in log2 units on the 16 lanes of each output row group;
//   * PV on fp32 VALU: lane = channel pair, one coalesced 256-byte V row
//     load per token (the slot id is wave-uniform), weights from LDS.
// A merge kernel combines the chunks' (m, l, o) by log-sum-exp.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <algorithm>
#include <cmath>
#include <string>

#include "common.h"
#include "internal.h"

namespace oscar {
namespace {

constexpr int kStepTokens = 32;
constexpr int kWaves = 4;                 // KV heads per workgroup
constexpr int kRowElems = 2 * kHeadDim;   // K and V of one (slot, KV head)

struct Bf16Args {
    const uint16_t *kv;
    const void *q;
    const int32_t *req_ids;
    const int32_t *seq_lens;
    const int32_t *req_to_slot;
    void *out;
    float *part_o;     // [B][items][Hq][128]
    float *part_ml;    // [B][items][Hq][2]
    int64_t r2s_stride;
    int64_t num_slots;
    float scale_log2;
    int32_t q_dtype;
    int32_t out_dtype;
    int32_t batch;
    int32_t hkv;
    int32_t hq;
    int32_t g;
    int32_t max_requests;
    int32_t chunk;
    int32_t items;
    int32_t head_chunks;
};

__device__ __forceinline__ float load_f32(const void *p, int dtype, size_t idx) {
    if (dtype == OSCAR_F32) return static_cast<const float *>(p)[idx];
    const uint16_t u = static_cast<const uint16_t *>(p)[idx];
    if (dtype == OSCAR_BF16) return bf16_bits_to_f32(u);
    return __half2float(__ushort_as_half(u));
}

__device__ __forceinline__ int request_of(const Bf16Args &a, int b, int &req) {
    req = a.req_ids[b];
    const int L = a.seq_lens[b];
    if (req < 0 || req >= a.max_requests || L < 0) return 0;
    return int(min<int64_t>(L, a.r2s_stride));
}

template <int K>
__device__ __forceinline__ float ror16(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x120 + K, 0xF, 0xF, false));
}
__device__ __forceinline__ float max16(float v) {
    v = fmaxf(v, ror16<1>(v));
    v = fmaxf(v, ror16<2>(v));
    v = fmaxf(v, ror16<4>(v));
    return fmaxf(v, ror16<8>(v));
}
__device__ __forceinline__ float sum16(float v) {
    v += ror16<1>(v);
    v += ror16<2>(v);
    v += ror16<4>(v);
    return v + ror16<8>(v);
}
__device__ __forceinline__ float bcast(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

template <int GQ>
__global__ __launch_bounds__(64 * kWaves) void bf16_partial_kernel(Bf16Args a) {
    // weights p of the current step: [wave][token][head row]
    __shared__ __attribute__((aligned(16))) float ps_all[kWaves][kStepTokens][16];
    const int id = blockIdx.x;
    const int hc = id % a.head_chunks;
    const int rest = id / a.head_chunks;
    const int b = rest % a.batch;
    const int j = rest / a.batch;
    int req = 0;
    const int L = request_of(a, b, req);
    const int p0 = j * a.chunk;
    const int p1 = min(L, p0 + a.chunk);
    const int w = threadIdx.x >> 6;
    const int hk = hc * kWaves + w;
    if (p0 >= p1 || hk >= a.hkv) return;   // no workgroup barrier below: waves exit on their own
    const int lane = threadIdx.x & 63;
    const int col = lane & 15;             // MFMA column (token) / A row (head)
    const int kq = lane >> 4;              // MFMA k-slot group
    float(*ps)[16] = ps_all[w];

    // A operands: row = query head hk * GQ + col (zero past GQ), k-slots of
    // step s = channels 32 s + 8 kq .. + 7
    bf16x8 ahi[4], alo[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = 0.0f;
            if (col < GQ)
                x = load_f32(a.q, a.q_dtype, (size_t(b) * a.hq + hk * GQ + col) * kHeadDim + 32 * s + 8 * kq + e) *
                    a.scale_log2;
            const uint16_t hi = bf16_bits_rn(x);
            const uint16_t lo = bf16_bits_rn(x - bf16_bits_to_f32(hi));
            ahi[s][e] = bits_to_bf16(hi);
            alo[s][e] = bits_to_bf16(lo);
        }
    }

    float m_run[4], l_lane[4];      // head row 4 kq + r, per lane of its row group
    float o0[GQ], o1[GQ];           // channels 2 lane, 2 lane + 1 of query head hk * GQ + h
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        m_run[r] = -INFINITY;
        l_lane[r] = 0.0f;
    }
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
        o0[h] = 0.0f;
        o1[h] = 0.0f;
    }

    const int32_t *tab = a.req_to_slot + size_t(req) * a.r2s_stride;
    const uint16_t *kv_head = a.kv + size_t(hk) * kRowElems;
    const size_t slot_stride = size_t(a.hkv) * kRowElems;
    // slot of token (lane % 32) of the step at position c; -1 past the item
    auto slot_at = [&](int c) -> int {
        const int p = c + (lane & 31);
        return p < p1 ? __builtin_nontemporal_load(tab + p) : -1;
    };
    int slot_next = slot_at(p0);

    for (int cb = p0; cb < p1; cb += kStepTokens) {
        const int slot_raw = slot_next;
        if (cb + kStepTokens < p1) slot_next = slot_at(cb + kStepTokens);
        const bool ok = slot_raw >= 0 && slot_raw < a.num_slots;
        const int slot = ok ? slot_raw : 0;                       // a readable row for masked tokens
        const uint64_t okmask = __ballot(ok) & 0xFFFFFFFFull;     // token t usable <=> bit t

        // ---- loads: K fragments (token 16 tb + col, 16 bytes of k-slot group kq of step s)
        u32x4 kf[2][4];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const int st = __shfl(slot, 16 * tb + col);
            const u32x4 *src = reinterpret_cast<const u32x4 *>(kv_head + size_t(st) * slot_stride + 8 * kq);
#pragma unroll
            for (int s = 0; s < 4; ++s) kf[tb][s] = __builtin_nontemporal_load(src + 4 * s);
        }
        // V: channels 2 lane, 2 lane + 1 of every token of the step
        uint32_t vw[kStepTokens];
#pragma unroll
        for (int u = 0; u < kStepTokens; ++u) {
            const int su = __builtin_amdgcn_readlane(slot, u);
            vw[u] = __builtin_nontemporal_load(
                reinterpret_cast<const uint32_t *>(kv_head + size_t(su) * slot_stride + kHeadDim) + lane);
        }

        // ---- QK: logits (log2 units) of head row 4 kq + r, token 16 tb + col
        f32x4 d[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bf16x8 bk = __builtin_bit_cast(bf16x8, kf[tb][s]);
                acc = mfma_bf16(ahi[s], bk, acc);
                acc = mfma_bf16(alo[s], bk, acc);
            }
            d[tb] = acc;
        }

        // ---- online softmax
        float alpha[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float x[2];
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                const int t = 16 * tb + col;
                x[tb] = ((okmask >> t) & 1) ? d[tb][r] : -INFINITY;
            }
            const float mt = max16(fmaxf(x[0], x[1]));
            const float m_new = fmaxf(m_run[r], mt);
            alpha[r] = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run[r] - m_new);
            m_run[r] = m_new;
            float lsum = 0.0f;
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                const float p = x[tb] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(x[tb] - m_new);
                lsum += p;
                ps[16 * tb + col][4 * kq + r] = p;
            }
            l_lane[r] = fmaf(l_lane[r], alpha[r], lsum);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // ---- PV: rescale, then accumulate the step's tokens
#pragma unroll
        for (int h = 0; h < GQ; ++h) {
            const float al = bcast(alpha[h & 3], 16 * (h >> 2));
            o0[h] *= al;
            o1[h] *= al;
        }
#pragma unroll
        for (int u = 0; u < kStepTokens; ++u) {
            const bool use = (okmask >> u) & 1;
            const uint32_t v = use ? vw[u] : 0u;                  // masked rows may hold anything
            const float v0 = bf16_bits_to_f32(v & 0xFFFFu), v1 = __uint_as_float(v & 0xFFFF0000u);
            float p[GQ];
#pragma unroll
            for (int h4 = 0; h4 < GQ; h4 += 4) {
                const f32x4 q4 = *reinterpret_cast<const f32x4 *>(&ps[u][h4]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (h4 + e < GQ) p[h4 + e] = q4[e];
            }
#pragma unroll
            for (int h = 0; h < GQ; ++h) {
                o0[h] = fmaf(p[h], v0, o0[h]);
                o1[h] = fmaf(p[h], v1, o1[h]);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // ---- partials of query heads hk * GQ + h
    const size_t row0 = (size_t(b) * a.items + j) * a.hq + size_t(hk) * GQ;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float l = sum16(l_lane[r]);
        const int h = 4 * kq + r;
        if (col == 0 && h < GQ) {
            a.part_ml[(row0 + h) * 2 + 0] = m_run[r];
            a.part_ml[(row0 + h) * 2 + 1] = l;
        }
    }
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
        float2 *dst = reinterpret_cast<float2 *>(a.part_o + (row0 + h) * kHeadDim) + lane;
        *dst = make_float2(o0[h], o1[h]);
    }
}

// One workgroup per (request, KV head); thread (h, c) merges channel c of
// query head h over the request's items, 16 items' loads in flight at a time.
__global__ __launch_bounds__(512) void bf16_merge_kernel(Bf16Args a) {
    const int b = blockIdx.x / a.hkv;
    const int hk = blockIdx.x % a.hkv;
    const int c = threadIdx.x & (kHeadDim - 1);
    int req = 0;
    const int L = request_of(a, b, req);
    const int n_items = min(a.items, (L + a.chunk - 1) / a.chunk);
    for (int h = threadIdx.x >> 7; h < a.g; h += 4) {
        const size_t row_h = size_t(b) * a.items * a.hq + size_t(hk) * a.g + h;
        float M = -INFINITY;
#pragma unroll 16
        for (int jj = 0; jj < n_items; ++jj) M = fmaxf(M, a.part_ml[(row_h + size_t(jj) * a.hq) * 2]);
        float l = 0.0f, acc = 0.0f;
        if (M != -INFINITY) {
#pragma unroll 16
            for (int jj = 0; jj < n_items; ++jj) {
                const size_t row = row_h + size_t(jj) * a.hq;
                const float e = __builtin_amdgcn_exp2f(a.part_ml[row * 2] - M);
                l = fmaf(e, a.part_ml[row * 2 + 1], l);
                acc = fmaf(e, a.part_o[row * kHeadDim + c], acc);
            }
        }
        const float o = l > 0.0f ? acc / l : 0.0f;
        const size_t idx = (size_t(b) * a.hq + size_t(hk) * a.g + h) * kHeadDim + c;
        if (a.out_dtype == OSCAR_F32)
            static_cast<float *>(a.out)[idx] = o;
        else if (a.out_dtype == OSCAR_BF16)
            static_cast<uint16_t *>(a.out)[idx] = bf16_bits_rn(o);
        else
            static_cast<__half *>(a.out)[idx] = __float2half_rn(o);
    }
}

struct AppendArgs {
    uint16_t *kv;
    const void *k;
    const void *v;
    const int32_t *slots;
    int64_t num_slots;
    int64_t quads;     // n_tokens * Hkv * 2 * 32: four channels each
    int32_t hkv;
    int32_t dtype;
};

// Thread = four consecutive channels of one (token, KV head, K or V).
__global__ __launch_bounds__(256) void bf16_append_kernel(AppendArgs a) {
    for (int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; e < a.quads;
         e += int64_t(gridDim.x) * blockDim.x) {
        const int c4 = int(e & 31);
        const int64_t r = e >> 5;                  // (token, head, t) row
        const int t = int(r & 1);
        const int64_t th = r >> 1;                 // token * hkv + head
        const int64_t tok = th / a.hkv;
        const int slot = a.slots[tok];
        if (slot < 0 || slot >= a.num_slots) continue;
        const int h = int(th - tok * a.hkv);
        const size_t src = size_t(th) * kHeadDim + 4 * c4;
        const void *in = t ? a.v : a.k;
        uint16_t bits[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) bits[i] = bf16_bits_rn(load_f32(in, a.dtype, src + i));
        uint2 packed;
        packed.x = uint32_t(bits[0]) | (uint32_t(bits[1]) << 16);
        packed.y = uint32_t(bits[2]) | (uint32_t(bits[3]) << 16);
        *reinterpret_cast<uint2 *>(a.kv + (size_t(slot) * a.hkv + h) * kRowElems + t * kHeadDim + 4 * c4) = packed;
    }
}

struct Bf16Plan {
    int32_t chunk = 0;
    int32_t items = 0;
    int32_t max_len = 0;
    size_t ws_part_o = 0;
    size_t ws_part_ml = 0;
    size_t ws_bytes = 0;
};

oscar_status make_bf16_plan(const oscar_layout &lay, int32_t batch, const int32_t *lens,
                            const oscar_launch_opts *opts, Bf16Plan *plan) {
    if (batch < 1) return fail(OSCAR_ERR_INVALID_ARG, "batch must be >= 1");
    if (!lens) return fail(OSCAR_ERR_INVALID_ARG, "seq_lens_host is null");
    int64_t total = 0, max_len = 0;
    for (int32_t b = 0; b < batch; ++b) {
        if (lens[b] < 1) return fail(OSCAR_ERR_INVALID_ARG, "every sequence length must be >= 1");
        total += lens[b];
        max_len = std::max<int64_t>(max_len, lens[b]);
    }
    int64_t chunk;
    if (opts && opts->history_chunk > 0) {
        if (opts->history_chunk % kStepTokens)
            return fail(OSCAR_ERR_INVALID_ARG, "history_chunk must be a multiple of 32");
        chunk = opts->history_chunk;
    } else {
        // about 1,024 work items over the batch (a few per compute unit and
        // head chunk), each a whole number of 32-token steps
        chunk = (total + 1023) / 1024;
        chunk = (chunk + kStepTokens - 1) / kStepTokens * kStepTokens;
        chunk = std::min<int64_t>(8192, std::max<int64_t>(256, chunk));
    }
    const int64_t items = (max_len + chunk - 1) / chunk;
    const int64_t head_chunks = (lay.num_kv_heads + kWaves - 1) / kWaves;
    if (items * batch * head_chunks > INT32_MAX)
        return fail(OSCAR_ERR_UNSUPPORTED, "batch x work items exceeds one launch grid");
    auto align = [](size_t x) { return (x + 255) / 256 * 256; };
    plan->chunk = int32_t(chunk);
    plan->items = int32_t(items);
    plan->max_len = int32_t(max_len);
    size_t off = 0;
    plan->ws_part_o = off;
    off += align(size_t(batch) * items * lay.num_q_heads * kHeadDim * sizeof(float));
    plan->ws_part_ml = off;
    off += align(size_t(batch) * items * lay.num_q_heads * 2 * sizeof(float));
    plan->ws_bytes = off;
    return OSCAR_OK;
}

template <int GQ>
hipError_t launch_bf16_partial(const Bf16Args &a, int blocks, hipStream_t stream) {
    hipLaunchKernelGGL(bf16_partial_kernel<GQ>, dim3(blocks), dim3(64 * kWaves), 0, stream, a);
    return hipGetLastError();
}

bool valid_dtype(oscar_dtype d) { return d == OSCAR_F32 || d == OSCAR_BF16 || d == OSCAR_F16; }

}  // namespace
}  // namespace oscar

using namespace oscar;

extern "C" size_t oscar_bf16_pool_bytes(const oscar_layout *layout) {
    if (check_layout(layout) != OSCAR_OK) return 0;
    return size_t(layout->num_slots) * layout->num_kv_heads * kRowElems * sizeof(uint16_t);
}

extern "C" oscar_status oscar_bf16_append(hipStream_t stream, const oscar_layout *layout, uint16_t *kv_pool,
                                          const void *k, const void *v, oscar_dtype dtype, int32_t n_tokens,
                                          const int32_t *slots) {
    oscar_status st = check_layout(layout);
    if (st != OSCAR_OK) return st;
    if (n_tokens < 0) return fail(OSCAR_ERR_INVALID_ARG, "n_tokens must be >= 0");
    if (n_tokens == 0) return OSCAR_OK;
    if (!kv_pool || !k || !v || !slots) return fail(OSCAR_ERR_INVALID_ARG, "a required pointer is null");
    if (!valid_dtype(dtype)) return fail(OSCAR_ERR_INVALID_ARG, "dtype must be F32, BF16 or F16");
    AppendArgs a;
    a.kv = kv_pool;
    a.k = k;
    a.v = v;
    a.slots = slots;
    a.num_slots = layout->num_slots;
    a.hkv = layout->num_kv_heads;
    a.dtype = dtype;
    a.quads = int64_t(n_tokens) * layout->num_kv_heads * 2 * (kHeadDim / 4);
    const int64_t blocks = std::min<int64_t>((a.quads + 255) / 256, 8192);
    hipLaunchKernelGGL(bf16_append_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(OSCAR_ERR_HIP, std::string("bf16 append launch: ") + hipGetErrorString(e));
    return OSCAR_OK;
}

extern "C" oscar_status oscar_bf16_decode_workspace_size(const oscar_layout *layout, int32_t batch,
                                                         const int32_t *seq_lens_host,
                                                         const oscar_launch_opts *opts, size_t *bytes) {
    oscar_status st = check_layout(layout);
    if (st != OSCAR_OK) return st;
    if (!bytes) return fail(OSCAR_ERR_INVALID_ARG, "bytes is null");
    Bf16Plan plan;
    st = make_bf16_plan(*layout, batch, seq_lens_host, opts, &plan);
    if (st != OSCAR_OK) return st;
    *bytes = plan.ws_bytes;
    return OSCAR_OK;
}

extern "C" oscar_status oscar_bf16_decode_attn(hipStream_t stream, const oscar_layout *layout,
                                               const uint16_t *kv_pool, const void *q, oscar_dtype q_dtype,
                                               int32_t batch, const int32_t *req_ids, const int32_t *seq_lens,
                                               const int32_t *seq_lens_host, const int32_t *req_to_slot,
                                               int64_t req_to_slot_stride, float sm_scale, void *out,
                                               oscar_dtype out_dtype, void *workspace, size_t workspace_bytes,
                                               const oscar_launch_opts *opts) {
    oscar_status st = check_layout(layout);
    if (st != OSCAR_OK) return st;
    if (!kv_pool || !q || !req_ids || !seq_lens || !req_to_slot || !out)
        return fail(OSCAR_ERR_INVALID_ARG, "a required pointer is null");
    if (layout->num_slots < 1) return fail(OSCAR_ERR_INVALID_ARG, "the BF16 pool needs num_slots >= 1");
    if (!valid_dtype(q_dtype)) return fail(OSCAR_ERR_INVALID_ARG, "q_dtype must be F32, BF16 or F16");
    if (!valid_dtype(out_dtype)) return fail(OSCAR_ERR_INVALID_ARG, "out_dtype must be F32, BF16 or F16");
    if (!std::isfinite(sm_scale)) return fail(OSCAR_ERR_INVALID_ARG, "sm_scale must be finite");
    Bf16Plan plan;
    st = make_bf16_plan(*layout, batch, seq_lens_host, opts, &plan);
    if (st != OSCAR_OK) return st;
    if (req_to_slot_stride < plan.max_len)
        return fail(OSCAR_ERR_INVALID_ARG, "req_to_slot_stride is smaller than the longest sequence");
    if (!workspace || workspace_bytes < plan.ws_bytes)
        return fail(OSCAR_ERR_WORKSPACE, "workspace is smaller than the size the library reported");
    if (reinterpret_cast<uintptr_t>(workspace) % 256)
        return fail(OSCAR_ERR_INVALID_ARG, "workspace must be 256-byte aligned");

    Bf16Args a;
    a.kv = kv_pool;
    a.q = q;
    a.req_ids = req_ids;
    a.seq_lens = seq_lens;
    a.req_to_slot = req_to_slot;
    a.out = out;
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    a.part_o = reinterpret_cast<float *>(ws + plan.ws_part_o);
    a.part_ml = reinterpret_cast<float *>(ws + plan.ws_part_ml);
    a.r2s_stride = req_to_slot_stride;
    a.num_slots = layout->num_slots;
    a.scale_log2 = sm_scale * 1.4426950408889634f;
    a.q_dtype = q_dtype;
    a.out_dtype = out_dtype;
    a.batch = batch;
    a.hkv = layout->num_kv_heads;
    a.hq = layout->num_q_heads;
    a.g = layout->num_q_heads / layout->num_kv_heads;
    a.max_requests = layout->max_requests;
    a.chunk = plan.chunk;
    a.items = plan.items;
    a.head_chunks = (a.hkv + kWaves - 1) / kWaves;

    if (opts && opts->kernel_begin && hipEventRecord(opts->kernel_begin, stream) != hipSuccess)
        return fail(OSCAR_ERR_HIP, "hipEventRecord failed");
    const int blocks = plan.items * batch * a.head_chunks;
    hipError_t e;
    switch (a.g) {
        case 1: e = launch_bf16_partial<1>(a, blocks, stream); break;
        case 2: e = launch_bf16_partial<2>(a, blocks, stream); break;
        case 3: e = launch_bf16_partial<3>(a, blocks, stream); break;
        case 4: e = launch_bf16_partial<4>(a, blocks, stream); break;
        case 5: e = launch_bf16_partial<5>(a, blocks, stream); break;
        case 6: e = launch_bf16_partial<6>(a, blocks, stream); break;
        case 7: e = launch_bf16_partial<7>(a, blocks, stream); break;
        default: e = launch_bf16_partial<8>(a, blocks, stream); break;
    }
    if (e != hipSuccess) return fail(OSCAR_ERR_HIP, std::string("bf16 partial launch: ") + hipGetErrorString(e));
    if (opts && opts->kernel_end && hipEventRecord(opts->kernel_end, stream) != hipSuccess)
        return fail(OSCAR_ERR_HIP, "hipEventRecord failed");
    hipLaunchKernelGGL(bf16_merge_kernel, dim3(batch * a.hkv), dim3(512), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(OSCAR_ERR_HIP, std::string("bf16 merge launch: ") + hipGetErrorString(e));
    return OSCAR_OK;
}
