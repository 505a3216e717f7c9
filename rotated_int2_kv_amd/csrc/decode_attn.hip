// oscar_decode_attn: decode attention over the three-region cache (Together
// AI OSCAR page, "What OSCAR does differently" for the rotated-basis logits
// and "Serving system" for the sink / INT2 history / recent layout; query head
// h reads KV head h / g as in the Qiita article, "Fix 4").
//
// Three kernels on the caller's stream:
//   1. prep:    q' = q R_K * sm_scale * log2(e) per (request, KV head), plus
//               per-group sums of q' (for the zero-point term).
//   2. partial: split-K.  Work item j of request b is the sink window (j = 0),
//               the recent window (j = 1) or history chunk j - 2.  One wave per
//               KV head; the workgroup holds all KV heads of the item so that
//               the slot-major records are read as whole cache lines.
//               History tiles of 32 tokens run on f16 MFMA:
//                 QK: A = s * code, dequantised in the operand and exact: the
//                     scale is split into s_hi (9 significant bits) and s_lo
//                     (the 2 low bits), so c s_hi and c s_lo are exact fp16
//                     values and both are accumulated; B = q' split into fp16
//                     hi + lo columns; one extra MFMA adds sum_g z_g Qbar_g.
//                 PV: A = softmax weights split hi + lo rows, B = s * code of 8
//                     tokens per lane, split the same way; one extra MFMA adds
//                     sum_t p_t z_t.
//               BF16 windows run on fp32 VALU.  Each item writes (m, l, o')
//               with m in log2 units.
//   3. merge:   log-sum-exp merge of the items and o = o' R_V^T.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <cmath>

#include "common.cuh"
#include "internal.h"

namespace oscar {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kTileTokens = 32;      // history tokens per MFMA tile
constexpr int kBf16Chunk = 64;       // BF16-window tokens per VALU step

struct DecodeArgs {
    const void *q;
    const int32_t *req_ids;
    const int32_t *seq_lens;
    const int32_t *req_to_slot;
    const float *r_k;
    const float *r_v;
    const uint8_t *records;
    const uint16_t *sink;
    const uint16_t *recent;
    void *out;
    float *qrot;       // [B][Hq][128], log2-scaled rotated query
    float *qsum;       // [B][Hq][4], group sums of qrot
    float *part_o;     // [B][items][Hq][128]
    float *part_ml;    // [B][items][Hq][2] (m, l)
    int64_t r2s_stride;
    int64_t num_slots;
    float scale_log2;
    int32_t q_dtype;
    int32_t out_dtype;
    int32_t batch;
    int32_t hkv;
    int32_t hq;
    int32_t g;
    int32_t sink_tokens;
    int32_t recent_tokens;
    int32_t max_requests;
    int32_t chunk;
    int32_t items;
    int32_t waves;     // KV heads per workgroup
    int32_t head_chunks;
};

// Position range [p0, p1) of work item j of a request of length L.
__device__ __forceinline__ void item_range(const DecodeArgs &a, int L, int j, int &p0, int &p1) {
    const int S = a.sink_tokens, W = a.recent_tokens;
    const int hist_end = max(S, L - W);
    if (j == 0) {
        p0 = 0;
        p1 = min(S, L);
    } else if (j == 1) {
        p0 = L > S ? hist_end : L;
        p1 = L;
    } else {
        p0 = S + (j - 2) * a.chunk;
        p1 = min(p0 + a.chunk, hist_end);
    }
}

__device__ __forceinline__ int request_length(const DecodeArgs &a, int b, int &req) {
    req = a.req_ids[b];
    int L = a.seq_lens[b];
    if (req < 0 || req >= a.max_requests || L < 0) return 0;
    // never read past a row of the index table
    return int(min<int64_t>(L, a.r2s_stride));
}

__device__ __forceinline__ float load_as_f32(const void *p, int dtype, size_t idx) {
    if (dtype == OSCAR_F32) return static_cast<const float *>(p)[idx];
    const uint16_t u = static_cast<const uint16_t *>(p)[idx];
    if (dtype == OSCAR_BF16) return bf16_bits_to_f32(u);
    return __half2float(__ushort_as_half(u));
}

// ---------------------------------------------------------------------------
// 1. query rotation
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(128) void prep_kernel(DecodeArgs a) {
    __shared__ float qs[kMaxGroup][kHeadDim];
    __shared__ float qr[kMaxGroup][kHeadDim];
    const int b = blockIdx.x / a.hkv;
    const int hk = blockIdx.x % a.hkv;
    const int c = threadIdx.x;
    for (int h = 0; h < a.g; ++h)
        qs[h][c] = load_as_f32(a.q, a.q_dtype, (size_t(b) * a.hq + hk * a.g + h) * kHeadDim + c);
    __syncthreads();
    const float *R = a.r_k + size_t(hk) * kHeadDim * kHeadDim;
    float acc[kMaxGroup];
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) acc[h] = 0.0f;
    for (int i = 0; i < kHeadDim; ++i) {
        const float r = R[size_t(i) * kHeadDim + c];
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h)
            if (h < a.g) acc[h] = fmaf(qs[h][i], r, acc[h]);
    }
    for (int h = 0; h < a.g; ++h) {
        const float v = acc[h] * a.scale_log2;
        qr[h][c] = v;
        a.qrot[(size_t(b) * a.hq + hk * a.g + h) * kHeadDim + c] = v;
    }
    __syncthreads();
    if (c < a.g * kGroups) {
        const int h = c / kGroups, grp = c % kGroups;
        float s = 0.0f;
        for (int i = 0; i < kGroup; ++i) s += qr[h][grp * kGroup + i];
        a.qsum[(size_t(b) * a.hq + hk * a.g + h) * kGroups + grp] = s;
    }
}

// ---------------------------------------------------------------------------
// 2. split-K partials
// ---------------------------------------------------------------------------
__device__ __forceinline__ f16x2 as_h2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }
__device__ __forceinline__ uint32_t as_u32(f16x2 h) { return __builtin_bit_cast(uint32_t, h); }

// Move bit `from` of v to bit 8 (from is a constant after unrolling).
__device__ __forceinline__ uint32_t to_bit8(uint32_t v, int from) {
    return from <= 8 ? v << (8 - from) : v >> (from - 8);
}

// 4 + c in each fp16 half for the two codes at bits 8-9 and 24-25 of `x`:
// the code becomes the low mantissa bits of 4.0, whose ulp is 2^-8.
__device__ __forceinline__ f16x2 code_pair(uint32_t x) {
    return as_h2((x & 0x03000300u) | 0x44004400u);
}

// c * s for a code pair e = 4 + c: (4 + c) s - 4 s in one fused multiply-add
// (c2 = -4 s), rounded once; exact whenever c * s fits in fp16, which holds
// for s with at most 9 significant bits.
__device__ __forceinline__ uint32_t dq(f16x2 e, f16x2 s2, f16x2 c2) {
    return as_u32(__builtin_elementwise_fma(e, s2, c2));
}

// Split fp16 scales (two per word) into s_hi (low 2 mantissa bits cleared) and
// s_lo = s - s_hi (exact); returns the four multipliers and offsets.
struct ScaleSplit {
    f16x2 s_hi, s_lo, c_hi, c_lo;
};
__device__ __forceinline__ ScaleSplit split_scale(uint32_t s_bits2) {
    const f16x2 neg4 = as_h2(0xC400C400u);   // (-4, -4)
    ScaleSplit r;
    r.s_hi = as_h2(s_bits2 & 0xFFFCFFFCu);
    r.s_lo = as_h2(s_bits2) - r.s_hi;
    r.c_hi = r.s_hi * neg4;
    r.c_lo = r.s_lo * neg4;
    return r;
}

__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
    return uint32_t(__half_as_ushort(__float2half_rn(lo))) |
           (uint32_t(__half_as_ushort(__float2half_rn(hi))) << 16);
}

__device__ __forceinline__ f16x8 u4_as_h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    return __builtin_bit_cast(f16x8, u32x4{a, b, c, d});
}

// History item on the matrix cores.  GQ = query heads per KV head.
//
// The whole workgroup streams the tile's slot records (all of its KV heads:
// whole cache lines of the slot-major pool) with 16-byte loads, three per
// thread per 32-token tile, into a two-stage LDS ring; each wave then
// computes its own KV head from LDS.  Loads of tile i + 2 are in flight while
// tile i is computed.  Tokens past the item or with an out-of-range slot are
// zero-filled in LDS and masked out of the softmax.
template <int GQ>
__device__ void int2_item(const DecodeArgs &a, int b, int req, int j, int hc, int p0, int p1,
                          uint8_t *smem) {
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int n = lane & 15;
    const int kb = lane >> 4;
    const int nthreads = 64 * a.waves;
    const int h0 = hc * a.waves;
    const int nh = min(a.waves, a.hkv - h0);      // KV heads of this workgroup
    const bool active = w < nh;
    const int hk = h0 + (active ? w : 0);
    const int ts = nh * kHeadRecord + 16;          // LDS bytes per token (padded)
    const int stage_bytes = kTileTokens * ts;
    const int chunks_tok = nh * (kHeadRecord / 16);
    const int chunks_tile = kTileTokens * chunks_tok;
    const int64_t rec_bytes = int64_t(a.hkv) * kHeadRecord;
    const uint8_t *gbase = a.records + h0 * kHeadRecord;
    const int32_t *r2s = a.req_to_slot + int64_t(req) * a.r2s_stride;
    const int n_tiles = (p1 - p0 + kTileTokens - 1) / kTileTokens;

    // column n of the QK B operand: head n (hi part) or head n - GQ (lo part)
    const bool col_hi = n < GQ;
    const bool col_lo = n >= GQ && n < 2 * GQ;
    const int col_head = col_hi ? n : (col_lo ? n - GQ : 0);
    const float *qr = a.qrot + (size_t(b) * a.hq + hk * GQ + col_head) * kHeadDim;
    f16x8 qB[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        uint32_t wq[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            // k-slots (2p, 2p+1) of MFMA r hold channels base + p and base + 8 + p
            const int base = 32 * kb + 16 * (r >> 1) + 4 * (r & 1);
            float x0 = 0.0f, x1 = 0.0f;
            if (col_hi || col_lo) {
                x0 = qr[base + p];
                x1 = qr[base + 8 + p];
                if (col_lo) {
                    x0 -= __half2float(__float2half_rn(x0));
                    x1 -= __half2float(__float2half_rn(x1));
                }
            }
            wq[p] = pack_h2(x0, x1);
        }
        qB[r] = u4_as_h8(wq[0], wq[1], wq[2], wq[3]);
    }
    f16x8 qBz;
    {
        uint32_t wq[4] = {0, 0, 0, 0};
        if ((col_hi || col_lo) && kb == 0) {
            const float *qsum = a.qsum + (size_t(b) * a.hq + hk * GQ + col_head) * kGroups;
            float x[4];
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
                x[grp] = qsum[grp];
                if (col_lo) x[grp] -= __half2float(__float2half_rn(x[grp]));
            }
            wq[0] = pack_h2(x[0], x[1]);
            wq[1] = pack_h2(x[2], x[3]);
        }
        qBz = u4_as_h8(wq[0], wq[1], wq[2], wq[3]);
    }
    const int partner = col_hi ? lane + GQ : (col_lo ? lane - GQ : lane);

    // Every load below is unconditional (out-of-range positions and slots are
    // clamped to a safe address and masked afterwards), so each iteration
    // issues the same straight-line sequence of loads and the loads of the
    // next tile stay outstanding through the current tile's compute.
    //
    // raw slot id of token `lane & 31` of tile t; in_tile(t) says which are real
    auto tile_slot = [&](int t) -> int {
        const int pos = p0 + t * kTileTokens + (lane & (kTileTokens - 1));
        return r2s[pos < p1 ? pos : p0];
    };
    auto tile_mask = [&](int t) -> uint32_t {   // positions of tile t inside [p0, p1)
        const int cnt = min(kTileTokens, p1 - (p0 + t * kTileTokens));
        return cnt <= 0 ? 0u : (cnt >= 32 ? 0xFFFFFFFFu : ((1u << cnt) - 1u));
    };
    // this thread's three 16-byte pieces of a tile
    u32x4 rr[3];
    bool rr_ok[3];
    auto issue = [&](int slot_reg, uint32_t in_tile) {
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            const int q = u * nthreads + tid;
            const int qc = q < chunks_tile ? q : 0;
            const int tok = qc / chunks_tok;
            const int c = qc - tok * chunks_tok;
            const int slot = __shfl(slot_reg, tok);
            const bool ok = q < chunks_tile && ((in_tile >> tok) & 1u) && slot >= 0 &&
                            int64_t(slot) < a.num_slots;
            rr_ok[u] = ok;
            rr[u] = *reinterpret_cast<const u32x4 *>(gbase + int64_t(ok ? slot : 0) * rec_bytes + 16 * c);
        }
    };
    auto stash = [&](int stage) {
        uint8_t *dst = smem + stage * stage_bytes;
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            const int q = u * nthreads + tid;
            const int tok = q / chunks_tok;
            const int c = q - tok * chunks_tok;
            const u32x4 v = rr_ok[u] ? rr[u] : u32x4{0, 0, 0, 0};
            if (q < chunks_tile) *reinterpret_cast<u32x4 *>(dst + tok * ts + 16 * c) = v;
        }
    };
    // tokens of a tile with a real position and an in-range slot
    auto valid_mask = [&](int slot_reg, uint32_t in_tile) -> uint32_t {
        const bool ok = lane < kTileTokens && ((in_tile >> lane) & 1u) && slot_reg >= 0 &&
                        int64_t(slot_reg) < a.num_slots;
        return uint32_t(__ballot(ok));
    };
    auto barrier = []() {
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS writes are done
        __builtin_amdgcn_s_barrier();
    };

    float m_run = -INFINITY;
    float l_lane = 0.0f;
    f32x4 oacc[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) oacc[jj] = f32x4{0, 0, 0, 0};
    f32x4 zacc = f32x4{0, 0, 0, 0};

    // prologue: tile 0 into stage 0, tile 1 in flight, slots of tile 2 loaded
    const int s0 = tile_slot(0);
    const int s1 = tile_slot(1);
    issue(s0, tile_mask(0));
    uint32_t mask_cur = valid_mask(s0, tile_mask(0));
    stash(0);
    barrier();
    int s_far = tile_slot(2);
    issue(s1, tile_mask(1));
    uint32_t mask_next = valid_mask(s1, tile_mask(1));

    for (int it = 0; it < n_tiles; ++it) {
        if (it > 0) {
            // tile it arrived in registers one iteration ago: put it in LDS,
            // then start loading tile it + 1
            stash(it & 1);
            barrier();
            // slot ids first, record loads last: the loads stay outstanding
            // through the compute below and are waited for by the next stash
            const int s_new = tile_slot(it + 2);
            issue(s_far, tile_mask(it + 1));
            mask_cur = mask_next;
            mask_next = valid_mask(s_far, tile_mask(it + 1));
            s_far = s_new;
        }
        if (active) {
            const uint8_t *stage = smem + (it & 1) * stage_bytes + w * kHeadRecord;
            // ---- QK: rows = tokens (two halves of 16), cols = (hi|lo, head)
            float lg[2][4];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const uint8_t *row = stage + (16 * hf + n) * ts;
                const u32x2 kc = *reinterpret_cast<const u32x2 *>(row + 8 * kb);
                const u32x4 ksz = *reinterpret_cast<const u32x4 *>(row + 2 * kCodeBytes);
                const uint32_t szk = kb == 0 ? ksz[0] : (kb == 1 ? ksz[1] : (kb == 2 ? ksz[2] : ksz[3]));
                const ScaleSplit sk = split_scale((szk & 0xFFFFu) | (szk << 16));
                f32x4 acc = f32x4{0, 0, 0, 0};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint32_t d = (r < 2) ? kc[0] : kc[1];
                    const int sh = 8 * (r & 1);
                    f16x2 e[4];
#pragma unroll
                    for (int p = 0; p < 4; ++p) e[p] = code_pair(to_bit8(d, sh + 2 * p));
                    const f16x8 Ahi = u4_as_h8(dq(e[0], sk.s_hi, sk.c_hi), dq(e[1], sk.s_hi, sk.c_hi),
                                               dq(e[2], sk.s_hi, sk.c_hi), dq(e[3], sk.s_hi, sk.c_hi));
                    const f16x8 Alo = u4_as_h8(dq(e[0], sk.s_lo, sk.c_lo), dq(e[1], sk.s_lo, sk.c_lo),
                                               dq(e[2], sk.s_lo, sk.c_lo), dq(e[3], sk.s_lo, sk.c_lo));
                    acc = mfma_f16(Ahi, qB[r], acc);
                    acc = mfma_f16(Alo, qB[r], acc);
                }
                {
                    uint32_t z01 = 0, z23 = 0;
                    if (kb == 0) {
                        z01 = (ksz[0] >> 16) | (ksz[1] & 0xFFFF0000u);
                        z23 = (ksz[2] >> 16) | (ksz[3] & 0xFFFF0000u);
                    }
                    acc = mfma_f16(u4_as_h8(z01, z23, 0, 0), qBz, acc);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool ok = (mask_cur >> (16 * hf + 4 * kb + i)) & 1u;
                    const float part = __shfl(acc[i], partner);
                    lg[hf][i] = ok ? acc[i] + part : -INFINITY;
                }
            }

            // ---- online softmax (per column; all 4 row groups agree after the reduction)
            float mx = lg[0][0];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int i = 0; i < 4; ++i) mx = fmaxf(mx, lg[hf][i]);
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run, mx);
            if (__any(m_new > m_run)) {
                const float alpha = (m_new > m_run) ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
                l_lane *= alpha;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float ar = __shfl(alpha, 4 * kb + i);   // alpha of PV row 4 kb + i
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj) oacc[jj][i] *= ar;
                    zacc[i] *= ar;
                }
                m_run = m_new;
            }
            float pv[8];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float x = lg[hf][i];
                    const float p = (x == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(x - m_run);
                    pv[4 * hf + i] = p;
                    l_lane += p;
                }
            // PV A operand: row n = (hi|lo, head), k-slots = tokens 4 kb + s (s < 4)
            // and 16 + 4 kb + s - 4 (s >= 4)
            uint32_t aw[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                float x0 = pv[2 * p], x1 = pv[2 * p + 1];
                if (col_lo) {
                    x0 -= __half2float(__float2half_rn(x0));
                    x1 -= __half2float(__float2half_rn(x1));
                } else if (!col_hi) {
                    x0 = 0.0f;
                    x1 = 0.0f;
                }
                aw[p] = pack_h2(x0, x1);
            }
            const f16x8 AP = u4_as_h8(aw[0], aw[1], aw[2], aw[3]);

            // ---- PV B operands: lane (n, kb) reads word n (channels 8n .. 8n+7)
            // of the V codes and the (s, z) of group n / 4 for its 8 tokens
            uint32_t vw[4], sp[4], zp[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                uint32_t wv[2], szv[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int sidx = 2 * p + e;
                    const int tt = sidx < 4 ? 4 * kb + sidx : 16 + 4 * kb + (sidx - 4);
                    const uint8_t *row = stage + tt * ts;
                    wv[e] = *reinterpret_cast<const uint16_t *>(row + kCodeBytes + 2 * n);
                    szv[e] = *reinterpret_cast<const uint32_t *>(row + 2 * kCodeBytes + kSzBytes + 4 * (n >> 2));
                }
                vw[p] = wv[0] | (wv[1] << 16);
                sp[p] = (szv[0] & 0xFFFFu) | (szv[1] << 16);
                zp[p] = (szv[0] >> 16) | (szv[1] & 0xFFFF0000u);
            }
            const f16x8 BZ = u4_as_h8(zp[0], zp[1], zp[2], zp[3]);
            ScaleSplit sv[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) sv[p] = split_scale(sp[p]);
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                f16x2 e[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) e[p] = code_pair(to_bit8(vw[p], 2 * jj));
                const f16x8 Bhi = u4_as_h8(dq(e[0], sv[0].s_hi, sv[0].c_hi), dq(e[1], sv[1].s_hi, sv[1].c_hi),
                                           dq(e[2], sv[2].s_hi, sv[2].c_hi), dq(e[3], sv[3].s_hi, sv[3].c_hi));
                const f16x8 Blo = u4_as_h8(dq(e[0], sv[0].s_lo, sv[0].c_lo), dq(e[1], sv[1].s_lo, sv[1].c_lo),
                                           dq(e[2], sv[2].s_lo, sv[2].c_lo), dq(e[3], sv[3].s_lo, sv[3].c_lo));
                oacc[jj] = mfma_f16(AP, Bhi, oacc[jj]);
                oacc[jj] = mfma_f16(AP, Blo, oacc[jj]);
            }
            zacc = mfma_f16(AP, BZ, zacc);
        }
    }
    if (!active) return;

    // ---- write the partial (m, l, o') of the GQ heads
    float l_col = l_lane + __shfl_xor(l_lane, 16);
    l_col += __shfl_xor(l_col, 32);
    const size_t row0 = (size_t(b) * a.items + j) * a.hq + hk * GQ;
    if (kb == 0 && col_hi) {
        a.part_ml[(row0 + n) * 2 + 0] = m_run;
        a.part_ml[(row0 + n) * 2 + 1] = l_col;
    }
    // PV output: lane (n, kb) holds rows 4 kb + i, channels 8 n + jj; row h
    // (hi) and row GQ + h (lo) add up to head h
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * kb + i;
        const int e = (GQ + i) & 3;
        const int src = n + 16 * (kb + ((GQ + i) >> 2));
        float o[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            float lo_part = 0.0f;
            switch (e) {  // register index must be static
                case 0: lo_part = __shfl(oacc[jj][0] + zacc[0], src); break;
                case 1: lo_part = __shfl(oacc[jj][1] + zacc[1], src); break;
                case 2: lo_part = __shfl(oacc[jj][2] + zacc[2], src); break;
                default: lo_part = __shfl(oacc[jj][3] + zacc[3], src); break;
            }
            o[jj] = oacc[jj][i] + zacc[i] + lo_part;
        }
        if (r < GQ) {
            float *dst = a.part_o + (row0 + r) * kHeadDim + 8 * n;
            *reinterpret_cast<f32x4 *>(dst) = f32x4{o[0], o[1], o[2], o[3]};
            *reinterpret_cast<f32x4 *>(dst + 4) = f32x4{o[4], o[5], o[6], o[7]};
        }
    }
}

// BF16 window item on fp32 VALU: lanes over tokens for QK, over channel pairs
// for PV.  `pbuf` is this wave's LDS scratch [kMaxGroup][64].
__device__ void bf16_item(const DecodeArgs &a, int b, int req, int j, int hk, int p0, int p1,
                          bool active, float *pbuf) {
    const int lane = threadIdx.x & 63;
    const int g = a.g;
    const float *qr = a.qrot + (size_t(b) * a.hq + hk * g) * kHeadDim;
    const bool is_sink = (j == 0);
    float m_run[kMaxGroup], l_lane[kMaxGroup], o0[kMaxGroup], o1[kMaxGroup];
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
        m_run[h] = -INFINITY;
        l_lane[h] = 0.0f;
        o0[h] = 0.0f;
        o1[h] = 0.0f;
    }
    auto row_ptr = [&](int pos, int t) -> const uint16_t * {
        if (is_sink)
            return a.sink + ((size_t(req) * a.sink_tokens + pos) * a.hkv + hk) * 2 * kHeadDim + t * kHeadDim;
        return a.recent + ((size_t(req) * a.recent_tokens + pos % a.recent_tokens) * a.hkv + hk) * 2 * kHeadDim +
               t * kHeadDim;
    };
    for (int cb = p0; cb < p1; cb += kBf16Chunk) {
        const int pos = cb + lane;
        const bool ok = active && pos < p1;
        float acc[kMaxGroup];
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h) acc[h] = 0.0f;
        if (ok) {
            const uint16_t *kr = row_ptr(pos, 0);
            for (int i = 0; i < kHeadDim; i += 8) {
                const u32x4 kw = *reinterpret_cast<const u32x4 *>(kr + i);
                float kf[8];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    kf[2 * u] = bf16_bits_to_f32(kw[u] & 0xFFFFu);
                    kf[2 * u + 1] = bf16_bits_to_f32(kw[u] >> 16);
                }
#pragma unroll
                for (int h = 0; h < kMaxGroup; ++h) {
                    if (h < g) {
#pragma unroll
                        for (int u = 0; u < 8; ++u) acc[h] = fmaf(qr[h * kHeadDim + i + u], kf[u], acc[h]);
                    }
                }
            }
        }
        float alpha[kMaxGroup];
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h) {
            const float x = ok ? acc[h] : -INFINITY;
            float mx = x;
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
            const float m_new = fmaxf(m_run[h], mx);
            alpha[h] = (m_new > m_run[h]) ? __builtin_amdgcn_exp2f(m_run[h] - m_new) : 1.0f;
            m_run[h] = m_new;
            const float p = (x == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(x - m_new);
            l_lane[h] = l_lane[h] * alpha[h] + p;
            if (h < g) pbuf[h * kBf16Chunk + lane] = p;
        }
        __syncthreads();
        // PV: lane holds channels 2 lane, 2 lane + 1
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h) {
            o0[h] *= alpha[h];
            o1[h] *= alpha[h];
        }
        if (active) {
            const int cnt = min(kBf16Chunk, p1 - cb);
            for (int tt = 0; tt < cnt; ++tt) {
                const uint32_t vw = *reinterpret_cast<const uint32_t *>(row_ptr(cb + tt, 1) + 2 * lane);
                const float v0 = bf16_bits_to_f32(vw & 0xFFFFu), v1 = bf16_bits_to_f32(vw >> 16);
#pragma unroll
                for (int h = 0; h < kMaxGroup; ++h) {
                    if (h < g) {
                        const float p = pbuf[h * kBf16Chunk + tt];
                        o0[h] = fmaf(p, v0, o0[h]);
                        o1[h] = fmaf(p, v1, o1[h]);
                    }
                }
            }
        }
        __syncthreads();
    }
    if (!active) return;
    const size_t row0 = (size_t(b) * a.items + j) * a.hq + hk * g;
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
        if (h >= g) break;
        float l = l_lane[h];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) l += __shfl_xor(l, off);
        if (lane == 0) {
            a.part_ml[(row0 + h) * 2 + 0] = m_run[h];
            a.part_ml[(row0 + h) * 2 + 1] = l;
        }
        float *dst = a.part_o + (row0 + h) * kHeadDim + 2 * lane;
        dst[0] = o0[h];
        dst[1] = o1[h];
    }
}

template <int GQ>
__global__ __launch_bounds__(512) void partial_kernel(DecodeArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int id = blockIdx.x;
    const int hc = id % a.head_chunks;
    const int rest = id / a.head_chunks;
    const int b = rest % a.batch;
    const int j = rest / a.batch;
    int req = 0;
    const int L = request_length(a, b, req);
    int p0, p1;
    item_range(a, L, j, p0, p1);
    if (p0 >= p1) return;                       // uniform over the workgroup
    const int w = threadIdx.x >> 6;
    const int hk = hc * a.waves + w;
    const bool active = hk < a.hkv;
    if (j < 2) {
        float *pbuf = reinterpret_cast<float *>(smem) + w * (kMaxGroup * kBf16Chunk);
        bf16_item(a, b, req, j, active ? hk : 0, p0, p1, active, pbuf);
    } else if (a.num_slots > 0) {
        int2_item<GQ>(a, b, req, j, hc, p0, p1, smem);
    }
}

// ---------------------------------------------------------------------------
// 3. merge + un-rotation
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(128) void merge_kernel(DecodeArgs a) {
    __shared__ float ob[kMaxGroup][kHeadDim];
    const int b = blockIdx.x / a.hkv;
    const int hk = blockIdx.x % a.hkv;
    const int c = threadIdx.x;
    int req = 0;
    const int L = request_length(a, b, req);
    for (int h = 0; h < a.g; ++h) {
        const size_t head = size_t(hk) * a.g + h;
        float M = -INFINITY;
        for (int j = 0; j < a.items; ++j) {
            int p0, p1;
            item_range(a, L, j, p0, p1);
            if (p0 >= p1) continue;
            M = fmaxf(M, a.part_ml[((size_t(b) * a.items + j) * a.hq + head) * 2]);
        }
        float acc = 0.0f, l = 0.0f;
        if (M != -INFINITY) {
            for (int j = 0; j < a.items; ++j) {
                int p0, p1;
                item_range(a, L, j, p0, p1);
                if (p0 >= p1) continue;
                const size_t row = (size_t(b) * a.items + j) * a.hq + head;
                const float m = a.part_ml[row * 2];
                if (m == -INFINITY) continue;
                const float wgt = __builtin_amdgcn_exp2f(m - M);
                l = fmaf(wgt, a.part_ml[row * 2 + 1], l);
                acc = fmaf(wgt, a.part_o[row * kHeadDim + c], acc);
            }
        }
        ob[h][c] = l > 0.0f ? acc / l : 0.0f;
    }
    __syncthreads();
    // o[c] = sum_i o'[i] R_V[c][i]
    const float *R = a.r_v + (size_t(hk) * kHeadDim + c) * kHeadDim;
    float o[kMaxGroup];
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) o[h] = 0.0f;
    for (int i = 0; i < kHeadDim; i += 4) {
        const f32x4 r = *reinterpret_cast<const f32x4 *>(R + i);
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h) {
            if (h < a.g) {
                o[h] = fmaf(ob[h][i], r[0], o[h]);
                o[h] = fmaf(ob[h][i + 1], r[1], o[h]);
                o[h] = fmaf(ob[h][i + 2], r[2], o[h]);
                o[h] = fmaf(ob[h][i + 3], r[3], o[h]);
            }
        }
    }
    for (int h = 0; h < a.g; ++h) {
        const size_t idx = (size_t(b) * a.hq + hk * a.g + h) * kHeadDim + c;
        if (a.out_dtype == OSCAR_F32)
            static_cast<float *>(a.out)[idx] = o[h];
        else if (a.out_dtype == OSCAR_BF16)
            static_cast<uint16_t *>(a.out)[idx] = bf16_bits_rn(o[h]);
        else
            static_cast<uint16_t *>(a.out)[idx] = __half_as_ushort(__float2half_rn(o[h]));
    }
}

// Dynamic LDS of the partial kernel: two stages of 32 padded token records
// for the INT2 items, or the per-wave softmax buffers of the BF16 items.
size_t partial_lds_bytes(const DecodeArgs &a) {
    const size_t stages = 2 * size_t(kTileTokens) * (size_t(a.waves) * kHeadRecord + 16);
    const size_t pbuf = size_t(a.waves) * kMaxGroup * kBf16Chunk * sizeof(float);
    return stages > pbuf ? stages : pbuf;
}

template <int GQ>
hipError_t launch_partial(const DecodeArgs &a, int blocks, hipStream_t stream) {
    hipLaunchKernelGGL(partial_kernel<GQ>, dim3(blocks), dim3(64 * a.waves), partial_lds_bytes(a), stream, a);
    return hipGetLastError();
}

}  // namespace
}  // namespace oscar

using namespace oscar;

extern "C" oscar_status oscar_decode_attn(hipStream_t stream, const oscar_layout *layout,
                                          const oscar_pool *pool, const void *q, oscar_dtype q_dtype,
                                          int32_t batch, const int32_t *req_ids,
                                          const int32_t *seq_lens, const int32_t *seq_lens_host,
                                          const int32_t *req_to_slot, int64_t req_to_slot_stride,
                                          const float *R_K, const float *R_V, float sm_scale,
                                          void *out, oscar_dtype out_dtype, void *workspace,
                                          size_t workspace_bytes, const oscar_launch_opts *opts) {
    oscar_status st = check_layout(layout);
    if (st != OSCAR_OK) return st;
    if (!pool || !q || !req_ids || !seq_lens || !req_to_slot || !R_K || !R_V || !out)
        return fail(OSCAR_ERR_INVALID_ARG, "a required pointer is null");
    if (!pool->records || !pool->recent || (layout->sink_tokens > 0 && !pool->sink))
        return fail(OSCAR_ERR_INVALID_ARG, "a pool pointer is null");
    if (q_dtype != OSCAR_F32 && q_dtype != OSCAR_BF16 && q_dtype != OSCAR_F16)
        return fail(OSCAR_ERR_INVALID_ARG, "q_dtype must be F32, BF16 or F16");
    if (out_dtype != OSCAR_F32 && out_dtype != OSCAR_BF16 && out_dtype != OSCAR_F16)
        return fail(OSCAR_ERR_INVALID_ARG, "out_dtype must be F32, BF16 or F16");
    if (!std::isfinite(sm_scale)) return fail(OSCAR_ERR_INVALID_ARG, "sm_scale must be finite");
    DecodePlan plan;
    st = make_decode_plan(*layout, batch, seq_lens_host, opts, &plan);
    if (st != OSCAR_OK) return st;
    if (req_to_slot_stride < plan.max_len)
        return fail(OSCAR_ERR_INVALID_ARG, "req_to_slot_stride is smaller than the longest sequence");
    if (!workspace || workspace_bytes < plan.ws_bytes)
        return fail(OSCAR_ERR_WORKSPACE, "workspace is smaller than oscar_decode_workspace_size");
    if (reinterpret_cast<uintptr_t>(workspace) % 256)
        return fail(OSCAR_ERR_INVALID_ARG, "workspace must be 256-byte aligned");

    DecodeArgs a;
    a.q = q;
    a.req_ids = req_ids;
    a.seq_lens = seq_lens;
    a.req_to_slot = req_to_slot;
    a.r_k = R_K;
    a.r_v = R_V;
    a.records = pool->records;
    a.sink = pool->sink;
    a.recent = pool->recent;
    a.out = out;
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    a.qrot = reinterpret_cast<float *>(ws + plan.ws_qrot);
    a.qsum = reinterpret_cast<float *>(ws + plan.ws_qsum);
    a.part_o = reinterpret_cast<float *>(ws + plan.ws_part_o);
    a.part_ml = reinterpret_cast<float *>(ws + plan.ws_part_ml);
    a.r2s_stride = req_to_slot_stride;
    a.num_slots = layout->num_slots;
    a.scale_log2 = sm_scale * kLog2e;
    a.q_dtype = q_dtype;
    a.out_dtype = out_dtype;
    a.batch = batch;
    a.hkv = layout->num_kv_heads;
    a.hq = layout->num_q_heads;
    a.g = layout->num_q_heads / layout->num_kv_heads;
    a.sink_tokens = layout->sink_tokens;
    a.recent_tokens = layout->recent_tokens;
    a.max_requests = layout->max_requests;
    a.chunk = plan.chunk;
    a.items = plan.items;
    a.waves = a.hkv < 8 ? a.hkv : 8;
    a.head_chunks = (a.hkv + a.waves - 1) / a.waves;

    hipLaunchKernelGGL(prep_kernel, dim3(batch * a.hkv), dim3(128), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(OSCAR_ERR_HIP, std::string("prep launch: ") + hipGetErrorString(e));

    if (opts && opts->kernel_begin && hipEventRecord(opts->kernel_begin, stream) != hipSuccess)
        return fail(OSCAR_ERR_HIP, "hipEventRecord failed");
    const int blocks = plan.items * batch * a.head_chunks;
    switch (a.g) {
        case 1: e = launch_partial<1>(a, blocks, stream); break;
        case 2: e = launch_partial<2>(a, blocks, stream); break;
        case 3: e = launch_partial<3>(a, blocks, stream); break;
        case 4: e = launch_partial<4>(a, blocks, stream); break;
        case 5: e = launch_partial<5>(a, blocks, stream); break;
        case 6: e = launch_partial<6>(a, blocks, stream); break;
        case 7: e = launch_partial<7>(a, blocks, stream); break;
        default: e = launch_partial<8>(a, blocks, stream); break;
    }
    if (e != hipSuccess) return fail(OSCAR_ERR_HIP, std::string("partial launch: ") + hipGetErrorString(e));
    if (opts && opts->kernel_end && hipEventRecord(opts->kernel_end, stream) != hipSuccess)
        return fail(OSCAR_ERR_HIP, "hipEventRecord failed");

    hipLaunchKernelGGL(merge_kernel, dim3(batch * a.hkv), dim3(128), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(OSCAR_ERR_HIP, std::string("merge launch: ") + hipGetErrorString(e));
    return OSCAR_OK;
}
