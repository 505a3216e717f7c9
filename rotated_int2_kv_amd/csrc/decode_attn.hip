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
//               History tiles of 32 tokens run on f16 MFMA with the INT2 codes
//               as exact fp16 denormal operands (see int2_item).
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
    float *qsum;       // [B][Hq][8]: group sums of qrot, then 2^K, 2^(24-K) (operand scaling)
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
        a.qsum[(size_t(b) * a.hq + hk * a.g + h) * 8 + grp] = s;
    }
    if (c < a.g) {
        // power-of-two operand scale 2^K with max|q'| 2^K < 2^15, so that
        // q' 2^(K - e) (e = 0..8) fits fp16 and its low part stays normal
        float mx = 0.0f;
        for (int i = 0; i < kHeadDim; ++i) mx = fmaxf(mx, fabsf(qr[c][i]));
        int e = 0;
        frexpf(mx, &e);                          // mx < 2^e
        const int K = mx > 0.0f ? max(-20, min(24, 15 - e)) : 24;
        float *info = a.qsum + (size_t(b) * a.hq + hk * a.g + c) * 8;
        info[4] = ldexpf(1.0f, K);
        info[5] = ldexpf(1.0f, 24 - K);
    }
}

// ---------------------------------------------------------------------------
// 2. split-K partials
// ---------------------------------------------------------------------------
__device__ __forceinline__ f16x2 as_h2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }
__device__ __forceinline__ uint32_t as_u32(f16x2 h) { return __builtin_bit_cast(uint32_t, h); }

__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
    return uint32_t(__half_as_ushort(__float2half_rn(lo))) |
           (uint32_t(__half_as_ushort(__float2half_rn(hi))) << 16);
}

__device__ __forceinline__ f16x8 u4_as_h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    return __builtin_bit_cast(f16x8, u32x4{a, b, c, d});
}

// Exponent offset of code pair j inside a 32-bit word of 16 LSB-first codes:
// pairs (j, j + 8) sit at bits 2j and 16 + 2j; j = 0..4 are masked in place,
// j = 5..7 after a right shift by 6.  Masked, each 16-bit half is an fp16
// denormal of value c 2^(e_j - 24).
__host__ __device__ constexpr int pair_exp(int j) { return j <= 4 ? 2 * j : 2 * j - 6; }

__device__ __forceinline__ uint32_t code_bits(uint32_t w, uint32_t w_sh6, int j) {
    return j <= 4 ? (w & (0x00030003u << (2 * j))) : (w_sh6 & (0x00030003u << (2 * j - 6)));
}

__device__ __forceinline__ float dpp_ror4_add(float v) {
    return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_ror8_add(float v) {
    return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
}

// History item on the matrix cores.  GQ = query heads per KV head, handled in
// sets of 4.
//
// Loads: the whole workgroup streams the tile's slot records (all of its KV
// heads: whole cache lines of the slot-major pool) with 16-byte loads, three
// per thread per 32-token tile, into a two-stage LDS ring; loads of tile i + 1
// are in flight while tile i is computed.  Tokens past the item or with an
// out-of-range slot are zero-filled in LDS and masked out of the softmax.
//
// QK (per half of 16 tokens): A = the token's K codes as exact fp16 denormals
// (one AND per pair, no scale); B = q' (hi and lo fp16 parts, times 2^(K - e))
// placed block-diagonally so that column (g, h) collects the dot product of
// group g only.  Each lane then applies s and z of its (token, group) in fp32
// and a DPP rotate-add sums the four groups: every step is exact except the
// final fp32 additions.
// PV: rows (g, h) of A hold p s_g (hi and lo parts), B holds the V codes of 8
// tokens per lane as exact denormals; the output of column (channel) c is read
// from the row whose group is c's group.  A second pair of MFMAs adds p z.
template <int GQ>
__device__ void int2_item(const DecodeArgs &a, int b, int req, int j, int hc, int p0, int p1,
                          uint8_t *smem) {
    constexpr int HS = (GQ + 3) / 4;          // sets of 4 query heads
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int n = lane & 15;
    const int kb = lane >> 4;
    const int cg = n >> 2;                    // group of QK column / PV row n
    const int ch = n & 3;                     // head (within a set) of column / row n
    const int nthreads = 64 * a.waves;
    const int h0 = hc * a.waves;
    const int nh = min(a.waves, a.hkv - h0);  // KV heads of this workgroup
    const bool active = w < nh;
    const int hk = h0 + (active ? w : 0);
    const int ts = nh * kHeadRecord + 16;     // LDS bytes per token (padded)
    const int stage_bytes = kTileTokens * ts;
    const int chunks_tok = nh * (kHeadRecord / 16);
    const int chunks_tile = kTileTokens * chunks_tok;
    const int64_t rec_bytes = int64_t(a.hkv) * kHeadRecord;
    const uint8_t *gbase = a.records + h0 * kHeadRecord;
    const int32_t *r2s = a.req_to_slot + int64_t(req) * a.r2s_stride;
    const int n_tiles = (p1 - p0 + kTileTokens - 1) / kTileTokens;

    // ---- per-item operands
    f16x8 qB[HS][4][2];
    float qz[HS];       // Qbar[h][cg] 2^(K - 24): zero-point term in the MFMA's units
    float qout[HS];     // 2^(24 - K): back to logit units
#pragma unroll
    for (int hs = 0; hs < HS; ++hs) {
        const int h = 4 * hs + ch;
        const bool hv = h < GQ;
        const size_t row = size_t(b) * a.hq + hk * GQ + (hv ? h : 0);
        const float *qr = a.qrot + row * kHeadDim;
        const float *info = a.qsum + row * 8;
        const float k2 = info[4];
        qz[hs] = hv ? info[cg] / info[5] : 0.0f;
        qout[hs] = info[5];
        const bool nz = hv && cg == kb;       // block-diagonal: K-block kb is group kb
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            uint32_t whi[4], wlo[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int jj = 4 * (r & 1) + p;
                const int c0 = 32 * kb + 16 * (r >> 1) + jj;
                const float sc = k2 * __builtin_ldexpf(1.0f, -pair_exp(jj));
                const float x0 = nz ? qr[c0] * sc : 0.0f;
                const float x1 = nz ? qr[c0 + 8] * sc : 0.0f;
                whi[p] = pack_h2(x0, x1);
                const float h0f = __half2float(__ushort_as_half(uint16_t(whi[p] & 0xFFFFu)));
                const float h1f = __half2float(__ushort_as_half(uint16_t(whi[p] >> 16)));
                wlo[p] = pack_h2(x0 - h0f, x1 - h1f);
            }
            qB[hs][r][0] = u4_as_h8(whi[0], whi[1], whi[2], whi[3]);
            qB[hs][r][1] = u4_as_h8(wlo[0], wlo[1], wlo[2], wlo[3]);
        }
    }

    // ---- load pipeline (all loads unconditional: out-of-range positions and
    // slots read a safe address and are zeroed when written to LDS)
    auto tile_slot = [&](int t) -> int {
        const int pos = p0 + t * kTileTokens + (lane & (kTileTokens - 1));
        return r2s[pos < p1 ? pos : p0];
    };
    auto tile_mask = [&](int t) -> uint32_t {   // positions of tile t inside [p0, p1)
        const int cnt = min(kTileTokens, p1 - (p0 + t * kTileTokens));
        return cnt <= 0 ? 0u : (cnt >= 32 ? 0xFFFFFFFFu : ((1u << cnt) - 1u));
    };
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
    auto valid_mask = [&](int slot_reg, uint32_t in_tile) -> uint32_t {
        const bool ok = lane < kTileTokens && ((in_tile >> lane) & 1u) && slot_reg >= 0 &&
                        int64_t(slot_reg) < a.num_slots;
        return uint32_t(__ballot(ok));
    };
    auto barrier = []() {
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS writes are done
        __builtin_amdgcn_s_barrier();
    };

    float m_run[HS], l_lane[HS];
    f32x4 oacc[HS][8], zacc[HS];
#pragma unroll
    for (int hs = 0; hs < HS; ++hs) {
        m_run[hs] = -INFINITY;
        l_lane[hs] = 0.0f;
        zacc[hs] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) oacc[hs][jj] = f32x4{0, 0, 0, 0};
    }

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
            // then start loading tile it + 1 (slot ids first, record loads last,
            // so that the record loads stay outstanding through the compute)
            stash(it & 1);
            barrier();
            const int s_new = tile_slot(it + 2);
            issue(s_far, tile_mask(it + 1));
            mask_cur = mask_next;
            mask_next = valid_mask(s_far, tile_mask(it + 1));
            s_far = s_new;
        }
        if (!active) continue;
        const uint8_t *stage = smem + (it & 1) * stage_bytes + w * kHeadRecord;

        // ---- QK
        float lg[HS][8];      // logits of tokens 4 kb + i (i < 4) and 16 + 4 kb + i
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const u32x2 kc = *reinterpret_cast<const u32x2 *>(stage + (16 * hf + n) * ts + 8 * kb);
            const uint32_t d0s = kc[0] >> 6, d1s = kc[1] >> 6;
            f16x8 A[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t d = r < 2 ? kc[0] : kc[1];
                const uint32_t ds = r < 2 ? d0s : d1s;
                A[r] = u4_as_h8(code_bits(d, ds, 4 * (r & 1) + 0), code_bits(d, ds, 4 * (r & 1) + 1),
                                code_bits(d, ds, 4 * (r & 1) + 2), code_bits(d, ds, 4 * (r & 1) + 3));
            }
            // (s, z) of the output lane's 4 tokens for group cg
            uint32_t szk[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                szk[i] = *reinterpret_cast<const uint32_t *>(stage + (16 * hf + 4 * kb + i) * ts +
                                                            2 * kCodeBytes + 4 * cg);
#pragma unroll
            for (int hs = 0; hs < HS; ++hs) {
                f32x4 acc = f32x4{0, 0, 0, 0};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    acc = mfma_f16(A[r], qB[hs][r][0], acc);
                    acc = mfma_f16(A[r], qB[hs][r][1], acc);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float sf = __half2float(__ushort_as_half(uint16_t(szk[i] & 0xFFFFu)));
                    const float zf = __half2float(__ushort_as_half(uint16_t(szk[i] >> 16)));
                    float x = fmaf(acc[i], sf, zf * qz[hs]);
                    x = dpp_ror8_add(dpp_ror4_add(x));          // sum over the 4 groups
                    const bool ok = (mask_cur >> (16 * hf + 4 * kb + i)) & 1u;
                    lg[hs][4 * hf + i] = ok ? x * qout[hs] : -INFINITY;
                }
            }
        }

        // ---- online softmax and PV A operands
        // (s, z) of V for group cg and the 8 tokens of this lane
        uint32_t szv[8], vw[8];
#pragma unroll
        for (int sidx = 0; sidx < 8; ++sidx) {
            const int tt = sidx < 4 ? 4 * kb + sidx : 16 + 4 * kb + (sidx - 4);
            const uint8_t *row = stage + tt * ts;
            szv[sidx] = *reinterpret_cast<const uint32_t *>(row + 2 * kCodeBytes + kSzBytes + 4 * cg);
            vw[sidx] = *reinterpret_cast<const uint16_t *>(row + kCodeBytes + 2 * n);
        }
        f16x8 AS[HS][2], AZ[HS][2];
#pragma unroll
        for (int hs = 0; hs < HS; ++hs) {
            float mx = lg[hs][0];
#pragma unroll
            for (int i = 1; i < 8; ++i) mx = fmaxf(mx, lg[hs][i]);
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run[hs], mx);
            if (__any(m_new > m_run[hs])) {
                const float alpha = (m_new > m_run[hs]) ? __builtin_amdgcn_exp2f(m_run[hs] - m_new) : 1.0f;
                l_lane[hs] *= alpha;
                // PV output row (g, h) = (kb, i): alpha of head i lives in lane i
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float ai = __builtin_bit_cast(
                        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), i));
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj) oacc[hs][jj][i] *= ai;
                    zacc[hs][i] *= ai;
                }
                m_run[hs] = m_new;
            }
            uint32_t wsh[4], wsl[4], wzh[4], wzl[4];
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) {
                float pr[2], ps[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const float x = lg[hs][2 * pp + e];
                    const float p = (x == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(x - m_run[hs]);
                    l_lane[hs] += p;
                    pr[e] = p;
                    ps[e] = p * __half2float(__ushort_as_half(uint16_t(szv[2 * pp + e] & 0xFFFFu)));
                }
                wsh[pp] = pack_h2(ps[0], ps[1]);
                wzh[pp] = pack_h2(pr[0], pr[1]);
                const float sh0 = __half2float(__ushort_as_half(uint16_t(wsh[pp] & 0xFFFFu)));
                const float sh1 = __half2float(__ushort_as_half(uint16_t(wsh[pp] >> 16)));
                const float zh0 = __half2float(__ushort_as_half(uint16_t(wzh[pp] & 0xFFFFu)));
                const float zh1 = __half2float(__ushort_as_half(uint16_t(wzh[pp] >> 16)));
                wsl[pp] = pack_h2(ps[0] - sh0, ps[1] - sh1);
                wzl[pp] = pack_h2(pr[0] - zh0, pr[1] - zh1);
            }
            AS[hs][0] = u4_as_h8(wsh[0], wsh[1], wsh[2], wsh[3]);
            AS[hs][1] = u4_as_h8(wsl[0], wsl[1], wsl[2], wsl[3]);
            AZ[hs][0] = u4_as_h8(wzh[0], wzh[1], wzh[2], wzh[3]);
            AZ[hs][1] = u4_as_h8(wzl[0], wzl[1], wzl[2], wzl[3]);
        }

        // ---- PV: B = V codes of channel 8 n + jj for the lane's 8 tokens
        uint32_t xw[4], xs[4];
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
            xw[pp] = vw[2 * pp] | (vw[2 * pp + 1] << 16);
            xs[pp] = xw[pp] >> 6;
        }
        const f16x8 BZ = u4_as_h8((szv[0] >> 16) | (szv[1] & 0xFFFF0000u), (szv[2] >> 16) | (szv[3] & 0xFFFF0000u),
                                  (szv[4] >> 16) | (szv[5] & 0xFFFF0000u), (szv[6] >> 16) | (szv[7] & 0xFFFF0000u));
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const f16x8 Bj = u4_as_h8(code_bits(xw[0], xs[0], jj), code_bits(xw[1], xs[1], jj),
                                      code_bits(xw[2], xs[2], jj), code_bits(xw[3], xs[3], jj));
#pragma unroll
            for (int hs = 0; hs < HS; ++hs) {
                oacc[hs][jj] = mfma_f16(AS[hs][0], Bj, oacc[hs][jj]);
                oacc[hs][jj] = mfma_f16(AS[hs][1], Bj, oacc[hs][jj]);
            }
        }
#pragma unroll
        for (int hs = 0; hs < HS; ++hs) {
            zacc[hs] = mfma_f16(AZ[hs][0], BZ, zacc[hs]);
            zacc[hs] = mfma_f16(AZ[hs][1], BZ, zacc[hs]);
        }
    }
    if (!active) return;

    // ---- write the partial (m, l, o') of the GQ heads
    const size_t row0 = (size_t(b) * a.items + j) * a.hq + hk * GQ;
#pragma unroll
    for (int hs = 0; hs < HS; ++hs) {
        float l_col = l_lane[hs] + __shfl_xor(l_lane[hs], 16);
        l_col += __shfl_xor(l_col, 32);
        const int h = 4 * hs + ch;
        if (kb == 0 && cg == 0 && h < GQ) {
            a.part_ml[(row0 + h) * 2 + 0] = m_run[hs];
            a.part_ml[(row0 + h) * 2 + 1] = l_col;
        }
        // output lane (n, kb) holds rows (g = kb, h = i); the row whose group
        // matches channel 8 n + jj (group n / 4) carries the result
        if (kb == cg) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (4 * hs + i >= GQ) break;
                float o[8];
#pragma unroll
                for (int jj = 0; jj < 8; ++jj)
                    o[jj] = oacc[hs][jj][i] * __builtin_ldexpf(1.0f, 24 - pair_exp(jj)) + zacc[hs][i];
                float *dst = a.part_o + (row0 + 4 * hs + i) * kHeadDim + 8 * n;
                *reinterpret_cast<f32x4 *>(dst) = f32x4{o[0], o[1], o[2], o[3]};
                *reinterpret_cast<f32x4 *>(dst + 4) = f32x4{o[4], o[5], o[6], o[7]};
            }
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
