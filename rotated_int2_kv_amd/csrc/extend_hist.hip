// History part of an extend call: many new tokens against the INT2 prefix on
// the matrix cores.
//
// The decode kernel's history path is shaped for one query row per KV head
// and reads every history tile once per row; a prefill chunk has thousands of
// rows over the same prefix.  Here one workgroup takes 256 query rows of one
// KV head (256 / g new tokens x g heads) and one history work item, and for
// every 32-token tile of the item:
//   1. the tile's 96-byte head records (K, V codes and (s, z)) are staged in
//      LDS; records of the next tile are in flight meanwhile;
//   2. the workgroup dequantises the tile once: x = s c + z, scaled by 1/8
//      (exact) so that any fp16 (s, z) stays inside the fp16 range, split into
//      fp16 hi + lo.  K goes to a token-major tile, V to a channel-major
//      (transposed) tile;
//   3. each wave (16 rows) runs flash attention on v_mfma_f32_16x16x32_f16:
//      S^T = K q'^T with hi.hi + hi.lo + lo.hi products (about 22 bits of
//      each operand), online softmax in log2 units on the 16-row state, and
//      O += P V with P taken straight from the S^T output registers (their
//      token order is the k-slot order of the PV product, and the V fragments
//      are read in that order), again with three products.
// Partials (m, l, o) go to the decode layout, where the merge combines them
// with the BF16 windows' and the new tokens' items.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <cmath>
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace oscar {
namespace {

constexpr int kTile = 32;                    // history tokens per tile
constexpr int kThreads = 512;                // 8 waves x 16 query rows per workgroup (BF16 items)
constexpr int kHistThreads = 1024;           // 16 waves x 16 query rows per workgroup (history items)
constexpr int kKdStride = kHeadDim + 8;      // halves per K row (272 bytes: conflict-free 16-byte reads)
constexpr int kVtStride = kTile + 4;         // halves per V^T row (72 bytes: conflict-free 8-byte reads)
constexpr float kDqScale = 0.125f;           // dequantised values are stored times 1/8
constexpr float kSlack = 15.0f;              // log2 headroom of the softmax reference (weights < 2^15)

__device__ __forceinline__ uint32_t pk_f16(float x0, float x1) {
    const f16x2 h = {static_cast<_Float16>(x0), static_cast<_Float16>(x1)};
    return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ float f16_lo(uint32_t w) { return __half2float(__ushort_as_half(uint16_t(w))); }
__device__ __forceinline__ float f16_hi(uint32_t w) { return __half2float(__ushort_as_half(uint16_t(w >> 16))); }

// (x0, x1) ~ hi + lo, both fp16 pairs rounded to nearest.  x - hi is exact
// in fp32, so one fused x * 1 - hi rounded to fp16 gives the same lo; the 1 is
// kept opaque so that the compiler emits that (one mixed-precision fma per
// half, reading hi's fp16 halves in place) instead of folding it to a
// subtraction with separate conversions.
__device__ __forceinline__ void split2(float x0, float x1, uint32_t &hi, uint32_t &lo) {
    float one = 1.0f;
    asm("" : "+s"(one));
    hi = pk_f16(x0, x1);
    lo = pk_f16(fmaf(x0, one, -f16_lo(hi)), fmaf(x1, one, -f16_hi(hi)));
}

__device__ __forceinline__ float sz_s(uint32_t w) { return f16_lo(w); }
__device__ __forceinline__ float sz_z(uint32_t w) { return f16_hi(w); }

// The wave's 16 query rows: row rho = 16 w + col is new token
// rb * tok_per_block + rho / g, query head hk * g + rho % g.  Lane (col, kq)
// holds that row's q' (times 2^K) as the B operand of S^T = K q'^T: k-slots
// = channels 32 s + 8 kq .. + 7, split into fp16 hi + lo.
struct Rows {
    f16x8 bq_hi[4], bq_lo[4];
    float unscale;      // logit (log2 units) = S^T element x unscale
    int tok;
    bool row_ok;
};

__device__ __forceinline__ void load_rows(const ExtendHistArgs &a, int tpb, int rb, int hk, int w, int col, int kq,
                                          Rows &r) {
    const int rho = 16 * w + col;
    const int tl = rho / a.g;
    const int head = rho - tl * a.g;
    r.tok = rb * tpb + tl;
    r.row_ok = tl < tpb && r.tok < a.n_new;
    const size_t qrow = size_t(r.row_ok ? r.tok : 0) * a.hq + size_t(hk) * a.g + head;
    float qscale = 0.0f;
    r.unscale = 1.0f;                                       // rows past the block: q = 0, S = 0
    if (r.row_ok) {
        qscale = a.qsum[qrow * 8 + 4];                      // 2^K: max |q'| 2^K < 2^15
        r.unscale = a.qsum[qrow * 8 + 5] * (1.0f / (16777216.0f * kDqScale));   // 2^-K x 8
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        uint32_t h[4], l[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float x0 = 0.0f, x1 = 0.0f;
            if (r.row_ok) {
                const float2 q2 = *reinterpret_cast<const float2 *>(a.qrot + qrow * kHeadDim + 32 * s + 8 * kq + 2 * e);
                x0 = q2.x * qscale;
                x1 = q2.y * qscale;
            }
            split2(x0, x1, h[e], l[e]);
        }
        r.bq_hi[s] = __builtin_bit_cast(f16x8, u32x4{h[0], h[1], h[2], h[3]});
        r.bq_lo[s] = __builtin_bit_cast(f16x8, u32x4{l[0], l[1], l[2], l[3]});
    }
}

// Partials of work item j: (m, l) of row 16 w + col from the lanes of kq 0;
// o rows 16 w + 4 kq + i, channels 16 n + col (stored times 8, undoing the
// 1/8 of the V tile).
__device__ __forceinline__ void store_partials(const ExtendHistArgs &a, int tpb, int rb, int hk, int j, int w, int col, int kq,
                                               const Rows &r, float m_run, float l_run, const f32x4 *o) {
    if (kq == 0 && r.row_ok) {
        const int rho = 16 * w + col;
        const int head = rho - (rho / a.g) * a.g;
        float *ml = a.part_ml + ((size_t(r.tok) * a.items + j) * a.hq + size_t(hk) * a.g + head) * 2;
        ml[0] = m_run;
        ml[1] = l_run;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int rr = 16 * w + 4 * kq + i;
        const int tli = rr / a.g;
        const int hi = rr - tli * a.g;
        const int toki = rb * tpb + tli;
        if (tli < tpb && toki < a.n_new) {
            float *dst = a.part_o + ((size_t(toki) * a.items + j) * a.hq + size_t(hk) * a.g + hi) * kHeadDim;
#pragma unroll
            for (int n = 0; n < 8; ++n) dst[16 * n + col] = o[n][i] * (1.0f / kDqScale);
        }
    }
}

// o *= al (row 4 kq + i by al[i]) for two output blocks, skipped by a scalar
// branch when `moved` (wave-uniform) is 0: a row's reference moves in few
// tiles.  The branch sits inside the asm so that the compiler sees straight
// code (an `if` around the products made it spill the accumulators).
__device__ __forceinline__ void rescale_if(f32x4 &oa, f32x4 &ob, const float (&al)[4], int moved) {
    float a0 = oa[0], a1 = oa[1], a2 = oa[2], a3 = oa[3], b0 = ob[0], b1 = ob[1], b2 = ob[2], b3 = ob[3];
    asm volatile(
        "s_cmp_eq_u32 %[mv], 0\n\t"
        "s_cbranch_scc1 .Lrescale_skip_%=\n\t"
        "v_mul_f32_e32 %[a0], %[a0], %[s0]\n\t"
        "v_mul_f32_e32 %[a1], %[a1], %[s1]\n\t"
        "v_mul_f32_e32 %[a2], %[a2], %[s2]\n\t"
        "v_mul_f32_e32 %[a3], %[a3], %[s3]\n\t"
        "v_mul_f32_e32 %[b0], %[b0], %[s0]\n\t"
        "v_mul_f32_e32 %[b1], %[b1], %[s1]\n\t"
        "v_mul_f32_e32 %[b2], %[b2], %[s2]\n\t"
        "v_mul_f32_e32 %[b3], %[b3], %[s3]\n\t"
        ".Lrescale_skip_%=:"
        : [a0] "+v"(a0), [a1] "+v"(a1), [a2] "+v"(a2), [a3] "+v"(a3), [b0] "+v"(b0), [b1] "+v"(b1),
          [b2] "+v"(b2), [b3] "+v"(b3)
        : [s0] "v"(al[0]), [s1] "v"(al[1]), [s2] "v"(al[2]), [s3] "v"(al[3]), [mv] "s"(moved)
        : "scc");
    oa = f32x4{a0, a1, a2, a3};
    ob = f32x4{b0, b1, b2, b3};
}

// One 32-token tile of flash attention for the wave's 16 query rows.
// kd: K tile [hi, lo][token][channel]; vt: V tile [hi, lo][channel][token]
// (fp16, times 1/8).  S^T = K q'^T leaves lane (col, kq) with tokens
// 16 u + 4 kq + i of row col; the products start from bias[u][i], 0 for a
// usable token and -inf for one that is masked, so a masked logit is -inf
// and its weight exp2(-inf) = 0 with no select.  With
// kKLo false the K lo tile is zero (BF16 sources are exact in fp16) and its
// products are skipped.  V is one fp16 per value: its rounding (relative
// 2^-12, unbiased) enters the output as a weighted average, so it stays near
// 2^-12 of the output's scale, while a K rounding error is amplified by the
// logit's magnitude and keeps its lo part.
template <bool kKLo>
__device__ __forceinline__ void flash_step(const _Float16 (*kd)[kTile][kKdStride],
                                           const _Float16 (*vt)[kHeadDim][kVtStride], const f16x8 *bq_hi,
                                           const f16x8 *bq_lo, float unscale, const f32x4 *bias, float &m_run,
                                           float &l_run, f32x4 *o, int col, int kq) {
    f32x4 d[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        f32x4 acc = bias[u];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const f16x8 kh = *reinterpret_cast<const f16x8 *>(&kd[0][16 * u + col][32 * s + 8 * kq]);
            acc = mfma_f16(kh, bq_hi[s], acc);
            acc = mfma_f16(kh, bq_lo[s], acc);
            if constexpr (kKLo) {
                const f16x8 kl = *reinterpret_cast<const f16x8 *>(&kd[1][16 * u + col][32 * s + 8 * kq]);
                acc = mfma_f16(kl, bq_hi[s], acc);
            }
        }
        d[u] = acc;
    }
    // row maximum of the tile in S^T units (unscale > 0 keeps the order)
    float mt = fmaxf(d[0][0], d[0][1]);
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 2 * (u == 0); i < 4; ++i) mt = fmaxf(mt, d[u][i]);
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    mt *= unscale;                                          // log2 units
    // The reference maximum moves only when a logit exceeds it by more than
    // kSlack (weights stay below 2^kSlack, inside fp16), so alpha is mostly 1.
    const bool move = mt > m_run + kSlack;
    const float m_new = move ? mt : m_run;
    const float alpha = move ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
    m_run = m_new;
    // while every token of the row so far is masked, m is -inf: a finite
    // stand-in keeps exp2(-inf - m) from becoming NaN
    const float m_ref = m_new == -INFINITY ? 0.0f : m_new;
    float p[2][4];
    float lsum = 0.0f;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[u][i] = __builtin_amdgcn_exp2f(fmaf(d[u][i], unscale, -m_ref));
            lsum += p[u][i];
        }
    }
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    l_run = fmaf(l_run, alpha, lsum);

    // O += P V: A = P (row col, k-slot 4 u + i = token 16 u + 4 kq + i)
    uint32_t ph[4], pl[4];
    split2(p[0][0], p[0][1], ph[0], pl[0]);
    split2(p[0][2], p[0][3], ph[1], pl[1]);
    split2(p[1][0], p[1][1], ph[2], pl[2]);
    split2(p[1][2], p[1][3], ph[3], pl[3]);
    const f16x8 a_hi = __builtin_bit_cast(f16x8, u32x4{ph[0], ph[1], ph[2], ph[3]});
    const f16x8 a_lo = __builtin_bit_cast(f16x8, u32x4{pl[0], pl[1], pl[2], pl[3]});
    float al[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * kq + i);        // alpha of output row 4 kq + i
    const int moved = __builtin_amdgcn_readfirstlane(__any(move) ? 1 : 0);
#pragma unroll
    for (int n = 0; n < 8; n += 2) rescale_if(o[n], o[n + 1], al, moved);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
        const int ch = 16 * n + col;
        const u32x2 v0 = *reinterpret_cast<const u32x2 *>(&vt[0][ch][4 * kq]);
        const u32x2 v1 = *reinterpret_cast<const u32x2 *>(&vt[0][ch][16 + 4 * kq]);
        const f16x8 vh = __builtin_bit_cast(f16x8, u32x4{v0[0], v0[1], v1[0], v1[1]});
        o[n] = mfma_f16(a_hi, vh, o[n]);
        o[n] = mfma_f16(a_lo, vh, o[n]);
    }
}

// At most 128 VGPRs (launch bound of 4 waves per SIMD): one workgroup of 16
// waves per compute unit, so that each tile's dequantisation (K by waves
// 0-7, V by waves 8-15) serves 256 query rows.
// NG = groups per head vector (4, 2, 1 for G = 32, 64, 128), SZB = bytes of
// one group's (s, z) (4: fp16, 2: E4M3 codes): head records of 96, 80 or 72
// bytes, staged in 16-byte units (8-byte units for 72).
template <int NG, int SZB>
__global__ __launch_bounds__(kHistThreads, 4) void extend_hist_kernel(ExtendHistArgs a) {
    constexpr int kRec = 2 * kCodeBytes + 2 * NG * SZB;
    // (s, z) stored at p, times 1/8 (exact); group g of tensor t (0 = K, 1 = V)
    // sits at byte 64 + (t NG + g) SZB of a head record
    auto load_sz = [](const uint8_t *p) -> float2 {
        if constexpr (SZB == 4) {
            const uint32_t w = *reinterpret_cast<const uint32_t *>(p);
            return make_float2(sz_s(w) * kDqScale, sz_z(w) * kDqScale);
        } else {
            const uint32_t w = e4m3x2_to_f16x2(*reinterpret_cast<const uint16_t *>(p));
            return make_float2(sz_s(w) * kDqScale, sz_z(w) * kDqScale);
        }
    };
    constexpr int kUnit = kRec % 16 == 0 ? 16 : 8;
    constexpr int kUnits = kRec / kUnit;
    using Unit = std::conditional_t<kUnit == 16, u32x4, u32x2>;
    // two of everything: tile k is computed from one buffer while tile k + 1
    // is dequantised into the other, one workgroup barrier per tile
    __shared__ __attribute__((aligned(16))) uint8_t raw_all[2][kTile * kRec];
    __shared__ __attribute__((aligned(16))) float bias_all[2][kTile];
    __shared__ __attribute__((aligned(16))) _Float16 kd_all[2][2][kTile][kKdStride];
    __shared__ __attribute__((aligned(16))) _Float16 vt_all[2][1][kHeadDim][kVtStride];

    const int id = blockIdx.x;
    const int rb = id % a.hist_row_blocks;
    const int rest = id / a.hist_row_blocks;
    const int hk = rest % a.hkv;
    const int jj = rest / a.hkv;
    const int j = 2 + jj;                                   // work item index in the decode layout
    const int hist_end = max(a.sink, a.prefix_len - a.recent);
    const int p0 = a.sink + jj * a.chunk;
    const int p1 = min(p0 + a.chunk, hist_end);
    if (p0 >= p1) return;                                   // uniform over the workgroup

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int col = lane & 15;
    const int kq = lane >> 4;

    Rows r;
    load_rows(a, a.hist_tok_per_block, rb, hk, w, col, kq, r);
    float m_run = -INFINITY, l_run = 0.0f;
    f32x4 o[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) o[n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // ---- producers: thread < 32 kUnits stages unit pu of token pt's head record
    const bool producer = tid < kTile * kUnits;
    const int pt = tid / kUnits;
    const int pu = tid - kUnits * pt;
    const size_t rec_bytes = size_t(a.hkv) * kRec;
    auto slot_of = [&](int c) -> int {
        const int p = c + pt;
        return (producer && p < p1) ? __builtin_nontemporal_load(a.slot_row + p) : -1;
    };
    auto usable = [&](int slot) { return slot >= 0 && slot < a.num_slots; };
    auto load_rec = [&](int slot) -> Unit {
        const uint8_t *base = usable(slot) ? a.records + size_t(slot) * rec_bytes + size_t(hk) * kRec : a.zero_rec;
        return __builtin_nontemporal_load(reinterpret_cast<const Unit *>(base + kUnit * pu));
    };
    // records of the next tile to stage, its usability, and the slot ids of the one after
    int slot_cur = slot_of(p0);
    Unit rec = producer ? load_rec(slot_cur) : Unit{};
    bool ok_cur = usable(slot_cur);
    int slot_nxt = slot_of(p0 + kTile);
    // stage the records held in `rec` (tile at cb) into buffer b, then start loading the next
    auto stage = [&](int b, int cb) {
        if (producer) {
            *reinterpret_cast<Unit *>(raw_all[b] + pt * kRec + kUnit * pu) = rec;
            if (pu == 0) bias_all[b][pt] = ok_cur ? 0.0f : -INFINITY;
        }
        if (cb + kTile < p1) {
            if (producer) rec = load_rec(slot_nxt);
            ok_cur = usable(slot_nxt);
            slot_nxt = slot_of(cb + 2 * kTile);
        }
    };
    auto dequant = [&](int b) {
        const uint8_t *raw = raw_all[b];
        _Float16(*kd)[kTile][kKdStride] = kd_all[b];
        _Float16(*vt)[kHeadDim][kVtStride] = vt_all[b];
        // ---- 2. dequantise.  K rows (token t, channels 8 part .. +7), by
        // threads 0..511: the group's four levels (s c + z) / 8, c = 0..3, as
        // fp16 hi and lo pairs, then one byte-select (v_perm) per two channels
        // picks their levels
        if (tid < 512) {
            const int t = tid >> 4, part = tid & 15;
            const uint32_t cw = *reinterpret_cast<const uint16_t *>(raw + t * kRec + 2 * part);
            const float2 sz = load_sz(raw + t * kRec + 2 * kCodeBytes + SZB * (part * NG / 16));
            const float s = sz.x, z = sz.y;
            uint32_t h01, l01, h23, l23;
            split2(z, s + z, h01, l01);                       // s + z: fmaf(s, 1, z)
            split2(fmaf(s, 2.0f, z), fmaf(s, 3.0f, z), h23, l23);
            const uint32_t c0s = cw & 0x3333u;                 // code of channel 2e at bits 4e
            const uint32_t c1s = (cw >> 2) & 0x3333u;          // code of channel 2e + 1 at bits 4e
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // selector bytes 2 c0, 2 c0 + 1, 2 c1, 2 c1 + 1 (levels 0, 1 in h01, 2, 3 in h23)
                const uint32_t y = ((c0s >> (4 * e)) & 3u) | (((c1s >> (4 * e)) & 3u) << 16);
                const uint32_t sel = y * 0x0202u + 0x01000100u;
                hi[e] = __builtin_amdgcn_perm(h23, h01, sel);
                lo[e] = __builtin_amdgcn_perm(l23, l01, sel);
            }
            *reinterpret_cast<u32x4 *>(&kd[0][t][8 * part]) = u32x4{hi[0], hi[1], hi[2], hi[3]};
            *reinterpret_cast<u32x4 *>(&kd[1][t][8 * part]) = u32x4{lo[0], lo[1], lo[2], lo[3]};
        }
        // V^T rows (channels 2 cp, 2 cp + 1; tokens 4 tq .. 4 tq + 3), by threads
        // 512..1023, one fp16 per value; 8-byte row writes (at most 2 lanes of
        // 16 per bank)
        else {
            const int cp = (tid - 512) & 63, tq = (tid - 512) >> 6;
            const int byte = 32 + (cp >> 1), sh = 4 * (cp & 1);
            const int sz_off = 2 * kCodeBytes + SZB * NG + SZB * (cp * NG / 64);
            float x0[4], x1[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int t = 4 * tq + k;
                const uint32_t c = uint32_t(raw[t * kRec + byte]) >> sh;
                const float2 sz = load_sz(raw + t * kRec + sz_off);
                const float s = sz.x, z = sz.y;
                x0[k] = fmaf(s, float(c & 3u), z);
                x1[k] = fmaf(s, float((c >> 2) & 3u), z);
            }
            *reinterpret_cast<u32x2 *>(&vt[0][2 * cp][4 * tq]) = u32x2{pk_f16(x0[0], x0[1]), pk_f16(x0[2], x0[3])};
            *reinterpret_cast<u32x2 *>(&vt[0][2 * cp + 1][4 * tq]) = u32x2{pk_f16(x1[0], x1[1]), pk_f16(x1[2], x1[3])};
        }
    };

    stage(0, p0);
    __syncthreads();
    dequant(0);
    // one tile from buffer `buf` (a compile-time constant: the loop runs two tiles per
    // iteration, so every LDS address is an immediate offset)
    auto tile = [&](auto bufc, int cb) {
        constexpr int buf = decltype(bufc)::value;
        const bool more = cb + kTile < p1;
        if (more) stage(buf ^ 1, cb + kTile);
        // logit biases of tile cb, 0 or -inf for tokens that are not usable
        // (past the item included); read before the barrier: the staging of
        // tile cb + 2 overwrites them once every wave has passed it
        const f32x4 bias[2] = {*reinterpret_cast<const f32x4 *>(&bias_all[buf][4 * kq]),
                               *reinterpret_cast<const f32x4 *>(&bias_all[buf][16 + 4 * kq])};
        __syncthreads();
        flash_step<true>(kd_all[buf], vt_all[buf], r.bq_hi, r.bq_lo, r.unscale, bias, m_run, l_run, o, col, kq);
        if (more) dequant(buf ^ 1);                         // overlaps the step's matrix-core work
    };
    for (int cb = p0; cb < p1; cb += 2 * kTile) {
        tile(std::integral_constant<int, 0>{}, cb);
        if (cb + kTile < p1) tile(std::integral_constant<int, 1>{}, cb + kTile);
    }

    store_partials(a, a.hist_tok_per_block, rb, hk, j, w, col, kq, r, m_run, l_run, o);
}

// BF16 items: kind 0 = sink window [0, min(S, P)), kind 1 = recent window
// [max(S, P - W), P), kind 2 = the new tokens themselves, causal (row token
// i sees new tokens 0..i).  Rows are exact in fp16 once scaled by 1/8 (bf16
// has fewer mantissa bits), so there is no lo tile.  Each thread loads 32
// bytes of a K row and 4 bytes of 8 V rows per tile, one tile ahead.
__global__ __launch_bounds__(kThreads, 4) void extend_bf16_kernel(ExtendHistArgs a) {
    __shared__ __attribute__((aligned(16))) _Float16 kd[1][kTile][kKdStride];
    __shared__ __attribute__((aligned(16))) _Float16 vt[1][kHeadDim][kVtStride];

    const int id = blockIdx.x;
    const int rb = id % a.row_blocks;
    const int rest = id / a.row_blocks;
    const int hk = rest % a.hkv;
    const int kind = rest / a.hkv;
    const int P = a.prefix_len;
    int p0, p1, j;
    if (kind == 0) {
        p0 = 0;
        p1 = min(a.sink, P);
        j = 0;
    } else if (kind == 1) {
        p0 = max(a.sink, P - a.recent);
        p1 = P;
        j = 1;
    } else {
        p0 = 0;
        p1 = min(a.n_new, (rb + 1) * a.tok_per_block);
        j = a.extra_item;
    }
    if (p0 >= p1) return;                                   // uniform over the workgroup

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int col = lane & 15;
    const int kq = lane >> 4;
    Rows r;
    load_rows(a, a.tok_per_block, rb, hk, w, col, kq, r);
    float m_run = -INFINITY, l_run = 0.0f;
    f32x4 o[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) o[n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    auto row_ptr = [&](int pos) -> const uint16_t * {
        size_t row;
        if (kind == 0)
            row = (size_t(a.req) * a.sink + pos) * a.hkv + hk;
        else if (kind == 1)
            row = (size_t(a.req) * a.recent + pos % a.recent) * a.hkv + hk;
        else
            row = size_t(pos) * a.hkv + hk;
        const uint16_t *base = kind == 0 ? a.sink_store : kind == 1 ? a.recent_store : a.newkv;
        return base + row * (2 * kHeadDim);
    };
    // K: token kt, channels 8 kp .. +7; V: channels 2 cp, 2 cp + 1 of tokens 4 tg .. +3
    const int kt = tid >> 4, kp = tid & 15;
    const int cp = tid & 63, tg = tid >> 6;
    u32x4 kreg;
    uint32_t vreg[4];
    auto load_tile = [&](int c) {
        const int pk = c + kt;
        kreg = pk < p1 ? __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(row_ptr(pk) + 8 * kp))
                       : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int pv = c + 4 * tg + k;
            vreg[k] = pv < p1 ? __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(row_ptr(pv) + kHeadDim) + cp)
                              : 0u;
        }
    };
    auto bf = [](uint32_t u, int half) { return __uint_as_float(half ? (u & 0xFFFF0000u) : (u << 16)) * kDqScale; };
    load_tile(p0);
    for (int cb = p0; cb < p1; cb += kTile) {
        __syncthreads();                                    // every wave is done with the previous tile
        {
            uint32_t hk4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) hk4[e] = pk_f16(bf(kreg[e], 0), bf(kreg[e], 1));
            *reinterpret_cast<u32x4 *>(&kd[0][kt][8 * kp]) = u32x4{hk4[0], hk4[1], hk4[2], hk4[3]};
            uint32_t h0[2], h1[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                h0[e] = pk_f16(bf(vreg[2 * e], 0), bf(vreg[2 * e + 1], 0));
                h1[e] = pk_f16(bf(vreg[2 * e], 1), bf(vreg[2 * e + 1], 1));
            }
            *reinterpret_cast<u32x2 *>(&vt[0][2 * cp][4 * tg]) = u32x2{h0[0], h0[1]};
            *reinterpret_cast<u32x2 *>(&vt[0][2 * cp + 1][4 * tg]) = u32x2{h1[0], h1[1]};
        }
        if (cb + kTile < p1) load_tile(cb + kTile);
        __syncthreads();
        f32x4 bias[2];
        const int lim = kind == 2 ? r.tok : INT32_MAX;      // causal: key position <= row token
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int pos = cb + 16 * u + 4 * kq + i;
                bias[u][i] = (pos < p1 && pos <= lim) ? 0.0f : -INFINITY;
            }
        flash_step<false>(kd, vt, r.bq_hi, r.bq_lo, r.unscale, bias, m_run, l_run, o, col, kq);
    }
    store_partials(a, a.tok_per_block, rb, hk, j, w, col, kq, r, m_run, l_run, o);
}

// Merge of the work items and un-rotation, o = o' R_V^T, for 8 new tokens
// (8 g query rows) of one KV head per workgroup, so that R_V is read once per
// 8 tokens instead of once per token.  Thread (c, rq) first merges channel c
// of rows rq, rq + 4, ... into LDS, then computes output channel c of those
// rows from its row of R_V.
constexpr int kMergeTokens = 8;

__global__ __launch_bounds__(512) void extend_merge_kernel(ExtendHistArgs a) {
    __shared__ float ob[kMergeTokens * kMaxGroup][kHeadDim];
    const int rbm = blockIdx.x;
    const int hk = blockIdx.y;
    const int c = threadIdx.x & (kHeadDim - 1);
    const int rq = threadIdx.x >> 7;
    const int g = a.g;
    const int rows = kMergeTokens * g;
    const int P = a.prefix_len;
    const bool sink_ok = min(a.sink, P) > 0;
    const bool recent_ok = P > a.sink;
    const int hist = max(0, max(a.sink, P - a.recent) - a.sink);
    const int n_hist = (a.num_slots > 0 && hist > 0) ? a.hist_items : 0;
    auto item_ok = [&](int jj) {
        return jj == a.extra_item || (jj == 0 && sink_ok) || (jj == 1 && recent_ok) || (jj >= 2 && jj < 2 + n_hist);
    };
    for (int rr = rq; rr < rows; rr += 4) {
        const int tok = rbm * kMergeTokens + rr / g;
        const int h = rr - (rr / g) * g;
        float o = 0.0f;
        if (tok < a.n_new) {
            const size_t row_h = size_t(tok) * a.items * a.hq + size_t(hk) * g + h;    // item 0
            float M = -INFINITY;
            for (int jj = 0; jj <= a.extra_item; ++jj)
                if (item_ok(jj)) M = fmaxf(M, a.part_ml[(row_h + size_t(jj) * a.hq) * 2]);
            float l = 0.0f, acc = 0.0f;
            if (M != -INFINITY) {
                for (int jj = 0; jj <= a.extra_item; ++jj) {
                    if (!item_ok(jj)) continue;
                    const size_t row = row_h + size_t(jj) * a.hq;
                    const float e = __builtin_amdgcn_exp2f(a.part_ml[row * 2] - M);
                    l = fmaf(e, a.part_ml[row * 2 + 1], l);
                    acc = fmaf(e, a.part_o[row * kHeadDim + c], acc);
                }
            }
            o = l > 0.0f ? acc / l : 0.0f;
        }
        ob[rr][c] = o;
    }
    __syncthreads();
    const float *R = a.r_v + (size_t(hk) * kHeadDim + c) * kHeadDim;
    float acc[kMergeTokens * kMaxGroup / 4];
#pragma unroll
    for (int k = 0; k < kMergeTokens * kMaxGroup / 4; ++k) acc[k] = 0.0f;
    for (int i = 0; i < kHeadDim; i += 4) {
        const f32x4 r = *reinterpret_cast<const f32x4 *>(R + i);
#pragma unroll
        for (int k = 0; k < kMergeTokens * kMaxGroup / 4; ++k) {
            const int rr = rq + 4 * k;
            if (rr < rows) {
                acc[k] = fmaf(ob[rr][i], r[0], acc[k]);
                acc[k] = fmaf(ob[rr][i + 1], r[1], acc[k]);
                acc[k] = fmaf(ob[rr][i + 2], r[2], acc[k]);
                acc[k] = fmaf(ob[rr][i + 3], r[3], acc[k]);
            }
        }
    }
#pragma unroll
    for (int k = 0; k < kMergeTokens * kMaxGroup / 4; ++k) {
        const int rr = rq + 4 * k;
        const int tok = rbm * kMergeTokens + rr / g;
        if (rr >= rows || tok >= a.n_new) continue;
        const size_t idx = (size_t(tok) * a.hq + size_t(hk) * g + (rr - (rr / g) * g)) * kHeadDim + c;
        if (a.out_dtype == OSCAR_F32)
            static_cast<float *>(a.out)[idx] = acc[k];
        else if (a.out_dtype == OSCAR_BF16)
            static_cast<uint16_t *>(a.out)[idx] = bf16_bits_rn(acc[k]);
        else
            static_cast<__half *>(a.out)[idx] = __float2half_rn(acc[k]);
    }
}

}  // namespace

hipError_t launch_extend_merge(const ExtendHistArgs &a, hipStream_t stream) {
    const unsigned blocks = unsigned((a.n_new + kMergeTokens - 1) / kMergeTokens);
    hipLaunchKernelGGL(extend_merge_kernel, dim3(blocks, a.hkv), dim3(512), 0, stream, a);
    return hipGetLastError();
}

int64_t extend_bf16_blocks(const ExtendHistArgs &a) { return int64_t(a.row_blocks) * 3 * a.hkv; }

hipError_t launch_extend_bf16(const ExtendHistArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL(extend_bf16_kernel, dim3(unsigned(extend_bf16_blocks(a))), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

int64_t extend_history_blocks(const ExtendHistArgs &a) {
    return int64_t(a.hist_row_blocks) * a.hist_items * a.hkv;
}

hipError_t launch_extend_history(const ExtendHistArgs &a, hipStream_t stream) {
    const int64_t blocks = extend_history_blocks(a);
    if (blocks <= 0) return hipSuccess;
    if (a.scale_bits == 8) {
        hipLaunchKernelGGL((extend_hist_kernel<2, 2>), dim3(unsigned(blocks)), dim3(kHistThreads), 0, stream, a);
        return hipGetLastError();
    }
    switch (a.group_size) {
        case 64: hipLaunchKernelGGL((extend_hist_kernel<2, 4>), dim3(unsigned(blocks)), dim3(kHistThreads), 0, stream, a); break;
        case 128: hipLaunchKernelGGL((extend_hist_kernel<1, 4>), dim3(unsigned(blocks)), dim3(kHistThreads), 0, stream, a); break;
        default: hipLaunchKernelGGL((extend_hist_kernel<4, 4>), dim3(unsigned(blocks)), dim3(kHistThreads), 0, stream, a); break;
    }
    return hipGetLastError();
}

}  // namespace oscar
