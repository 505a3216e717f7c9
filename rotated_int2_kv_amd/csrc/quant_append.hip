// oscar_quant_append: rotate, clip, INT2-quantise, pack and route new K/V
// tokens (Together AI OSCAR page, "Serving system"; group-wise INT2 with
// per-group scale and zero, "Why is INT2 KV-cache quantization hard?").
//
// One workgroup = one (token chunk, KV head, tensor K or V); its four waves
// own the four groups of 32 rotated output channels.  Each wave keeps the
// transposed rotation columns of its group in registers as MFMA A operands:
// the fp32 rotation is split exactly into three bf16 terms r1 + r2 + r3, so
// with bf16 inputs the product x R is formed without approximation and
// accumulated in fp32 on the matrix cores (v_mfma_f32_32x32x16_bf16: 32
// output channels x 32 tokens per product, 16 input channels deep).  Tiles
// of 32 tokens are staged through LDS as the B operand (x^T).  The rows of A
// are ordered so that each lane ends up with 16 contiguous rotated channels
// of one token: the two lanes l and l + 32 hold the two halves of a token's
// group, so the group's statistics, scale, zero and code thresholds are
// formed by two lanes (each lane forms two of the thresholds and swaps them
// with its partner), and each lane writes its 16 codes as one 32-bit word.
// With groups of 64 or 128 channels (NGW = 2 or 4 waves per group) the waves
// of a group also exchange their minima and maxima through LDS.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <algorithm>

#include "common.h"
#include "internal.h"

namespace oscar {
namespace {

constexpr int kTile = 32;             // tokens per MFMA tile
constexpr int kWaves = 4;             // one per output group
constexpr int kThreads = 64 * kWaves;
constexpr int kRowBytes = 2 * kHeadDim + 16;   // padded LDS row of one token (bf16 plane)
constexpr int kPlaneBytes = kTile * kRowBytes;

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

struct AppendArgs {
    const void *k;
    const void *v;
    const int32_t *req_ids;
    const int32_t *positions;
    const int32_t *slots;
    const int32_t *seq_len_after;
    const float *r_k;
    const float *r_v;
    float *rotated_out;
    uint8_t *records;
    uint16_t *sink;
    uint16_t *recent;
    int64_t num_slots;
    int32_t n_tokens;
    int32_t hkv;
    int32_t sink_tokens;
    int32_t recent_tokens;
    int32_t max_requests;
    int32_t chunk;
    int32_t n_chunks;
    int32_t in_dtype;
    float alpha;
};

// The fp32 value nearest above (or equal to) t: t rounded to nearest, then one
// ulp toward +infinity if that fell below t.  t is never in (0, 2^-25) here,
// so a rounded value of zero is exact and needs no step.
__device__ __forceinline__ float round_up_f32(double t) {
    const float f = float(t);
    return double(f) < t ? __int_as_float(__float_as_int(f) + (f >= 0.0f ? 1 : -1)) : f;
}

// Four 2-bit codes into a word, the code of x3 first: with thresholds
// u0 <= u1 <= u2 the code (number of thresholds at or below x) has high bit
// x >= u1 and low bit x >= u2 if that holds, else x >= u0.  Each code enters
// as two doublings of the word with the bit as carry-in (v_addc_co_u32 takes
// it straight from the compare's lane mask): 5 instructions per code.  Every
// lane mask is read three or more instructions after the compare that writes
// it, past the wait a VALU-written mask needs before a VALU reads it.
__device__ __forceinline__ uint32_t codes4_into(uint32_t p, float x3, float x2, float x1, float x0, float u0,
                                                float u1, float u2) {
    uint64_t m3, m2, m1, m0, n3, n2, n1, n0, co;
    float s3, s2, s1, s0;
    asm("v_cmp_ge_f32_e64 %[m3], %[x3], %[u1]\n\t"
        "v_cmp_ge_f32_e64 %[m2], %[x2], %[u1]\n\t"
        "v_cmp_ge_f32_e64 %[m1], %[x1], %[u1]\n\t"
        "v_cmp_ge_f32_e64 %[m0], %[x0], %[u1]\n\t"
        "v_cndmask_b32_e64 %[s3], %[u0], %[u2], %[m3]\n\t"
        "v_cndmask_b32_e64 %[s2], %[u0], %[u2], %[m2]\n\t"
        "v_cndmask_b32_e64 %[s1], %[u0], %[u2], %[m1]\n\t"
        "v_cndmask_b32_e64 %[s0], %[u0], %[u2], %[m0]\n\t"
        "v_cmp_ge_f32_e64 %[n3], %[x3], %[s3]\n\t"
        "v_cmp_ge_f32_e64 %[n2], %[x2], %[s2]\n\t"
        "v_cmp_ge_f32_e64 %[n1], %[x1], %[s1]\n\t"
        "v_cmp_ge_f32_e64 %[n0], %[x0], %[s0]\n\t"
        "v_addc_co_u32_e64 %[p], %[co], %[p], %[p], %[m3]\n\t"
        "v_addc_co_u32_e64 %[p], %[co], %[p], %[p], %[n3]\n\t"
        "v_addc_co_u32_e64 %[p], %[co], %[p], %[p], %[m2]\n\t"
        "v_addc_co_u32_e64 %[p], %[co], %[p], %[p], %[n2]\n\t"
        "v_addc_co_u32_e64 %[p], %[co], %[p], %[p], %[m1]\n\t"
        "v_addc_co_u32_e64 %[p], %[co], %[p], %[p], %[n1]\n\t"
        "v_addc_co_u32_e64 %[p], %[co], %[p], %[p], %[m0]\n\t"
        "v_addc_co_u32_e64 %[p], %[co], %[p], %[p], %[n0]"
        : [p] "+v"(p), [m3] "=&s"(m3), [m2] "=&s"(m2), [m1] "=&s"(m1), [m0] "=&s"(m0), [n3] "=&s"(n3),
          [n2] "=&s"(n2), [n1] "=&s"(n1), [n0] "=&s"(n0), [co] "=&s"(co), [s3] "=&v"(s3), [s2] "=&v"(s2),
          [s1] "=&v"(s1), [s0] "=&v"(s0)
        : [x3] "v"(x3), [x2] "v"(x2), [x1] "v"(x1), [x0] "v"(x0), [u0] "v"(u0), [u1] "v"(u1), [u2] "v"(u2));
    return p;
}

// Split an fp32 value into three bf16 terms whose sum is the value.
__device__ __forceinline__ void split3(float x, uint16_t &a, uint16_t &b, uint16_t &c) {
    a = bf16_bits_rn(x);
    const float r1 = x - bf16_bits_to_f32(a);
    b = bf16_bits_rn(r1);
    const float r2 = r1 - bf16_bits_to_f32(b);
    c = bf16_bits_rn(r2);
}

// SZB: bytes of one group's (s, z): 4 (two fp16) or 2 (two E4M3 codes)
template <int XT, int NGW, int SZB>
__global__ __launch_bounds__(kThreads) void quant_append_kernel(AppendArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t lds_buf[2][XT * kPlaneBytes];
    __shared__ float2 grp_stat[kWaves][kTile];             // per wave and token: (min, max)

    // XCD-aware block order: blocks are dealt round-robin to the 8 XCDs, so
    // all 2*Hkv workgroups of one token chunk land on the same XCD and its L2
    // assembles the slot records of that chunk.
    const int id = blockIdx.x;
    const int xcd = id & 7;
    const int li = id >> 3;
    const int ht = li % (2 * a.hkv);
    const int chunk_id = xcd + 8 * (li / (2 * a.hkv));
    if (chunk_id >= a.n_chunks) return;
    const int h = ht >> 1;
    const int t = ht & 1;
    const int tok_begin = chunk_id * a.chunk;
    const int tok_end = min(a.n_tokens, tok_begin + a.chunk);

    const int tid = threadIdx.x;
    const int w = tid >> 6;          // output group
    const int lane = tid & 63;
    const int tt = lane & 31;        // token of the tile (MFMA column)
    const int hh = lane >> 5;        // half of the group: channels 16 hh .. 16 hh + 15

    // A operands: transposed rotation rows of this wave's 32 output channels.
    // Output element 4 j + i of lane (tt, hh) is row 8 j + 4 hh + i; that row
    // holds output channel 32 w + 16 hh + 4 j + i, so the lane's 16 elements
    // are the channels 32 w + 16 hh + 0..15 in order.
    const float *R = (t == 0 ? a.r_k : a.r_v) + size_t(h) * kHeadDim * kHeadDim;
    bf16x8 rf[8][3];
    {
        const int r = lane & 31;
        const int oc = 32 * w + 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int ic = 16 * ks + 8 * hh + j;
                uint16_t x0, x1, x2;
                split3(R[size_t(ic) * kHeadDim + oc], x0, x1, x2);
                rf[ks][0][j] = bits_to_bf16(x0);
                rf[ks][1][j] = bits_to_bf16(x1);
                rf[ks][2][j] = bits_to_bf16(x2);
            }
        }
    }

    // staging: a tile is 32 token rows x 16 units of 8 channels; thread tid
    // stages units tid and tid + 256 (row u / 16, channels 8 (u % 16) ..).
    // Addresses: a per-thread base (head h, channels 8 (tid % 16) ..) plus
    // token x the bytes of one token's heads (one 32 x 32 -> 64-bit multiply-add).
    const bool f32_in = a.in_dtype == OSCAR_F32;
    const uint32_t esz = f32_in ? 4u : 2u;
    const uint32_t x_tok_bytes = uint32_t(a.hkv) * kHeadDim * esz;
    const uint8_t *const x_base = static_cast<const uint8_t *>(t == 0 ? a.k : a.v) +
                                  (uint32_t(h) * kHeadDim + 8u * uint32_t(tid & 15)) * esz;
    auto load_tile = [&](int tb, u32x4 (&r)[2][2]) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int tok = tb + (tid >> 4) + 16 * q;
            r[q][0] = u32x4{0, 0, 0, 0};
            r[q][1] = u32x4{0, 0, 0, 0};
            if (tok < tok_end) {
                const u32x4 *p = reinterpret_cast<const u32x4 *>(x_base + uint64_t(uint32_t(tok)) * x_tok_bytes);
                r[q][0] = __builtin_nontemporal_load(p);            // input read once
                if (f32_in) r[q][1] = __builtin_nontemporal_load(p + 1);
            }
        }
    };
    auto store_tile = [&](uint8_t *lds, const u32x4 (&r)[2][2]) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int u = tid + 256 * q;
            uint8_t *dst = lds + (u >> 4) * kRowBytes + 16 * (u & 15);
            if constexpr (XT == 1) {
                *reinterpret_cast<u32x4 *>(dst) = r[q][0];
            } else {
                float f[8];
                if (a.in_dtype == OSCAR_F32) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        f[j] = __uint_as_float(r[q][0][j]);
                        f[4 + j] = __uint_as_float(r[q][1][j]);
                    }
                } else {  // fp16 input, converted exactly to fp32
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        f[2 * j] = __half2float(__ushort_as_half(uint16_t(r[q][0][j] & 0xFFFFu)));
                        f[2 * j + 1] = __half2float(__ushort_as_half(uint16_t(r[q][0][j] >> 16)));
                    }
                }
                uint16_t p0[8], p1[8], p2[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) split3(f[j], p0[j], p1[j], p2[j]);
                u32x4 w0, w1, w2;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    w0[j] = uint32_t(p0[2 * j]) | (uint32_t(p0[2 * j + 1]) << 16);
                    w1[j] = uint32_t(p1[2 * j]) | (uint32_t(p1[2 * j + 1]) << 16);
                    w2[j] = uint32_t(p2[2 * j]) | (uint32_t(p2[2 * j + 1]) << 16);
                }
                *reinterpret_cast<u32x4 *>(dst) = w0;
                *reinterpret_cast<u32x4 *>(dst + kPlaneBytes) = w1;
                *reinterpret_cast<u32x4 *>(dst + 2 * kPlaneBytes) = w2;
            }
        }
    };

    constexpr int kHeadRec = 2 * kCodeBytes + 2 * SZB * (kWaves / NGW);   // head record of this layout
    constexpr int kSzTensor = SZB * (kWaves / NGW);                        // (s, z) bytes per tensor
    const uint32_t rec_bytes = uint32_t(a.hkv) * kHeadRec;
    // this lane's code word and its group's (s, z) in the record of slot 0
    uint8_t *const code_base = a.records + (h * kHeadRec + t * kCodeBytes + 8 * w + 4 * hh);
    uint8_t *const sz_base = a.records + (h * kHeadRec + 2 * kCodeBytes + t * kSzTensor + SZB * (w / NGW));
    // the next tile of input in flight in registers (the waits are the
    // compiler's; a second tile would take the registers of a third wave per
    // SIMD); the LDS tile is double-buffered, so one barrier per tile both
    // publishes the new tile and retires the buffer it overwrites next
    constexpr int kDepth = 1;
    u32x4 pr[kDepth][2][2];
#pragma unroll
    for (int d = 0; d < kDepth; ++d) load_tile(tok_begin + d * kTile, pr[d]);

    // per-token routing data of this lane's token (tb + tt), fetched ahead:
    // request, position and slot two tiles early, the request's length one
    // tile early, so that no tile waits on a dependent global load
    // (32-bit byte offsets from the arrays' bases)
    auto at = [](const int32_t *base, int i) {
        return *reinterpret_cast<const int32_t *>(reinterpret_cast<const uint8_t *>(base) + 4u * uint32_t(i));
    };
    auto load_meta = [&](int tb, int &req, int &pos, int &slot) {
        const int tok = tb + tt;
        const int tc = tok < tok_end ? tok : tok_begin;
        req = at(a.req_ids, tc);
        pos = at(a.positions, tc);
        slot = at(a.slots, tc);
    };
    auto load_len = [&](int req) { return at(a.seq_len_after, (req >= 0 && req < a.max_requests) ? req : 0); };
    int req0, pos0, slot0, req1, pos1, slot1;
    load_meta(tok_begin, req0, pos0, slot0);
    load_meta(tok_begin + kTile, req1, pos1, slot1);
    int len0 = load_len(req0);

    for (int tb0 = tok_begin; tb0 < tok_end; tb0 += kDepth * kTile) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
        const int tb = tb0 + d * kTile;
        if (tb >= tok_end) break;
        uint8_t *lds = lds_buf[((tb - tok_begin) / kTile) & 1];
        store_tile(lds, pr[d]);
        __syncthreads();
        load_tile(tb + kDepth * kTile, pr[d]);
        int req2, pos2, slot2;
        load_meta(tb + 2 * kTile, req2, pos2, slot2);
        const int len1 = load_len(req1);

        // x'^T: 32 output channels x 32 tokens, 16 input channels per step
        f32x16 acc = {};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
            for (int xa = 0; xa < XT; ++xa) {
                const bf16x8 b = *reinterpret_cast<const bf16x8 *>(
                    lds + xa * kPlaneBytes + tt * kRowBytes + ks * 32 + hh * 16);
#pragma unroll
                for (int tr = 0; tr + xa < 3; ++tr) acc = mfma32_bf16(rf[ks][tr], b, acc);
            }
        }

        // lane (tt, hh): token tb + tt, rotated channels 32 w + 16 hh + 0..15
        float lo = fminf(acc[0], acc[1]), hi = fmaxf(acc[0], acc[1]);
#pragma unroll
        for (int j = 2; j < 16; ++j) {
            lo = fminf(lo, acc[j]);
            hi = fmaxf(hi, acc[j]);
        }
        lo = fminf(lo, __shfl_xor(lo, 32));
        hi = fmaxf(hi, __shfl_xor(hi, 32));
        if constexpr (NGW > 1) {
            // the other waves of this group: every wave passes here (no lane has
            // left the iteration yet)
            if (hh == 0) grp_stat[w][tt] = make_float2(lo, hi);
            __syncthreads();
#pragma unroll
            for (int o = 1; o < NGW; ++o) {
                const float2 st = grp_stat[(w & ~(NGW - 1)) | ((w + o) & (NGW - 1))][tt];
                lo = fminf(lo, st.x);
                hi = fmaxf(hi, st.y);
            }
        }

        const int tok = tb + tt;
        const int req = req0, pos = pos0, slot = slot0, L = len0;
        // the next tile's routing data moves up (every lane, before any early exit)
        req0 = req1; pos0 = pos1; slot0 = slot1; len0 = len1;
        req1 = req2; pos1 = pos2; slot1 = slot2;
        if (tok >= tok_end) continue;
        if (req < 0 || req >= a.max_requests || pos < 0) continue;
        const bool to_sink = pos < a.sink_tokens;
        if (!to_sink && (slot < 0 || int64_t(slot) >= a.num_slots)) continue;

        const int c0 = 32 * w + 16 * hh;
        if (a.rotated_out) {
            float *ro = a.rotated_out + ((size_t(tok) * a.hkv + h) * 2 + t) * kHeadDim + c0;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<f32x4 *>(ro + 4 * q) = f32x4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
        }
        // BF16 copy of the rotated values: only the sink and recent windows keep one
        auto store_bf16 = [&](uint16_t *dst) {
            u32x4 bf[2];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                bf[j >> 2][j & 3] = uint32_t(bf16_bits_rn(acc[2 * j])) | (uint32_t(bf16_bits_rn(acc[2 * j + 1])) << 16);
            reinterpret_cast<u32x4 *>(dst)[0] = bf[0];
            reinterpret_cast<u32x4 *>(dst)[1] = bf[1];
        };
        if (to_sink) {
            store_bf16(a.sink + ((size_t(req) * a.sink_tokens + pos) * a.hkv + h) * 2 * kHeadDim + t * kHeadDim + c0);
            continue;
        }

        // clip bounds, scale and zero (fp32 ops, each rounded once)
        const float lo_c = lo < 0.0f ? __fmul_rn(a.alpha, lo) : lo;
        const float hi_c = hi > 0.0f ? __fmul_rn(a.alpha, hi) : hi;
        const float range = __fsub_rn(hi_c, lo_c);
        // range / 3 rounded to nearest fp32: the fp64 product is within 2^-52
        // (relative) of the quotient, and a quotient by 3 of an fp32 value is
        // never within 2^-25 (relative) of a midpoint between fp32 values
        const float s32 = float(double(range) * (1.0 / 3.0));
        // the stored (s, z): fp16, or E4M3 codes (every E4M3 value is an fp16 value)
        uint32_t sz_word;
        double sd, zd;
        if constexpr (SZB == 4) {
            const __half s = __float2half_rn(s32);
            const __half z = __float2half_rn(lo_c);
            sz_word = uint32_t(__half_as_ushort(s)) | (uint32_t(__half_as_ushort(z)) << 16);
            sd = double(__half2float(s));
            zd = double(__half2float(z));
        } else {
            const uint32_t sc = e4m3_code_rn(s32), zc = e4m3_code_rn(lo_c);
            sz_word = sc | (zc << 8);
            sd = double(e4m3_to_f32(sc));
            zd = double(e4m3_to_f32(zc));
        }
        // thresholds z + (k + 1/2) s: exact in fp64 (fp16 operands, sums below
        // 2^19 on a 2^-25 grid), rounded up to fp32 so that "x >= T" is exact
        // for fp32 x; a scale of zero gives +inf thresholds (codes 0).  The two
        // lanes of a token's group share the work: each forms T1, lane hh = 0
        // forms T0 and lane hh = 1 forms T2, and they swap those (both lanes of
        // a token are active or inactive together: they share the routing data
        // above, so the swap reads an active lane)
        const bool zero_scale = sd == 0.0;
        const float ua = zero_scale ? INFINITY : round_up_f32(fma(hh ? 2.5 : 0.5, sd, zd));
        const float u1 = zero_scale ? INFINITY : round_up_f32(fma(1.5, sd, zd));
        const float pa = __shfl_xor(ua, 32);
        const float u0 = hh ? pa : ua;
        const float u2 = hh ? ua : pa;
        // code = number of thresholds at or below the clipped value, code j
        // at bits 2 j, 2 j + 1.  With alpha = 1 the clip bounds are the group's
        // own min and max, so every value is inside them and the clip is
        // skipped (uniform branch).
        uint32_t packed = 0;
        if (a.alpha == 1.0f) {
#pragma unroll
            for (int j = 12; j >= 0; j -= 4)
                packed = codes4_into(packed, acc[j + 3], acc[j + 2], acc[j + 1], acc[j], u0, u1, u2);
        } else {
            auto clip = [&](float x) { return __builtin_amdgcn_fmed3f(x, lo_c, hi_c); };   // lo_c <= hi_c
#pragma unroll
            for (int j = 12; j >= 0; j -= 4)
                packed = codes4_into(packed, clip(acc[j + 3]), clip(acc[j + 2]), clip(acc[j + 1]), clip(acc[j]), u0, u1, u2);
        }
        const uint64_t rec_off = uint64_t(uint32_t(slot)) * rec_bytes;     // slot >= 0 here
        *reinterpret_cast<uint32_t *>(code_base + rec_off) = packed;
        if (hh == 0 && (w & (NGW - 1)) == 0) {            // one writer per group
            uint8_t *dst = sz_base + rec_off;
            if constexpr (SZB == 4)
                *reinterpret_cast<uint32_t *>(dst) = sz_word;
            else
                *reinterpret_cast<uint16_t *>(dst) = uint16_t(sz_word);
        }
        if (pos >= L - a.recent_tokens)
            store_bf16(a.recent + ((size_t(req) * a.recent_tokens + pos % a.recent_tokens) * a.hkv + h) * 2 * kHeadDim +
                       t * kHeadDim + c0);
    }
    }
}

// the kernel for (input dtype, group size, scale/zero bits)
const void *append_kernel(oscar_dtype in_dtype, int group_size, int sz_bits) {
    const bool bf = in_dtype == OSCAR_BF16;
    if (sz_bits == 8)                                   // group size 64 (checked with the layout)
        return bf ? reinterpret_cast<const void *>(quant_append_kernel<1, 2, 2>)
                  : reinterpret_cast<const void *>(quant_append_kernel<3, 2, 2>);
    switch (group_size) {
        case 64: return bf ? reinterpret_cast<const void *>(quant_append_kernel<1, 2, 4>)
                           : reinterpret_cast<const void *>(quant_append_kernel<3, 2, 4>);
        case 128: return bf ? reinterpret_cast<const void *>(quant_append_kernel<1, 4, 4>)
                            : reinterpret_cast<const void *>(quant_append_kernel<3, 4, 4>);
        default: return bf ? reinterpret_cast<const void *>(quant_append_kernel<1, 1, 4>)
                           : reinterpret_cast<const void *>(quant_append_kernel<3, 1, 4>);
    }
}

}  // namespace
}  // namespace oscar

using namespace oscar;

extern "C" oscar_status oscar_quant_append(hipStream_t stream, const oscar_layout *layout,
                                           const oscar_pool *pool, const void *k, const void *v,
                                           oscar_dtype in_dtype, int32_t n_tokens,
                                           const int32_t *req_ids, const int32_t *positions,
                                           const int32_t *slots, const int32_t *seq_len_after,
                                           const float *R_K, const float *R_V, float clip_ratio,
                                           float *rotated_out, const oscar_launch_opts *opts) {
    oscar_status st = check_layout(layout);
    if (st != OSCAR_OK) return st;
    if (!pool) return fail(OSCAR_ERR_INVALID_ARG, "pool is null");
    if (n_tokens < 0) return fail(OSCAR_ERR_INVALID_ARG, "n_tokens must be >= 0");
    if (in_dtype != OSCAR_F32 && in_dtype != OSCAR_BF16 && in_dtype != OSCAR_F16)
        return fail(OSCAR_ERR_INVALID_ARG, "in_dtype must be F32, BF16 or F16");
    if (!(clip_ratio > 0.0f && clip_ratio <= 1.0f))
        return fail(OSCAR_ERR_INVALID_ARG, "clip_ratio must be in (0, 1]");
    if (n_tokens == 0) return OSCAR_OK;
    if (!k || !v || !req_ids || !positions || !slots || !seq_len_after || !R_K || !R_V)
        return fail(OSCAR_ERR_INVALID_ARG, "a required pointer is null");
    if (!pool->records || (layout->sink_tokens > 0 && !pool->sink) || !pool->recent)
        return fail(OSCAR_ERR_INVALID_ARG, "a pool pointer is null");
    int chunk = 0;
    if (opts && opts->append_chunk) {
        chunk = opts->append_chunk;
        if (chunk < kTile || chunk % kTile)
            return fail(OSCAR_ERR_INVALID_ARG, "append_chunk must be a positive multiple of 32");
    } else {
        // one round of workgroups that are all resident at once: compute
        // units x workgroups per compute unit (from the kernel's registers)
        int dev = 0, cus = 0, per_cu = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return fail(OSCAR_ERR_HIP, "querying the device failed");
        const void *kern = append_kernel(in_dtype, layout->group_size, scale_bits(*layout));
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kThreads, 0) != hipSuccess)
            return fail(OSCAR_ERR_HIP, "occupancy query failed");
        const int slots = std::max(1, cus * std::max(1, per_cu));
        const int per = std::max(1, slots / (2 * layout->num_kv_heads));
        chunk = (n_tokens + per - 1) / per;
        chunk = std::max(kTile, (chunk + kTile - 1) / kTile * kTile);
    }
    const int n_chunks = (n_tokens + chunk - 1) / chunk;

    AppendArgs args;
    args.k = k;
    args.v = v;
    args.req_ids = req_ids;
    args.positions = positions;
    args.slots = slots;
    args.seq_len_after = seq_len_after;
    args.r_k = R_K;
    args.r_v = R_V;
    args.rotated_out = rotated_out;
    args.records = pool->records;
    args.sink = pool->sink;
    args.recent = pool->recent;
    args.num_slots = layout->num_slots;
    args.n_tokens = n_tokens;
    args.hkv = layout->num_kv_heads;
    args.sink_tokens = layout->sink_tokens;
    args.recent_tokens = layout->recent_tokens;
    args.max_requests = layout->max_requests;
    args.chunk = chunk;
    args.n_chunks = n_chunks;
    args.in_dtype = in_dtype;
    args.alpha = clip_ratio;

    const int blocks = 8 * ((n_chunks + 7) / 8) * 2 * layout->num_kv_heads;
    if (opts && opts->kernel_begin) {
        if (hipEventRecord(opts->kernel_begin, stream) != hipSuccess)
            return fail(OSCAR_ERR_HIP, "hipEventRecord failed");
    }
    void *kargs[] = {&args};
    hipError_t e = hipLaunchKernel(append_kernel(in_dtype, layout->group_size, scale_bits(*layout)), dim3(blocks), dim3(kThreads),
                                   kargs, 0, stream);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) return fail(OSCAR_ERR_HIP, std::string("quant_append launch: ") + hipGetErrorString(e));
    if (opts && opts->kernel_end) {
        if (hipEventRecord(opts->kernel_end, stream) != hipSuccess)
            return fail(OSCAR_ERR_HIP, "hipEventRecord failed");
    }
    return OSCAR_OK;
}
