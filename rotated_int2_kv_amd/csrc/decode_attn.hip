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
//               as exact fp16 denormal operands (see int2_item), for 96-, 80-
//               and 72-byte head records (G = 32, 64, 128).
//               With G = 128 and an odd number of KV heads the history runs on
//               a VALU kernel instead (hist_lowmeta_kernel).
//               BF16 windows run on fp32 VALU.  Each item writes (m, l, o')
//               with m in log2 units.
//   3. merge:   log-sum-exp merge of the items and o = o' R_V^T.
//
// oscar_extend_attn treats the new tokens of one request as rows that read
// the request's cached prefix as stored at the prefix length, plus one more
// work item per row: the new tokens up to and including its own, as BF16
// rotated keys and values (rotated here by extend_rotate_kernel).  It shares
// the query rotation and the merge; its work items run on the matrix-core
// kernels of extend_hist.hip, which take many rows per loaded tile.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <cmath>
#include <mutex>
#include <string>
#include <type_traits>
#include <vector>

#include "common.h"
#include "internal.h"

namespace oscar {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kTileTokens = 32;      // history tokens per MFMA tile
constexpr int kBf16Chunk = 64;       // BF16-window tokens per VALU step
constexpr int kPartialWaves = 4;     // KV heads (waves) per split-K workgroup

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
    uint8_t *zero_rec; // 256 zero bytes (cleared by the prep kernel)
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
    int32_t sink_items;   // items [0, sink_items): the sink window, kWindowItemTokens positions each
    int32_t win_items;    // items [sink_items, win_items): the recent window; then the history chunks
    int32_t win_last;     // partial_kernel's grid takes the history items first, the window items last
    int32_t waves;     // KV heads per workgroup
    int32_t head_chunks;
    int32_t group_size;
    int32_t scale_bits;       // 16 (fp16 s, z) or 8 (E4M3 s, z)
    // extend: every batch row is request fixed_req at length fixed_len, and
    // item extra_item reads the rotated new tokens 0 .. row (causal)
    int32_t fixed_req;        // -1 for decode
    int32_t fixed_len;
    int32_t extra_item;       // -1 for decode
    const uint16_t *newkv;    // [rows][Hkv][2][128] BF16 rotated K, V of the new tokens
};

// Position range [p0, p1) of work item j of a request of length L: the sink
// window [0, min(S, L)) and the recent window [max(S, L - W), L) in items of
// kWindowItemTokens positions (one item each when the plan has one), then the
// history [S, L - W) in chunks.
__device__ __forceinline__ void item_range(const DecodeArgs &a, int L, int j, int &p0, int &p1) {
    const int S = a.sink_tokens, W = a.recent_tokens;
    const int hist_end = max(S, L - W);
    if (j < a.sink_items) {
        const int end = min(S, L);
        p0 = a.sink_items == 1 ? 0 : min(end, j * kWindowItemTokens);
        p1 = a.sink_items == 1 ? end : min(end, p0 + kWindowItemTokens);
    } else if (j < a.win_items) {
        const int start = L > S ? hist_end : L;
        const int r = j - a.sink_items;
        p0 = a.win_items - a.sink_items == 1 ? start : min(L, start + r * kWindowItemTokens);
        p1 = a.win_items - a.sink_items == 1 ? L : min(L, p0 + kWindowItemTokens);
    } else {
        p0 = S + (j - a.win_items) * a.chunk;
        p1 = min(p0 + a.chunk, hist_end);
    }
}

__device__ __forceinline__ int request_length(const DecodeArgs &a, int b, int &req) {
    req = a.fixed_req >= 0 ? a.fixed_req : a.req_ids[b];
    int L = a.fixed_req >= 0 ? a.fixed_len : a.seq_lens[b];
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
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

__global__ __launch_bounds__(512) void prep_kernel(DecodeArgs a) {
    __shared__ float qs[kMaxGroup][kHeadDim];
    __shared__ float part[4][kMaxGroup][kHeadDim];
    __shared__ float half_max[kMaxGroup][2];
    const int b = blockIdx.x / a.hkv;
    const int hk = blockIdx.x % a.hkv;
    const int t = threadIdx.x;
    const int c = t & (kHeadDim - 1);        // output channel
    const int quarter = t >> 7;               // input channels [32 quarter, 32 quarter + 32)
    if (blockIdx.x == 0 && t < 64) reinterpret_cast<uint32_t *>(a.zero_rec)[t] = 0u;
    // this thread's slice of column c of R_K, all loads in flight at once
    const float *R = a.r_k + size_t(hk) * kHeadDim * kHeadDim;
    float r[kHeadDim / 4];
#pragma unroll
    for (int ii = 0; ii < kHeadDim / 4; ++ii) r[ii] = R[size_t(quarter * (kHeadDim / 4) + ii) * kHeadDim + c];
    for (int e = t; e < a.g * kHeadDim; e += 512) {
        const int h = e / kHeadDim, i = e % kHeadDim;
        qs[h][i] = load_as_f32(a.q, a.q_dtype, (size_t(b) * a.hq + hk * a.g + h) * kHeadDim + i);
    }
    __syncthreads();
    for (int h = 0; h < a.g; ++h) {
        float acc = 0.0f;
#pragma unroll
        for (int ii = 0; ii < kHeadDim / 4; ++ii) acc = fmaf(qs[h][quarter * (kHeadDim / 4) + ii], r[ii], acc);
        part[quarter][h][c] = acc;
    }
    __syncthreads();
    // the head index is uniform over each wave: 128 threads per head
    for (int h = t >> 7; h < a.g; h += 4) {
        const float v = (part[0][h][c] + part[1][h][c] + part[2][h][c] + part[3][h][c]) * a.scale_log2;
        const size_t row = size_t(b) * a.hq + hk * a.g + h;
        a.qrot[row * kHeadDim + c] = v;
        // sum over the 32 channels of c's group (32 aligned lanes of the wave)
        float gsum = v;
#pragma unroll
        for (int off = 16; off >= 1; off >>= 1) gsum += __shfl_xor(gsum, off);
        if ((c & (kGroup - 1)) == 0) a.qsum[row * 8 + c / kGroup] = gsum;
        const float mx = wave_max(fabsf(v));
        if ((t & 63) == 0) half_max[h][c >> 6] = mx;
    }
    __syncthreads();
    if (t < a.g) {
        // power-of-two operand scale 2^K with max|q'| 2^K < 2^15, so that
        // q' 2^(K - e) (e = 0..8) fits fp16
        const int h = t;
        const float mx = fmaxf(half_max[h][0], half_max[h][1]);
        int e = 0;
        frexpf(mx, &e);                          // mx < 2^e
        const int K = mx > 0.0f ? max(-20, min(24, 15 - e)) : 24;
        float *info = a.qsum + (size_t(b) * a.hq + hk * a.g + h) * 8;
        info[4] = ldexpf(1.0f, K);
        info[5] = ldexpf(1.0f, 24 - K);
    }
}

// ---------------------------------------------------------------------------
// 2. split-K partials
// ---------------------------------------------------------------------------

__device__ __forceinline__ float half_lo_f(uint32_t w) { return __half2float(__ushort_as_half(uint16_t(w))); }
__device__ __forceinline__ float half_hi_f(uint32_t w) { return __half2float(__ushort_as_half(uint16_t(w >> 16))); }

// Two fp32 values as an fp16 pair, each rounded to nearest (ties to even):
// one v_cvt_pk_f16_f32.
__device__ __forceinline__ uint32_t pk_rn(float x0, float x1) {
    const f16x2 h = {static_cast<_Float16>(x0), static_cast<_Float16>(x1)};
    return __builtin_bit_cast(uint32_t, h);
}

// x ~ hi + lo with hi, lo fp16 pairs: hi rounded to nearest, lo the exact
// fp32 residual rounded to nearest (relative error of hi + lo below 2^-21,
// and unbiased, so that errors of many such products do not add up in one
// direction).
struct HiLo2 {
    uint32_t hi, lo;
};
__device__ __forceinline__ HiLo2 split_hilo(float x0, float x1) {
    const uint32_t h = pk_rn(x0, x1);
    const uint32_t l = pk_rn(x0 - half_lo_f(h), x1 - half_hi_f(h));
    return {h, l};
}

__device__ __forceinline__ f16x8 u4_as_h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    return __builtin_bit_cast(f16x8, u32x4{a, b, c, d});
}

// Exponent offset of code pair j inside a 32-bit word of 16 LSB-first codes:
// pairs (j, j + 8) sit at bits 2j and 16 + 2j; j = 0..4 are masked in place,
// j = 5..7 after a right shift by 6.  Masked, each 16-bit half is an fp16
// denormal of value c 2^(e_j - 24).
__host__ __device__ constexpr int pair_exp(int j) { return j <= 4 ? 2 * j : 2 * j - 6; }

[[maybe_unused]] __device__ __forceinline__ uint32_t code_bits(uint32_t w, uint32_t w_sh6, int j) {
    return j <= 4 ? (w & (0x00030003u << (2 * j))) : (w_sh6 & (0x00030003u << (2 * j - 6)));
}
// Bit position of V code j (channel 4 n + j) in each 16-bit half of a PV
// B-operand dword.  The matrix core aligns the products of one instruction by
// their exponent fields, and every denormal carries the smallest exponent, so
// a code low in its mantissa loses as many bits of the alignment window as it
// has leading zeros: with the codes at bits 0, 2, 4, 6 the products of code 0
// kept about 15 bits, and the output of 131K-token requests drifted by up to
// 1.2e-3 of its scale.  Codes 0 and 1 are therefore taken after a left shift
// by 4 (bits 4 and 6), codes 2 and 3 in place.  (The QK products showed no
// such drift with their codes at bits 0..8.)
__host__ __device__ constexpr int pv_code_exp(int j) { return j <= 1 ? 2 * j + 4 : 2 * j; }

// The matrix-core products below span the channels of at most two groups each:
// channel halves 0..63 and 64..127 (P = 0, 1), and within a half the 16-channel
// quarter k = 0..3 lies in group (64 P + 16 k) / G.  The group's index within
// its half ("pair-local", 0 or 1) picks the A rows that carry it; with G >= 64
// a half holds one group.
template <int NG>
__host__ __device__ constexpr int pair_local_group(int quarter) { return NG == 4 ? quarter >> 1 : 0; }
template <int NG>
__host__ __device__ constexpr int half_group(int P, int gl) { return NG == 4 ? 2 * P + gl : NG == 2 ? P : 0; }

// reductions over the 16 lanes of a DPP row (every lane of the row gets the result)
template <int K>
__device__ __forceinline__ float row_ror(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x120 + K, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, row_ror<1>(v));
    v = fmaxf(v, row_ror<2>(v));
    v = fmaxf(v, row_ror<4>(v));
    return fmaxf(v, row_ror<8>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
    v += row_ror<1>(v);
    v += row_ror<2>(v);
    v += row_ror<4>(v);
    return v + row_ror<8>(v);
}
[[maybe_unused]] __device__ __forceinline__ float half_lo(uint32_t w) { return __half2float(__ushort_as_half(uint16_t(w))); }
[[maybe_unused]] __device__ __forceinline__ float half_hi(uint32_t w) { return __half2float(__ushort_as_half(uint16_t(w >> 16))); }

// History item on the matrix cores.  GQ = query heads per KV head, handled in
// sets of 4.  A workgroup holds four waves, one per KV head of the head chunk
// (the 384 bytes of four 96-byte head records that follow each other in a
// slot-major record); waves past the last KV head only help with the loads.
//
// Loads go straight from HBM into LDS (global_load_lds, no registers in
// between) and are shared by the workgroup: for each 32-token tile the four
// waves together fetch the chunk's 384 bytes of every token as whole 128-byte
// lines (wave w fetches tokens 8 w .. 8 w + 7), so that each request fills a
// line.  Token t of a tile occupies 384 bytes of the stage; within each of
// its three 128-byte lines the 16-byte units are permuted by XOR with a
// per-token value (tok_swizzle) chosen so that every read pattern below hits
// distinct banks, whether the LDS serves 128 or 256 bytes per cycle.  Four stages let three tiles be in flight while
// a fourth is computed; one workgroup barrier per tile publishes a landed
// tile and retires the stage that the next loads overwrite.  The slot ids of
// a tile go to a ring shared by the workgroup (each wave fetches 8 of them)
// two tiles before its records.  Tokens past the item read the record of
// the item's first position and tokens with an out-of-range slot id that of
// the last slot; both are masked out of the softmax (p = 0), and tiles with
// every token usable skip the mask.
//
// Every matrix-core product spans the channels of two groups at most (the
// halves 0..63 and 64..127 with G = 32), so that its A rows can carry two
// parts of one quantity instead of one row per group.
// QK (per half of 16 tokens): lane group kb holds K-code words P = 0, 1
// (channels 64 P + 16 kb .. + 15: group 2 P + kb / 2); B = a word's codes as
// exact fp16 denormals (one AND per pair, no scale); A = q' (hi and lo fp16
// parts in two products that share an output, times 2^(K - e)) in rows
// (h, x), x = the pair-local group, nonzero where it matches the lane group's.
// Lane (token n, head h) thereby receives its four group sums and applies s
// and z in fp32: one logit per lane, nothing repeated.
// PV: the lane of (token, head) forms p s_g (hi and lo fp16 parts) for the
// four groups and accumulates p z_g itself; the weights go through the
// wave's LDS into rows 4 q + h of two weight planes (plane = channel half,
// q = (pair-local group, part)), so that one product carries both parts.  B
// holds the V codes of 8 tokens per lane as exact denormals: column n of
// plane c is channel 64 c + 4 n + j, byte n % 4 of a V-code dword picked by
// one v_perm_b32 per token pair.  The hi and lo rows of a column's group are
// summed once, when the partial is written.  K-slot 8 kb + i of the PV
// products is token 16 (i % 2) + 2 ((i / 2) % 2) + 8 (i / 4) + (kb % 2) +
// 4 (kb / 2): a lane's two tokens n and 16 + n take adjacent K-slots, so that
// one 32-bit write stores both weights of a row, and the four lane groups read
// V codes of tokens t, t + 1, t + 4, t + 5 at once, which the token swizzle
// puts in disjoint LDS banks.  Weight rows hold 4 units of 16
// bytes (8 K-slots each), the physical unit of logical unit v in row 4 q + h
// being v ^ q.  The rows live in the stage itself: once a wave has read its K
// codes and both (s, z) of the tile into registers, those 128 units of its
// head are dead, and each weight unit takes a dead unit in a bank group chosen
// so that the 16-bit weight writes and the 128-bit operand reads hit distinct
// banks.
constexpr int kTokBytes = 4 * kHeadRecord;             // 384: one token of a head chunk
constexpr int kStage = kTileTokens * kTokBytes;        // 12 KiB per tile
constexpr int kStages = 4;                             // three tiles in flight while one is computed
constexpr int kRingBytes = kTileTokens * 4;            // slot ids of one tile
constexpr int kRing = 4;                               // slot-id ring of the workgroup
__host__ __device__ constexpr int int2_lds_bytes() { return kStages * kStage + kRing * kRingBytes; }

// The same pipeline for the lower-metadata records: 80 bytes (G = 64, two
// groups; the K and V (s, z) of a head share one 16-byte unit) and 72 bytes
// (G = 128, one group).  A token of a 4-head chunk is 320 or 288 bytes (20 or
// 18 units), stored in token order without a swizzle but with one padding
// unit after each token: a token stride of 21 or 19 units (84 or 76 dwords)
// puts the same word of tokens 0..15 in 16 distinct 4-bank groups, so the
// K-code, (s, z) and V-code reads hit distinct banks.  A tile takes 672 or 608
// of the stage's 768 unit positions; the padding units and the rest receive
// zero-record loads so that every lane still issues three.  With G >= 64 a
// channel half holds one group, so the A rows x = 1 of the QK products are
// zero and the PV weights use rows q = part only (G = 128: one plane serves
// both halves).  The PV weights get their own LDS area (a head has too few
// dead units per token): per wave two planes (channel halves) of 8 rows
// 4 q + h x 32 K-slots of fp16, the 16-byte units of rows 4..7 XOR-permuted by
// 1 so that the operand reads of rows r and r + 4 hit distinct banks.
constexpr int kWeightPlane = 8 * kTileTokens * 2;      // 512 bytes
constexpr int kWeightWave = 2 * kWeightPlane;          // 1 KiB
__host__ __device__ constexpr int int2_lds_bytes_lowmeta() { return int2_lds_bytes() + 4 * kWeightWave; }

// XOR applied to the unit index (within its 128-byte line) of token t: bits
// 0 and 1 of t % 8 swapped, bit 1 flipped for t % 16 >= 8.  Tokens t and
// t + 16 share it (token 16 + t is 16 x 384 bytes after token t).  It makes the
// units read by any 8 consecutive tokens distinct, the (line parity, unit)
// pairs of tokens 0..15 distinct, and the V-code units of tokens t, t + 1
// (and t + 4, t + 5) read by one PV load distinct.  (Token 16 + t of a stage
// is 16 kTokBytes after token t.)
__host__ __device__ constexpr int tok_swizzle(int t) {
    return (((t & 1) << 1) | ((t >> 1) & 1) | (t & 4)) ^ (2 * ((t >> 3) & 1));
}
// Tokens t and t + 16 share the swizzle (the PV reads take both in one instruction).
constexpr bool swizzle_period_16() {
    for (int t = 0; t < 16; ++t)
        if (tok_swizzle(t + 16) != tok_swizzle(t)) return false;
    return true;
}
static_assert(swizzle_period_16(), "V-code units of tokens t, t + 16");

// byte offset of 16-byte unit q (0..23) of token t inside a stage
__device__ __forceinline__ int unit_addr(int t, int q) {
    return t * kTokBytes + 16 * ((q & ~7) | ((q & 7) ^ tok_swizzle(t)));
}

// Byte offset inside a stage of physical unit u (0..3) of row r (0..15) of
// wave w's PV weight plane 0 (hi parts); plane 1 (lo parts) is 16 x 384 bytes
// further.  Row r's units go to K-code or (s, z) unit {0, 1, 4, 5}[r / 4] of
// w's head record, of the one token among 0..15 that puts the unit in bank
// group (4 r + (u ^ 2 ((r / 2) % 2))) % 16 (16-byte groups of a 256-byte
// window).  Those groups keep the weight writes (rows 4 g .. 4 g + 3, all
// units) and the operand reads (rows 8 j .. 8 j + 7 or 0 .. 15, one unit
// each) in distinct banks.
__device__ __forceinline__ int wunit_addr(int w, int r, int u) {
    const int q = 6 * w + ((r >> 2) & 1) + 4 * (r >> 3);
    const int bg = (4 * r + (u ^ (2 * ((r >> 1) & 1)))) & 15;
    const int par = (bg >> 3) ^ ((q >> 3) & 1);     // t % 2: line parity within the 256-byte window
    const int sw = (bg & 7) ^ (q & 7);              // tok_swizzle(t) needed
    const int t = par | ((sw & 1) << 1) | (sw & 4) | ((((sw >> 1) & 1) ^ par) << 3);
    return unit_addr(t, q);
}

typedef __attribute__((address_space(3))) void lds_void;
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// LDS byte addresses as 32-bit integers.  Per-lane addresses are computed
// once per item and hidden from the optimiser (`lds_pin`), so that inside the
// tile loop every LDS access is one instruction: a pinned register plus a
// constant offset (the stage), with no re-added base.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return uint32_t(reinterpret_cast<uintptr_t>((const lds_void *)p));
}
__device__ __forceinline__ uint32_t lds_pin(uint32_t x) {
    asm volatile("" : "+v"(x));
    return x;
}
template <class T>
__device__ __forceinline__ T lds_ld(uint32_t addr) {
    return *reinterpret_cast<const __attribute__((address_space(3))) T *>(uintptr_t(addr));
}
template <class T>
__device__ __forceinline__ void lds_st(uint32_t addr, T v) {
    *reinterpret_cast<__attribute__((address_space(3))) T *>(uintptr_t(addr)) = v;
}
__device__ __forceinline__ lds_void *lds_ptr(uint32_t addr) { return reinterpret_cast<lds_void *>(uintptr_t(addr)); }

// Cache policy of the record loads: non-temporal (each record is read once).
constexpr int kNonTemporal = 2;

// Wait until at most N vector-memory operations of this wave are pending.
// The compiler does not track global_load_lds, so the pipeline below waits
// by hand; the memory clobber keeps LDS accesses on their side of the wait.
template <int N>
__device__ __forceinline__ void wait_vmem() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// NG groups per head vector; SZB bytes per group's (s, z): 4 (fp16) or 2 (E4M3)
template <int GQ, int NG, int SZB>
__device__ __forceinline__ void int2_item(const DecodeArgs &a, int b, int req, int j, int hc, int p0, int p1,
                          uint8_t *smem) {
    static_assert(NG == 4 || NG == 2 || NG == 1, "four, two or one (s, z) groups per head vector");
    static_assert(SZB == 4 || (SZB == 2 && NG == 2), "E4M3 (s, z) with two groups");
    constexpr int HS = (GQ + 3) / 4;          // sets of 4 query heads
    constexpr int kRecH = 2 * kCodeBytes + 2 * NG * SZB;  // head record: 96, 80 or 72 bytes
    constexpr int kUnitsH = kRecH / 16;                   // whole units of a head record
    constexpr int kTokB = 4 * kRecH;                      // one token of the 4-head chunk
    constexpr int kRecUnits = kTokB / 16;                 // 24, 20 or 18 units of records
    constexpr int kTokUnits = NG == 4 ? 24 : kRecUnits + 1;   // LDS units per token (one padding unit)
    constexpr int kTokL = 16 * kTokUnits;                 // LDS bytes per token
    constexpr int kTileUnits = kTileTokens * kTokUnits;   // 768, 672 or 608 units per tile
    static_assert(kTileUnits <= 768, "a tile fits the stage");
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform over the wave
    const int lane = threadIdx.x & 63;
    const int n = lane & 15;
    const int kb = lane >> 4;
    const int hk = hc * kPartialWaves + w;    // this wave's KV head
    const bool active = hk < a.hkv;
    const int nh = min(kPartialWaves, a.hkv - hc * kPartialWaves);   // KV heads of the chunk
    const uint32_t rec_bytes = uint32_t(a.hkv) * kRecH;
    const int32_t *r2s = a.req_to_slot + int64_t(req) * a.r2s_stride;
    const int n_tiles = (p1 - p0 + kTileTokens - 1) / kTileTokens;
    const uint32_t st0 = lds_addr(smem);                                // stage 0
    const uint32_t ring = st0 + kStages * kStage;                         // slot-id ring of the workgroup
    const size_t head0 = size_t(b) * a.hq + size_t(active ? hk : 0) * GQ;

    // ---- per-item operands
    // QK A of word P (K codes 64 P + 16 kb .. + 15 in lane group kb), half sh
    // (pairs 4 sh .. 4 sh + 3): row n = (h = n / 4, x = n % 4) with x = (pair-local
    // group, part); nonzero where the row's group is the lane group's
    f16x8 qA[HS][2][2];
    float qz[HS][4];      // Qbar[head kb][g] 2^(K - 24): zero-point term in the MFMA's units
    float qout[HS];       // 2^(24 - K) of head kb: MFMA units -> logit units (log2)
#pragma unroll
    for (int hs = 0; hs < HS; ++hs) {
        {
            const int h = 4 * hs + (n >> 2);
            const bool hv = h < GQ && active;
            const float *qr = a.qrot + (head0 + (hv ? h : 0)) * kHeadDim;
            const float k2 = a.qsum[(head0 + (hv ? h : 0)) * 8 + 4];
            const bool nz = hv && ((n & 3) >> 1) == pair_local_group<NG>(kb);
            const bool lo_row = (n & 1) != 0;
#pragma unroll
            for (int P = 0; P < 2; ++P) {
#pragma unroll
                for (int sh = 0; sh < 2; ++sh) {
                    uint32_t wv[4];
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        const int jj = 4 * sh + p;
                        const int c0 = 64 * P + 16 * kb + jj;
                        const float sc = k2 * __builtin_ldexpf(1.0f, -pair_exp(jj));
                        const float x0 = nz ? qr[c0] * sc : 0.0f;
                        const float x1 = nz ? qr[c0 + 8] * sc : 0.0f;
                        const HiLo2 hl = split_hilo(x0, x1);
                        wv[p] = lo_row ? hl.lo : hl.hi;
                    }
                    qA[hs][P][sh] = u4_as_h8(wv[0], wv[1], wv[2], wv[3]);
                }
            }
        }
        {
            const int h = 4 * hs + kb;
            const bool hv = h < GQ && active;
            const float *info = a.qsum + (head0 + (hv ? h : 0)) * 8;
#pragma unroll
            for (int g = 0; g < NG; ++g)
                qz[hs][g] = hv ? (NG == 4 ? info[g]
                                 : NG == 2 ? info[2 * g] + info[2 * g + 1]
                                           : (info[0] + info[1]) + (info[2] + info[3])) / info[5]
                               : 0.0f;
            qout[hs] = hv ? info[5] : 1.0f;
        }
    }

    // ---- what this lane fetches: 16-byte unit P of the stage, for P =
    // 64 (3 w + u) + lane (u = 0..2), holds logical unit q of token tq[u];
    // units of KV heads past the chunk (never read) repeat the chunk's first head
    int tq[3];
    const uint8_t *src_base[3];
    bool in_tile[3];                          // false: a padding position of the 80- or 72-byte layout
#pragma unroll
    for (int u = 0; u < 3; ++u) {
        const int P = 64 * (3 * w + u) + lane;
        // the 96-byte layout fills the stage; the others pad each token by one unit
        in_tile[u] = NG == 4 || (P < kTileUnits && P % kTokUnits < kRecUnits);
        const int Pc = in_tile[u] ? P : 0;
        const int t = Pc / kTokUnits, U = Pc % kTokUnits;
        const int q = NG == 4 ? ((U & ~7) | ((U & 7) ^ tok_swizzle(t))) : U;
        tq[u] = t;
        // units past the chunk's heads (never read) repeat an in-range unit; with
        // 72-byte records the chunk holds an even number of heads (whole units)
        if constexpr (kRecH % 16 != 0)
            src_base[u] = a.records + hc * kTokB + 16 * (16 * q + 16 <= nh * kRecH ? q : 0);
        else
            src_base[u] = a.records + hc * kTokB + 16 * (q / kUnitsH < nh ? q : q % kUnitsH);
    }

    // ---- loads.  Iteration t issues S(t + 6), this wave's 8 of the slot ids
    // of tile t + 6, and R(t + 3), this wave's three record loads of tile
    // t + 3: three record tiles are in flight while tile t is computed.  The
    // record addresses of tile t + 4 are formed at the end of iteration t,
    // from slot ids that landed two iterations earlier, so that the record
    // loads leave right after the barrier.  Every iteration issues the same
    // four operations, including tiles past the end, and so does the
    // prologue: the wait counts are constants.  The slot ids of tile T go to
    // ring slot T % 4 and its records to stage T % 4.
    const uint32_t span = uint32_t(p1 - p0);
    auto slot_load = [&](int T, int rs) {
        const uint32_t off = uint32_t(T * kTileTokens + 8 * w + (lane & 7));
        const int32_t *src = r2s + p0 + (off < span ? off : 0u);   // past the item: position p0
        if (lane < 8) __builtin_amdgcn_global_load_lds(src, lds_ptr(ring + rs * kRingBytes + 32 * w), 4, 0, 0);
    };
    uint32_t slot_at[3];                      // ring addresses of the slot ids of tokens tq[u]
#pragma unroll
    for (int u = 0; u < 3; ++u) slot_at[u] = lds_pin(ring + 4 * tq[u]);
    const uint32_t slot_own = lds_pin(ring + 4 * (lane & 31));
    // record addresses of tile T (slot ids in ring slot rs) and its usable
    // tokens (bit t).  History items run only with num_slots >= 1.
    const uint32_t slot_max = uint32_t(a.num_slots - 1);
    struct Fetch {
        const uint8_t *src[3];
        uint32_t valid;
    };
    // the slot ids of a tile in ring slot rs: this lane's three record tokens
    // and its own token
    struct SlotIds {
        int slot[3];
        int own;
    };
    auto read_ids = [&](int rs) -> SlotIds {
        SlotIds ids;
#pragma unroll
        for (int u = 0; u < 3; ++u) ids.slot[u] = lds_ld<int>(slot_at[u] + rs * kRingBytes);
        ids.own = lds_ld<int>(slot_own + rs * kRingBytes);
        return ids;
    };
    auto form = [&](int T, const SlotIds &ids) -> Fetch {
        Fetch f;
        // out-of-range slot ids read the last slot's record: their tokens are
        // masked (p = 0), so what they hold does not enter the result
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            const uint32_t sl = min(uint32_t(ids.slot[u]), slot_max);
            const uint8_t *rec = src_base[u] + uint64_t(sl) * rec_bytes;
            f.src[u] = NG == 4 || in_tile[u] ? rec : a.zero_rec;
        }
        const uint32_t left = span - uint32_t(T * kTileTokens);   // positions left in the item (may wrap: none)
        const uint32_t n_ok = uint32_t(T * kTileTokens) < span ? left : 0u;
        f.valid = uint32_t(__ballot((uint32_t(lane & 31) < n_ok) & (uint32_t(ids.own) < uint32_t(a.num_slots))));
        return f;
    };
    auto prep = [&](int T, int rs) -> Fetch { return form(T, read_ids(rs)); };
    auto issue = [&](const Fetch &f, int k) {
#pragma unroll
        for (int u = 0; u < 3; ++u)
            __builtin_amdgcn_global_load_lds(f.src[u], lds_ptr(st0 + k * kStage + 1024 * (3 * w + u)), 16, 0, kNonTemporal);
    };
    // LDS is used by this wave alone and runs a wave's operations in order;
    // the fences keep the compiler from moving LDS accesses across them
    auto lds_order = [] {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    // running state, per lane = (token n, head kb of each set)
    // m_ref = m_run 2^(24 - K) in log2 units, or 0 (a finite stand-in) while
    // every token so far is masked; it changes only when the running max grows
    float m_run[HS], m_ref[HS], l_lane[HS], zl[HS][NG];
    f32x4 oacc[HS][8];    // PV output: lane (n, kb) rows 4 q + h = (kb, i), channels 64 c + 4 n + j
#pragma unroll
    for (int hs = 0; hs < HS; ++hs) {
        m_run[hs] = -INFINITY;
        m_ref[hs] = 0.0f;
        l_lane[hs] = 0.0f;
#pragma unroll
        for (int g = 0; g < NG; ++g) zl[hs][g] = 0.0f;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) oacc[hs][jj] = f32x4{0, 0, 0, 0};
    }

    // this lane's LDS addresses in stage 0 (head w of token t); token 16 + t
    // of a stage is 6144 bytes after token t (same swizzle)
    constexpr int kHalfTok = 16 * kTokL;
    // byte b of head w's record of token t in stage 0 (80-byte layout)
    auto rec_at = [&](int t, int byte) { return st0 + t * kTokL + kRecH * w + byte; };
    const int kb_tok = (kb & 1) + 4 * (kb >> 1);
    // K codes: word P of the lane = bytes 16 P + 4 kb .. + 3 (channels 64 P + 16 kb .. + 15)
    uint32_t qk_at[2], szk_at, szv_at, a_at;
    // second plane of the PV weights (channels 64..127)
    constexpr uint32_t wpl_off = NG == 4 ? kHalfTok : kWeightPlane;
    // V codes of the tokens t and t + 16 of K-slots 8 kb + 2 pp and 8 kb + 2 pp + 1
    // (t = 8 (pp / 2) + 2 (pp % 2) + kb_tok): byte n (channels 4 n .. 4 n + 3) of
    // plane c is byte n % 4 of the dword at pv_at[pp][c], token 16 + n 16 token
    // strides further.  With G = 32 that stride is 6144 bytes and token t + 16
    // has the swizzle of t, so each pair is one ds_read2st64_b32 whose offsets
    // also take the stage.
    uint32_t pv_at[4][2];
    // v_perm_b32 selector: bytes (n % 4 of the first token, 0, n % 4 of the second, 0)
    const uint32_t pv_sel = lds_pin(0x0c040c00u | uint32_t(n & 3) * 0x00010001u);
    // PV weights of tokens n and 16 + n (one dword) in row 4 q + kb (q = 0 .. NQ - 1)
    constexpr int NQ = NG == 4 ? 4 : 2;
    uint32_t w_at[NQ];
    const int w_unit = (n & 1) + 2 * ((n >> 2) & 1);            // K-slot / 8 of token n
    const int w_i = ((n >> 1) & 1) + 2 * (n >> 3);              // K-slot % 8
    if constexpr (NG == 4) {
#pragma unroll
        for (int P = 0; P < 2; ++P) qk_at[P] = lds_pin(st0 + unit_addr(n, 6 * w + P) + 4 * kb);
        szk_at = lds_pin(st0 + unit_addr(n, 6 * w + 4));
        szv_at = lds_pin(st0 + unit_addr(n, 6 * w + 5));
        // V-code units 2 and 3 of the head record (channels 0..63, 64..127)
#pragma unroll
        for (int pp = 0; pp < 4; ++pp)
#pragma unroll
            for (int c = 0; c < 2; ++c)
                pv_at[pp][c] = lds_pin(st0 + unit_addr(8 * (pp >> 1) + 2 * (pp & 1) + kb_tok, 6 * w + 2 + c) + (n & ~3));
        // K-slots 8 unit + 2 w_i, + 1 of the row (tokens n, 16 + n), unit XOR-permuted by q
#pragma unroll
        for (int q = 0; q < 4; ++q) w_at[q] = lds_pin(st0 + wunit_addr(w, 4 * q + kb, w_unit ^ q) + 4 * w_i);
        // A-operand read of row n, K-slots 8 kb .. 8 kb + 7
        a_at = lds_pin(st0 + wunit_addr(w, n, kb ^ (n >> 2)));
    } else {
        qk_at[0] = lds_pin(rec_at(n, 4 * kb));
        qk_at[1] = qk_at[0] + 16;
        szk_at = lds_pin(rec_at(n, 2 * kCodeBytes));
        szv_at = lds_pin(rec_at(n, 2 * kCodeBytes + SZB * NG));
#pragma unroll
        for (int pp = 0; pp < 4; ++pp)
#pragma unroll
            for (int c = 0; c < 2; ++c)
                pv_at[pp][c] = lds_pin(rec_at(8 * (pp >> 1) + 2 * (pp & 1) + kb_tok, kCodeBytes + 16 * c + (n & ~3)));
        const uint32_t wb = st0 + int2_lds_bytes() + w * kWeightWave;   // after the stages and the ring
        // row r's unit v at physical unit v ^ (r / 4)
#pragma unroll
        for (int q = 0; q < 2; ++q) w_at[q] = lds_pin(wb + (4 * q + kb) * 64 + 16 * (w_unit ^ q) + 4 * w_i);
        a_at = lds_pin(wb + (n & 7) * 64 + 16 * (kb ^ ((n >> 2) & 1)));
    }
    // token 16 + t of a stage: 16 token strides after token t
    constexpr uint32_t kHalfTokOff = 16 * kTokL;
    // the weight area of the 80-byte layout does not move with the stage
    constexpr bool kWeightsInStage = NG == 4;

    // one tile: QK, online softmax, PV (LDS stage K)
    auto compute = [&](auto K, uint32_t valid) {
        constexpr uint32_t so = decltype(K)::value * kStage;   // stage offset
        // ---- V codes for the PV products, read first so that their LDS latency
        // overlaps the QK products and the softmax.  Plane c (channels 64 c .. 64 c + 63) has A
        // rows 4 q + h, q = (pair-local group, part): the hi and lo fp16 parts
        // of the weights p s_g of the half's groups for K-slots 8 kb .. 8 kb + 7,
        // so that one product carries both parts.  B of plane c, pair j = the V
        // codes of channel 64 c + 4 n + j for the same tokens, two tokens (t in
        // the low half, t + 16 in the high half) per 32-bit word.
        uint32_t xw[2][4];
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const uint32_t lo = lds_ld<uint32_t>(pv_at[pp][c] + so);
                const uint32_t hi = lds_ld<uint32_t>(pv_at[pp][c] + so + kHalfTokOff);
                // token t + 16 enters as 3 - c: its 2-bit codes are inverted
                // where B is formed (the bits above the codes are never read)
                xw[c][pp] = __builtin_amdgcn_perm(hi, lo, pv_sel);
            }
        }
        // ---- QK: logit of (token 16 hf + n, head 4 hs + kb)
        float lg[HS][2];
        uint32_t szv[2][NG];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const uint32_t ho = so + hf * kHalfTok;
            const uint32_t kc[2] = {lds_ld<uint32_t>(qk_at[0] + ho), lds_ld<uint32_t>(qk_at[1] + ho)};
            uint32_t szk[NG];
            if constexpr (NG == 4) {
                const u32x4 k4 = lds_ld<u32x4>(szk_at + ho), v4 = lds_ld<u32x4>(szv_at + ho);
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    szk[g] = k4[g];
                    szv[hf][g] = v4[g];
                }
            } else if constexpr (SZB == 2) {
                // E4M3 (s0, z0, s1, z1) bytes -> fp16 pairs (exact)
                const uint32_t k4 = lds_ld<uint32_t>(szk_at + ho), v4 = lds_ld<uint32_t>(szv_at + ho);
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    szk[g] = e4m3x2_to_f16x2(k4 >> (16 * g));
                    szv[hf][g] = e4m3x2_to_f16x2(v4 >> (16 * g));
                }
            } else if constexpr (NG == 2) {
                const u32x2 k2 = lds_ld<u32x2>(szk_at + ho), v2 = lds_ld<u32x2>(szv_at + ho);
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    szk[g] = k2[g];
                    szv[hf][g] = v2[g];
                }
            } else {
                szk[0] = lds_ld<uint32_t>(szk_at + ho);
                szv[hf][0] = lds_ld<uint32_t>(szv_at + ho);
            }
            // B of word P, half sh: pairs 4 sh .. 4 sh + 3 of the word as exact denormals
            f16x8 B[2][2];
#pragma unroll
            for (int P = 0; P < 2; ++P) {
                const uint32_t ds = kc[P] >> 6;
#pragma unroll
                for (int sh = 0; sh < 2; ++sh)
                    B[P][sh] = u4_as_h8(code_bits(kc[P], ds, 4 * sh + 0), code_bits(kc[P], ds, 4 * sh + 1),
                                        code_bits(kc[P], ds, 4 * sh + 2), code_bits(kc[P], ds, 4 * sh + 3));
            }
#pragma unroll
            for (int hs = 0; hs < HS; ++hs) {
                // acc[P] element x = (pair-local group x / 2, part x % 2) of
                // group half_group(P, x / 2): its hi or lo dot product
                f32x4 acc[2];
#pragma unroll
                for (int P = 0; P < 2; ++P) {
                    acc[P] = mfma_f16(qA[hs][P][0], B[P][0], f32x4{0, 0, 0, 0});
                    acc[P] = mfma_f16(qA[hs][P][1], B[P][1], acc[P]);
                }
                // s_g, z_g are halves of szk[g].  The logit stays in the MFMA's
                // units (a factor 2^(K - 24) of the log2 logit, K fixed per head).
                float x = 0.0f;
#pragma unroll
                for (int g = 0; g < NG; ++g) x = fmaf(half_hi(szk[g]), qz[hs][g], x);
#pragma unroll
                for (int P = 0; P < 2; ++P) {
#pragma unroll
                    for (int gl = 0; gl < (NG == 4 ? 2 : 1); ++gl) {
                        const float sg = half_lo(szk[half_group<NG>(P, gl)]);
                        x = fmaf(acc[P][2 * gl], sg, x);
                        x = fmaf(acc[P][2 * gl + 1], sg, x);
                    }
                }
                lg[hs][hf] = x;
            }
        }
        // masked tokens (only in tiles that are not full) get -inf
        if (__builtin_expect(valid != 0xffffffffu, 0)) {
#pragma unroll
            for (int hs = 0; hs < HS; ++hs) {
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) lg[hs][hf] = ((valid >> (16 * hf + n)) & 1u) ? lg[hs][hf] : -INFINITY;
            }
        }
        // ---- online softmax
        bool grow[HS];
        float alpha[HS], pw[HS][2];
#pragma unroll
        for (int hs = 0; hs < HS; ++hs) {
            const float mx = row16_max(fmaxf(lg[hs][0], lg[hs][1]));
            const float m_new = fmaxf(m_run[hs], mx);
            grow[hs] = __any(m_new > m_run[hs]);
            if (__builtin_expect(grow[hs], 0)) {
                alpha[hs] = (m_new > m_run[hs]) ? __builtin_amdgcn_exp2f((m_run[hs] - m_new) * qout[hs]) : 1.0f;
                l_lane[hs] *= alpha[hs];
#pragma unroll
                for (int g = 0; g < NG; ++g) zl[hs][g] *= alpha[hs];
                m_run[hs] = m_new;
                m_ref[hs] = m_new == -INFINITY ? 0.0f : m_new * qout[hs];
            }
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const float p = __builtin_amdgcn_exp2f(fmaf(lg[hs][hf], qout[hs], -m_ref[hs]));   // 0 for masked tokens
                pw[hs][hf] = p;
                l_lane[hs] += p;
                // tokens 16..31 enter the PV products as -p s_g against 3 - c (see
                // below); their zero-point term carries the difference, z + 3 s
                if (hf == 0) {
#pragma unroll
                    for (int g = 0; g < NG; ++g) zl[hs][g] = fmaf(p, half_hi(szv[hf][g]), zl[hs][g]);
                } else {
#pragma unroll
                    for (int g = 0; g < NG; ++g)
                        zl[hs][g] = fmaf(p, fmaf(3.0f, half_lo(szv[hf][g]), half_hi(szv[hf][g])), zl[hs][g]);
                }
            }
        }
        // ---- PV
#pragma unroll
        for (int hs = 0; hs < HS; ++hs) {
            // w_g = p s_g as hi + lo fp16 parts, both rounded to nearest; lo = w_g - hi.
            // They overwrite this head's K codes and (s, z) of the stage, read above.
            // Sign balance: the matrix core sums its 32 products after aligning
            // them to the largest and truncating the low bits toward zero, so
            // products of one sign (p s c >= 0) would lose a little in the same
            // direction on every tile.  Tokens 16..31 enter as (-p s)(3 - c) =
            // p s c - 3 p s, the -3 p s is returned through the zero-point sum,
            // and the truncation errors cancel; the running sums also stay near
            // the output instead of growing to ~1.5 s l.
            const float p0 = pw[hs][0], p1 = -pw[hs][1];
            constexpr uint32_t wso = kWeightsInStage ? so : 0u;
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const float s0 = half_lo(szv[0][g]), s1 = half_lo(szv[1][g]);
                // (fmaf with a zero addend reads the fp16 s in place: one mixed-precision fma)
                const uint32_t whi = pk_rn(fmaf(p0, s0, 0.0f), fmaf(p1, s1, 0.0f));   // tokens n, 16 + n
                const uint32_t wlo = pk_rn(fmaf(p0, s0, -half_lo(whi)), fmaf(p1, s1, -half_hi(whi)));
                const int gl = NG == 4 ? (g & 1) : 0;
                const uint32_t pl = NG == 4 ? uint32_t(g >> 1) * wpl_off : NG == 2 ? uint32_t(g) * wpl_off : 0u;
                lds_st<uint32_t>(w_at[2 * gl] + pl + wso, whi);
                lds_st<uint32_t>(w_at[2 * gl + 1] + pl + wso, wlo);
            }
            lds_order();
            // rescale the output rows of heads whose running max grew; PV output
            // row 4 q + h = (kb, i): the factor of head i lives in row i of lanes
            if (__builtin_expect(grow[hs], 0)) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float ai = __builtin_bit_cast(
                        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha[hs]), 16 * i));
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj) oacc[hs][jj][i] *= ai;
                }
            }
            constexpr uint32_t aso = kWeightsInStage ? so : 0u;
            f16x8 A[2];
            A[0] = lds_ld<f16x8>(a_at + aso);
            // with one group, both halves use its weights
            A[1] = NG == 1 ? A[0] : lds_ld<f16x8>(a_at + aso + wpl_off);
#pragma unroll
            for (int c = 0; c < 2; ++c) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    // (x ^ inv) & m: one three-input bit operation per dword
                    const uint32_t m = 0x00030003u << pv_code_exp(j);
                    const uint32_t inv = j <= 1 ? 0xfff00000u : 0xffff0000u;
                    uint32_t x[4];
#pragma unroll
                    for (int pp = 0; pp < 4; ++pp) x[pp] = ((j <= 1 ? xw[c][pp] << 4 : xw[c][pp]) ^ inv) & m;
                    const f16x8 Bj = u4_as_h8(x[0], x[1], x[2], x[3]);
                    oacc[hs][4 * c + j] = mfma_f16(A[c], Bj, oacc[hs][4 * c + j]);
                }
            }
            // the next set's weights go to the same units: the reads above come first
            lds_order();
        }
    };

    // ---- pipeline.  At the top of iteration t, R(t) and S(t + 4) must have
    // landed: seven operations follow them (R(t + 1), S(t + 5), R(t + 2)).
    // The barrier then publishes tile t and the slot ids of tile t + 4 of
    // every wave, and guarantees that every wave is done with tile t - 1,
    // whose stage R(t + 3) overwrites, and with the slot ids of tile t + 2,
    // whose ring slot S(t + 6) overwrites.  The prologue leaves the same
    // operations in flight, so the counts hold from the start.  The loop is
    // unrolled by four so that stage and ring offsets are constants; tiles
    // with no usable token (past the end) are not computed.
    const bool run_compute = __builtin_amdgcn_readfirstlane(int(active)) != 0;
    auto sync = [] {
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    slot_load(0, 0);
    slot_load(1, 1);
    slot_load(2, 2);
    slot_load(3, 3);
    wait_vmem<0>();
    sync();
    Fetch f = prep(0, 0);
    uint32_t vq0 = f.valid;                   // usable tokens of tiles t .. t + 3
    issue(f, 0);
    f = prep(1, 1);
    uint32_t vq1 = f.valid;
    sync();                                   // ring slots 0 and 1 are read by every wave
    slot_load(4, 0);
    issue(f, 1);
    f = prep(2, 2);
    uint32_t vq2 = f.valid;
    slot_load(5, 1);
    issue(f, 2);
    f = prep(3, 3);
    uint32_t vq3 = f.valid;
    auto step = [&](int t, auto K) {
        constexpr int k = decltype(K)::value;             // t % 4
        wait_vmem<7>();
        sync();
        slot_load(t + 6, (k + 2) & 3);
        issue(f, (k + 3) & 3);                            // R(t + 3)
        // the slot ids of tile t + 4 are read before the compute, so that their
        // LDS latency overlaps it; its record addresses are formed after
        const SlotIds ids = read_ids(k);
        if (run_compute && vq0 != 0u) compute(K, vq0);
        f = form(t + 4, ids);
        vq0 = vq1;
        vq1 = vq2;
        vq2 = vq3;
        vq3 = f.valid;
    };
    for (int t = 0; t < n_tiles; t += 4) {
        step(t, std::integral_constant<int, 0>{});
        step(t + 1, std::integral_constant<int, 1>{});
        step(t + 2, std::integral_constant<int, 2>{});
        step(t + 3, std::integral_constant<int, 3>{});
    }
    // the trailing (unused) loads still write the stages: let them land
    wait_vmem<0>();
    if (!active) return;

    // ---- write the partial (m, l, o') of the GQ heads
    const size_t row0 = (size_t(b) * a.items + j) * a.hq + hk * GQ;
    // lane (n, kb) holds rows 4 kb + i = (q = kb, h = i) of column n: channel
    // 64 c + 4 n + j in oacc[hs][4 c + j].  That channel's group is
    // half_group(c, gl) with gl = pair_local_group(n / 4); its hi and lo rows
    // (q = 2 gl, 2 gl + 1) are in lanes kb = 2 gl and 2 gl + 1, 16 lanes apart
    const int gl_o = pair_local_group<NG>(n >> 2);
    const bool writer = kb == 2 * gl_o;
    auto swap16 = [](float v) {   // the value of lane l ^ 16
        return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
    };
#pragma unroll
    for (int hs = 0; hs < HS; ++hs) {
        const float l_row = row16_sum(l_lane[hs]);
        float zt[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) zt[g] = row16_sum(zl[hs][g]);
        if (n == 0 && 4 * hs + kb < GQ) {
            a.part_ml[(row0 + 4 * hs + kb) * 2 + 0] = m_run[hs] * qout[hs];   // log2 units
            a.part_ml[(row0 + 4 * hs + kb) * 2 + 1] = l_row;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (4 * hs + i >= GQ) break;
            // p z summed over the item for head i and each group (held by row i of lanes)
            float zg[NG];
#pragma unroll
            for (int g = 0; g < NG; ++g)
                zg[g] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, zt[g]), 16 * i));
            float o[8];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                float z = 0.0f;
#pragma unroll
                for (int gl = 0; gl < (NG == 4 ? 2 : 1); ++gl) z = gl == gl_o ? zg[half_group<NG>(c, gl)] : z;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const float v = oacc[hs][4 * c + jj][i];
                    o[4 * c + jj] = (v + swap16(v)) * __builtin_ldexpf(1.0f, 24 - pv_code_exp(jj)) + z;
                }
            }
            if (writer) {
                float *dst = a.part_o + (row0 + 4 * hs + i) * kHeadDim + 4 * n;
                *reinterpret_cast<f32x4 *>(dst) = f32x4{o[0], o[1], o[2], o[3]};
                *reinterpret_cast<f32x4 *>(dst + 64) = f32x4{o[4], o[5], o[6], o[7]};
            }
        }
    }
}

// BF16 window item on fp32 VALU: at most kWindowItemTokens = 64 positions of
// the sink or recent window, one wave per KV head.  Two memory round trips:
// QK with lane = position (its K row, 16 x 16 bytes, against q' staged in
// this wave's LDS), then PV with lane = channel pair and the V rows of all the
// item's positions in flight at once, each row's offset broadcast from the
// lane that computed it.  The softmax runs while the V rows arrive.
// `pbuf` is this wave's LDS scratch: q' [kMaxGroup][128] then p [64][kMaxGroup].
static_assert(kWindowItemTokens == kBf16Chunk, "a window item is one chunk of 64 positions");
constexpr int kBf16WaveFloats = kMaxGroup * kHeadDim + kMaxGroup * kBf16Chunk;

// Ends a block of PV products: the accumulators pass through an empty asm
// statement with a memory clobber, so the next block's LDS reads cannot be
// hoisted above this block's products (held all at once they would need 256
// registers).
template <int NH>
__device__ __forceinline__ void pv_block_end(float (&o0)[NH], float (&o1)[NH]) {
    if constexpr (NH == 4)
        asm volatile("" : "+v"(o0[0]), "+v"(o0[1]), "+v"(o0[2]), "+v"(o0[3]), "+v"(o1[0]), "+v"(o1[1]),
                     "+v"(o1[2]), "+v"(o1[3])::"memory");
    else
        asm volatile("" : "+v"(o0[0]), "+v"(o0[1]), "+v"(o0[2]), "+v"(o0[3]), "+v"(o0[4]), "+v"(o0[5]),
                     "+v"(o0[6]), "+v"(o0[7]), "+v"(o1[0]), "+v"(o1[1]), "+v"(o1[2]), "+v"(o1[3]),
                     "+v"(o1[4]), "+v"(o1[5]), "+v"(o1[6]), "+v"(o1[7])::"memory");
}

// o[h] += p[t][h] v_t over the 64 positions for NH heads (the group padded to
// 4 or 8; the padding heads' weights are zero), lane = channel pair, in blocks
// of 4 positions whose weights are read while the previous block's products
// run.  Positions past the item's end have p = 0 and the first position's V row.
template <int NH>
__device__ __forceinline__ void bf16_pv(const uint32_t (&vw)[kBf16Chunk], const float *ps, float (&o0)[NH],
                                        float (&o1)[NH]) {
    constexpr int kBlk = 4, kQ = NH / 4;
    f32x4 pw[2][kBlk][kQ];
#pragma unroll
    for (int u = 0; u < kBlk; ++u)
#pragma unroll
        for (int q = 0; q < kQ; ++q) pw[0][u][q] = *reinterpret_cast<const f32x4 *>(ps + u * kMaxGroup + 4 * q);
#pragma unroll
    for (int blk = 0; blk < kBf16Chunk / kBlk; ++blk) {
        if (blk + 1 < kBf16Chunk / kBlk) {
#pragma unroll
            for (int u = 0; u < kBlk; ++u)
#pragma unroll
                for (int q = 0; q < kQ; ++q)
                    pw[(blk + 1) & 1][u][q] =
                        *reinterpret_cast<const f32x4 *>(ps + ((blk + 1) * kBlk + u) * kMaxGroup + 4 * q);
        }
#pragma unroll
        for (int u = 0; u < kBlk; ++u) {
            const uint32_t v = vw[blk * kBlk + u];
            const float v0 = bf16_bits_to_f32(v & 0xFFFFu), v1 = bf16_bits_to_f32(v >> 16);
#pragma unroll
            for (int q = 0; q < kQ; ++q)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    o0[4 * q + e] = fmaf(pw[blk & 1][u][q][e], v0, o0[4 * q + e]);
                    o1[4 * q + e] = fmaf(pw[blk & 1][u][q][e], v1, o1[4 * q + e]);
                }
        }
        pv_block_end<NH>(o0, o1);
    }
}

template <int NH>
__device__ __forceinline__ void bf16_item(const DecodeArgs &a, int b, int req, int j, int hk, int p0, int p1,
                                          bool active, float *pbuf) {
    const int lane = threadIdx.x & 63;
    const int g = a.g;
    float *qs = pbuf;
    float *ps = pbuf + kMaxGroup * kHeadDim;
    const float *qr = a.qrot + (size_t(b) * a.hq + hk * g) * kHeadDim;
    for (int e = lane; e < NH * kHeadDim; e += 64) qs[e] = e < g * kHeadDim ? qr[e] : 0.0f;   // padding: q' = 0
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // row of window position pos: base + ring index x row_elems (K at +0, V at
    // +128); windows of at most 4096 rows and 16 KV heads keep it below 2^24
    const bool is_sink = j < a.sink_items;
    const uint32_t ring = uint32_t(is_sink ? a.sink_tokens : a.recent_tokens);
    const uint16_t *base = (is_sink ? a.sink : a.recent) + (size_t(req) * ring * a.hkv + hk) * 2 * kHeadDim;
    const uint32_t row_elems = uint32_t(a.hkv) * 2 * kHeadDim;
    const int cnt = p1 - p0;                             // 1 .. 64
    const bool ok = active && lane < cnt;
    const uint32_t pos = uint32_t(p0 + (lane < cnt ? lane : 0));   // past the end: the first position
    const uint32_t roff = (is_sink ? pos : pos % ring) * row_elems;
    // ---- QK: the whole K row of this lane's position in flight at once
    u32x4 kw[kHeadDim / 8];
#pragma unroll
    for (int i = 0; i < kHeadDim / 8; ++i) kw[i] = *reinterpret_cast<const u32x4 *>(base + roff + 8 * i);
    float acc[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) acc[h] = 0.0f;
#pragma unroll
    for (int i = 0; i < kHeadDim / 8; ++i) {
        float kf[8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            kf[2 * u] = bf16_bits_to_f32(kw[i][u] & 0xFFFFu);
            kf[2 * u + 1] = bf16_bits_to_f32(kw[i][u] >> 16);
        }
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            const f32x4 qa = *reinterpret_cast<const f32x4 *>(qs + h * kHeadDim + 8 * i);
            const f32x4 qb = *reinterpret_cast<const f32x4 *>(qs + h * kHeadDim + 8 * i + 4);
            acc[h] = fmaf(qa[0], kf[0], acc[h]);
            acc[h] = fmaf(qa[1], kf[1], acc[h]);
            acc[h] = fmaf(qa[2], kf[2], acc[h]);
            acc[h] = fmaf(qa[3], kf[3], acc[h]);
            acc[h] = fmaf(qb[0], kf[4], acc[h]);
            acc[h] = fmaf(qb[1], kf[5], acc[h]);
            acc[h] = fmaf(qb[2], kf[6], acc[h]);
            acc[h] = fmaf(qb[3], kf[7], acc[h]);
        }
    }
    // ---- V rows of every position, in flight during the softmax
    uint32_t vw[kBf16Chunk];
#pragma unroll
    for (int t = 0; t < kBf16Chunk; ++t) {
        const uint32_t ro = uint32_t(__builtin_amdgcn_readlane(int(roff), t));
        vw[t] = *reinterpret_cast<const uint32_t *>(base + ro + kHeadDim + 2 * lane);
    }
    // ---- softmax over the item's positions (log2 units), p token-major in LDS
    float m[NH], l[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        const float x = ok ? acc[h] : -INFINITY;
        float mx = row16_max(x);                         // DPP within rows, then across the 4 rows
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float p = ok ? __builtin_amdgcn_exp2f(x - mx) : 0.0f;
        m[h] = mx;
        l[h] = p;
        ps[lane * kMaxGroup + h] = h < g ? p : 0.0f;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // ---- PV
    float o0[NH], o1[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        o0[h] = 0.0f;
        o1[h] = 0.0f;
    }
    bf16_pv<NH>(vw, ps, o0, o1);
    if (!active) return;
    const size_t row0 = (size_t(b) * a.items + j) * a.hq + hk * g;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        if (h >= g) break;
        float lsum = row16_sum(l[h]);
        lsum += __shfl_xor(lsum, 16);
        lsum += __shfl_xor(lsum, 32);
        if (lane == 0) {
            a.part_ml[(row0 + h) * 2 + 0] = m[h];
            a.part_ml[(row0 + h) * 2 + 1] = lsum;
        }
        float *dst = a.part_o + (row0 + h) * kHeadDim + 2 * lane;
        dst[0] = o0[h];
        dst[1] = o1[h];
    }
}

template <int GQ, int NG, int SZB>
__global__ __launch_bounds__(64 * kPartialWaves) void partial_kernel(DecodeArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int id = blockIdx.x;
    const int hc = id % a.head_chunks;
    const int rest = id / a.head_chunks;
    // grid row jg holds one item of every request, request b at column
    // (b + jg) mod batch: the XCDs take workgroups round-robin by index, so
    // rotating the columns spreads each request's items over the XCDs (with a
    // multiple of 8 columns a request would otherwise stay on one XCD, and a
    // ragged batch would load the XCDs unevenly)
    const int jg = rest / a.batch;
    const int b = (rest % a.batch + a.batch - jg % a.batch) % a.batch;
    // grid order: the long history items first, so that the short window items
    // fill the compute units that the last history items leave idle
    const int n_hist = a.items - a.win_items;
    const int j = !a.win_last ? jg : jg < n_hist ? a.win_items + jg : jg - n_hist;
    int req = 0;
    const int L = request_length(a, b, req);
    int p0, p1;
    item_range(a, L, j, p0, p1);
    if (p0 >= p1) return;                       // uniform over the workgroup
    const int w = threadIdx.x >> 6;
    const int hk = hc * kPartialWaves + w;
    const bool active = hk < a.hkv;
    if (j < a.win_items) {
        float *pbuf = reinterpret_cast<float *>(smem) + w * kBf16WaveFloats;
        if (a.g <= 4)                               // the group padded to 4 or 8 heads
            bf16_item<4>(a, b, req, j, active ? hk : 0, p0, p1, active, pbuf);
        else
            bf16_item<8>(a, b, req, j, active ? hk : 0, p0, p1, active, pbuf);
    } else if (a.num_slots > 0) {
        int2_item<GQ, NG, SZB>(a, b, req, j, hc, p0, p1, smem);   // every wave: the loads are shared
    }
}

// History items of the 72-byte layout (G = 128, one group per head vector)
// when the number of KV heads is odd; the kernel also takes G = 64 (NG = 2).
// fp32 VALU, 64 tokens per step.  QK: lane = token, the 128 codes of
// its K against q' in LDS, factored per group as s_g (q'_g . c_g) + z_g Q_g
// (Q_g the group's sum of q').  PV: lane = channel pair, the step's V codes and
// (s, z) staged in LDS, v = s c + z formed per token.
constexpr int kLmChunk = 64;

template <int NG, int SZB>
__global__ __launch_bounds__(64 * kPartialWaves) void hist_lowmeta_kernel(DecodeArgs a) {
    constexpr int kRec = 2 * kCodeBytes + 2 * NG * SZB;    // head record bytes
    constexpr int kG = kHeadDim / NG;                       // channels per group
    __shared__ __attribute__((aligned(16))) float qs_all[kPartialWaves][kMaxGroup][kHeadDim];
    __shared__ __attribute__((aligned(16))) float ps_all[kPartialWaves][kLmChunk][kMaxGroup];
    __shared__ uint32_t vc_all[kPartialWaves][kLmChunk][kCodeBytes / 4];
    __shared__ float2 vsz_all[kPartialWaves][kLmChunk][NG];
    const int id = blockIdx.x;
    const int hc = id % a.head_chunks;
    const int rest = id / a.head_chunks;
    const int jg = rest / a.batch;
    const int b = (rest % a.batch + a.batch - jg % a.batch) % a.batch;   // rotated columns, as partial_kernel
    const int j = a.win_items + jg;
    int req = 0;
    const int L = request_length(a, b, req);
    int p0, p1;
    item_range(a, L, j, p0, p1);
    const int w = threadIdx.x >> 6;
    const int hk = hc * kPartialWaves + w;
    if (p0 >= p1 || hk >= a.hkv) return;                    // no workgroup barrier below
    const int lane = threadIdx.x & 63;
    const int g = a.g;
    float(*qs)[kHeadDim] = qs_all[w];
    float(*ps)[kMaxGroup] = ps_all[w];
    uint32_t(*vc)[kCodeBytes / 4] = vc_all[w];
    float2(*vsz)[NG] = vsz_all[w];
    const size_t row0q = size_t(b) * a.hq + size_t(hk) * g;
    for (int e = lane; e < g * kHeadDim; e += 64) qs[e / kHeadDim][e % kHeadDim] = a.qrot[row0q * kHeadDim + e];
    float qg[kMaxGroup][NG];                                // group sums of q' (from the 32-channel sums)
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h)
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            float sum = 0.0f;
            if (h < g)
#pragma unroll
                for (int sub = 0; sub < kG / kGroup; ++sub) sum += a.qsum[(row0q + h) * 8 + gi * (kG / kGroup) + sub];
            qg[h][gi] = sum;
        }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    float m_run[kMaxGroup], l_lane[kMaxGroup], o0[kMaxGroup], o1[kMaxGroup];
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
        m_run[h] = -INFINITY;
        l_lane[h] = 0.0f;
        o0[h] = 0.0f;
        o1[h] = 0.0f;
    }
    const int32_t *tab = a.req_to_slot + size_t(req) * a.r2s_stride;
    const size_t rec_bytes = size_t(a.hkv) * kRec;
    for (int cb = p0; cb < p1; cb += kLmChunk) {
        const int cnt = min(kLmChunk, p1 - cb);
        const int slot = lane < cnt ? tab[cb + lane] : -1;
        const bool ok = slot >= 0 && slot < a.num_slots;
        const uint8_t *base = ok ? a.records + size_t(slot) * rec_bytes + size_t(hk) * kRec : a.zero_rec;
        u32x2 kc[4], vv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            kc[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(base) + i);
            vv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(base + kCodeBytes) + i);
        }
        uint32_t ksz[NG];                                   // (s, z) of K as an fp16 pair
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            if constexpr (SZB == 4) {
                ksz[gi] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(base + 2 * kCodeBytes) + gi);
                const uint32_t vw = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(base + 2 * kCodeBytes + 4 * NG) + gi);
                vsz[lane][gi] = make_float2(__half2float(__ushort_as_half(uint16_t(vw))),
                                            __half2float(__ushort_as_half(uint16_t(vw >> 16))));
            } else {                                        // E4M3 codes, s first
                const uint32_t kw = __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(base + 2 * kCodeBytes) + gi);
                const uint32_t vw = __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(base + 2 * kCodeBytes + 2 * NG) + gi);
                ksz[gi] = e4m3x2_to_f16x2(kw);
                const uint32_t vh = e4m3x2_to_f16x2(vw);
                vsz[lane][gi] = make_float2(half_lo_f(vh), half_hi_f(vh));
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            vc[lane][2 * i] = vv[i][0];
            vc[lane][2 * i + 1] = vv[i][1];
        }
        // ---- QK: lane = token
        float dot[kMaxGroup][NG];
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h)
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) dot[h][gi] = 0.0f;
#pragma unroll
        for (int wd = 0; wd < 8; ++wd) {                    // 16 channels per code word
            const uint32_t cw = kc[wd >> 1][wd & 1];
            const int gi = (16 * wd) / kG;
            float c[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) c[e] = float((cw >> (2 * e)) & 3u);
#pragma unroll
            for (int h = 0; h < kMaxGroup; ++h) {
                if (h < g) {
#pragma unroll
                    for (int e4 = 0; e4 < 16; e4 += 4) {
                        const f32x4 q4 = *reinterpret_cast<const f32x4 *>(&qs[h][16 * wd + e4]);
                        dot[h][gi] = fmaf(q4[0], c[e4], dot[h][gi]);
                        dot[h][gi] = fmaf(q4[1], c[e4 + 1], dot[h][gi]);
                        dot[h][gi] = fmaf(q4[2], c[e4 + 2], dot[h][gi]);
                        dot[h][gi] = fmaf(q4[3], c[e4 + 3], dot[h][gi]);
                    }
                }
            }
        }
        float alpha[kMaxGroup];
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h) {
            float x = 0.0f;
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                const float sg = __half2float(__ushort_as_half(uint16_t(ksz[gi])));
                const float zg = __half2float(__ushort_as_half(uint16_t(ksz[gi] >> 16)));
                x = fmaf(sg, dot[h][gi], x);
                x = fmaf(zg, qg[h][gi], x);
            }
            x = ok ? x : -INFINITY;
            const float mx = wave_max(x);
            const float m_new = fmaxf(m_run[h], mx);
            alpha[h] = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run[h] - m_new);
            m_run[h] = m_new;
            const float p = x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(x - m_new);
            l_lane[h] = fmaf(l_lane[h], alpha[h], p);
            if (h < g) ps[lane][h] = p;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // ---- PV: lane = channels 2 lane, 2 lane + 1
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h) {
            o0[h] *= alpha[h];
            o1[h] *= alpha[h];
        }
        const int cword = lane >> 3, cshift = 4 * (lane & 7), cg = (2 * lane) / kG;
        for (int u = 0; u < cnt; ++u) {
            const uint32_t cw = vc[u][cword] >> cshift;
            const float2 sz = vsz[u][cg];
            const float v0 = fmaf(sz.x, float(cw & 3u), sz.y), v1 = fmaf(sz.x, float((cw >> 2) & 3u), sz.y);
            float p[kMaxGroup];
#pragma unroll
            for (int h4 = 0; h4 < kMaxGroup; h4 += 4) {
                if (h4 < g) {
                    const f32x4 p4 = *reinterpret_cast<const f32x4 *>(&ps[u][h4]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) p[h4 + e] = p4[e];
                }
            }
#pragma unroll
            for (int h = 0; h < kMaxGroup; ++h) {
                if (h < g) {
                    o0[h] = fmaf(p[h], v0, o0[h]);
                    o1[h] = fmaf(p[h], v1, o1[h]);
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    const size_t row0 = (size_t(b) * a.items + j) * a.hq + size_t(hk) * g;
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
        if (h >= g) break;
        const float l = wave_sum(l_lane[h]);
        if (lane == 0) {
            a.part_ml[(row0 + h) * 2 + 0] = m_run[h];
            a.part_ml[(row0 + h) * 2 + 1] = l;
        }
        float2 *dst = reinterpret_cast<float2 *>(a.part_o + (row0 + h) * kHeadDim) + lane;
        *dst = make_float2(o0[h], o1[h]);
    }
}

// ---------------------------------------------------------------------------
// 3. merge + un-rotation
// ---------------------------------------------------------------------------
// One workgroup per (request, KV head).  Wave h first reduces the running
// maxima and sums of query head h over the items in one pass (each lane keeps
// a running (m, l) of its items); then thread (h, c) accumulates channel c
// over the items, 16 items' loads in flight at a time.
__global__ __launch_bounds__(512) void merge_kernel(DecodeArgs a) {
    __shared__ float ob[kMaxGroup][kHeadDim];
    __shared__ float red[4][kMaxGroup][kHeadDim];
    __shared__ float m_head[kMaxGroup], l_head[kMaxGroup];
    const int b = blockIdx.x / a.hkv;
    const int hk = blockIdx.x % a.hkv;
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int c = t & (kHeadDim - 1);
    int req = 0;
    const int L = request_length(a, b, req);
    // items that hold a partial: the window items that hold positions (item_range
    // fills them from the start: the first n_sink of the sink's, the first
    // n_recent of the recent window's), then every history chunk (written only
    // when the INT2 pool exists)
    const int hist_end = max(a.sink_tokens, L - a.recent_tokens);
    const int sink_len = min(a.sink_tokens, L), recent_len = L > a.sink_tokens ? L - hist_end : 0;
    const int recent_items = a.win_items - a.sink_items;
    const int n_sink = a.sink_items == 1 ? int(sink_len > 0) : (sink_len + kWindowItemTokens - 1) / kWindowItemTokens;
    const int n_recent =
        recent_items == 1 ? int(recent_len > 0) : (recent_len + kWindowItemTokens - 1) / kWindowItemTokens;
    const int hist = hist_end - a.sink_tokens;
    // capped at the planned items: a device length longer than the host copy
    // the plan was made from must not read partials past this request's rows
    const int item_cap = a.extra_item >= 0 ? a.extra_item : a.items;
    const int n_hist_items =
        a.num_slots > 0 ? min(item_cap, a.win_items + (hist + a.chunk - 1) / a.chunk) : a.win_items;
    // the extend's new-token item is the last one and always holds a partial;
    // items between the request's chunks and it hold none
    const int n_items = a.extra_item >= 0 ? a.extra_item + 1 : n_hist_items;
    const size_t row_b = size_t(b) * a.items * a.hq + size_t(hk) * a.g;   // item 0, head 0
    auto item_ok = [&](int j) {
        return j == a.extra_item || (j >= a.win_items && j < n_hist_items) || j < n_sink ||
               (j >= a.sink_items && j < a.sink_items + n_recent);
    };

    const int wv = t >> 6;
    if (wv < a.g) {
        float mx = -INFINITY, l = 0.0f;          // this lane's items, l relative to mx
        for (int j = lane; j < n_items; j += 64) {
            if (!item_ok(j)) continue;
            const float2 ml = *reinterpret_cast<const float2 *>(a.part_ml + (row_b + size_t(j) * a.hq + wv) * 2);
            if (ml.x == -INFINITY) continue;     // every token of the item masked: weight 0
            if (ml.x > mx) {
                l = fmaf(l, __builtin_amdgcn_exp2f(mx - ml.x), ml.y);
                mx = ml.x;
            } else {
                l = fmaf(ml.y, __builtin_amdgcn_exp2f(ml.x - mx), l);
            }
        }
        const float M = wave_max(mx);
        l = wave_sum(mx == -INFINITY ? 0.0f : l * __builtin_amdgcn_exp2f(mx - M));
        if (lane == 0) {
            m_head[wv] = M;
            l_head[wv] = l;
        }
    }
    __syncthreads();
    // o'[h] = sum over items of 2^(m_j - M) o'_j / l.  The items that hold a
    // partial, numbered k = 0 .. n_part-1, are split among `splits` threads per
    // (head, 4 channels), so that a long request's items are read with several
    // times the loads in flight; the splits add up through LDS in a fixed order.
    {
        const int n_hist = n_hist_items - a.win_items;
        const int n_part = n_sink + n_recent + n_hist + (a.extra_item >= 0 ? 1 : 0);
        const int units = a.g * (kHeadDim / 4);                 // (head, 4 channels)
        const int splits = 512 / units;                         // 2 .. 16
        const int u = t % units, sp = t / units;
        const int h = u / (kHeadDim / 4), c4 = 4 * (u % (kHeadDim / 4));
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        if (sp < splits) {
            const float M = m_head[h];
            const size_t row_h = row_b + h;
#pragma unroll 8
            for (int k = sp; k < n_part; k += splits) {
                // k -> item: the sink's, the recent window's, the history chunks, the new tokens
                int j = k < n_sink ? k : k - n_sink + a.sink_items;
                j = k < n_sink + n_recent ? j : k - n_sink - n_recent + a.win_items;
                j = k < n_sink + n_recent + n_hist ? j : a.extra_item;
                const size_t row = row_h + size_t(j) * a.hq;
                // every item that exists wrote finite (m, l, o'); a fully masked
                // one has m = -inf and weight exp2(-inf) = 0
                const float e = __builtin_amdgcn_exp2f(a.part_ml[row * 2] - M);
                const f32x4 o = *reinterpret_cast<const f32x4 *>(a.part_o + row * kHeadDim + c4);
                acc[0] = fmaf(e, o[0], acc[0]);
                acc[1] = fmaf(e, o[1], acc[1]);
                acc[2] = fmaf(e, o[2], acc[2]);
                acc[3] = fmaf(e, o[3], acc[3]);
            }
            *reinterpret_cast<f32x4 *>(&red[0][0][0] + (sp * units + u) * 4) = acc;
        }
        __syncthreads();
        for (int e = t; e < a.g * kHeadDim; e += 512) {
            const int hh = e / kHeadDim, cc = e % kHeadDim;
            const float M = m_head[hh], l = l_head[hh];
            float sum = 0.0f;
            for (int q = 0; q < splits; ++q) sum += (&red[0][0][0])[(q * units + hh * (kHeadDim / 4) + cc / 4) * 4 + cc % 4];
            ob[hh][cc] = (M != -INFINITY && l > 0.0f) ? sum / l : 0.0f;
        }
    }
    __syncthreads();
    // o[h][c] = sum_i o'[h][i] R_V[c][i]: thread (part, c) reads the quarter
    // i = 32 part .. 32 part + 31 of row c of R_V once and forms that part of
    // the sum for every query head; the four parts add up through LDS
    {
        const int part = t >> 7;
        const float *R = a.r_v + (size_t(hk) * kHeadDim + c) * kHeadDim + 32 * part;
        f32x4 r[8];
#pragma unroll
        for (int i4 = 0; i4 < 8; ++i4) r[i4] = *reinterpret_cast<const f32x4 *>(R + 4 * i4);
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h) {
            if (h >= a.g) break;
            const float *ov = ob[h] + 32 * part;
            float o = 0.0f;
#pragma unroll
            for (int i4 = 0; i4 < 8; ++i4) {
                o = fmaf(ov[4 * i4], r[i4][0], o);
                o = fmaf(ov[4 * i4 + 1], r[i4][1], o);
                o = fmaf(ov[4 * i4 + 2], r[i4][2], o);
                o = fmaf(ov[4 * i4 + 3], r[i4][3], o);
            }
            red[part][h][c] = o;
        }
    }
    __syncthreads();
    for (int h = t >> 7; h < a.g; h += 4) {
        const float o = (red[0][h][c] + red[1][h][c]) + (red[2][h][c] + red[3][h][c]);
        const size_t idx = (size_t(b) * a.hq + hk * a.g + h) * kHeadDim + c;
        if (a.out_dtype == OSCAR_F32)
            static_cast<float *>(a.out)[idx] = o;
        else if (a.out_dtype == OSCAR_BF16)
            static_cast<uint16_t *>(a.out)[idx] = bf16_bits_rn(o);
        else
            static_cast<uint16_t *>(a.out)[idx] = __half_as_ushort(__float2half_rn(o));
    }
}

// ---------------------------------------------------------------------------
// 4. extend: rotated BF16 keys and values of the new tokens
// ---------------------------------------------------------------------------
// One workgroup per (token, KV head, K or V); thread c forms channel c of
// x R in fp32 and rounds it to BF16, as the recent window stores it.
struct RotateArgs {
    const void *k;
    const void *v;
    const float *r_k;
    const float *r_v;
    uint16_t *out;     // [n][Hkv][2][128]
    int32_t hkv;
    int32_t dtype;
};

__global__ __launch_bounds__(kHeadDim) void extend_rotate_kernel(RotateArgs a) {
    __shared__ float xs[kHeadDim];
    const int t = blockIdx.x & 1;
    const int hk = (blockIdx.x >> 1) % a.hkv;
    const int i = (blockIdx.x >> 1) / a.hkv;
    const int c = threadIdx.x;
    xs[c] = load_as_f32(t ? a.v : a.k, a.dtype, (size_t(i) * a.hkv + hk) * kHeadDim + c);
    __syncthreads();
    const float *R = (t ? a.r_v : a.r_k) + size_t(hk) * kHeadDim * kHeadDim + c;
    float acc = 0.0f;
#pragma unroll 16
    for (int r = 0; r < kHeadDim; ++r) acc = fmaf(xs[r], R[size_t(r) * kHeadDim], acc);
    a.out[((size_t(i) * a.hkv + hk) * 2 + t) * kHeadDim + c] = bf16_bits_rn(acc);
}

// Dynamic LDS of the partial kernel: the four record stages and the slot-id
// ring of the INT2 items, or each wave's softmax buffer for the BF16 items.
size_t partial_lds_bytes(const DecodeArgs &a) {
    const size_t int2 = a.group_size == kGroup ? int2_lds_bytes() : int2_lds_bytes_lowmeta();
    const size_t pbuf = size_t(kPartialWaves) * kBf16WaveFloats * sizeof(float);
    return int2 > pbuf ? int2 : pbuf;
}

template <int GQ>
hipError_t launch_partial(const DecodeArgs &a, int blocks, hipStream_t stream) {
    const size_t lds = partial_lds_bytes(a);
    if (a.group_size == 64 && a.scale_bits == 8)
        hipLaunchKernelGGL((partial_kernel<GQ, 2, 2>), dim3(blocks), dim3(64 * kPartialWaves), lds, stream, a);
    else if (a.group_size == 64)
        hipLaunchKernelGGL((partial_kernel<GQ, 2, 4>), dim3(blocks), dim3(64 * kPartialWaves), lds, stream, a);
    else if (a.group_size == 128)
        hipLaunchKernelGGL((partial_kernel<GQ, 1, 4>), dim3(blocks), dim3(64 * kPartialWaves), lds, stream, a);
    else
        hipLaunchKernelGGL((partial_kernel<GQ, 4, 4>), dim3(blocks), dim3(64 * kPartialWaves), lds, stream, a);
    return hipGetLastError();
}

}  // namespace
}  // namespace oscar

using namespace oscar;

namespace {

oscar_status check_decode_common(const oscar_layout *layout, const oscar_pool *pool, const void *q,
                                 oscar_dtype q_dtype, const int32_t *req_to_slot, const float *R_K,
                                 const float *R_V, float sm_scale, void *out, oscar_dtype out_dtype) {
    oscar_status st = check_layout(layout);
    if (st != OSCAR_OK) return st;
    if (!pool || !q || !req_to_slot || !R_K || !R_V || !out)
        return fail(OSCAR_ERR_INVALID_ARG, "a required pointer is null");
    if (!pool->records || !pool->recent || (layout->sink_tokens > 0 && !pool->sink))
        return fail(OSCAR_ERR_INVALID_ARG, "a pool pointer is null");
    if (q_dtype != OSCAR_F32 && q_dtype != OSCAR_BF16 && q_dtype != OSCAR_F16)
        return fail(OSCAR_ERR_INVALID_ARG, "q_dtype must be F32, BF16 or F16");
    if (out_dtype != OSCAR_F32 && out_dtype != OSCAR_BF16 && out_dtype != OSCAR_F16)
        return fail(OSCAR_ERR_INVALID_ARG, "out_dtype must be F32, BF16 or F16");
    if (!std::isfinite(sm_scale)) return fail(OSCAR_ERR_INVALID_ARG, "sm_scale must be finite");
    return OSCAR_OK;
}

oscar_status check_workspace(const DecodePlan &plan, int64_t req_to_slot_stride, void *workspace,
                             size_t workspace_bytes) {
    if (req_to_slot_stride < plan.max_len)
        return fail(OSCAR_ERR_INVALID_ARG, "req_to_slot_stride is smaller than the longest sequence");
    if (!workspace || workspace_bytes < plan.ws_bytes)
        return fail(OSCAR_ERR_WORKSPACE, "workspace is smaller than the size the library reported");
    if (reinterpret_cast<uintptr_t>(workspace) % 256)
        return fail(OSCAR_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    return OSCAR_OK;
}

DecodeArgs make_args(const oscar_layout *layout, const oscar_pool *pool, const void *q, oscar_dtype q_dtype,
                     int32_t batch, const int32_t *req_to_slot, int64_t req_to_slot_stride,
                     const float *R_K, const float *R_V, float sm_scale, void *out, oscar_dtype out_dtype,
                     void *workspace, const DecodePlan &plan) {
    DecodeArgs a;
    a.q = q;
    a.req_ids = nullptr;
    a.seq_lens = nullptr;
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
    a.zero_rec = ws + plan.ws_zero;
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
    a.sink_items = plan.sink_items;
    a.win_items = plan.sink_items + plan.recent_items;
    a.win_last = 1;
    a.waves = kPartialWaves;
    a.head_chunks = (a.hkv + kPartialWaves - 1) / kPartialWaves;
    a.group_size = layout->group_size;
    a.scale_bits = scale_bits(*layout);
    a.fixed_req = -1;
    a.fixed_len = 0;
    a.extra_item = plan.extra_item;
    a.newkv = plan.extra_item >= 0 ? reinterpret_cast<const uint16_t *>(ws + plan.ws_newkv) : nullptr;
    return a;
}

// prep, split-K partials and merge on `stream`
oscar_status launch_decode(const DecodeArgs &a, const DecodePlan &plan, hipStream_t stream,
                           const oscar_launch_opts *opts, const ExtendHistArgs *xh = nullptr) {
    if (int64_t(plan.items) * a.batch * a.head_chunks > INT32_MAX)
        return fail(OSCAR_ERR_UNSUPPORTED, "batch x work items exceeds one launch grid");
    hipLaunchKernelGGL(prep_kernel, dim3(a.batch * a.hkv), dim3(512), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(OSCAR_ERR_HIP, std::string("prep launch: ") + hipGetErrorString(e));

    if (opts && opts->kernel_begin && hipEventRecord(opts->kernel_begin, stream) != hipSuccess)
        return fail(OSCAR_ERR_HIP, "hipEventRecord failed");
    const int blocks = plan.items * a.batch * a.head_chunks;
    if (xh) {
        // extend: every work item on the matrix cores, a block of new tokens per workgroup
        if (xh->hist_items > 0 && xh->num_slots > 0) {
            e = launch_extend_history(*xh, stream);
            if (e != hipSuccess)
                return fail(OSCAR_ERR_HIP, std::string("extend history launch: ") + hipGetErrorString(e));
        }
        e = launch_extend_bf16(*xh, stream);
        if (e != hipSuccess) return fail(OSCAR_ERR_HIP, std::string("extend bf16 launch: ") + hipGetErrorString(e));
    } else if (head_record_bytes(a.group_size, a.scale_bits) % 16 != 0 && (a.hkv & 1)) {
        // 72-byte records and an odd number of KV heads (a 4-head chunk would
        // end inside a 16-byte unit): the BF16 window items on partial_kernel,
        // the history items on hist_lowmeta_kernel
        const int bf_blocks = a.win_items * a.batch * a.head_chunks;
        DecodeArgs aw = a;
        aw.win_last = 0;                            // this grid holds the window items alone
        switch (a.g) {
            case 1: e = launch_partial<1>(aw, bf_blocks, stream); break;
            case 2: e = launch_partial<2>(aw, bf_blocks, stream); break;
            case 3: e = launch_partial<3>(aw, bf_blocks, stream); break;
            case 4: e = launch_partial<4>(aw, bf_blocks, stream); break;
            case 5: e = launch_partial<5>(aw, bf_blocks, stream); break;
            case 6: e = launch_partial<6>(aw, bf_blocks, stream); break;
            case 7: e = launch_partial<7>(aw, bf_blocks, stream); break;
            default: e = launch_partial<8>(aw, bf_blocks, stream); break;
        }
        if (e != hipSuccess) return fail(OSCAR_ERR_HIP, std::string("partial launch: ") + hipGetErrorString(e));
        const int h_blocks = (plan.items - a.win_items) * a.batch * a.head_chunks;
        if (h_blocks > 0 && a.num_slots > 0) {
            if (a.scale_bits == 8)
                hipLaunchKernelGGL((hist_lowmeta_kernel<2, 2>), dim3(h_blocks), dim3(64 * kPartialWaves), 0, stream, a);
            else
                hipLaunchKernelGGL((hist_lowmeta_kernel<1, 4>), dim3(h_blocks), dim3(64 * kPartialWaves), 0, stream, a);
            e = hipGetLastError();
            if (e != hipSuccess) return fail(OSCAR_ERR_HIP, std::string("history launch: ") + hipGetErrorString(e));
        }
    } else {
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
    }
    if (opts && opts->kernel_end && hipEventRecord(opts->kernel_end, stream) != hipSuccess)
        return fail(OSCAR_ERR_HIP, "hipEventRecord failed");

    if (xh) {
        e = launch_extend_merge(*xh, stream);
        if (e != hipSuccess) return fail(OSCAR_ERR_HIP, std::string("extend merge launch: ") + hipGetErrorString(e));
        return OSCAR_OK;
    }
    hipLaunchKernelGGL(merge_kernel, dim3(a.batch * a.hkv), dim3(512), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(OSCAR_ERR_HIP, std::string("merge launch: ") + hipGetErrorString(e));
    return OSCAR_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// Decode that allocates nothing: the workspace is a file-scope device array.
// Each GPU holds its own copy at its own address, found once per device with
// hipGetSymbolAddress; host code uses only that address, never the array's
// name (which on the host is a stand-in, not a device address).
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[OSCAR_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_at[kMaxScratchDevices] = {};

// address of the current device's copy of `scratch` (set up on first use)
oscar_status scratch_address(void **at) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return fail(OSCAR_ERR_HIP, "hipGetDevice failed");
    if (dev < 0 || dev >= kMaxScratchDevices) return fail(OSCAR_ERR_UNSUPPORTED, "device index beyond 64");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_at[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(OSCAR_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
        g_scratch_at[dev] = p;
    }
    *at = g_scratch_at[dev];
    return OSCAR_OK;
}

}  // namespace

extern "C" oscar_status oscar_decode_attn_noalloc(hipStream_t stream, const oscar_layout *layout,
                                                  const oscar_pool *pool, const void *q, oscar_dtype q_dtype,
                                                  int32_t batch, const int32_t *req_ids,
                                                  const int32_t *seq_lens, const int32_t *seq_lens_host,
                                                  const int32_t *req_to_slot, int64_t req_to_slot_stride,
                                                  const float *R_K, const float *R_V, float sm_scale,
                                                  void *out, oscar_dtype out_dtype,
                                                  const oscar_launch_opts *opts) {
    oscar_status st = check_decode_common(layout, pool, q, q_dtype, req_to_slot, R_K, R_V, sm_scale, out,
                                          out_dtype);
    if (st != OSCAR_OK) return st;
    if (!req_ids || !seq_lens) return fail(OSCAR_ERR_INVALID_ARG, "a required pointer is null");
    DecodePlan plan;
    st = make_decode_plan(*layout, batch, seq_lens_host, opts, &plan);
    if (st != OSCAR_OK) return st;
    if (plan.ws_bytes > OSCAR_NOALLOC_SCRATCH_BYTES)
        return fail(OSCAR_ERR_WORKSPACE, "this batch needs " + std::to_string(plan.ws_bytes) +
                                             " bytes of workspace, more than the " +
                                             std::to_string(size_t(OSCAR_NOALLOC_SCRATCH_BYTES)) +
                                             " bytes of the library's scratch array (use oscar_decode_attn "
                                             "with a workspace)");
    void *ws = nullptr;
    st = scratch_address(&ws);
    if (st != OSCAR_OK) return st;
    st = check_workspace(plan, req_to_slot_stride, ws, OSCAR_NOALLOC_SCRATCH_BYTES);
    if (st != OSCAR_OK) return st;
    DecodeArgs a = make_args(layout, pool, q, q_dtype, batch, req_to_slot, req_to_slot_stride, R_K, R_V,
                             sm_scale, out, out_dtype, ws, plan);
    a.req_ids = req_ids;
    a.seq_lens = seq_lens;
    return launch_decode(a, plan, stream, opts);
}

extern "C" oscar_status oscar_decode_attn(hipStream_t stream, const oscar_layout *layout,
                                          const oscar_pool *pool, const void *q, oscar_dtype q_dtype,
                                          int32_t batch, const int32_t *req_ids,
                                          const int32_t *seq_lens, const int32_t *seq_lens_host,
                                          const int32_t *req_to_slot, int64_t req_to_slot_stride,
                                          const float *R_K, const float *R_V, float sm_scale,
                                          void *out, oscar_dtype out_dtype, void *workspace,
                                          size_t workspace_bytes, const oscar_launch_opts *opts) {
    oscar_status st = check_decode_common(layout, pool, q, q_dtype, req_to_slot, R_K, R_V, sm_scale, out,
                                          out_dtype);
    if (st != OSCAR_OK) return st;
    if (!req_ids || !seq_lens) return fail(OSCAR_ERR_INVALID_ARG, "a required pointer is null");
    DecodePlan plan;
    st = make_decode_plan(*layout, batch, seq_lens_host, opts, &plan);
    if (st != OSCAR_OK) return st;
    st = check_workspace(plan, req_to_slot_stride, workspace, workspace_bytes);
    if (st != OSCAR_OK) return st;
    DecodeArgs a = make_args(layout, pool, q, q_dtype, batch, req_to_slot, req_to_slot_stride, R_K, R_V,
                             sm_scale, out, out_dtype, workspace, plan);
    a.req_ids = req_ids;
    a.seq_lens = seq_lens;
    return launch_decode(a, plan, stream, opts);
}

extern "C" oscar_status oscar_extend_attn(hipStream_t stream, const oscar_layout *layout,
                                          const oscar_pool *pool, const void *q, oscar_dtype q_dtype,
                                          const void *k_new, const void *v_new, oscar_dtype kv_dtype,
                                          int32_t n_new, int32_t req_id, int32_t prefix_len,
                                          const int32_t *req_to_slot, int64_t req_to_slot_stride,
                                          const float *R_K, const float *R_V, float sm_scale,
                                          void *out, oscar_dtype out_dtype, void *workspace,
                                          size_t workspace_bytes, const oscar_launch_opts *opts) {
    oscar_status st = check_decode_common(layout, pool, q, q_dtype, req_to_slot, R_K, R_V, sm_scale, out,
                                          out_dtype);
    if (st != OSCAR_OK) return st;
    if (!k_new || !v_new) return fail(OSCAR_ERR_INVALID_ARG, "a required pointer is null");
    if (kv_dtype != OSCAR_F32 && kv_dtype != OSCAR_BF16 && kv_dtype != OSCAR_F16)
        return fail(OSCAR_ERR_INVALID_ARG, "kv_dtype must be F32, BF16 or F16");
    if (n_new < 1) return fail(OSCAR_ERR_INVALID_ARG, "n_new must be >= 1");
    if (req_id < 0 || req_id >= layout->max_requests)
        return fail(OSCAR_ERR_INVALID_ARG, "req_id must be in [0, max_requests)");
    if (prefix_len < 0) return fail(OSCAR_ERR_INVALID_ARG, "prefix_len must be >= 0");
    if (int64_t(prefix_len) + n_new > int64_t(INT32_MAX))
        return fail(OSCAR_ERR_INVALID_ARG, "prefix_len + n_new must fit int32");
    if (int64_t(n_new) * layout->num_kv_heads * 2 > INT32_MAX)
        return fail(OSCAR_ERR_UNSUPPORTED, "n_new x KV heads exceeds one launch grid");
    const std::vector<int32_t> lens(size_t(n_new), prefix_len);
    DecodePlan plan;
    st = make_decode_plan(*layout, n_new, lens.data(), opts, &plan, true);
    if (st != OSCAR_OK) return st;
    st = check_workspace(plan, req_to_slot_stride, workspace, workspace_bytes);
    if (st != OSCAR_OK) return st;
    DecodeArgs a = make_args(layout, pool, q, q_dtype, n_new, req_to_slot, req_to_slot_stride, R_K, R_V,
                             sm_scale, out, out_dtype, workspace, plan);
    a.fixed_req = req_id;
    a.fixed_len = prefix_len;

    // work items on the matrix cores: 256 / g new tokens per history
    // workgroup, 128 / g per workgroup of the BF16 items
    ExtendHistArgs xh;
    xh.records = pool->records;
    xh.slot_row = req_to_slot + size_t(req_id) * req_to_slot_stride;
    xh.zero_rec = a.zero_rec;
    xh.qrot = a.qrot;
    xh.qsum = a.qsum;
    xh.part_o = a.part_o;
    xh.part_ml = a.part_ml;
    xh.num_slots = layout->num_slots;
    xh.hkv = a.hkv;
    xh.hq = a.hq;
    xh.g = a.g;
    xh.items = a.items;
    xh.chunk = a.chunk;
    xh.sink = a.sink_tokens;
    xh.recent = a.recent_tokens;
    xh.prefix_len = prefix_len;
    xh.n_new = n_new;
    xh.tok_per_block = 128 / a.g;
    xh.row_blocks = (n_new + xh.tok_per_block - 1) / xh.tok_per_block;
    xh.hist_tok_per_block = 256 / a.g;
    xh.hist_row_blocks = (n_new + xh.hist_tok_per_block - 1) / xh.hist_tok_per_block;
    xh.hist_items = plan.extra_item - 2;
    xh.sink_store = pool->sink;
    xh.recent_store = pool->recent;
    xh.newkv = a.newkv;
    xh.req = req_id;
    xh.extra_item = plan.extra_item;
    xh.r_v = R_V;
    xh.out = out;
    xh.out_dtype = out_dtype;
    xh.group_size = layout->group_size;
    xh.scale_bits = scale_bits(*layout);
    if (extend_history_blocks(xh) > INT32_MAX || extend_bf16_blocks(xh) > INT32_MAX)
        return fail(OSCAR_ERR_UNSUPPORTED, "new tokens x work items exceeds one launch grid");

    RotateArgs r;
    r.k = k_new;
    r.v = v_new;
    r.r_k = R_K;
    r.r_v = R_V;
    r.out = reinterpret_cast<uint16_t *>(static_cast<uint8_t *>(workspace) + plan.ws_newkv);
    r.hkv = layout->num_kv_heads;
    r.dtype = kv_dtype;
    hipLaunchKernelGGL(extend_rotate_kernel, dim3(n_new * layout->num_kv_heads * 2), dim3(kHeadDim), 0,
                       stream, r);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(OSCAR_ERR_HIP, std::string("rotate launch: ") + hipGetErrorString(e));
    return launch_decode(a, plan, stream, opts, &xh);
}
