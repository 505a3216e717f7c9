// Internal declarations shared by the host code and the kernel launchers of
// liboscar.  Not part of the ABI.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include <hip/hip_runtime.h>

#include "../../include/oscar.h"

namespace oscar {

constexpr int kHeadDim = 128;
constexpr int kGroup = 32;
constexpr int kGroups = kHeadDim / kGroup;          // 4
constexpr int kCodeBytes = kHeadDim / 4;            // 32 bytes of codes per head-vector
constexpr int kSzBytes = 4 * kGroups;               // 16 bytes of (s, z) per head-vector
constexpr int kHeadRecord = 2 * kCodeBytes + 2 * kSzBytes;  // 96
constexpr int kMaxKvHeads = 16;
constexpr int kMaxGroup = 8;                        // query heads per KV head

oscar_status fail(oscar_status st, const std::string &msg);
oscar_status ok();

// Full validation of a layout (shape support included).
oscar_status check_layout(const oscar_layout *lay);

// Bits of each stored scale and zero (0 in the struct means 16).
inline int scale_bits(const oscar_layout &lay) { return lay.scale_bits == 0 ? 16 : lay.scale_bits; }

// Head record of group size G: K codes, V codes, then (s, z) of K and of V per
// group: 96 bytes at G = 32, 80 at 64, 72 at 128 with fp16 (s, z); 72 at
// G = 64 with E4M3 (s, z).
inline int head_record_bytes(int group_size, int sz_bits = 16) {
    return 2 * kCodeBytes + 2 * 2 * (sz_bits / 8) * (kHeadDim / group_size);
}

inline int64_t record_bytes(const oscar_layout &lay) {
    return static_cast<int64_t>(lay.num_kv_heads) * head_record_bytes(lay.group_size, scale_bits(lay));
}

// Decode splits the sink and recent windows into work items of this many
// positions, so that a request's window work runs on several compute units.
constexpr int kWindowItemTokens = 64;

// Decode planning: compute units of the device (MI355X) and split-K workgroups
// that one compute unit holds at once (the history kernel takes 156 registers
// per lane with up to 4 query heads per KV head, three workgroups of 4 waves
// per CU, and over 200 with 5 to 8, two).
constexpr int kDeviceCUs = 256;
inline int decode_workgroups_per_cu(int group) { return group <= 4 ? 3 : 2; }

// Split-K plan of one decode call (pure function of the host lengths).
struct DecodePlan {
    int32_t chunk = 0;           // history tokens per work item
    int32_t items = 0;           // work items per request: sink, recent, chunks
    int32_t sink_items = 1;      // items 0 .. sink_items-1 cover the sink window
    int32_t recent_items = 1;    // the next recent_items cover the recent window
    int32_t max_len = 0;
    size_t ws_qrot = 0;          // byte offsets into the workspace
    size_t ws_qsum = 0;
    size_t ws_part_o = 0;
    size_t ws_part_ml = 0;
    size_t ws_zero = 0;          // 256 bytes the decode clears: stand-in record of unusable tokens
    size_t ws_newkv = 0;         // extend: BF16 rotated K, V of the new tokens
    int32_t extra_item = -1;     // extend: work item of the new tokens (the last one)
    size_t ws_bytes = 0;
};

// Work split and workspace layout of a decode step, or (extend = true) of an
// extend call whose `batch` rows are new tokens reading a prefix of length
// seq_lens_host[row] (which may then be 0) plus the new tokens themselves.
oscar_status make_decode_plan(const oscar_layout &lay, int32_t batch,
                              const int32_t *seq_lens_host, const oscar_launch_opts *opts,
                              DecodePlan *plan, bool extend = false);

// Extend attention on the matrix cores (extend_hist.hip): for every work
// item (history chunks; sink, recent and new-token windows), a workgroup
// takes a block of new tokens of one KV head and writes their split-K
// partials in the decode layout (part_o [rows][items][Hq][128], part_ml
// [rows][items][Hq][2]).
struct ExtendHistArgs {
    const uint8_t *records;
    const int32_t *slot_row;      // req_to_slot row of the request
    const uint8_t *zero_rec;      // 256 zero bytes (cleared before this kernel runs)
    const float *qrot;            // [rows][Hq][128] log2-scaled rotated queries
    const float *qsum;            // [rows][Hq][8]; [4] = 2^K, [5] = 2^(24-K)
    float *part_o;
    float *part_ml;
    int64_t num_slots;
    int32_t hkv;
    int32_t hq;
    int32_t g;
    int32_t items;
    int32_t chunk;
    int32_t sink;
    int32_t recent;
    int32_t prefix_len;
    int32_t n_new;
    int32_t tok_per_block;        // new tokens per workgroup of the BF16 items: 128 / g
    int32_t row_blocks;
    int32_t hist_tok_per_block;   // new tokens per workgroup of the history items: 256 / g
    int32_t hist_row_blocks;
    int32_t hist_items;
    // BF16 items (sink window, recent window, the new tokens themselves)
    const uint16_t *sink_store;   // [max_requests][S][Hkv][2][128]
    const uint16_t *recent_store; // [max_requests][W][Hkv][2][128], row p mod W
    const uint16_t *newkv;        // [n_new][Hkv][2][128] rotated new tokens
    int32_t req;
    int32_t extra_item;           // work item of the new tokens
    // merge and un-rotation
    const float *r_v;             // [Hkv][128][128]
    void *out;                    // [n_new][Hq][128] of out_dtype
    int32_t out_dtype;
    int32_t group_size;
    int32_t scale_bits;           // 16 (fp16 s, z) or 8 (E4M3 s, z)
};
// Grid sizes of the two launches (row blocks x items x hkv).
int64_t extend_history_blocks(const ExtendHistArgs &a);
int64_t extend_bf16_blocks(const ExtendHistArgs &a);
hipError_t launch_extend_history(const ExtendHistArgs &a, hipStream_t stream);
hipError_t launch_extend_bf16(const ExtendHistArgs &a, hipStream_t stream);
hipError_t launch_extend_merge(const ExtendHistArgs &a, hipStream_t stream);

}  // namespace oscar
