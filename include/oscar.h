/*
 * oscar.h - C ABI of the OSCAR INT2 KV-cache hot path for AMD Instinct MI355X
 * (gfx950).
 *
 * The method (Together AI's OSCAR announcement, sections "What OSCAR does
 * differently" and "Serving system: mixed-precision cache layout"):
 *   - every new key head-vector k is rotated by R_K = U_Q H P_br and every
 *     value head-vector v by R_V = U_S H P_br, then clipped, quantised to INT2
 *     with a scale and zero per group of channels, and packed;
 *   - each request's cache has three regions: the first 64 tokens (sink) and
 *     the last 256 tokens (recent) stay in BF16, every token between them
 *     (history) is kept in INT2;
 *   - decode attention rotates the query by R_K, computes the logits in the
 *     rotated basis against the dequantised cache, and brings the output back
 *     with R_V^T.
 *
 * Conventions of this ABI
 *   - Vectors are rows: x' = x R.  Matrices are row-major.
 *   - Every pointer argument of a device-side call is a device pointer on the
 *     current HIP device unless it is marked "host".  The caller owns all
 *     memory; the library never allocates device memory.
 *   - All arguments are validated on the host before any HIP call; invalid
 *     arguments return a status and launch nothing.  Device work is
 *     asynchronous on `stream`; execution faults surface at the caller's
 *     synchronisation.  No call aborts or throws across the ABI.
 *   - Calls are re-entrant.  The only global state is a thread-local error
 *     message (oscar_last_error).  Two calls that write the same pool bytes
 *     concurrently race; serialise them on one stream.
 *   - Supported shapes: head_dim 128, group_size 32, 64 or 128 with fp16
 *     scale/zero, or 64 with E4M3 scale/zero (scale_bits = 8),
 *     1 <= num_kv_heads <= 16, num_q_heads = g * num_kv_heads with
 *     1 <= g <= 8.  Other shapes return OSCAR_ERR_UNSUPPORTED.
 */
#ifndef OSCAR_H
#define OSCAR_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    OSCAR_OK = 0,
    OSCAR_ERR_INVALID_ARG = 1,  /* null pointer, negative size, inconsistent layout */
    OSCAR_ERR_UNSUPPORTED = 2,  /* shape outside the supported set above */
    OSCAR_ERR_WORKSPACE = 3,    /* workspace smaller than oscar_decode_workspace_size */
    OSCAR_ERR_HIP = 4,          /* a HIP launch or query failed */
    OSCAR_ERR_NUMERIC = 5       /* eigensolver did not converge */
} oscar_status;

typedef enum {
    OSCAR_F32 = 0,
    OSCAR_BF16 = 1,
    OSCAR_F16 = 2,
    /* Not formats.  They make every int32 value a value of this type, so that
       an out-of-range argument from a C caller is a defined value that the
       library rejects with OSCAR_ERR_INVALID_ARG (in C++ an enum's values are
       otherwise only those its enumerators' bits can hold). */
    OSCAR_DTYPE_RANGE_MIN_ = INT32_MIN,
    OSCAR_DTYPE_RANGE_MAX_ = INT32_MAX
} oscar_dtype;

/* Shape of one attention layer's cache. */
typedef struct {
    int32_t head_dim;       /* d; must be 128 */
    int32_t group_size;     /* G, channels per scale/zero group: 32, 64 or 128 */
    int32_t num_kv_heads;   /* Hkv, 1..16 */
    int32_t num_q_heads;    /* Hq = g * Hkv, 1 <= g <= 8 */
    int32_t sink_tokens;    /* S, BF16 sink window (the pages use 64); 0..4096 */
    int32_t recent_tokens;  /* W, BF16 recent window (the pages use 256); 1..4096 */
    int64_t num_slots;      /* INT2 pool capacity in tokens (page_size = 1) */
    int32_t max_requests;   /* rows of the sink/recent stores */
    int32_t scale_bits;     /* bits of each stored scale and zero: 16 (fp16) or
                               8 (E4M3, G = 64 only); 0 means 16 */
} oscar_layout;

/*
 * Cache storage.  Byte formats (little endian):
 *
 * records: [num_slots][Hkv * B] bytes, B = 64 + 8 * (128 / G) (96 at G = 32,
 *   80 at 64, 72 at 128; the smaller metadata is the lower bits per element
 *   of the OSCAR page's summary).  The record of a slot holds one B-byte
 *   head record per KV head, head h at byte B h, n_g = 128 / G:
 *     [0, 32)   K codes      [32, 64)  V codes
 *     [64, 64 + 4 n_g)  K (s, z)     [64 + 4 n_g, 64 + 8 n_g)  V (s, z)
 *   Codes: the 128 rotated channels, 2 bits each, four per byte, least
 *   significant bits first: byte j holds channels 4j .. 4j+3 at bit offsets
 *   0, 2, 4, 6.  (s, z): for each of the n_g groups of G contiguous rotated
 *   channels, fp16 scale s then fp16 zero z.  Element value = s * code + z.
 *   With scale_bits = 8 (G = 64) each (s, z) is two E4M3 codes instead, s
 *   first (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; largest
 *   finite value 448, only S.1111.111 is NaN), so B = 72:
 *     [64, 68)  K (s0, z0, s1, z1)     [68, 72)  V (s0, z0, s1, z1)
 *   The quantiser rounds s and z to E4M3 to nearest (ties to even),
 *   saturating at +-448, then picks codes against the rounded values.
 * sink:    [max_requests][S][Hkv][2][128] bf16 (2 = K, V), rotated basis,
 *          position p < S at index p.
 * recent:  [max_requests][W][Hkv][2][128] bf16 ring, rotated basis,
 *          position p at index p mod W.
 */
typedef struct {
    uint8_t *records;
    uint16_t *sink;
    uint16_t *recent;
} oscar_pool;

/* Optional launch controls (pass NULL for defaults). */
typedef struct {
    /* If non-null, recorded on `stream` immediately before and after the
       dominant kernel of the call (decode: the split-K partial kernel;
       append: the rotate/quantise kernel), for live per-kernel timing. */
    hipEvent_t kernel_begin;
    hipEvent_t kernel_end;
    /* Decode only: history tokens per split-K work item (multiple of 32,
       32..65536); 0 = chosen from the sequence lengths. */
    int32_t history_chunk;
    /* Append only: tokens per workgroup (multiple of 32); 0 = automatic. */
    int32_t append_chunk;
} oscar_launch_opts;

/* Returns OSCAR_OK if `layout` is valid and supported, else the status and
   a message in oscar_last_error(). */
oscar_status oscar_layout_check(const oscar_layout *layout);

/* Bytes of one part of the storage: part 0 = records, 1 = sink, 2 = recent.
   Returns 0 for an invalid layout or part. */
size_t oscar_pool_bytes(const oscar_layout *layout, int32_t part);

/*
 * oscar_build_rotation (host only, fp64).
 *
 * R = U H P for a symmetric d x d covariance `cov` (host, row-major), where
 *   U: eigenvectors of cov (Together AI OSCAR page, "What OSCAR does
 *      differently": U_Q from C_Q = (1/N) sum q_n^T q_n for keys, U_S from
 *      C_S = (1/N) V^T S^T S V for values), eigenvalues in descending order,
 *      each column signed so that its largest-magnitude entry is positive
 *      (first index on ties);
 *   H: Sylvester Hadamard matrix / sqrt(d) (Qiita article, "Fix 3");
 *   P: bit-reversal permutation of the channel index, (x P)[rev(i)] = x[i],
 *      which gives every contiguous group one channel of every importance tier.
 * flags select the factors: OSCAR_ROT_EIG | OSCAR_ROT_HAD | OSCAR_ROT_PBR is
 * OSCAR; OSCAR_ROT_HAD alone a data-independent Hadamard rotation; 0 the
 * identity.  cov is read only if OSCAR_ROT_EIG is set.  d: power of two,
 * 1..1024.  R_out: host, d*d doubles.  eigvals_out: host, d doubles or NULL
 * (descending eigenvalues; zeros if OSCAR_ROT_EIG is not set).
 * Eigenvectors come from the cyclic Jacobi method; it stops when a sweep finds
 * every off-diagonal entry negligible next to its diagonal pair or the
 * off-diagonal norm is below 1e-15 of the matrix norm (at most 100 sweeps,
 * else OSCAR_ERR_NUMERIC).  A non-finite or non-symmetric (beyond 1e-12
 * relative) cov returns OSCAR_ERR_INVALID_ARG.
 */
#define OSCAR_ROT_EIG 1u
#define OSCAR_ROT_HAD 2u
#define OSCAR_ROT_PBR 4u
#define OSCAR_ROT_OSCAR 7u
oscar_status oscar_build_rotation(const double *cov, int32_t d, uint32_t flags,
                                  double *R_out, double *eigvals_out);

/*
 * oscar_quant_append: rotate, clip, quantise and route n new tokens
 * (Together AI OSCAR page, "Serving system": INT2 after rotation and
 * clipping; BF16 sink and recent windows).
 *
 * k, v:          [n_tokens][Hkv][128] of in_dtype (F32, BF16 or F16).
 * req_ids:       [n_tokens] int32, row of the sink/recent stores, < max_requests.
 * positions:     [n_tokens] int32 >= 0, position of the token in its request.
 * slots:         [n_tokens] int32, INT2 pool slot, < num_slots (ignored for
 *                positions < S).
 * seq_len_after: [max_requests] int32, cache length of each request once this
 *                call's tokens are in (decides the recent window).
 * R_K, R_V:      [Hkv][128][128] fp32 rotations.
 * clip_ratio:    alpha in (0, 1]; 1 disables clipping.
 * rotated_out:   NULL or [n_tokens][Hkv][2][128] fp32: the rotated values
 *                x' = fl32(x R) (for testing).
 * Per token and tensor: x' = x R in fp32; then per group of 32 channels
 *   lo, hi = min, max of x'; lo_c = fl32(alpha lo) if lo < 0 else lo;
 *   hi_c = fl32(alpha hi) if hi > 0 else hi; x_c = min(max(x', lo_c), hi_c);
 *   s = fp16_rn(fl32((hi_c - lo_c) / 3)); z = fp16_rn(lo_c);
 *   code = #{k in 0,1,2 : x_c >= z + (k + 1/2) s} (exact), 0 if s == 0.
 * Routing: p < S -> sink[req][p] = bf16_rn(x'); p >= S -> the slot's record;
 *   p >= S and p >= seq_len_after[req] - W -> also recent[req][p mod W].
 * Tokens whose req_id, position or (for p >= S) slot is out of range are
 * skipped.  Tokens of one call must not share a slot or a (req, position).
 */
oscar_status oscar_quant_append(hipStream_t stream, const oscar_layout *layout,
                                const oscar_pool *pool, const void *k, const void *v,
                                oscar_dtype in_dtype, int32_t n_tokens,
                                const int32_t *req_ids, const int32_t *positions,
                                const int32_t *slots, const int32_t *seq_len_after,
                                const float *R_K, const float *R_V, float clip_ratio,
                                float *rotated_out, const oscar_launch_opts *opts);

/*
 * Workspace bytes that oscar_decode_attn needs for this batch.
 * seq_lens_host: host, [batch] int32 >= 1.  opts may be NULL.
 */
oscar_status oscar_decode_workspace_size(const oscar_layout *layout, int32_t batch,
                                         const int32_t *seq_lens_host,
                                         const oscar_launch_opts *opts, size_t *bytes);

/*
 * oscar_decode_attn: one decode step of attention for `batch` requests.
 *
 * q:             [batch][Hq][128] of q_dtype (F32, BF16 or F16).
 * req_ids:       [batch] int32, rows of the stores and of req_to_slot.
 * seq_lens:      [batch] int32, cache length L of each request (device copy).
 * seq_lens_host: host, [batch] int32, the same lengths (used for planning;
 *                if they differ from seq_lens the output is undefined but all
 *                accesses stay in bounds).
 * req_to_slot:   [max_requests][req_to_slot_stride] int32 slot ids per
 *                position (page_size = 1); entries for history positions
 *                [S, L - W) are read, out-of-range slot ids are skipped.
 * R_K, R_V:      [Hkv][128][128] fp32.
 * sm_scale:      logit scale (1/sqrt(128) is the usual choice).
 * out:           [batch][Hq][128] of out_dtype (F32, BF16 or F16).
 * workspace:     >= oscar_decode_workspace_size bytes, 256-byte aligned.
 * Computes, for q head h reading KV head h / g (Qiita article, "Fix 4"):
 *   q' = q R_K; logits over sink [0, min(S, L)), history [S, max(S, L - W))
 *   (dequantised INT2) and recent [max(S, L - W), L) (BF16); softmax;
 *   o' = sum_p softmax_p v'_p; out = o' R_V^T.
 */
oscar_status oscar_decode_attn(hipStream_t stream, const oscar_layout *layout,
                               const oscar_pool *pool, const void *q, oscar_dtype q_dtype,
                               int32_t batch, const int32_t *req_ids,
                               const int32_t *seq_lens, const int32_t *seq_lens_host,
                               const int32_t *req_to_slot, int64_t req_to_slot_stride,
                               const float *R_K, const float *R_V, float sm_scale,
                               void *out, oscar_dtype out_dtype, void *workspace,
                               size_t workspace_bytes, const oscar_launch_opts *opts);

/*
 * oscar_decode_attn_noalloc: the same decode step for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Arguments, computation and results are
 * those of oscar_decode_attn (bit for bit: the same kernels and plan); the
 * workspace is instead a device array inside the library, one per GPU, of
 * OSCAR_NOALLOC_SCRATCH_BYTES (32 MiB; the 32 x 100K-token batch of
 * 32 q / 8 KV heads needs about 9.6 MB, oscar_decode_workspace_size tells any
 * other), held by each GPU the library runs on until the process ends.
 * A batch whose workspace would exceed it returns OSCAR_ERR_WORKSPACE and
 * launches nothing; a larger history_chunk in opts makes fewer work items and
 * a smaller workspace (a ragged batch of 64 requests up to 131K tokens, 24 q /
 * 4 KV heads, needs 52 MB with the default plan and fits with 8192).  The call makes no allocation (no hipMalloc, hipFree or
 * allocating library routine); its first use on a device looks up that
 * device's array address (hipGetSymbolAddress) once.  Every call on one GPU
 * shares its array, so calls that overlap on one GPU (different streams, or
 * threads without ordering) race and may return wrong results; serialise
 * them, e.g. on one stream.
 */
#define OSCAR_NOALLOC_SCRATCH_BYTES (32u << 20)
oscar_status oscar_decode_attn_noalloc(hipStream_t stream, const oscar_layout *layout,
                                       const oscar_pool *pool, const void *q, oscar_dtype q_dtype,
                                       int32_t batch, const int32_t *req_ids,
                                       const int32_t *seq_lens, const int32_t *seq_lens_host,
                                       const int32_t *req_to_slot, int64_t req_to_slot_stride,
                                       const float *R_K, const float *R_V, float sm_scale,
                                       void *out, oscar_dtype out_dtype,
                                       const oscar_launch_opts *opts);

/* Split-K plan that oscar_decode_attn uses: history tokens per work item and
   work items per request: ceil(sink_tokens / 64) items of the sink window (at
   least one), ceil(recent_tokens / 64) of the recent window, then the history
   chunks.  Items of 64 positions let one request's window attention run on
   several compute units. */
oscar_status oscar_decode_plan(const oscar_layout *layout, int32_t batch,
                               const int32_t *seq_lens_host,
                               const oscar_launch_opts *opts, int32_t *history_chunk,
                               int32_t *items_per_request);

/*
 * Workspace bytes that oscar_extend_attn needs for n_new new tokens over a
 * prefix of prefix_len tokens.  opts may be NULL.
 */
oscar_status oscar_extend_workspace_size(const oscar_layout *layout, int32_t n_new, int32_t prefix_len,
                                         const oscar_launch_opts *opts, size_t *bytes);

/*
 * oscar_extend_attn: attention of n_new new tokens of one request (a
 * prefill or extend chunk) over the request's cached prefix and, causally,
 * over themselves.  Follows the prefill path that the Qiita article (its first
 * pitfall, INT2 KV using memory outside the pool) and its KV-pool follow-up
 * (section on the buffer that is not the pool) describe: each chunk attends to
 * the whole cached prefix, which those pages expand to dense 16-bit outside
 * the pool before attention.  Here the stored prefix is read in place, with
 * dequantisation fused into the attention, so no buffer grows with P.
 *
 * q:             [n_new][Hq][128] of q_dtype (F32, BF16 or F16); row i is
 *                the new token at position prefix_len + i.
 * k_new, v_new:  [n_new][Hkv][128] of kv_dtype (F32, BF16 or F16), the new
 *                tokens' raw keys and values.
 * req_id:        the request's row of the stores and of req_to_slot.
 * prefix_len:    cached tokens before the chunk (>= 0).  The prefix is read
 *                as the pool holds it at that length: sink [0, min(S, P))
 *                and recent [max(S, P - W), P) BF16, history [S, P - W) INT2.
 *                Call this before oscar_quant_append of the same tokens (the
 *                append overwrites the recent ring).
 * req_to_slot:   as for oscar_decode_attn; the stride must cover prefix_len.
 * out:           [n_new][Hq][128] of out_dtype.
 * workspace:     >= oscar_extend_workspace_size bytes, 256-byte aligned.
 * Computes, for new token i and q head h reading KV head h / g: keys and
 *   values of positions [0, P) from the prefix as stored, and of new tokens
 *   0 .. i as bf16_rn(x R) (x R formed in fp32); softmax over all of them
 *   with q' = q R_K; out = o' R_V^T.
 */
oscar_status oscar_extend_attn(hipStream_t stream, const oscar_layout *layout,
                               const oscar_pool *pool, const void *q, oscar_dtype q_dtype,
                               const void *k_new, const void *v_new, oscar_dtype kv_dtype,
                               int32_t n_new, int32_t req_id, int32_t prefix_len,
                               const int32_t *req_to_slot, int64_t req_to_slot_stride,
                               const float *R_K, const float *R_V, float sm_scale,
                               void *out, oscar_dtype out_dtype, void *workspace,
                               size_t workspace_bytes, const oscar_launch_opts *opts);

/*
 * BF16 paged KV cache: the baseline that the OSCAR announcement's "Results"
 * section measures its decode speed-up and batch-32 throughput against.  The
 * same page_size-1 slots hold every token's K and V in BF16, unrotated:
 *   kv_pool: [num_slots][Hkv][2][128] bf16 bits (K then V of each KV head),
 *            oscar_bf16_pool_bytes(layout) bytes, caller-owned.
 * Only head_dim, num_kv_heads, num_q_heads, num_slots and max_requests of the
 * layout matter here (it must still pass oscar_layout_check).
 */
size_t oscar_bf16_pool_bytes(const oscar_layout *layout);   /* 0 if the layout is invalid */

/*
 * oscar_bf16_append: kv_pool[slots[i]][h][0] = bf16_rn(k[i][h]),
 * kv_pool[slots[i]][h][1] = bf16_rn(v[i][h]) for every token i and KV head h.
 * k, v: [n_tokens][Hkv][128] of dtype (F32, BF16 or F16).  Slots outside
 * [0, num_slots) are skipped.  n_tokens = 0 is a no-op.  Asynchronous on
 * `stream`.
 */
oscar_status oscar_bf16_append(hipStream_t stream, const oscar_layout *layout, uint16_t *kv_pool,
                               const void *k, const void *v, oscar_dtype dtype, int32_t n_tokens,
                               const int32_t *slots);

/* Workspace bytes oscar_bf16_decode_attn needs for these lengths.  opts may be NULL. */
oscar_status oscar_bf16_decode_workspace_size(const oscar_layout *layout, int32_t batch,
                                              const int32_t *seq_lens_host,
                                              const oscar_launch_opts *opts, size_t *bytes);

/*
 * oscar_bf16_decode_attn: o[b][h] = softmax(sm_scale q[b][h] K^T) V over the
 * positions [0, L_b) of request req_ids[b], K and V rows read from the slots
 * req_to_slot[req][p] (tokens with a slot outside [0, num_slots) are left
 * out), query head h reading KV head h / g.  No rotation.  Arguments as for
 * oscar_decode_attn; history_chunk in opts sets the positions per work item
 * (a multiple of 32).  Requires num_slots >= 1.
 */
oscar_status oscar_bf16_decode_attn(hipStream_t stream, const oscar_layout *layout,
                                    const uint16_t *kv_pool, const void *q, oscar_dtype q_dtype,
                                    int32_t batch, const int32_t *req_ids, const int32_t *seq_lens,
                                    const int32_t *seq_lens_host, const int32_t *req_to_slot,
                                    int64_t req_to_slot_stride, float sm_scale, void *out,
                                    oscar_dtype out_dtype, void *workspace, size_t workspace_bytes,
                                    const oscar_launch_opts *opts);

/*
 * Calibration statistics (OSCAR page, "What OSCAR does differently"): the
 * key basis comes from the query covariance C_Q = (1/N) sum q^T q and the
 * value basis from C_S = (1/N) V^T S^T S V = (1/N) sum o^T o over the
 * attention outputs o = S V.  Both are Gram sums of 128-wide rows, the g
 * query heads of a KV head pooled into its rows.
 *
 * oscar_covariance_accumulate: acc[h] += sum over n < n_rows and the query
 * heads q of KV head h of x[n][q]^T x[n][q] (128 x 128, row-major).
 *   x:    [n_rows][Hq][128] of dtype (F32, BF16 or F16), device.
 *   acc:  [Hkv][128][128] fp64, device, accumulated into (the caller zeroes
 *         it first and divides by the row count, n_rows * g, at the end).
 *   workspace: >= oscar_covariance_workspace_size bytes, 256-byte aligned.
 * Products are exact in fp32 (fp32 matrix cores), each slab of rows sums in
 * fp32 and the slabs add in fp64.  n_rows = 0 is a no-op.  Asynchronous.
 */
oscar_status oscar_covariance_workspace_size(const oscar_layout *layout, int64_t n_rows, size_t *bytes);
oscar_status oscar_covariance_accumulate(hipStream_t stream, const oscar_layout *layout, const void *x,
                                         oscar_dtype dtype, int64_t n_rows, double *acc, void *workspace,
                                         size_t workspace_bytes);

/*
 * oscar_gather_read_reference: a measurement reference, not a step of the
 * method.  Reads whole rows of `rows` ([num_rows][row_bytes], device, 16-byte
 * aligned; row_bytes = 768, the slot-major record of 8 KV heads of 96-byte
 * head records) at the row indices idx[0..n-1] (device int32; an index
 * outside 0..num_rows-1 reads the last row), 16 bytes per load with the
 * non-temporal policy, and writes one XOR of what it read per thread to
 * `sink` (device, OSCAR_GATHER_REF_SINK_WORDS uint32).  It is the access
 * pattern of the INT2 history stream of oscar_decode_attn (OSCAR page,
 * "Serving system": a token-granular pool read through the request's index
 * table) with no arithmetic, so its rate bounds what that stream can reach on
 * the device.  Asynchronous on `stream`; invalid arguments return a status
 * and launch nothing.
 */
#define OSCAR_GATHER_REF_SINK_WORDS (2048 * 256)
oscar_status oscar_gather_read_reference(hipStream_t stream, const void *rows, int64_t row_bytes,
                                         int64_t num_rows, const int32_t *idx, int64_t n, uint32_t *sink,
                                         int64_t sink_words);

/* Thread-local message of the last non-OK status of this thread. */
const char *oscar_last_error(void);

/* Library version string. */
const char *oscar_version(void);

#ifdef __cplusplus
}
#endif

#endif /* OSCAR_H */
