// Host-side part of liboscar: error reporting, layout validation, storage
// sizes, the split-K planner and oscar_build_rotation (fp64 cyclic Jacobi).
#include <algorithm>
#include <cmath>
#include <cstring>
#include <string>
#include <vector>

#include "internal.h"

namespace oscar {

namespace {
thread_local std::string g_last_error;
}

oscar_status fail(oscar_status st, const std::string &msg) {
    g_last_error = msg;
    return st;
}

oscar_status ok() { return OSCAR_OK; }

oscar_status check_layout(const oscar_layout *lay) {
    if (!lay) return fail(OSCAR_ERR_INVALID_ARG, "layout is null");
    if (lay->head_dim <= 0 || lay->group_size <= 0 || lay->num_kv_heads <= 0 ||
        lay->num_q_heads <= 0)
        return fail(OSCAR_ERR_INVALID_ARG, "head_dim, group_size and head counts must be > 0");
    if (lay->head_dim != kHeadDim)
        return fail(OSCAR_ERR_UNSUPPORTED, "head_dim must be 128");
    if (lay->head_dim % lay->group_size != 0)
        return fail(OSCAR_ERR_INVALID_ARG, "group_size must divide head_dim");
    if (lay->group_size != 32 && lay->group_size != 64 && lay->group_size != 128)
        return fail(OSCAR_ERR_UNSUPPORTED, "group_size must be 32, 64 or 128");
    if (lay->scale_bits != 0 && lay->scale_bits != 16 && lay->scale_bits != 8)
        return fail(OSCAR_ERR_INVALID_ARG, "scale_bits must be 16 or 8 (0 means 16)");
    if (lay->scale_bits == 8 && lay->group_size != 64)
        return fail(OSCAR_ERR_UNSUPPORTED, "8-bit scale/zero needs group_size 64");
    if (lay->num_q_heads % lay->num_kv_heads != 0)
        return fail(OSCAR_ERR_INVALID_ARG, "num_q_heads must be a multiple of num_kv_heads");
    if (lay->num_kv_heads > kMaxKvHeads)
        return fail(OSCAR_ERR_UNSUPPORTED, "num_kv_heads must be <= 16");
    if (lay->num_q_heads / lay->num_kv_heads > kMaxGroup)
        return fail(OSCAR_ERR_UNSUPPORTED, "at most 8 query heads per KV head");
    if (lay->sink_tokens < 0 || lay->sink_tokens > 4096)
        return fail(OSCAR_ERR_INVALID_ARG, "sink_tokens must be in [0, 4096]");
    if (lay->recent_tokens < 1 || lay->recent_tokens > 4096)
        return fail(OSCAR_ERR_INVALID_ARG, "recent_tokens must be in [1, 4096]");
    if (lay->num_slots < 0 || lay->num_slots > (int64_t(1) << 40))
        return fail(OSCAR_ERR_INVALID_ARG, "num_slots must be in [0, 2^40]");
    if (lay->num_slots > int64_t(INT32_MAX))
        return fail(OSCAR_ERR_UNSUPPORTED, "slot ids are int32: num_slots <= 2^31-1");
    if (lay->max_requests < 1) return fail(OSCAR_ERR_INVALID_ARG, "max_requests must be >= 1");
    return OSCAR_OK;
}

oscar_status make_decode_plan(const oscar_layout &lay, int32_t batch,
                              const int32_t *seq_lens_host, const oscar_launch_opts *opts,
                              DecodePlan *plan, bool extend) {
    if (batch < 1) return fail(OSCAR_ERR_INVALID_ARG, "batch must be >= 1");
    if (!seq_lens_host) return fail(OSCAR_ERR_INVALID_ARG, "seq_lens_host is null");
    const int64_t S = lay.sink_tokens, W = lay.recent_tokens;
    int64_t max_hist = 0, max_len = 0;
    for (int32_t b = 0; b < batch; ++b) {
        const int64_t L = seq_lens_host[b];
        if (L < (extend ? 0 : 1))
            return fail(OSCAR_ERR_INVALID_ARG, extend ? "prefix_len must be >= 0" : "every sequence length must be >= 1");
        const int64_t hist = std::max<int64_t>(0, std::max(S, L - W) - S);
        max_hist = std::max(max_hist, hist);
        max_len = std::max(max_len, L);
    }
    int64_t chunk = 0;
    if (opts && opts->history_chunk) {
        chunk = opts->history_chunk;
        if (chunk < 32 || chunk > 65536 || chunk % 32)
            return fail(OSCAR_ERR_INVALID_ARG, "history_chunk must be a multiple of 32 in [32, 65536]");
    } else if (extend) {
        // every row reads the same prefix and a history workgroup serves
        // 256 / g new tokens: about 2048 history workgroups (eight rounds of
        // one per compute unit) in total, so that few partials go through the merge
        const int64_t g = lay.num_q_heads / lay.num_kv_heads;
        const int64_t row_blocks = (batch + 256 / g - 1) / (256 / g);
        const int64_t want = std::max<int64_t>(1, (2048 + row_blocks * lay.num_kv_heads - 1) /
                                                      (row_blocks * lay.num_kv_heads));
        chunk = (max_hist + want - 1) / want;
        chunk = std::max<int64_t>(256, (chunk + 31) / 32 * 32);
    } else {
        // Rounds of the workgroups the device holds at once.  When every
        // request has the same number of nearly full history items (a uniform
        // batch), one round: its items start and end together, and the short
        // window items, last in the grid, fill the compute units the history
        // items leave idle.  Otherwise four rounds, so that the partial last
        // items of ragged requests leave small gaps.  Each case takes the
        // smallest chunk (a multiple of 32, at least 256) whose items fit.
        const int64_t head_chunks = (lay.num_kv_heads + 3) / 4;
        const int64_t g = lay.num_q_heads / lay.num_kv_heads;
        const int64_t resident =
            std::max<int64_t>(1, int64_t(kDeviceCUs) * decode_workgroups_per_cu(int(g)) / head_chunks);
        auto items_for = [&](int64_t c) {
            int64_t n = 0;
            for (int32_t b = 0; b < batch; ++b) {
                const int64_t hist = std::max<int64_t>(0, std::max(S, int64_t(seq_lens_host[b]) - W) - S);
                n += (hist + c - 1) / c;
            }
            return n;
        };
        const int64_t c_max = std::max<int64_t>(256, (max_hist + 31) / 32 * 32);
        // the fewest rounds any chunk allows (more than one only when the batch
        // has more requests than the device holds workgroups)
        const int64_t rounds = std::max<int64_t>(1, (items_for(c_max) + resident - 1) / resident);
        auto chunk_for = [&](int64_t n_rounds) {   // smallest chunk whose items fit n_rounds
            int64_t lo = 256 / 32, hi = c_max / 32;   // in units of 32 positions
            while (lo < hi) {
                const int64_t mid = (lo + hi) / 2;
                if (items_for(32 * mid) <= n_rounds * resident)
                    hi = mid;
                else
                    lo = mid + 1;
            }
            return 32 * lo;
        };
        chunk = chunk_for(rounds);
        int64_t per_request = -1, hist_sum = 0, n_items = 0;
        bool uniform = true;
        for (int32_t b = 0; b < batch; ++b) {
            const int64_t hist = std::max<int64_t>(0, std::max(S, int64_t(seq_lens_host[b]) - W) - S);
            if (hist == 0) continue;
            const int64_t k = (hist + chunk - 1) / chunk;
            uniform = uniform && (per_request < 0 || k == per_request);
            per_request = k;
            hist_sum += hist;
            n_items += k;
        }
        if (!uniform || 10 * hist_sum < 9 * n_items * chunk) chunk = chunk_for(4 * rounds);
    }
    // decode: windows in items of kWindowItemTokens positions; extend: one item each
    const int64_t sink_items = extend ? 1 : std::max<int64_t>(1, (S + kWindowItemTokens - 1) / kWindowItemTokens);
    const int64_t recent_items = extend ? 1 : (W + kWindowItemTokens - 1) / kWindowItemTokens;
    const int64_t items = sink_items + recent_items + (max_hist + chunk - 1) / chunk + (extend ? 1 : 0);
    const int64_t hq = lay.num_q_heads;
    auto align = [](size_t x) { return (x + 255) / 256 * 256; };
    plan->chunk = static_cast<int32_t>(chunk);
    plan->items = static_cast<int32_t>(items);
    plan->sink_items = static_cast<int32_t>(sink_items);
    plan->recent_items = static_cast<int32_t>(recent_items);
    plan->max_len = static_cast<int32_t>(max_len);
    size_t off = 0;
    plan->ws_qrot = off;
    off += align(size_t(batch) * hq * kHeadDim * sizeof(float));
    plan->ws_qsum = off;
    off += align(size_t(batch) * hq * 8 * sizeof(float));
    plan->ws_part_o = off;
    off += align(size_t(batch) * items * hq * kHeadDim * sizeof(float));
    plan->ws_part_ml = off;
    off += align(size_t(batch) * items * hq * 2 * sizeof(float));
    plan->ws_zero = off;
    off += 256;
    if (extend) {
        plan->extra_item = static_cast<int32_t>(items - 1);
        plan->ws_newkv = off;
        off += align(size_t(batch) * lay.num_kv_heads * 2 * kHeadDim * sizeof(uint16_t));
    }
    plan->ws_bytes = off;
    return OSCAR_OK;
}

namespace {

// Cyclic Jacobi eigen-decomposition of a symmetric matrix (row-major a[n*n],
// overwritten).  On return the diagonal of `a` holds the eigenvalues and the
// columns of v the eigenvectors.  Returns false if it did not converge.
bool jacobi_eigen(std::vector<double> &a, std::vector<double> &v, int n) {
    v.assign(size_t(n) * n, 0.0);
    for (int i = 0; i < n; ++i) v[size_t(i) * n + i] = 1.0;
    double fro = 0.0;
    for (double x : a) fro += x * x;
    fro = std::sqrt(fro);
    if (fro == 0.0) return true;
    for (int sweep = 0; sweep < 100; ++sweep) {
        double off = 0.0;
        for (int p = 0; p < n; ++p)
            for (int q = 0; q < n; ++q)
                if (p != q) off += a[size_t(p) * n + q] * a[size_t(p) * n + q];
        if (std::sqrt(off) <= 1e-15 * fro) return true;
        bool rotated = false;
        for (int p = 0; p < n - 1; ++p) {
            for (int q = p + 1; q < n; ++q) {
                double &apq = a[size_t(p) * n + q];
                const double app = a[size_t(p) * n + p], aqq = a[size_t(q) * n + q];
                if (apq == 0.0) continue;
                // negligible next to both diagonal entries: set to zero
                if (std::fabs(app) + 100.0 * std::fabs(apq) == std::fabs(app) &&
                    std::fabs(aqq) + 100.0 * std::fabs(apq) == std::fabs(aqq)) {
                    apq = 0.0;
                    a[size_t(q) * n + p] = 0.0;
                    continue;
                }
                rotated = true;
                // t = tan(phi) of the rotation that zeroes a_pq
                const double theta = (aqq - app) / (2.0 * apq);
                const double t = (theta >= 0 ? 1.0 : -1.0) /
                                 (std::fabs(theta) + std::sqrt(theta * theta + 1.0));
                const double c = 1.0 / std::sqrt(t * t + 1.0);
                const double s = t * c;
                const double apq_v = apq;
                for (int k = 0; k < n; ++k) {
                    if (k == p || k == q) continue;
                    const double akp = a[size_t(k) * n + p], akq = a[size_t(k) * n + q];
                    const double nkp = c * akp - s * akq, nkq = s * akp + c * akq;
                    a[size_t(k) * n + p] = nkp;
                    a[size_t(p) * n + k] = nkp;
                    a[size_t(k) * n + q] = nkq;
                    a[size_t(q) * n + k] = nkq;
                }
                a[size_t(p) * n + p] = app - t * apq_v;
                a[size_t(q) * n + q] = aqq + t * apq_v;
                a[size_t(p) * n + q] = 0.0;
                a[size_t(q) * n + p] = 0.0;
                for (int k = 0; k < n; ++k) {
                    const double vkp = v[size_t(k) * n + p], vkq = v[size_t(k) * n + q];
                    v[size_t(k) * n + p] = c * vkp - s * vkq;
                    v[size_t(k) * n + q] = s * vkp + c * vkq;
                }
            }
        }
        if (!rotated) return true;
    }
    return false;
}

int bit_reverse(int i, int bits) {
    int r = 0;
    for (int b = 0; b < bits; ++b) {
        r = (r << 1) | (i & 1);
        i >>= 1;
    }
    return r;
}

}  // namespace
}  // namespace oscar

using namespace oscar;

extern "C" {

const char *oscar_last_error(void) { return g_last_error.c_str(); }

const char *oscar_version(void) { return "oscar-int2-kv 0.1 (gfx950)"; }

oscar_status oscar_layout_check(const oscar_layout *layout) { return check_layout(layout); }

size_t oscar_pool_bytes(const oscar_layout *layout, int32_t part) {
    if (check_layout(layout) != OSCAR_OK) return 0;
    const size_t hkv = size_t(layout->num_kv_heads);
    switch (part) {
        case 0: return size_t(layout->num_slots) * size_t(record_bytes(*layout));
        case 1: return size_t(layout->max_requests) * layout->sink_tokens * hkv * 2 * kHeadDim * 2;
        case 2: return size_t(layout->max_requests) * layout->recent_tokens * hkv * 2 * kHeadDim * 2;
        default: fail(OSCAR_ERR_INVALID_ARG, "part must be 0, 1 or 2"); return 0;
    }
}

oscar_status oscar_build_rotation(const double *cov, int32_t d, uint32_t flags, double *R_out,
                                  double *eigvals_out) {
    if (d < 1 || d > 1024 || (d & (d - 1)) != 0)
        return fail(OSCAR_ERR_INVALID_ARG, "d must be a power of two in [1, 1024]");
    if (flags & ~OSCAR_ROT_OSCAR) return fail(OSCAR_ERR_INVALID_ARG, "unknown rotation flag");
    if (!R_out) return fail(OSCAR_ERR_INVALID_ARG, "R_out is null");
    const size_t n = size_t(d);
    std::vector<double> u(n * n, 0.0), evals(n, 0.0);
    for (size_t i = 0; i < n; ++i) u[i * n + i] = 1.0;
    if (flags & OSCAR_ROT_EIG) {
        if (!cov) return fail(OSCAR_ERR_INVALID_ARG, "cov is null");
        double scale = 0.0;
        for (size_t i = 0; i < n * n; ++i) {
            if (!std::isfinite(cov[i])) return fail(OSCAR_ERR_INVALID_ARG, "cov is not finite");
            scale = std::max(scale, std::fabs(cov[i]));
        }
        std::vector<double> a(n * n);
        for (size_t i = 0; i < n; ++i)
            for (size_t j = 0; j < n; ++j) {
                const double x = cov[i * n + j], y = cov[j * n + i];
                if (std::fabs(x - y) > 1e-12 * scale)
                    return fail(OSCAR_ERR_INVALID_ARG, "cov is not symmetric");
                a[i * n + j] = 0.5 * (x + y);
            }
        std::vector<double> v;
        if (!jacobi_eigen(a, v, d))
            return fail(OSCAR_ERR_NUMERIC, "Jacobi eigensolver did not converge in 100 sweeps");
        // sort descending by eigenvalue (stable on ties)
        std::vector<int> order(n);
        for (size_t i = 0; i < n; ++i) order[i] = int(i);
        std::stable_sort(order.begin(), order.end(),
                         [&](int x, int y) { return a[size_t(x) * n + x] > a[size_t(y) * n + y]; });
        for (size_t c = 0; c < n; ++c) {
            const size_t src = size_t(order[c]);
            evals[c] = a[src * n + src];
            // sign: the entry of largest magnitude is positive (first on ties)
            size_t lead = 0;
            double best = -1.0;
            for (size_t r = 0; r < n; ++r) {
                const double m = std::fabs(v[r * n + src]);
                if (m > best) { best = m; lead = r; }
            }
            const double sgn = v[lead * n + src] < 0 ? -1.0 : 1.0;
            for (size_t r = 0; r < n; ++r) u[r * n + c] = sgn * v[r * n + src];
        }
    }
    if (flags & OSCAR_ROT_HAD) {
        // each row of U times the Sylvester Hadamard matrix (fast Walsh-Hadamard
        // butterfly on the row), then divide by sqrt(d)
        const double norm = 1.0 / std::sqrt(double(d));
        for (size_t r = 0; r < n; ++r) {
            double *row = &u[r * n];
            for (size_t h = 1; h < n; h <<= 1)
                for (size_t i = 0; i < n; i += 2 * h)
                    for (size_t j = i; j < i + h; ++j) {
                        const double x = row[j], y = row[j + h];
                        row[j] = x + y;
                        row[j + h] = x - y;
                    }
            for (size_t j = 0; j < n; ++j) row[j] *= norm;
        }
    }
    if (flags & OSCAR_ROT_PBR) {
        int bits = 0;
        while ((1 << bits) < d) ++bits;
        std::vector<double> row(n);
        for (size_t r = 0; r < n; ++r) {
            for (size_t j = 0; j < n; ++j) row[size_t(bit_reverse(int(j), bits))] = u[r * n + j];
            std::memcpy(&u[r * n], row.data(), n * sizeof(double));
        }
    }
    std::memcpy(R_out, u.data(), n * n * sizeof(double));
    if (eigvals_out) std::memcpy(eigvals_out, evals.data(), n * sizeof(double));
    return OSCAR_OK;
}

oscar_status oscar_decode_workspace_size(const oscar_layout *layout, int32_t batch,
                                         const int32_t *seq_lens_host,
                                         const oscar_launch_opts *opts, size_t *bytes) {
    oscar_status st = check_layout(layout);
    if (st != OSCAR_OK) return st;
    if (!bytes) return fail(OSCAR_ERR_INVALID_ARG, "bytes is null");
    DecodePlan plan;
    st = make_decode_plan(*layout, batch, seq_lens_host, opts, &plan);
    if (st != OSCAR_OK) return st;
    *bytes = plan.ws_bytes;
    return OSCAR_OK;
}

oscar_status oscar_extend_workspace_size(const oscar_layout *layout, int32_t n_new, int32_t prefix_len,
                                         const oscar_launch_opts *opts, size_t *bytes) {
    oscar_status st = check_layout(layout);
    if (st != OSCAR_OK) return st;
    if (!bytes) return fail(OSCAR_ERR_INVALID_ARG, "bytes is null");
    if (n_new < 1) return fail(OSCAR_ERR_INVALID_ARG, "n_new must be >= 1");
    const std::vector<int32_t> lens(size_t(n_new), prefix_len);
    DecodePlan plan;
    st = make_decode_plan(*layout, n_new, lens.data(), opts, &plan, true);
    if (st != OSCAR_OK) return st;
    *bytes = plan.ws_bytes;
    return OSCAR_OK;
}

oscar_status oscar_decode_plan(const oscar_layout *layout, int32_t batch,
                               const int32_t *seq_lens_host, const oscar_launch_opts *opts,
                               int32_t *history_chunk, int32_t *items_per_request) {
    oscar_status st = check_layout(layout);
    if (st != OSCAR_OK) return st;
    DecodePlan plan;
    st = make_decode_plan(*layout, batch, seq_lens_host, opts, &plan);
    if (st != OSCAR_OK) return st;
    if (history_chunk) *history_chunk = plan.chunk;
    if (items_per_request) *items_per_request = plan.items;
    return OSCAR_OK;
}

}  // extern "C"
