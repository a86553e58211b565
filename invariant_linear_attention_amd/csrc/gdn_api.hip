// gdn_api.hip -- the C ABI (include/gdn.h): argument checks, launch planning and
// dispatch to the per-dk kernels.  Everything here runs on the host before any work
// is enqueued; nothing here reads device memory, allocates or synchronises.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "gdn.h"
#include "gdn_internal.hpp"

namespace gdn {
namespace {

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void *p, uint64_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, a + static_cast<uintptr_t>(bytes)};
}

bool overlap(Range a, Range b) {
    if (a.lo == a.hi || b.lo == b.hi || a.lo == 0 || b.lo == 0) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void *p, uintptr_t to) { return (reinterpret_cast<uintptr_t>(p) % to) == 0; }

bool dk_supported(int dk) { return dk == 16 || dk == 32 || dk == 64 || dk == 128; }

bool plan_available(int dk, bool decode, int io, Plan plan) {
    switch (dk) {
        case 16: return plan_available_dk16(decode, io, plan);
        case 32: return plan_available_dk32(decode, io, plan);
        case 64: return plan_available_dk64(decode, io, plan);
        case 128: return plan_available_dk128(decode, io, plan);
        default: return false;
    }
}

int rows_per_group(Plan plan) { return plan.waves * (64 / plan.lanes) * plan.rows; }

bool plan_fits(int dk, int dv, bool decode, int io, Plan plan) {
    return plan.lanes > 0 && plan.rows > 0 && plan.waves > 0 && plan_available(dk, decode, io, plan) &&
           dv % rows_per_group(plan) == 0;
}

// Automatic launch shape.  Rows are independent, so this only trades per-wave
// efficiency against parallelism.  Measured on MI355X (dk = dv = 128, bf16): 8
// lanes x 1 row per lane is fastest when the batch has rows to spare, then 16
// lanes x 2 rows; when rows are scarce (one long sequence) 16 lanes x 1 row puts
// the most waves on the chip.  Smaller heads take the same order over the shapes
// compiled for them (dk = 64: 8 or 4 lanes per row; dk = 16, 32: 4).
constexpr int64_t kWavesWanted = 4096;  // four per SIMD: lets longest-first ordering balance the tail

Plan auto_plan(int dk, int dv, bool decode, int io, int64_t units) {
    const int64_t rows_total = units * dv;
    if (decode) {
        // One row per lane and one wave per workgroup: the state stream is the whole
        // cost, and this shape measured fastest at B = 64 and 256 and gives small
        // batches the most workgroups.
        for (Plan pl : {Plan{4, 1, 1}, Plan{4, 1, 2}, Plan{4, 2, 1}})
            if (plan_fits(dk, dv, true, io, pl)) return pl;
        return Plan{4, 1, 1};
    }
    const Plan prefer[] = {Plan{8, 1, 4}, Plan{16, 2, 4}, Plan{16, 1, 4}, Plan{8, 1, 2}, Plan{4, 1, 4},
                           Plan{4, 1, 2}, Plan{4, 1, 1}, Plan{16, 1, 2}, Plan{8, 1, 1}};
    Plan best{0, 0, 0};
    int64_t best_waves = -1;
    for (Plan pl : prefer) {
        if (!plan_fits(dk, dv, false, io, pl)) continue;
        const int64_t waves = rows_total * pl.lanes / (64 * pl.rows);
        if (waves >= kWavesWanted) return pl;
        if (waves > best_waves) {  // otherwise keep the shape with the most waves
            best = pl;
            best_waves = waves;
        }
    }
    return best_waves >= 0 ? best : Plan{4, 1, 1};
}

gdn_status check_common(const gdn_dims *d) {
    if (!d) return GDN_ERR_NULL;
    if (d->reserved != 0) return GDN_ERR_SHAPE;
    if (d->n_seqs < 0 || d->total_tokens < 0 || d->hk <= 0 || d->hv <= 0 || d->dk <= 0 || d->dv <= 0)
        return GDN_ERR_SHAPE;
    if (d->hv % d->hk != 0 || d->dv % 16 != 0) return GDN_ERR_SHAPE;
    if (d->io_dtype != GDN_F32 && d->io_dtype != GDN_BF16) return GDN_ERR_DTYPE;
    if (!dk_supported(d->dk)) return GDN_ERR_UNSUPPORTED;
    if (d->hv > 65535 || d->n_seqs > 65535) return GDN_ERR_SHAPE;  // decode grid y / z limits
    if (const gdn_preproc *pre = d->pre) {
        if (pre->flags & ~(GDN_PRE_QK_L2NORM | GDN_PRE_GATE_LOGITS)) return GDN_ERR_UNSUPPORTED;
        if (!isfinite(pre->eps) || pre->eps < 0.f) return GDN_ERR_SHAPE;
        if ((pre->flags & GDN_PRE_GATE_LOGITS) && !pre->A_log) return GDN_ERR_NULL;
        if (!aligned(pre->A_log, 4) || !aligned(pre->dt_bias, 4)) return GDN_ERR_ALIGN;
    }
    return GDN_OK;
}

// Device arrays the preprocessing reads (A_log, dt_bias), for the alias checks.
Range pre_range(const gdn_dims *d, int which) {
    const gdn_preproc *pre = d->pre;
    if (!pre || !(pre->flags & GDN_PRE_GATE_LOGITS)) return Range{0, 0};
    return range_of(which == 0 ? pre->A_log : pre->dt_bias, (uint64_t)d->hv * 4);
}

template <class Params>
void apply_pre(const gdn_dims *d, Params &p) {
    if (const gdn_preproc *pre = d->pre) {
        p.pre_flags = pre->flags;
        p.pre_eps = pre->eps;
        if (pre->flags & GDN_PRE_GATE_LOGITS) {
            p.A_log = pre->A_log;
            p.dt_bias = pre->dt_bias;
        }
    }
}

gdn_status resolve_plan(const gdn_dims *d, bool decode, int64_t units, Plan *plan) {
    const Plan a = auto_plan(d->dk, d->dv, decode, d->io_dtype, units);
    if (d->plan_lanes == 0 && d->plan_rows == 0 && d->plan_waves == 0) {
        if (!plan_fits(d->dk, d->dv, decode, d->io_dtype, a)) return GDN_ERR_UNSUPPORTED;
        *plan = a;
        return GDN_OK;
    }
    // Partly pinned: fill the free fields from the automatic shape where it fits.
    Plan p{d->plan_lanes ? d->plan_lanes : (decode ? 4 : a.lanes), d->plan_rows ? d->plan_rows : a.rows,
           d->plan_waves};
    if (d->plan_rows == 0 && !plan_fits(d->dk, d->dv, decode, d->io_dtype, Plan{p.lanes, p.rows, 1})) p.rows = 1;
    if (p.waves == 0) {
        for (int w : {a.waves, 4, 2, 1, 8})
            if (plan_fits(d->dk, d->dv, decode, d->io_dtype, Plan{p.lanes, p.rows, w})) {
                p.waves = w;
                break;
            }
        if (p.waves == 0) return GDN_ERR_UNSUPPORTED;
    }
    if (!plan_fits(d->dk, d->dv, decode, d->io_dtype, p)) return GDN_ERR_UNSUPPORTED;
    *plan = p;
    return GDN_OK;
}

hipError_t dispatch_prefill(int dk, const PrefillParams &p, int io, Plan plan, hipStream_t s) {
    switch (dk) {
        case 16: return launch_prefill_dk16(p, io, plan, s);
        case 32: return launch_prefill_dk32(p, io, plan, s);
        case 64: return launch_prefill_dk64(p, io, plan, s);
        default: return launch_prefill_dk128(p, io, plan, s);
    }
}

hipError_t dispatch_decode(int dk, const DecodeParams &p, int io, Plan plan, hipStream_t s) {
    switch (dk) {
        case 16: return launch_decode_dk16(p, io, plan, s);
        case 32: return launch_decode_dk32(p, io, plan, s);
        case 64: return launch_decode_dk64(p, io, plan, s);
        default: return launch_decode_dk128(p, io, plan, s);
    }
}

}  // namespace
namespace {

// Planning and launch shared by both varlen entry points (arguments already checked).
gdn_status launch_varlen(const gdn_dims *dims, PrefillParams &p, void *stream) {
    const gdn_dims &d = *dims;
    const int64_t T = d.total_tokens, N = d.n_seqs;
    Plan plan;
    const gdn_status st = resolve_plan(dims, false, N * d.hv, &plan);
    if (st != GDN_OK) return st;
    p.total_tokens = T; p.n_seqs = (int32_t)N; p.hk = d.hk; p.hv = d.hv; p.dv = d.dv;
    // Longest-first ordering pays off when there are a few sequences of some length.
    p.rank_by_length = (N > 1 && N <= kMaxRankedSeqs && T >= 32 * N) ? 1 : 0;
    const hipError_t e = dispatch_prefill(d.dk, p, d.io_dtype, plan, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

}  // namespace
}  // namespace gdn

namespace gdn {
namespace {
gdn_status fwd_varlen(const gdn_dims *dims, const void *q, const void *k, const void *v, const float *g,
                      const float *beta, const float *h0, const int32_t *cu_seqlens, void *out, float *hT,
                      float *save_p, void *stream) {
    gdn_status st = check_common(dims);
    if (st != GDN_OK) return st;
    const gdn_dims &d = *dims;
    const int64_t T = d.total_tokens, N = d.n_seqs;
    if (N == 0) return T == 0 ? GDN_OK : GDN_ERR_SHAPE;
    if (!cu_seqlens) return GDN_ERR_NULL;
    if (T > 0 && (!q || !k || !v || !g || !beta || !out)) return GDN_ERR_NULL;

    const uint64_t esz = d.io_dtype == GDN_BF16 ? 2 : 4;
    const uint64_t qk_bytes = (uint64_t)T * d.hk * d.dk * esz;
    const uint64_t vo_bytes = (uint64_t)T * d.hv * d.dv * esz;
    const uint64_t gb_bytes = (uint64_t)T * d.hv * 4;
    const uint64_t s_bytes = (uint64_t)N * d.hv * d.dv * d.dk * 4;

    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(h0, 16) ||
        !aligned(hT, 16) || !aligned(save_p, 4) || !aligned(g, 4) || !aligned(beta, 4) || !aligned(cu_seqlens, 4))
        return GDN_ERR_ALIGN;

    const Range rq = range_of(q, qk_bytes), rk = range_of(k, qk_bytes), rv = range_of(v, vo_bytes);
    const Range rg = range_of(g, gb_bytes), rb = range_of(beta, gb_bytes);
    const Range rh0 = range_of(h0, h0 ? s_bytes : 0), rhT = range_of(hT, hT ? s_bytes : 0);
    const Range rcu = range_of(cu_seqlens, (uint64_t)(N + 1) * 4), ro = range_of(out, vo_bytes);
    const Range rp = range_of(save_p, save_p ? (uint64_t)T * d.hv * d.dv * 4 : 0);
    const Range ra = pre_range(dims, 0), rdb = pre_range(dims, 1);
    for (Range in : {rq, rk, rv, rg, rb, rh0, rcu, rhT, ra, rdb, rp})
        if (overlap(ro, in)) return GDN_ERR_ALIAS;
    for (Range in : {rq, rk, rv, rg, rb, rcu, ra, rdb, rp})
        if (overlap(rhT, in)) return GDN_ERR_ALIAS;
    for (Range in : {rq, rk, rv, rg, rb, rh0, rcu, ra, rdb})
        if (overlap(rp, in)) return GDN_ERR_ALIAS;
    if (h0 && hT && h0 != hT && overlap(rh0, rhT)) return GDN_ERR_ALIAS;

    PrefillParams p{};
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta; p.h0 = h0;
    p.cu_seqlens = cu_seqlens; p.out = out; p.hT = hT;
    p.pool_size = (int32_t)N;
    p.save_p = save_p;
    apply_pre(dims, p);
    return launch_varlen(dims, p, stream);
}
}  // namespace
}  // namespace gdn

extern "C" {

gdn_status gdn_fwd_varlen(const gdn_dims *dims, const void *q, const void *k, const void *v, const float *g,
                          const float *beta, const float *h0, const int32_t *cu_seqlens, void *out, float *hT,
                          void *stream) {
    return gdn::fwd_varlen(dims, q, k, v, g, beta, h0, cu_seqlens, out, hT, nullptr, stream);
}

gdn_status gdn_fwd_varlen_train(const gdn_dims *dims, const void *q, const void *k, const void *v, const float *g,
                                const float *beta, const float *h0, const int32_t *cu_seqlens, void *out, float *hT,
                                float *saved_p, void *stream) {
    if (dims && dims->pre) return GDN_ERR_UNSUPPORTED;
    if (dims && dims->total_tokens > 0 && !saved_p) return GDN_ERR_NULL;
    return gdn::fwd_varlen(dims, q, k, v, g, beta, h0, cu_seqlens, out, hT, saved_p, stream);
}

gdn_status gdn_fwd_varlen_pool(const gdn_dims *dims, const void *q, const void *k, const void *v, const float *g,
                               const float *beta, const int32_t *cu_seqlens, float *state_pool,
                               const int32_t *src_idx, const int32_t *dst_idx, const int32_t *pos0,
                               const int32_t *snap_idx, int32_t snap_block, int32_t snap_per_seq, void *out,
                               void *stream) {
    using namespace gdn;
    gdn_status st = check_common(dims);
    if (st != GDN_OK) return st;
    const gdn_dims &d = *dims;
    const int64_t T = d.total_tokens, N = d.n_seqs;
    if (d.pool_size <= 0 || snap_block < 0 || snap_per_seq < 0) return GDN_ERR_SHAPE;
    if (snap_block > 0 && (snap_block % kSnapshotGranule != 0 || snap_per_seq == 0)) return GDN_ERR_SHAPE;
    if (N == 0) return T == 0 ? GDN_OK : GDN_ERR_SHAPE;
    if (!cu_seqlens || !state_pool) return GDN_ERR_NULL;
    if (snap_block > 0 && !snap_idx) return GDN_ERR_NULL;
    if (T > 0 && (!q || !k || !v || !g || !beta || !out)) return GDN_ERR_NULL;

    const uint64_t esz = d.io_dtype == GDN_BF16 ? 2 : 4;
    const uint64_t qk_bytes = (uint64_t)T * d.hk * d.dk * esz;
    const uint64_t vo_bytes = (uint64_t)T * d.hv * d.dv * esz;
    const uint64_t gb_bytes = (uint64_t)T * d.hv * 4;
    const uint64_t pool_bytes = (uint64_t)d.pool_size * d.hv * d.dv * d.dk * 4;
    const uint64_t idx_bytes = (uint64_t)N * 4;

    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(state_pool, 16) ||
        !aligned(g, 4) || !aligned(beta, 4) || !aligned(cu_seqlens, 4) || !aligned(src_idx, 4) ||
        !aligned(dst_idx, 4) || !aligned(pos0, 4) || !aligned(snap_idx, 4))
        return GDN_ERR_ALIGN;

    const Range rq = range_of(q, qk_bytes), rk = range_of(k, qk_bytes), rv = range_of(v, vo_bytes);
    const Range rg = range_of(g, gb_bytes), rb = range_of(beta, gb_bytes);
    const Range rp = range_of(state_pool, pool_bytes), rcu = range_of(cu_seqlens, (uint64_t)(N + 1) * 4);
    const Range rs = range_of(src_idx, src_idx ? idx_bytes : 0), rd = range_of(dst_idx, dst_idx ? idx_bytes : 0);
    const Range r0 = range_of(pos0, pos0 ? idx_bytes : 0);
    const Range rn = range_of(snap_idx, snap_block > 0 ? idx_bytes * (uint64_t)snap_per_seq : 0);
    const Range ro = range_of(out, vo_bytes);
    const Range ra = pre_range(dims, 0), rdb = pre_range(dims, 1);
    for (Range in : {rq, rk, rv, rg, rb, rp, rcu, rs, rd, r0, rn, ra, rdb})
        if (overlap(ro, in)) return GDN_ERR_ALIAS;
    for (Range in : {rq, rk, rv, rg, rb, rcu, rs, rd, r0, rn, ra, rdb})
        if (overlap(rp, in)) return GDN_ERR_ALIAS;

    PrefillParams p{};
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta;
    p.h0 = state_pool; p.hT = state_pool; p.snap = state_pool;
    p.cu_seqlens = cu_seqlens; p.out = out;
    p.src_idx = src_idx; p.dst_idx = dst_idx; p.pos0 = pos0;
    // Without an index array the slot is the sequence index: the pool must hold them.
    if ((!src_idx || !dst_idx) && d.pool_size < N) return GDN_ERR_SHAPE;
    p.pool_size = d.pool_size;
    if (snap_block > 0) {
        p.snap_idx = snap_idx; p.snap_block = snap_block; p.snap_per_seq = snap_per_seq;
    }
    apply_pre(dims, p);
    return launch_varlen(dims, p, stream);
}

gdn_status gdn_decode_step(const gdn_dims *dims, const void *q, const void *k, const void *v, const float *g,
                           const float *beta, float *state_pool, const int32_t *state_idx, void *out,
                           void *stream) {
    using namespace gdn;
    gdn_status st = check_common(dims);
    if (st != GDN_OK) return st;
    const gdn_dims &d = *dims;
    const int64_t B = d.n_seqs;
    if (d.total_tokens != B) return GDN_ERR_SHAPE;
    if (d.pool_size < 0) return GDN_ERR_SHAPE;
    if (B == 0) return GDN_OK;
    if (!q || !k || !v || !g || !beta || !out || !state_pool) return GDN_ERR_NULL;
    if (d.pool_size == 0 && !state_idx) return GDN_ERR_SHAPE;
    if (!state_idx && d.pool_size < B) return GDN_ERR_SHAPE;  // identity map needs B entries

    const uint64_t esz = d.io_dtype == GDN_BF16 ? 2 : 4;
    const uint64_t qk_bytes = (uint64_t)B * d.hk * d.dk * esz;
    const uint64_t vo_bytes = (uint64_t)B * d.hv * d.dv * esz;
    const uint64_t gb_bytes = (uint64_t)B * d.hv * 4;
    const uint64_t pool_bytes = (uint64_t)d.pool_size * d.hv * d.dv * d.dk * 4;

    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(state_pool, 16) ||
        !aligned(g, 4) || !aligned(beta, 4) || !aligned(state_idx, 4))
        return GDN_ERR_ALIGN;

    const Range rq = range_of(q, qk_bytes), rk = range_of(k, qk_bytes), rv = range_of(v, vo_bytes);
    const Range rg = range_of(g, gb_bytes), rb = range_of(beta, gb_bytes);
    const Range rp = range_of(state_pool, pool_bytes), ri = range_of(state_idx, state_idx ? (uint64_t)B * 4 : 0);
    const Range ro = range_of(out, vo_bytes);
    const Range ra = pre_range(dims, 0), rdb = pre_range(dims, 1);
    for (Range in : {rq, rk, rv, rg, rb, rp, ri, ra, rdb})
        if (overlap(ro, in)) return GDN_ERR_ALIAS;
    for (Range in : {rq, rk, rv, rg, rb, ri, ra, rdb})
        if (overlap(rp, in)) return GDN_ERR_ALIAS;

    Plan plan;
    st = resolve_plan(dims, true, B * d.hv, &plan);
    if (st != GDN_OK) return st;

    DecodeParams p{};
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta;
    p.pool = state_pool; p.state_idx = state_idx; p.out = out;
    p.batch = (int32_t)B; p.hk = d.hk; p.hv = d.hv; p.dv = d.dv; p.pool_size = d.pool_size;
    apply_pre(dims, p);
    const hipError_t e = dispatch_decode(d.dk, p, d.io_dtype, plan, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

gdn_status gdn_query_plan(const gdn_dims *dims, int32_t decode, int32_t *shape) {
    using namespace gdn;
    if (!shape) return GDN_ERR_NULL;
    const gdn_status st = check_common(dims);
    if (st != GDN_OK) return st;
    Plan plan;
    const gdn_status sp = resolve_plan(dims, decode != 0, (int64_t)dims->n_seqs * dims->hv, &plan);
    if (sp != GDN_OK) return sp;
    shape[0] = plan.lanes;
    shape[1] = plan.rows;
    shape[2] = plan.waves;
    return GDN_OK;
}

gdn_status gdn_short_conv(const gdn_conv_dims *dims, const void *x, const float *w, const float *bias,
                          const int32_t *cu_seqlens, void *state_pool, const int32_t *src_idx,
                          const int32_t *dst_idx, void *y, void *stream) {
    using namespace gdn;
    if (!dims) return GDN_ERR_NULL;
    const gdn_conv_dims &d = *dims;
    const int64_t T = d.total_tokens, N = d.n_seqs, C = d.channels, K = d.taps;
    if (N < 0 || T < 0 || C <= 0 || K < 2 || K > 8 || d.pool_size <= 0 || N > 65535) return GDN_ERR_SHAPE;
    if (d.flags & ~GDN_CONV_SILU) return GDN_ERR_UNSUPPORTED;
    if (d.io_dtype != GDN_F32 && d.io_dtype != GDN_BF16) return GDN_ERR_DTYPE;
    if (N == 0) return T == 0 ? GDN_OK : GDN_ERR_SHAPE;
    if (!cu_seqlens || !w || !state_pool) return GDN_ERR_NULL;
    if (T > 0 && (!x || !y)) return GDN_ERR_NULL;
    if ((!src_idx || !dst_idx) && d.pool_size < N) return GDN_ERR_SHAPE;
    if ((T + 15) / 16 * ((C + 255) / 256) > 0xFFFFFFFFll) return GDN_ERR_SHAPE;  // 1-D grid

    const uintptr_t esz = d.io_dtype == GDN_BF16 ? 2 : 4;
    if (C % (16 / esz) != 0) return GDN_ERR_SHAPE;  // whole 16-byte channel vectors
    if (!aligned(x, 16) || !aligned(y, 16) || !aligned(state_pool, 16) || !aligned(w, 4) || !aligned(bias, 4) ||
        !aligned(cu_seqlens, 4) || !aligned(src_idx, 4) || !aligned(dst_idx, 4))
        return GDN_ERR_ALIGN;
    const Range rx = range_of(x, (uint64_t)T * C * esz), ry = range_of(y, (uint64_t)T * C * esz);
    const Range rw = range_of(w, (uint64_t)C * K * 4), rb = range_of(bias, bias ? (uint64_t)C * 4 : 0);
    const Range rp = range_of(state_pool, (uint64_t)d.pool_size * C * (K - 1) * esz);
    const Range rc = range_of(cu_seqlens, (uint64_t)(N + 1) * 4);
    const Range rs = range_of(src_idx, src_idx ? (uint64_t)N * 4 : 0), rd = range_of(dst_idx, dst_idx ? (uint64_t)N * 4 : 0);
    for (Range in : {rx, rw, rb, rp, rc, rs, rd})
        if (overlap(ry, in)) return GDN_ERR_ALIAS;
    for (Range in : {rx, rw, rb, rc, rs, rd})
        if (overlap(rp, in)) return GDN_ERR_ALIAS;

    ConvParams p{};
    p.x = x; p.w = w; p.bias = bias; p.cu_seqlens = cu_seqlens; p.src_idx = src_idx; p.dst_idx = dst_idx;
    p.state = state_pool; p.y = y; p.total_tokens = T; p.n_seqs = (int32_t)N; p.channels = (int32_t)C;
    p.taps = (int32_t)K; p.pool_size = d.pool_size; p.silu = (d.flags & GDN_CONV_SILU) ? 1 : 0;
    const hipError_t e = launch_short_conv(p, d.io_dtype, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

// Dimension checks of the convolution's backward that need no pointer.
static gdn_status conv_bwd_check(const gdn_conv_dims *dims) {
    if (!dims) return GDN_ERR_NULL;
    const gdn_conv_dims &d = *dims;
    if (d.n_seqs < 0 || d.total_tokens < 0 || d.channels <= 0 || d.taps < 2 || d.taps > 8 || d.pool_size <= 0 ||
        d.n_seqs > 65535)
        return GDN_ERR_SHAPE;
    if (d.flags & ~GDN_CONV_SILU) return GDN_ERR_UNSUPPORTED;
    if (d.io_dtype != GDN_F32 && d.io_dtype != GDN_BF16) return GDN_ERR_DTYPE;
    if (d.n_seqs == 0 && d.total_tokens != 0) return GDN_ERR_SHAPE;
    if ((d.total_tokens + 63) / 64 > 0x7FFFFFFFll || (d.channels + 255) / 256 > 65535) return GDN_ERR_SHAPE;
    return GDN_OK;
}

gdn_status gdn_short_conv_backward_workspace_size(const gdn_conv_dims *dims, uint64_t *bytes) {
    using namespace gdn;
    if (!bytes) return GDN_ERR_NULL;
    const gdn_status st = conv_bwd_check(dims);
    if (st != GDN_OK) return st;
    *bytes = conv_bwd_workspace_bytes(dims->total_tokens, dims->channels, dims->taps);
    return GDN_OK;
}

gdn_status gdn_short_conv_backward(const gdn_conv_dims *dims, const void *x, const float *w, const float *bias,
                                   const int32_t *cu_seqlens, const void *state_pool, const int32_t *src_idx,
                                   const float *dy, float *dx, float *dw, float *dbias, float *dstate,
                                   void *workspace, uint64_t workspace_bytes, void *stream) {
    using namespace gdn;
    const gdn_status st = conv_bwd_check(dims);
    if (st != GDN_OK) return st;
    const gdn_conv_dims &d = *dims;
    const int64_t T = d.total_tokens, N = d.n_seqs, C = d.channels, K = d.taps;
    if (!w || !dw) return GDN_ERR_NULL;
    if (N > 0 && (!cu_seqlens || !state_pool)) return GDN_ERR_NULL;
    if (T > 0 && (!x || !dy || !dx)) return GDN_ERR_NULL;
    if (N > 0 && !src_idx && d.pool_size < N) return GDN_ERR_SHAPE;
    const uint64_t ws = conv_bwd_workspace_bytes(T, C, (int)K);
    if (ws > 0 && !workspace) return GDN_ERR_NULL;
    if (workspace_bytes < ws) return GDN_ERR_SHAPE;
    const uintptr_t esz = d.io_dtype == GDN_BF16 ? 2 : 4;
    if (!aligned(x, esz) || !aligned(state_pool, esz) || !aligned(w, 4) || !aligned(bias, 4) ||
        !aligned(cu_seqlens, 4) || !aligned(src_idx, 4) || !aligned(dy, 4) || !aligned(dx, 4) || !aligned(dw, 4) ||
        !aligned(dbias, 4) || !aligned(dstate, 4) || !aligned(workspace, 4))
        return GDN_ERR_ALIGN;
    const Range inputs[] = {range_of(x, (uint64_t)T * C * esz), range_of(w, (uint64_t)C * K * 4),
                            range_of(bias, bias ? (uint64_t)C * 4 : 0),
                            range_of(cu_seqlens, N > 0 ? (uint64_t)(N + 1) * 4 : 0),
                            range_of(state_pool, (uint64_t)d.pool_size * C * (K - 1) * esz),
                            range_of(src_idx, src_idx ? (uint64_t)N * 4 : 0), range_of(dy, (uint64_t)T * C * 4)};
    const Range outputs[] = {range_of(dx, (uint64_t)T * C * 4), range_of(dw, (uint64_t)C * K * 4),
                             range_of(dbias, dbias ? (uint64_t)C * 4 : 0),
                             range_of(dstate, dstate ? (uint64_t)N * C * (K - 1) * 4 : 0),
                             range_of(workspace, ws)};
    for (size_t i = 0; i < 5; ++i) {
        for (const Range &in : inputs)
            if (overlap(outputs[i], in)) return GDN_ERR_ALIAS;
        for (size_t j = i + 1; j < 5; ++j)
            if (overlap(outputs[i], outputs[j])) return GDN_ERR_ALIAS;
    }
    ConvBwdParams p{};
    p.x = x; p.w = w; p.bias = bias; p.cu_seqlens = cu_seqlens; p.src_idx = src_idx; p.state = state_pool;
    p.dy = dy; p.dx = dx; p.dw = dw; p.dbias = dbias; p.dstate = dstate;
    p.partial = static_cast<float *>(workspace);
    p.total_tokens = T; p.n_seqs = (int32_t)N; p.channels = (int32_t)C; p.taps = (int32_t)K;
    p.pool_size = d.pool_size; p.silu = (d.flags & GDN_CONV_SILU) ? 1 : 0;
    const hipError_t e = launch_short_conv_backward(p, d.io_dtype, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

gdn_status gdn_bwd_workspace_size(const gdn_dims *dims, uint64_t *bytes) {
    using namespace gdn;
    if (!bytes) return GDN_ERR_NULL;
    const gdn_status st = check_common(dims);
    if (st != GDN_OK) return st;
    *bytes = backward_workspace(dims->total_tokens, dims->n_seqs, dims->hv, dims->dk, dims->dv).total;
    return GDN_OK;
}

}  // extern "C"

namespace gdn {
namespace {

// Dimension checks of the backward that need no pointer (shared by both entry points).
gdn_status bwd_check_dims(const gdn_dims *dims) {
    gdn_status st = check_common(dims);
    if (st != GDN_OK) return st;
    const gdn_dims &d = *dims;
    if (d.pre || d.plan_lanes || d.plan_rows || d.plan_waves) return GDN_ERR_UNSUPPORTED;
    auto bwd_dim = [](int x) { return x == 32 || x == 64 || x == 128; };
    if (!bwd_dim(d.dk) || !bwd_dim(d.dv)) return GDN_ERR_UNSUPPORTED;
    if (d.n_seqs == 0 && d.total_tokens != 0) return GDN_ERR_SHAPE;
    return GDN_OK;
}

gdn_status bwd_varlen_impl(const gdn_dims *dims, const void *q, const void *k, const void *v, const float *g,
                           const float *beta, const float *h0, const int32_t *cu_seqlens, const void *dout,
                           const float *dhT, const float *saved_p, const float *hT, float *dq, float *dk, float *dv,
                           float *dg, float *dbeta, float *dh0, void *workspace, uint64_t workspace_bytes,
                           void *stream) {
    gdn_status st = bwd_check_dims(dims);
    if (st != GDN_OK) return st;
    const gdn_dims &d = *dims;
    const int64_t T = d.total_tokens, N = d.n_seqs;
    if (N == 0) return GDN_OK;
    if (!cu_seqlens || !workspace) return GDN_ERR_NULL;
    if (T > 0 && (!q || !k || !v || !g || !beta || !dout || !dq || !dk || !dv || !dg || !dbeta))
        return GDN_ERR_NULL;
    if (saved_p && dhT && !hT) return GDN_ERR_NULL;  // <dhT, hT> needs the forward's hT
    const BwdWorkspace ws = backward_workspace(T, N, d.hv, d.dk, d.dv);
    if (workspace_bytes < ws.total) return GDN_ERR_SHAPE;
    if (N * d.hv * (int64_t)(d.dv / 32 > d.dk / 32 ? d.dv / 32 : d.dk / 32) > 0x7FFFFFFFll ||
        (T * d.hk + 3) / 4 > 0x7FFFFFFFll)
        return GDN_ERR_SHAPE;  // 1-D grids

    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(dout, 16) || !aligned(h0, 16) ||
        !aligned(dhT, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(dh0, 16) ||
        !aligned(workspace, 16) || !aligned(saved_p, 16) || !aligned(hT, 16) || !aligned(g, 4) ||
        !aligned(beta, 4) || !aligned(dg, 4) || !aligned(dbeta, 4) || !aligned(cu_seqlens, 4))
        return GDN_ERR_ALIGN;

    const uint64_t esz = d.io_dtype == GDN_BF16 ? 2 : 4;
    const uint64_t qk_n = (uint64_t)T * d.hk * d.dk, vo_n = (uint64_t)T * d.hv * d.dv;
    const uint64_t gb_bytes = (uint64_t)T * d.hv * 4, s_bytes = (uint64_t)N * d.hv * d.dv * d.dk * 4;
    const Range inputs[] = {range_of(q, qk_n * esz), range_of(k, qk_n * esz), range_of(v, vo_n * esz),
                            range_of(g, gb_bytes), range_of(beta, gb_bytes), range_of(h0, h0 ? s_bytes : 0),
                            range_of(cu_seqlens, (uint64_t)(N + 1) * 4), range_of(dout, vo_n * esz),
                            range_of(dhT, dhT ? s_bytes : 0), range_of(saved_p, saved_p ? vo_n * 4 : 0),
                            range_of(hT, hT ? s_bytes : 0)};
    const Range outputs[] = {range_of(dq, qk_n * 4), range_of(dk, qk_n * 4), range_of(dv, vo_n * 4),
                             range_of(dg, gb_bytes), range_of(dbeta, gb_bytes), range_of(dh0, dh0 ? s_bytes : 0),
                             range_of(workspace, ws.total)};
    for (size_t i = 0; i < sizeof(outputs) / sizeof(outputs[0]); ++i) {
        for (const Range &in : inputs)
            if (overlap(outputs[i], in)) return GDN_ERR_ALIAS;
        for (size_t j = i + 1; j < sizeof(outputs) / sizeof(outputs[0]); ++j)
            if (overlap(outputs[i], outputs[j])) return GDN_ERR_ALIAS;
    }

    char *w = static_cast<char *>(workspace);
    BwdParams p{};
    p.q = q; p.k = k; p.v = v; p.dout = dout; p.g = g; p.beta = beta; p.h0 = h0; p.dhT = dhT;
    p.cu_seqlens = cu_seqlens;
    p.grad_q = dq; p.grad_k = dk; p.grad_v = dv; p.grad_g = dg; p.grad_beta = dbeta; p.grad_h0 = dh0;
    p.rbuf = reinterpret_cast<float *>(w + ws.p);
    p.dubuf = reinterpret_cast<float *>(w + ws.du);
    p.dkbuf = reinterpret_cast<float *>(w + ws.dk);
    p.dqbuf = reinterpret_cast<float *>(w + ws.dq);
    p.cbuf = reinterpret_cast<float *>(w + ws.c);
    p.hT = reinterpret_cast<float *>(w + ws.hT);
    p.saved_p = saved_p;
    if (saved_p) p.hT = const_cast<float *>(hT);  // F0 is skipped: <dhT, hT> reads the caller's hT
    p.total_tokens = T; p.n_seqs = (int32_t)N; p.hk = d.hk; p.hv = d.hv; p.dk = d.dk; p.dv = d.dv;
    p.rank_by_length = (N > 1 && N <= kMaxRankedSeqs && T >= 32 * N) ? 1 : 0;
    const hipError_t e = launch_backward(p, d.io_dtype, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

// The allocation-free backward's workspace: one fixed array per device, resident
// for the life of the process.  Host code never passes `scratch` itself to a
// kernel (on the host that name is only a stand-in); it takes the array's device
// address from hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_addr[kMaxDevices];

// Device address of the current device's scratch array, or null on a HIP error.
void *scratch_address() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void *ptr = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (ptr) return ptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_addr[dev].store(ptr, std::memory_order_release);  // every thread finds the same address
    return ptr;
}

}  // namespace
}  // namespace gdn

extern "C" {

gdn_status gdn_bwd_varlen(const gdn_dims *dims, const void *q, const void *k, const void *v, const float *g,
                          const float *beta, const float *h0, const int32_t *cu_seqlens, const void *dout,
                          const float *dhT, const float *saved_p, const float *hT, float *dq, float *dk, float *dv,
                          float *dg, float *dbeta, float *dh0, void *workspace, uint64_t workspace_bytes,
                          void *stream) {
    return gdn::bwd_varlen_impl(dims, q, k, v, g, beta, h0, cu_seqlens, dout, dhT, saved_p, hT, dq, dk, dv, dg, dbeta,
                                dh0, workspace, workspace_bytes, stream);
}

gdn_status gdn_bwd_varlen_noalloc(const gdn_dims *dims, const void *q, const void *k, const void *v, const float *g,
                                  const float *beta, const float *h0, const int32_t *cu_seqlens, const void *dout,
                                  const float *dhT, const float *saved_p, const float *hT, float *dq, float *dk,
                                  float *dv, float *dg, float *dbeta, float *dh0, void *stream) {
    using namespace gdn;
    // Sizes first, on the host only: a call that would not fit is refused before
    // any HIP call.
    gdn_status st = bwd_check_dims(dims);
    if (st != GDN_OK) return st;
    if (dims->n_seqs == 0) return GDN_OK;
    const BwdWorkspace ws = backward_workspace(dims->total_tokens, dims->n_seqs, dims->hv, dims->dk, dims->dv);
    if (ws.total > (uint64_t)GDN_NOALLOC_SCRATCH_BYTES) return GDN_ERR_CAPACITY;
    void *ptr = scratch_address();
    if (!ptr) return GDN_ERR_HIP;
    return bwd_varlen_impl(dims, q, k, v, g, beta, h0, cu_seqlens, dout, dhT, saved_p, hT, dq, dk, dv, dg, dbeta,
                           dh0, ptr, (uint64_t)GDN_NOALLOC_SCRATCH_BYTES, stream);
}

gdn_status gdn_chunked_workspace_size(const gdn_dims *dims, uint64_t *bytes) {
    using namespace gdn;
    if (!bytes) return GDN_ERR_NULL;
    const gdn_status st = check_common(dims);
    if (st != GDN_OK) return st;
    *bytes = (uint64_t)chunk_ws_slots(dims->total_tokens, dims->n_seqs) * dims->hv * kChunkRec * 4;
    return GDN_OK;
}

gdn_status gdn_fwd_chunked(const gdn_dims *dims, const void *q, const void *k, const void *v, const float *g,
                           const float *beta, const int32_t *cu_seqlens, const gdn_chunk_state *in,
                           const gdn_chunk_state *out, void *o, void *workspace, uint64_t workspace_bytes,
                           void *stream) {
    using namespace gdn;
    gdn_status st = check_common(dims);
    if (st != GDN_OK) return st;
    const gdn_dims &d = *dims;
    if (d.pre || d.plan_lanes || d.plan_rows) return GDN_ERR_UNSUPPORTED;
    if (d.plan_waves != 0 && d.plan_waves != 1 && d.plan_waves != 2 && d.plan_waves != 4) return GDN_ERR_UNSUPPORTED;
    if ((d.dk != 64 && d.dk != 128) || d.dv % 16 != 0 || d.hv / d.hk > 16) return GDN_ERR_UNSUPPORTED;
    const int64_t T = d.total_tokens, N = d.n_seqs;
    if (N == 0) return T == 0 ? GDN_OK : GDN_ERR_SHAPE;
    // cu_seqlens may be NULL only for one token per sequence (T == N): token n is sequence n's
    // only token.
    if ((!cu_seqlens && T != N) || !out || !out->S || !out->k || !out->r || !out->a || !out->b || !out->count ||
        !workspace)
        return GDN_ERR_NULL;
    if (T > 0 && (!q || !k || !v || !g || !beta || !o)) return GDN_ERR_NULL;
    // an incoming state with an open chunk needs its k, r, a and b
    if (in && in->count && (!in->k || !in->r || !in->a || !in->b)) return GDN_ERR_NULL;
    const int64_t slots = chunk_ws_slots(T, N);
    if (workspace_bytes < (uint64_t)slots * d.hv * kChunkRec * 4) return GDN_ERR_SHAPE;
    if (slots > 0x7FFFFFFFll || N * d.hv * (int64_t)(d.dv / 16) > 0x7FFFFFFFll) return GDN_ERR_SHAPE;

    const uint64_t esz = d.io_dtype == GDN_BF16 ? 2 : 4;
    const uint64_t s_bytes = (uint64_t)N * d.hv * d.dv * d.dk * 4;
    const uint64_t k_bytes = (uint64_t)N * GDN_CHUNK * d.hk * d.dk * 4;
    const uint64_t r_bytes = (uint64_t)N * GDN_CHUNK * d.hv * d.dv * 4;
    const uint64_t a_bytes = (uint64_t)N * GDN_CHUNK * d.hv * 4, c_bytes = (uint64_t)N * 4;
    const gdn_chunk_state none{};
    const gdn_chunk_state &i = in ? *in : none;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(g, 4) ||
        !aligned(beta, 4) || !aligned(cu_seqlens, 4) || !aligned(out->S, 16) || !aligned(out->k, 16) ||
        !aligned(out->r, 4) || !aligned(out->a, 4) || !aligned(out->b, 4) || !aligned(out->count, 4) ||
        !aligned(i.S, 16) || !aligned(i.k, 16) || !aligned(i.r, 4) || !aligned(i.a, 4) || !aligned(i.b, 4) ||
        !aligned(i.count, 4) || !aligned(workspace, 16))
        return GDN_ERR_ALIGN;
    // in place: the same S, k, r, a and b arrays, one token per sequence, distinct counts
    const bool inplace = in && i.S == out->S && i.k == out->k && i.r == out->r && i.a == out->a && i.b == out->b;
    if (inplace && (T != N || i.count == out->count)) return GDN_ERR_ALIAS;
    const uint64_t qk_n = (uint64_t)T * d.hk * d.dk, vo_n = (uint64_t)T * d.hv * d.dv;
    const Range ws = range_of(workspace, (uint64_t)slots * d.hv * kChunkRec * 4);
    const Range inputs[] = {range_of(q, qk_n * esz), range_of(k, qk_n * esz), range_of(v, vo_n * esz),
                            range_of(g, (uint64_t)T * d.hv * 4), range_of(beta, (uint64_t)T * d.hv * 4),
                            range_of(cu_seqlens, (uint64_t)(N + 1) * 4),
                            range_of(inplace ? nullptr : i.S, i.S ? s_bytes : 0),
                            range_of(inplace ? nullptr : i.k, i.k ? k_bytes : 0),
                            range_of(inplace ? nullptr : i.r, i.r ? r_bytes : 0),
                            range_of(inplace ? nullptr : i.a, i.a ? a_bytes : 0),
                            range_of(inplace ? nullptr : i.b, i.b ? a_bytes : 0),
                            range_of(i.count, i.count ? c_bytes : 0)};
    const Range outputs[] = {range_of(o, vo_n * esz), range_of(out->S, s_bytes), range_of(out->k, k_bytes),
                             range_of(out->r, r_bytes), range_of(out->a, a_bytes), range_of(out->b, a_bytes),
                             range_of(out->count, c_bytes), ws};
    for (size_t x = 0; x < sizeof(outputs) / sizeof(outputs[0]); ++x) {
        for (const Range &r : inputs)
            if (overlap(outputs[x], r)) return GDN_ERR_ALIAS;
        for (size_t y = x + 1; y < sizeof(outputs) / sizeof(outputs[0]); ++y)
            if (overlap(outputs[x], outputs[y])) return GDN_ERR_ALIAS;
    }

    ChunkedParams p{};
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta; p.cu_seqlens = cu_seqlens;
    p.in_S = i.S; p.in_k = i.k; p.in_r = i.r; p.in_a = i.a; p.in_b = i.b; p.in_count = i.count;
    p.out_S = out->S; p.out_k = out->k; p.out_r = out->r; p.out_a = out->a; p.out_b = out->b;
    p.out_count = out->count;
    p.out = o;
    p.ws = static_cast<float *>(workspace);
    p.ws_slots = slots;
    p.total_tokens = T; p.n_seqs = (int32_t)N; p.hk = d.hk; p.hv = d.hv; p.dk = d.dk; p.dv = d.dv;
    p.rank_by_length = (cu_seqlens && N > 1 && N <= kMaxRankedSeqs && T >= 32 * N) ? 1 : 0;
    p.inplace = inplace ? 1 : 0;
    // Waves per 16-row tile: split the dk quarters over more waves when the call
    // has few tiles to spread over the chip's 1024 SIMDs (never changes a bit).
    const int64_t units = N * d.hv * (int64_t)(d.dv / 16);
    p.waves = d.plan_waves ? d.plan_waves : (units < 1024 ? 4 : (units <= 4096 ? 2 : 1));
    // one token per sequence on average (a decode step): the lean main kernel, whose
    // workgroups are latency-bound on the state read rather than on the chunk walk
    p.lean = T <= N ? 1 : 0;
    const hipError_t e = launch_chunked(p, d.io_dtype, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

}  // extern "C"

namespace gdn {
namespace {

// Workspace of the chunked backward, byte offsets (each 256-byte aligned).
struct BwdChunkWorkspace {
    uint64_t rec, ck, xv, hdot, dq, dk, dbeta, dg, total;
};

// Workgroups per (sequence, value head) in the chunked backward's reverse walk: each
// takes a share of the state rows (dims->plan_rows; 0 = 2 for dv = 128, else 1).
int bwd_chunked_parts(const gdn_dims &d) { return d.plan_rows ? d.plan_rows : (d.dv == 128 ? 2 : 1); }

uint64_t round256(uint64_t x) { return (x + 255) & ~(uint64_t)255; }

BwdChunkWorkspace bwd_chunked_workspace(int64_t T, int64_t N, int hk, int hv, int dk, int dv, int parts) {
    BwdChunkWorkspace w{};
    const uint64_t slots = (uint64_t)chunk_ws_slots(T, N);
    const bool split = hv > hk || parts > 1;  // dq, dk per (value head, part), summed afterwards
    uint64_t o = 0;
    w.rec = o; o = round256(o + slots * hv * kChunkRecBwd * 4);
    w.ck = o; o = round256(o + slots * hv * (uint64_t)dv * dk * 4);
    w.xv = o; o = round256(o + slots * hv * (uint64_t)dv * kChunkLen * 4);  // x: [row][token] tiles per slot
    w.hdot = o; o = round256(o + (uint64_t)N * hv * (dv / 16) * 4 * 4);
    w.dq = o; o = round256(o + (split ? (uint64_t)parts * T * hv * dk * 4 : 0));
    w.dk = o; o = round256(o + (split ? (uint64_t)parts * T * hv * dk * 4 : 0));
    w.dbeta = o; o = round256(o + (parts > 1 ? (uint64_t)parts * T * hv * 4 : 0));
    w.dg = o; o = round256(o + (parts > 1 ? (uint64_t)parts * T * hv * 4 : 0));
    w.total = o;
    return w;
}

gdn_status bwd_chunked_check_dims(const gdn_dims *dims) {
    gdn_status st = check_common(dims);
    if (st != GDN_OK) return st;
    const gdn_dims &d = *dims;
    if (d.pre || (d.plan_lanes != 0 && d.plan_lanes != 1)) return GDN_ERR_UNSUPPORTED;
    if (d.plan_waves != 0 && d.plan_waves != 1 && d.plan_waves != 2 && d.plan_waves != 4) return GDN_ERR_UNSUPPORTED;
    if ((d.dk != 64 && d.dk != 128) || (d.dv != 32 && d.dv != 64 && d.dv != 128) || d.hv / d.hk > 16)
        return GDN_ERR_UNSUPPORTED;
    if (d.plan_rows != 0 && d.plan_rows != 1 && !(d.plan_rows == 2 && d.dv >= 64)) return GDN_ERR_UNSUPPORTED;
    if (d.n_seqs == 0 && d.total_tokens != 0) return GDN_ERR_SHAPE;
    return GDN_OK;
}

}  // namespace
}  // namespace gdn

extern "C" {

gdn_status gdn_bwd_chunked_workspace_size(const gdn_dims *dims, uint64_t *bytes) {
    using namespace gdn;
    if (!bytes) return GDN_ERR_NULL;
    const gdn_status st = bwd_chunked_check_dims(dims);
    if (st != GDN_OK) return st;
    const gdn_dims &d = *dims;
    *bytes = bwd_chunked_workspace(d.total_tokens, d.n_seqs, d.hk, d.hv, d.dk, d.dv, bwd_chunked_parts(d)).total;
    return GDN_OK;
}

gdn_status gdn_bwd_chunked(const gdn_dims *dims, const void *q, const void *k, const void *v, const float *g,
                           const float *beta, const float *h0, const int32_t *cu_seqlens, const void *dout,
                           const float *dhT, float *dq, float *dk, float *dv, float *dg, float *dbeta, float *dh0,
                           void *workspace, uint64_t workspace_bytes, void *stream) {
    using namespace gdn;
    gdn_status st = bwd_chunked_check_dims(dims);
    if (st != GDN_OK) return st;
    const gdn_dims &d = *dims;
    const int64_t T = d.total_tokens, N = d.n_seqs;
    if (N == 0) return GDN_OK;
    if (!cu_seqlens || !workspace) return GDN_ERR_NULL;
    if (T > 0 && (!q || !k || !v || !g || !beta || !dout || !dq || !dk || !dv || !dg || !dbeta))
        return GDN_ERR_NULL;
    const int parts = bwd_chunked_parts(d);
    const BwdChunkWorkspace ws = bwd_chunked_workspace(T, N, d.hk, d.hv, d.dk, d.dv, parts);
    if (workspace_bytes < ws.total) return GDN_ERR_SHAPE;
    const int64_t slots = chunk_ws_slots(T, N);
    if (slots > 0x7FFFFFFFll || N * d.hv * (int64_t)(d.dv / 16) > 0x7FFFFFFFll ||
        (T * d.hk * d.dk / 4 + 255) / 256 > 0x7FFFFFFFll)
        return GDN_ERR_SHAPE;  // 1-D grids
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(dout, 16) || !aligned(h0, 16) ||
        !aligned(dhT, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(dh0, 16) ||
        !aligned(workspace, 16) || !aligned(g, 4) || !aligned(beta, 4) || !aligned(dg, 4) || !aligned(dbeta, 4) ||
        !aligned(cu_seqlens, 4))
        return GDN_ERR_ALIGN;

    const uint64_t esz = d.io_dtype == GDN_BF16 ? 2 : 4;
    const uint64_t qk_n = (uint64_t)T * d.hk * d.dk, vo_n = (uint64_t)T * d.hv * d.dv;
    const uint64_t gb_bytes = (uint64_t)T * d.hv * 4, s_bytes = (uint64_t)N * d.hv * d.dv * d.dk * 4;
    const Range inputs[] = {range_of(q, qk_n * esz), range_of(k, qk_n * esz), range_of(v, vo_n * esz),
                            range_of(g, gb_bytes), range_of(beta, gb_bytes), range_of(h0, h0 ? s_bytes : 0),
                            range_of(cu_seqlens, (uint64_t)(N + 1) * 4), range_of(dout, vo_n * esz),
                            range_of(dhT, dhT ? s_bytes : 0)};
    const Range outputs[] = {range_of(dq, qk_n * 4), range_of(dk, qk_n * 4), range_of(dv, vo_n * 4),
                             range_of(dg, gb_bytes), range_of(dbeta, gb_bytes), range_of(dh0, dh0 ? s_bytes : 0),
                             range_of(workspace, ws.total)};
    for (size_t i = 0; i < sizeof(outputs) / sizeof(outputs[0]); ++i) {
        for (const Range &in : inputs)
            if (overlap(outputs[i], in)) return GDN_ERR_ALIAS;
        for (size_t j = i + 1; j < sizeof(outputs) / sizeof(outputs[0]); ++j)
            if (overlap(outputs[i], outputs[j])) return GDN_ERR_ALIAS;
    }

    char *w = static_cast<char *>(workspace);
    const hipStream_t strm = static_cast<hipStream_t>(stream);
    const int rank = (N > 1 && N <= kMaxRankedSeqs && T >= 32 * N) ? 1 : 0;
    const int64_t units = N * d.hv * (int64_t)(d.dv / 16);
    // (the walk stores states instead of outputs and holds fewer registers than the
    // chunked form, so it keeps 4 waves per tile up to more tiles: measured)
    const int fw_waves = d.plan_waves ? d.plan_waves : (units <= 2048 ? 4 : (units <= 8192 ? 2 : 1));

    // forward walk: records, the state at every chunk's start, x = v - Gam P, <dhT, hT>
    ChunkedParams f{};
    f.q = q; f.k = k; f.v = v; f.g = g; f.beta = beta; f.cu_seqlens = cu_seqlens;
    f.in_S = h0;
    f.ws = reinterpret_cast<float *>(w + ws.rec);
    f.ws_slots = slots;
    f.total_tokens = T; f.n_seqs = (int32_t)N; f.hk = d.hk; f.hv = d.hv; f.dk = d.dk; f.dv = d.dv;
    f.rank_by_length = rank;
    f.waves = fw_waves;
    f.ck = reinterpret_cast<float *>(w + ws.ck);
    f.xv = reinterpret_cast<float *>(w + ws.xv);
    f.dhT = dhT;
    f.hdot = reinterpret_cast<float *>(w + ws.hdot);
    hipError_t e = launch_chunked_bwd_walk(f, d.io_dtype, strm);
    if (e != hipSuccess) return GDN_ERR_HIP;

    BwdChunkParams p{};
    p.q = q; p.k = k; p.v = v; p.dout = dout; p.beta = beta; p.dhT = dhT; p.cu_seqlens = cu_seqlens;
    p.rec = f.ws; p.ck = f.ck; p.xv = f.xv; p.hdot = f.hdot;
    p.grad_v = dv; p.grad_g = dg; p.grad_beta = dbeta; p.grad_h0 = dh0;
    p.grad_q = dq; p.grad_k = dk;
    const bool split = d.hv > d.hk || parts > 1;
    p.dqh = split ? reinterpret_cast<float *>(w + ws.dq) : dq;
    p.dkh = split ? reinterpret_cast<float *>(w + ws.dk) : dk;
    p.dbeta_part = reinterpret_cast<float *>(w + ws.dbeta);
    p.dg_part = reinterpret_cast<float *>(w + ws.dg);
    p.parts = parts;
    p.plain = d.plan_lanes;  // 1: no wave specialization in the reverse walk (same bits)
    p.ws_slots = slots; p.total_tokens = T;
    p.n_seqs = (int32_t)N; p.hk = d.hk; p.hv = d.hv; p.dk = d.dk; p.dv = d.dv;
    p.rank_by_length = rank;
    p.hdot_parts = (d.dv / 16) * 4;  // one per (16-row tile, dk quarter)
    e = launch_bwd_chunked(p, d.io_dtype, strm);
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

// The preprocessing passes' 1-D grids: q/k rows, gate elements, token blocks.
static bool pre_grid_fits(const gdn_dims &d) {
    const int64_t T = d.total_tokens;
    return (T * d.hk * (d.dk / 4) + 255) / 256 <= 0x7FFFFFFFll && (T * d.hv + 255) / 256 <= 0x7FFFFFFFll &&
           (T + 63) / 64 <= 0x7FFFFFFFll;
}

gdn_status gdn_preprocess(const gdn_dims *dims, const void *q, const void *k, const float *a, const float *b,
                          float *qn, float *kn, float *g, float *beta, void *stream) {
    using namespace gdn;
    const gdn_status st = check_common(dims);
    if (st != GDN_OK) return st;
    if (!pre_grid_fits(*dims)) return GDN_ERR_SHAPE;
    const gdn_dims &d = *dims;
    const int64_t T = d.total_tokens;
    if (T == 0) return GDN_OK;
    if (!q || !k || !a || !b || !qn || !kn || !g || !beta) return GDN_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(qn, 16) || !aligned(kn, 16) || !aligned(a, 4) ||
        !aligned(b, 4) || !aligned(g, 4) || !aligned(beta, 4))
        return GDN_ERR_ALIGN;
    const uint64_t esz = d.io_dtype == GDN_BF16 ? 2 : 4;
    const uint64_t qk_n = (uint64_t)T * d.hk * d.dk, gb = (uint64_t)T * d.hv * 4;
    const Range inputs[] = {range_of(q, qk_n * esz), range_of(k, qk_n * esz), range_of(a, gb), range_of(b, gb),
                            pre_range(dims, 0), pre_range(dims, 1)};
    const Range outputs[] = {range_of(qn, qk_n * 4), range_of(kn, qk_n * 4), range_of(g, gb), range_of(beta, gb)};
    for (size_t i = 0; i < 4; ++i) {
        for (const Range &in : inputs)
            if (overlap(outputs[i], in)) return GDN_ERR_ALIAS;
        for (size_t j = i + 1; j < 4; ++j)
            if (overlap(outputs[i], outputs[j])) return GDN_ERR_ALIAS;
    }
    PreParams p{};
    p.q = q; p.k = k; p.a = a; p.b = b;
    p.qn = qn; p.kn = kn; p.g = g; p.beta = beta;
    if (const gdn_preproc *pre = d.pre) {
        p.flags = pre->flags;
        p.eps = pre->eps;
        p.A_log = pre->A_log;
        p.dt_bias = pre->dt_bias;
    }
    p.total_tokens = T; p.hk = d.hk; p.hv = d.hv;
    return launch_preprocess(p, d.dk, d.io_dtype, false, static_cast<hipStream_t>(stream)) == hipSuccess
               ? GDN_OK
               : GDN_ERR_HIP;
}

gdn_status gdn_preprocess_backward(const gdn_dims *dims, const void *q, const void *k, const float *a,
                                   const float *b, const float *dqn, const float *dkn, const float *dg,
                                   const float *dbeta, float *dq, float *dk, float *da, float *db, float *dA_log,
                                   float *ddt_bias, void *stream) {
    using namespace gdn;
    const gdn_status st = check_common(dims);
    if (st != GDN_OK) return st;
    if (!pre_grid_fits(*dims)) return GDN_ERR_SHAPE;
    const gdn_dims &d = *dims;
    const int64_t T = d.total_tokens;
    const bool gated = d.pre && (d.pre->flags & GDN_PRE_GATE_LOGITS);
    if (T > 0 && (!q || !k || !a || !b || !dqn || !dkn || !dg || !dbeta || !dq || !dk || !da || !db))
        return GDN_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(dqn, 16) || !aligned(dkn, 16) || !aligned(dq, 16) ||
        !aligned(dk, 16) || !aligned(a, 4) || !aligned(b, 4) || !aligned(dg, 4) || !aligned(dbeta, 4) ||
        !aligned(da, 4) || !aligned(db, 4) || !aligned(dA_log, 4) || !aligned(ddt_bias, 4))
        return GDN_ERR_ALIGN;
    const uint64_t esz = d.io_dtype == GDN_BF16 ? 2 : 4;
    const uint64_t qk_n = (uint64_t)T * d.hk * d.dk, gb = (uint64_t)T * d.hv * 4, hb = (uint64_t)d.hv * 4;
    const Range inputs[] = {range_of(q, qk_n * esz), range_of(k, qk_n * esz), range_of(a, gb), range_of(b, gb),
                            range_of(dqn, qk_n * 4), range_of(dkn, qk_n * 4), range_of(dg, gb),
                            range_of(dbeta, gb), pre_range(dims, 0), pre_range(dims, 1)};
    const Range outputs[] = {range_of(dq, qk_n * 4), range_of(dk, qk_n * 4), range_of(da, gb), range_of(db, gb),
                             range_of(gated ? dA_log : nullptr, hb), range_of(gated ? ddt_bias : nullptr, hb)};
    for (size_t i = 0; i < 6; ++i) {
        for (const Range &in : inputs)
            if (overlap(outputs[i], in)) return GDN_ERR_ALIAS;
        for (size_t j = i + 1; j < 6; ++j)
            if (overlap(outputs[i], outputs[j])) return GDN_ERR_ALIAS;
    }
    PreParams p{};
    p.q = q; p.k = k; p.a = a; p.b = b;
    p.dqn = dqn; p.dkn = dkn; p.dg = dg; p.dbeta = dbeta;
    p.dq = dq; p.dk = dk; p.da = da; p.db = db;
    if (const gdn_preproc *pre = d.pre) {
        p.flags = pre->flags;
        p.eps = pre->eps;
        p.A_log = pre->A_log;
        p.dt_bias = pre->dt_bias;
    }
    // the parameter gradients (written even for T = 0: sums over no tokens)
    p.dA_log = gated ? dA_log : nullptr;
    p.ddt_bias = gated && d.pre->dt_bias ? ddt_bias : nullptr;
    p.total_tokens = T; p.hk = d.hk; p.hv = d.hv;
    return launch_preprocess(p, d.dk, d.io_dtype, true, static_cast<hipStream_t>(stream)) == hipSuccess
               ? GDN_OK
               : GDN_ERR_HIP;
}

const char *gdn_status_string(gdn_status status) {
    switch (status) {
        case GDN_OK: return "GDN_OK";
        case GDN_ERR_NULL: return "GDN_ERR_NULL: a required pointer is NULL";
        case GDN_ERR_SHAPE: return "GDN_ERR_SHAPE: sizes are negative or inconsistent";
        case GDN_ERR_DTYPE: return "GDN_ERR_DTYPE: io_dtype must be GDN_F32 or GDN_BF16";
        case GDN_ERR_ALIGN: return "GDN_ERR_ALIGN: a pointer is not aligned (16 bytes for arrays, 4 for g/beta/indices)";
        case GDN_ERR_ALIAS: return "GDN_ERR_ALIAS: an output overlaps an input";
        case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED: dk or launch shape not supported";
        case GDN_ERR_HIP: return "GDN_ERR_HIP: the HIP runtime refused the launch";
        case GDN_ERR_CAPACITY:
            return "GDN_ERR_CAPACITY: the call needs more than the allocation-free entry point's fixed scratch";
    }
    return "unknown gdn_status";
}

int32_t gdn_abi_version(void) { return GDN_ABI_VERSION; }

}  // extern "C"
