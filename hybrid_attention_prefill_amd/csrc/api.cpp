// api.cpp -- the C ABI of libhypic (declared in include/hypic.h): argument
// validation, kernel selection and launch on the caller's stream.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "../../include/hypic.h"
#include "api_internal.h"
#include "hypic_kernels.h"

namespace {

thread_local std::string g_last_error;

hypic_status fail(hypic_status st, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

hypic_status ok()
{
    return HYPIC_OK;
}

hypic_status from_hip(hipError_t e, const char* what)
{
    if (e == hipSuccess) return ok();
    if (e == hipErrorNotSupported) return fail(HYPIC_E_UNSUPPORTED, "%s: no kernel for this shape/dtype", what);
    return fail(HYPIC_E_DEVICE, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

bool valid_d(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

hypic_status check_dims(const hypic_dims* d)
{
    if (!d) return fail(HYPIC_E_INVALID, "dims is NULL");
    if (d->n_heads < 1) return fail(HYPIC_E_INVALID, "n_heads must be >= 1 (got %d)", d->n_heads);
    if (!valid_d(d->d_k) || !valid_d(d->d_v))
        return fail(HYPIC_E_INVALID, "d_k and d_v must be 16, 32, 64 or 128 (got %d, %d)", d->d_k, d->d_v);
    if (d->gate < HYPIC_GATE_HEAD || d->gate > HYPIC_GATE_DIAG)
        return fail(HYPIC_E_INVALID, "gate must be 0, 1 or 2 (got %d)", d->gate);
    if (d->delta < 0 || d->delta > 2) return fail(HYPIC_E_INVALID, "delta must be 0, 1 or 2 (got %d)", d->delta);
    if (d->in_dtype != HYPIC_F32 && d->in_dtype != HYPIC_BF16)
        return fail(HYPIC_E_INVALID, "in_dtype must be 0 (f32) or 1 (bf16) (got %d)", d->in_dtype);
    if (d->t_layout < HYPIC_T_DENSE || d->t_layout > HYPIC_T_DIAG)
        return fail(HYPIC_E_INVALID, "t_layout must be 0 (dense), 1 (scalar), 2 (split) or 3 (diag) (got %d)",
                    d->t_layout);
    if (d->t_layout == HYPIC_T_SCALAR && (d->delta || d->gate == HYPIC_GATE_DIAG))
        return fail(HYPIC_E_INVALID, "a scalar T exists only for scalar gates without the delta rule");
    if (d->t_layout == HYPIC_T_DIAG && (d->delta || d->gate != HYPIC_GATE_DIAG))
        return fail(HYPIC_E_INVALID, "a diagonal T exists only for the diagonal gate without the delta rule");
    return ok();
}

constexpr long long kMaxGrid = 0x7fffffffLL;

}  // namespace

hypic_status hypic::api_error(hypic_status st, const char* msg)
{
    return fail(st, "%s", msg);
}

extern "C" {

int32_t hypic_abi_version(void) { return HYPIC_ABI_VERSION; }

const char* hypic_last_error(void) { return g_last_error.c_str(); }

size_t hypic_build_workspace_bytes(const hypic_dims* dims, int32_t n_seg, int64_t n_tokens)
{
    if (!dims || dims->n_heads < 1 || n_seg < 1 || n_tokens < 0) return 0;
    if (!valid_d(dims->d_k) || !valid_d(dims->d_v) || dims->gate < HYPIC_GATE_HEAD || dims->gate > HYPIC_GATE_DIAG)
        return 0;
    if (!dims->delta)
        return hypic::decay_workspace_bytes(dims->d_k, dims->d_v, dims->n_heads, n_seg, n_tokens,
                                            dims->gate == HYPIC_GATE_DIAG);
    if (dims->d_k != dims->d_v || dims->gate != HYPIC_GATE_TOKEN || dims->in_dtype != HYPIC_BF16) return 0;
    return hypic::split_workspace_bytes(dims->d_k, dims->n_heads, n_seg, n_tokens);
}

hypic_status hypic_segment_build(const hypic_dims* dims, int32_t n_seg, const int64_t* seg_begin,
                                 const int64_t* seg_end, int64_t n_tokens, const void* k, const void* v,
                                 const void* g, const void* beta, void* T_out, float* S_out,
                                 void* workspace, size_t workspace_bytes, void* stream)
{
    if (hypic_status s = check_dims(dims)) return s;
    if (n_seg < 0) return fail(HYPIC_E_INVALID, "n_seg must be >= 0 (got %d)", n_seg);
    if (n_tokens < 0) return fail(HYPIC_E_INVALID, "n_tokens must be >= 0");
    if (n_seg == 0) return ok();
    if (!seg_begin || !seg_end) return fail(HYPIC_E_INVALID, "seg_begin / seg_end is NULL");
    if (!S_out) return fail(HYPIC_E_INVALID, "S_out is NULL");
    if (n_tokens > 0 && (!k || !v || !g)) return fail(HYPIC_E_INVALID, "k, v or g is NULL");
    if (dims->delta && n_tokens > 0 && !beta) return fail(HYPIC_E_INVALID, "beta is NULL with the delta rule");
    if ((long long)n_seg * dims->n_heads > kMaxGrid) return fail(HYPIC_E_INVALID, "n_seg * n_heads too large");
    const bool bf16 = dims->in_dtype == HYPIC_BF16;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (dims->delta && dims->d_k != dims->d_v) {
        // The columns of S evolve independently under the delta rule (the erase and the gate
        // act on its rows): a d_k x d_v state with d_v = m d_k is built as m blocks of d_k
        // columns with the square kernels, T with the first block; with d_v < d_k in one
        // launch whose missing value columns read as zeros and are not written.  No segment is cut.
        // (the KDA build runs d_k = 16, 32 on its d = 64 kernel: blocks of 64 value columns)
        const int bw = dims->gate == HYPIC_GATE_DIAG && dims->d_k < 64 ? 64 : dims->d_k;
        if ((dims->d_v > bw && dims->d_v % bw != 0) ||
            (dims->gate != HYPIC_GATE_TOKEN && dims->gate != HYPIC_GATE_DIAG))
            return fail(HYPIC_E_UNSUPPORTED, "the delta-rule builds need d_v < d_k or a multiple of it, and gate TOKEN or DIAG");
        const int m = dims->d_v > bw ? dims->d_v / bw : 1;
        const size_t esz = bf16 ? 2 : 4;
        for (int j = 0; j < m; ++j) {
            const void* vj = v ? static_cast<const char*>(v) + (size_t)j * bw * esz : nullptr;
            float* Sj = S_out + (size_t)j * bw;
            void* Tj = j == 0 ? T_out : nullptr;
            const hipError_t e =
                dims->gate == HYPIC_GATE_TOKEN
                    ? hypic::build_gdn(dims->d_k, bf16, n_seg, dims->n_heads, seg_begin, seg_end, n_tokens, k, vj, g,
                                       beta, Tj, dims->t_layout == HYPIC_T_SPLIT, Sj, hypic::BuildItems{},
                                       hypic::BuildOut{}, st, dims->d_v)
                    : hypic::build_kda(dims->d_k, bf16, dims->delta == 2, n_seg, dims->n_heads, seg_begin, seg_end,
                                       n_tokens, k, vj, g, beta, Tj, dims->t_layout == HYPIC_T_SPLIT, Sj, st,
                                       dims->d_v);
            if (e != hipSuccess) return from_hip(e, "hypic_segment_build");
        }
        return ok();
    }
    if (!dims->delta) {
        const size_t need = workspace ? hypic_build_workspace_bytes(dims, n_seg, n_tokens) : 0;
        if (need > 0) {
            if (workspace_bytes < need)
                return fail(HYPIC_E_INVALID, "build workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
            if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
                return fail(HYPIC_E_INVALID, "workspace must be 256-byte aligned");
        }
        return from_hip(hypic::build_decay(dims->d_k, dims->d_v, bf16, dims->gate, n_seg, dims->n_heads, seg_begin, seg_end,
                                           n_tokens, k, v, g, T_out, dims->t_layout, S_out,
                                           need > 0 ? workspace : nullptr, st),
                        "hypic_segment_build");
    }
    if (dims->delta && dims->gate == HYPIC_GATE_TOKEN) {
        const size_t need = workspace ? hypic_build_workspace_bytes(dims, n_seg, n_tokens) : 0;
        if (need > 0) {
            if (workspace_bytes < need)
                return fail(HYPIC_E_INVALID, "build workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
            if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
                return fail(HYPIC_E_INVALID, "workspace must be 256-byte aligned");
            return from_hip(hypic::build_gdn_split(dims->d_k, bf16, n_seg, dims->n_heads, seg_begin, seg_end,
                                                   n_tokens, k, v, g, beta, T_out,
                                                   dims->t_layout == HYPIC_T_SPLIT, S_out, workspace, st),
                            "hypic_segment_build");
        }
        return from_hip(hypic::build_gdn(dims->d_k, bf16, n_seg, dims->n_heads, seg_begin, seg_end,
                                         n_tokens, k, v, g, beta, T_out,
                                         dims->t_layout == HYPIC_T_SPLIT, S_out, hypic::BuildItems{},
                                         hypic::BuildOut{}, st),
                        "hypic_segment_build");
    }
    if (dims->delta && dims->gate == HYPIC_GATE_DIAG) {
        return from_hip(hypic::build_kda(dims->d_k, bf16, dims->delta == 2, n_seg, dims->n_heads, seg_begin, seg_end, n_tokens, k,
                                         v, g, beta, T_out, dims->t_layout == HYPIC_T_SPLIT, S_out, st),
                        "hypic_segment_build");
    }
    return fail(HYPIC_E_UNSUPPORTED, "hypic_segment_build: gate %d with delta %d is not implemented",
                dims->gate, dims->delta);
}

hypic_status hypic_segment_prefill(const hypic_dims* dims, int32_t n_seg, const int64_t* seg_begin,
                                   const int64_t* seg_end, int64_t n_tokens, const void* q, const void* k,
                                   const void* v, const void* g, const void* beta, float scale, void* T_out,
                                   float* S_out, float* out, void* stream)
{
    if (hypic_status s = check_dims(dims)) return s;
    if (n_seg < 0) return fail(HYPIC_E_INVALID, "n_seg must be >= 0 (got %d)", n_seg);
    if (n_tokens < 0) return fail(HYPIC_E_INVALID, "n_tokens must be >= 0");
    if (n_seg == 0) return ok();
    if (!seg_begin || !seg_end) return fail(HYPIC_E_INVALID, "seg_begin / seg_end is NULL");
    if (!S_out || !out) return fail(HYPIC_E_INVALID, "S_out or out is NULL");
    if (n_tokens > 0 && (!q || !k || !v || !g || !beta)) return fail(HYPIC_E_INVALID, "q, k, v, g or beta is NULL");
    if ((long long)n_seg * dims->n_heads > kMaxGrid) return fail(HYPIC_E_INVALID, "n_seg * n_heads too large");
    if (dims->gate != HYPIC_GATE_TOKEN || !dims->delta || dims->in_dtype != HYPIC_BF16 ||
        (dims->d_v > dims->d_k && dims->d_v % dims->d_k != 0) || (dims->d_k != 64 && dims->d_k != 128))
        return fail(HYPIC_E_UNSUPPORTED,
                    "hypic_segment_prefill: implemented for gate TOKEN with the delta rule, bf16, d_k in {64, 128} "
                    "and d_v below d_k or a multiple of it");
    if (dims->t_layout != HYPIC_T_DENSE && dims->t_layout != HYPIC_T_SPLIT)
        return fail(HYPIC_E_INVALID, "hypic_segment_prefill: T layout DENSE or SPLIT");
    // A wider state in blocks of d_k value columns (as in hypic_segment_build): output column
    // n depends on state column n only.
    for (int j = 0; j < (dims->d_v > dims->d_k ? dims->d_v / dims->d_k : 1); ++j) {
        const size_t c = (size_t)j * dims->d_k;
        hypic::BuildOut ob;
        ob.q = q;
        ob.scale = scale;
        ob.out = out + c;
        const hipError_t e =
            hypic::build_gdn(dims->d_k, true, n_seg, dims->n_heads, seg_begin, seg_end, n_tokens, k,
                             v ? static_cast<const char*>(v) + c * 2 : nullptr, g, beta, j == 0 ? T_out : nullptr,
                             dims->t_layout == HYPIC_T_SPLIT, S_out + c, hypic::BuildItems{}, ob,
                             reinterpret_cast<hipStream_t>(stream), dims->d_v);
        if (e != hipSuccess) return from_hip(e, "hypic_segment_prefill");
    }
    return ok();
}

hypic_status hypic_compose(const hypic_dims* dims, int32_t n_chain, int32_t n_step, const int32_t* pair_id,
                           int32_t n_pair, const void* T_cache, const float* S_cache, float* S_run,
                           void* stream)
{
    if (hypic_status s = check_dims(dims)) return s;
    if (n_chain < 0 || n_step < 0 || n_pair < 0)
        return fail(HYPIC_E_INVALID, "n_chain, n_step and n_pair must be >= 0");
    if (n_chain == 0 || n_step == 0) return ok();
    if (!pair_id || !S_run) return fail(HYPIC_E_INVALID, "pair_id or S_run is NULL");
    if (n_pair > 0 && (!T_cache || !S_cache)) return fail(HYPIC_E_INVALID, "T_cache or S_cache is NULL");
    if ((long long)n_chain * dims->n_heads * 8 > kMaxGrid ||
        (long long)n_chain * dims->n_heads * (dims->d_k * dims->d_v / 4) / 256 > kMaxGrid)
        return fail(HYPIC_E_INVALID, "too many chains");
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (dims->t_layout == HYPIC_T_SCALAR || dims->t_layout == HYPIC_T_DIAG)
        return from_hip(hypic::compose_scalar(dims->d_k, dims->d_v, dims->t_layout == HYPIC_T_DIAG, n_chain,
                                              dims->n_heads, n_step, pair_id, n_pair,
                                              static_cast<const float*>(T_cache), S_cache, S_run, st),
                        "hypic_compose");
    return from_hip(hypic::compose_dense(dims->d_k, dims->d_v, n_chain, dims->n_heads, n_step, pair_id, n_pair, T_cache,
                                         dims->t_layout == HYPIC_T_SPLIT, S_cache, S_run, nullptr, st),
                    "hypic_compose");
}

size_t hypic_seam_workspace_bytes(const hypic_dims* dims, int32_t n_chain, int32_t n_step, int32_t w)
{
    if (!dims || dims->n_heads < 1 || !valid_d(dims->d_k) || !valid_d(dims->d_v) ||
        (dims->d_v > dims->d_k && dims->d_v % dims->d_k != 0))
        return 0;
    if (n_chain < 0 || n_step < 0 || w < 1 || w > 16) return 0;
    return hypic::seam_plan(dims->d_k, n_chain, dims->n_heads, n_step, w).bytes;
}

hypic_status hypic_seam_advance(const hypic_dims* dims, int32_t n_chain, int32_t n_step, int32_t w,
                                const int64_t* seam_start, int64_t n_tokens, const void* q, const void* k,
                                const void* v, const void* g, const void* beta, float scale,
                                const int32_t* pair_id, int32_t n_pair, const void* T_cache,
                                const float* S_cache, float* S_run, float* out, void* workspace,
                                size_t workspace_bytes, void* stream)
{
    return hypic::seam_advance_with(dims, n_chain, n_step, w, seam_start, n_tokens, q, k, v, g, beta, scale,
                                    pair_id, n_pair, T_cache, S_cache, S_run, out, workspace, workspace_bytes,
                                    stream);
}

}  // extern "C"

namespace hypic {
static hypic_status seam_block(int d, int dv, int n_chain, int n_step, int H, int w, const int64_t* seam_start,
                               int64_t n_tokens, const void* q, const void* k, const void* v, const void* g,
                               const void* beta, bool bf16, float scale, const int32_t* pair_id, int n_pair,
                               const void* T_cache, bool t_split, const float* S_cache, float* S_run, float* out,
                               void* workspace, hipStream_t st);
}

hypic_status hypic::seam_advance_with(const hypic_dims* dims, int32_t n_chain, int32_t n_step, int32_t w,
                                      const int64_t* seam_start, int64_t n_tokens, const void* q, const void* k,
                                      const void* v, const void* g, const void* beta, float scale,
                                      const int32_t* pair_id, int32_t n_pair, const void* T_cache,
                                      const float* S_cache, float* S_run, float* out, void* workspace,
                                      size_t workspace_bytes, void* stream)
{
    if (hypic_status s = check_dims(dims)) return s;
    if (n_chain < 0 || n_step < 0 || n_pair < 0 || n_tokens < 0)
        return fail(HYPIC_E_INVALID, "n_chain, n_step, n_pair and n_tokens must be >= 0");
    if (w < 1 || w > 16) return fail(HYPIC_E_INVALID, "w must be in 1..16 (got %d)", w);
    if (n_chain == 0 || n_step == 0) return ok();
    if (!seam_start || !S_run || !out) return fail(HYPIC_E_INVALID, "seam_start, S_run or out is NULL");
    if (n_tokens > 0 && (!q || !k || !v || !g || !beta)) return fail(HYPIC_E_INVALID, "q, k, v, g or beta is NULL");
    if (pair_id && n_pair > 0 && (!T_cache || !S_cache)) return fail(HYPIC_E_INVALID, "T_cache or S_cache is NULL");
    if (dims->gate != HYPIC_GATE_TOKEN || !dims->delta)
        return fail(HYPIC_E_UNSUPPORTED, "hypic_seam_advance: only the scalar-gated delta rule is implemented");
    if (dims->t_layout == HYPIC_T_SCALAR || dims->t_layout == HYPIC_T_DIAG)
        return fail(HYPIC_E_UNSUPPORTED, "hypic_seam_advance needs a dense T (layout DENSE or SPLIT)");
    if (dims->d_v > dims->d_k && dims->d_v % dims->d_k != 0)
        return fail(HYPIC_E_UNSUPPORTED, "hypic_seam_advance: d_v must be below d_k or a multiple of it (got %d, %d)",
                    dims->d_k, dims->d_v);
    if ((long long)n_chain * n_step * dims->n_heads > kMaxGrid || (long long)n_chain * dims->n_heads * 8 > kMaxGrid)
        return fail(HYPIC_E_INVALID, "too many chains or steps");
    const size_t need = hypic_seam_workspace_bytes(dims, n_chain, n_step, w);
    if (!workspace || workspace_bytes < need)
        return fail(HYPIC_E_INVALID, "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return fail(HYPIC_E_INVALID, "workspace must be 256-byte aligned");
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const bool bf16 = dims->in_dtype == HYPIC_BF16;
    const int d = dims->d_k, H = dims->n_heads, dv = dims->d_v;
    // A state wider than d_k (d_v = m d_k) advances in m blocks of d_k columns, one after the
    // other through the same workspace: the columns of R, of the pairs' S, of the windows' U
    // and of the outputs evolve independently (T, the erase and the gates act on rows).  A
    // narrower one (d_v < d_k) in one pass whose column blocks end at its last column.
    for (int j = 0; j < (dv > d ? dv / d : 1); ++j) {
        const size_t c = (size_t)j * d;
        const void* vj = v ? static_cast<const char*>(v) + c * (bf16 ? 2 : 4) : nullptr;
        const hypic_status s = seam_block(d, dv, n_chain, n_step, H, w, seam_start, n_tokens, q, k, vj, g, beta,
                                          bf16, scale, pair_id, n_pair, T_cache, dims->t_layout == HYPIC_T_SPLIT,
                                          S_cache ? S_cache + c : nullptr, S_run + c, out + c, workspace, st);
        if (s != HYPIC_OK) return s;
    }
    return ok();
}

// One block of d state columns of hypic_seam_advance (S_cache, S_run and out point at the
// block's first column; their rows hold dv values).
hypic_status hypic::seam_block(int d, int dv, int n_chain, int n_step, int H, int w, const int64_t* seam_start,
                               int64_t n_tokens, const void* q, const void* k, const void* v, const void* g,
                               const void* beta, bool bf16, float scale, const int32_t* pair_id, int n_pair,
                               const void* T_cache, bool t_split, const float* S_cache, float* S_run, float* out,
                               void* workspace, hipStream_t st)
{
    const hypic::SeamPlan pl = hypic::seam_plan(d, n_chain, H, n_step, w, dv < d ? dv : 0);
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    hipError_t e = hypic::seam_prep(d, n_chain, n_step, H, seam_start, n_tokens, w, q, k, v, g, beta, bf16, scale,
                                    ws, st, dv);
    if (e != hipSuccess) return from_hip(e, "hypic_seam_advance (window preparation)");
    hypic::SeamArgs sa{seam_start, n_tokens, w, (int)bf16, scale, q, k, ws, out};
    sa.ld = dv;
    sa.nblk = pl.nblk;
    sa.blk = pl.blk;
    if (pl.nblk > 1) {
        sa.ox = reinterpret_cast<float*>(ws + pl.ox_off);
        sa.agg_T = ws + pl.agg_t_off;
        sa.agg_S = reinterpret_cast<float*>(ws + pl.agg_s_off);
    }
    const int np = pair_id ? n_pair : 0;
    e = hypic::seam_chain(d, pl.nb, n_chain, H, n_step, pair_id, np, T_cache, t_split, S_cache, S_run, sa, st);
    if (e != hipSuccess || pl.nblk == 1) return from_hip(e, "hypic_seam_advance");
    // blocked scan: block aggregates composed in order (the state entering every block
    // kept), then the windows of blocks >= 1 read out from those states
    float* trail = reinterpret_cast<float*>(ws + pl.trail_off);
    e = hypic::compose_dense(d, d, n_chain, H, pl.nblk - 1, nullptr, n_chain * (pl.nblk - 1), sa.agg_T, true, sa.agg_S,
                             S_run, trail, st, dv);
    if (e != hipSuccess) return from_hip(e, "hypic_seam_advance (composition of the block aggregates)");
    return from_hip(hypic::seam_readout(d, n_chain, H, n_step, pl.nblk, pl.blk, w, seam_start, n_tokens, sa.ox, trail,
                                        out, st, dv),
                    "hypic_seam_advance (window outputs)");
}

extern "C" {

// Diagnostic: runs the lane-layout self-test kernel into a device buffer of
// 2112 floats from 256 input floats (see selftest.hip).  Not part of the method.
hypic_status hypic_selftest_layouts(const float* in, float* out, void* stream)
{
    if (!in || !out) return fail(HYPIC_E_INVALID, "in or out is NULL");
    return from_hip(hypic::selftest_layouts(in, out, reinterpret_cast<hipStream_t>(stream)), "hypic_selftest_layouts");
}

}  // extern "C"
