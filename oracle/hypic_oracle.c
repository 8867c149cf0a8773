/*
 * hypic_oracle.c -- plain fp64 CPU oracle for the linear-attention state
 * algebra of HYPIC's position-independent caching.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library; it is deliberately slow and
 * written so that each routine can be checked against the source pages by eye.
 *
 * Sources (web pages retelling the HYPIC work; cited by short key):
 *   [ZH] "首 token 延迟降 3.25 倍！小红书联合北大、上交提出 HYPIC，让混合注意力
 *        大模型用上「位置无关缓存」" (nav.aitube.vip) -- sections 2.1, 2.2, 2.3.
 *   [ES] "Xiaohongshu, la Universidad de Pekín y la Universidad de Jiao Tong de
 *        Shanghai presentan HYPIC ..." (xix.ai, Spanish) -- paragraphs on the
 *        linear layers and on the seam windows.
 *
 * What the pages fix:
 *   - a linear-attention layer keeps one fixed-size recurrent state per head;
 *     every token applies its own transition matrix to it ([ZH] 2.1);
 *   - the segment operator T_C is the ordered product of the token transition
 *     matrices inside the segment, and S(C|0) is the final state when the
 *     segment starts from a zero state; both depend on the segment's tokens
 *     only ([ZH] 2.1, [ES] linear-layer paragraph);
 *   - composition law: S(C1 C2) = T(C2) S(C1) + S(C2) ([ZH] 2.1);
 *   - at reuse the first w tokens of every internal segment (the seam window)
 *     are stepped from the running state and their per-token outputs are sent
 *     upward ([ZH] 2.2, [ES] seam paragraph).
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes of the repository):
 *   - state S is d_k x d_v, transitions are d_k x d_k and act from the left,
 *     later tokens on the left of the product (forced by "T(C2) S(C1)");
 *   - transition of token t:  M_t = G_t (I - beta_t k_t k_t^T) with the
 *     delta rule (delta = 1, gate applied after the erase), M_t =
 *     (I - beta_t k_t k_t^T) G_t with delta = 2 (gate applied before the
 *     erase, the order of the Kimi Delta Attention write-ups; the same matrix
 *     for scalar gates), M_t = G_t without it; G_t = exp(g) (per-head constant
 *     or per-token scalar) or diag(exp(g_t)) (per-token, per key channel);
 *   - write term: beta_t k_t v_t^T with the delta rule, k_t v_t^T without;
 *   - output of a stepped token: o_t = S_t^T (scale q_t) with S_t the state
 *     after the token's update.
 *
 * Layouts (all row-major, fp64):
 *   q, k : [n_tok][H][d_k]     v : [n_tok][H][d_v]
 *   g    : [H] (gate 0) | [n_tok][H] (gate 1) | [n_tok][H][d_k] (gate 2)
 *   beta : [n_tok][H]
 *   S    : [..][H][d_k][d_v]   T : [..][H][d_k][d_k]  (or [..][H] if scalar)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int32_t n_heads, d_k, d_v;
    int32_t gate;  /* 0 head constant, 1 token scalar, 2 token per-channel */
    int32_t delta; /* 1: erase with beta k k^T, then gate, write beta k v^T;
                      2: gate, then erase, write beta k v^T; 0: gate, k v^T */
} ora_dims;

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* log-gate of token t, head h, key channel i */
static double log_gate(const ora_dims *d, const double *g, int64_t t, int h, int i)
{
    switch (d->gate) {
    case 0: return g[h];
    case 1: return g[t * d->n_heads + h];
    default: return g[(t * d->n_heads + h) * d->d_k + i];
    }
}

/* gate: X <- G_t X (row i scaled by exp of its log-gate) */
static void gate_rows(const ora_dims *d, int64_t t, int h, const double *g, double *X, int ncol)
{
    for (int i = 0; i < d->d_k; ++i) {
        const double G = exp(log_gate(d, g, t, h, i));
        for (int n = 0; n < ncol; ++n) X[i * ncol + n] *= G;
    }
}

/*
 * One token of one head, in place on a d_k x ncol matrix X (the state S, or
 * the running transition product T): X <- M_t X, then, if `v` is given, the
 * write term is added.  This is the definition of the per-token transition
 * ([ZH] 2.1) with the readings above.  `u` is scratch of length ncol.
 */
static void apply_token(const ora_dims *d, int64_t t, int h, const double *k,
                        const double *v, const double *g, const double *beta,
                        double *X, int ncol, double *u)
{
    const int dk = d->d_k, H = d->n_heads;
    const double *kt = k + (t * H + h) * (int64_t)dk;
    const double b = d->delta ? beta[t * H + h] : 0.0;
    if (d->delta == 2) gate_rows(d, t, h, g, X, ncol);
    if (d->delta) {
        /* erase: X <- (I - b k k^T) X */
        for (int n = 0; n < ncol; ++n) {
            double s = 0.0;
            for (int i = 0; i < dk; ++i) s += kt[i] * X[i * ncol + n];
            u[n] = s;
        }
        for (int i = 0; i < dk; ++i)
            for (int n = 0; n < ncol; ++n) X[i * ncol + n] -= b * kt[i] * u[n];
    }
    if (d->delta != 2) gate_rows(d, t, h, g, X, ncol);
    if (v) {
        /* write: X <- X + c k v^T, c = beta with the delta rule, else 1 */
        const double *vt = v + (t * H + h) * (int64_t)ncol;
        const double c = d->delta ? b : 1.0;
        for (int i = 0; i < dk; ++i)
            for (int n = 0; n < ncol; ++n) X[i * ncol + n] += c * kt[i] * vt[n];
    }
}

/* o = scale * S^T q for one token of one head */
static void token_output(const ora_dims *d, int64_t t, int h, const double *q,
                         double scale, const double *S, double *o)
{
    const int dk = d->d_k, dv = d->d_v;
    const double *qt = q + (t * d->n_heads + h) * (int64_t)dk;
    for (int n = 0; n < dv; ++n) {
        double s = 0.0;
        for (int i = 0; i < dk; ++i) s += S[i * dv + n] * qt[i];
        o[n] = scale * s;
    }
}

/*
 * Segment build ([ZH] 2.1): for every (segment, head), start from T = I and
 * S = 0 and step each token of [seg_begin, seg_end) in order.  The results are
 * T_C (ordered product of the token transitions) and S(C|0).
 * T_out may be NULL (state only).
 */
void oracle_build(const ora_dims *d, int32_t n_seg, const int64_t *seg_begin,
                  const int64_t *seg_end, const double *k, const double *v,
                  const double *g, const double *beta, double *T_out, double *S_out)
{
    const int H = d->n_heads, dk = d->d_k, dv = d->d_v;
    const int64_t n_unit = (int64_t)n_seg * H;
#pragma omp parallel
    {
        double *u = (double *)malloc(sizeof(double) * (size_t)(dk > dv ? dk : dv));
#pragma omp for schedule(dynamic, 1)
        for (int64_t unit = 0; unit < n_unit; ++unit) {
            const int s = (int)(unit / H), h = (int)(unit % H);
            double *S = S_out + unit * (int64_t)dk * dv;
            double *T = T_out ? T_out + unit * (int64_t)dk * dk : NULL;
            memset(S, 0, sizeof(double) * (size_t)dk * dv);
            if (T) {
                memset(T, 0, sizeof(double) * (size_t)dk * dk);
                for (int i = 0; i < dk; ++i) T[i * dk + i] = 1.0;
            }
            for (int64_t t = seg_begin[s]; t < seg_end[s]; ++t) {
                apply_token(d, t, h, k, v, g, beta, S, dv, u);
                if (T) apply_token(d, t, h, k, NULL, g, beta, T, dk, u);
            }
        }
        free(u);
    }
}

/*
 * Plain recurrence over tokens [t0, t1) for every head, starting from the
 * given state S[H][d_k][d_v] (updated in place).  If q and out are given,
 * out[(t - t0)][h][:] receives the output of token t.  This is the "full
 * recompute" the pages compare the composed state against ([ZH] 2.1).
 */
void oracle_run(const ora_dims *d, int64_t t0, int64_t t1, const double *q,
                const double *k, const double *v, const double *g,
                const double *beta, double scale, double *S, double *out)
{
    const int H = d->n_heads, dk = d->d_k, dv = d->d_v;
#pragma omp parallel
    {
        double *u = (double *)malloc(sizeof(double) * (size_t)(dk > dv ? dk : dv));
#pragma omp for schedule(static, 1)
        for (int h = 0; h < H; ++h) {
            double *Sh = S + (int64_t)h * dk * dv;
            for (int64_t t = t0; t < t1; ++t) {
                apply_token(d, t, h, k, v, g, beta, Sh, dv, u);
                if (q && out)
                    token_output(d, t, h, q, scale, Sh, out + ((t - t0) * H + h) * (int64_t)dv);
            }
        }
        free(u);
    }
}

/* S_run <- T S_run + S for one head: the composition law of [ZH] 2.1. */
static void compose_one(int dk, int dv, int t_scalar, const double *T,
                        const double *S, double *R, double *tmp)
{
    if (t_scalar) {
        for (int i = 0; i < dk * dv; ++i) R[i] = T[0] * R[i] + S[i];
        return;
    }
    for (int i = 0; i < dk; ++i)
        for (int n = 0; n < dv; ++n) {
            double s = 0.0;
            for (int j = 0; j < dk; ++j) s += T[i * dk + j] * R[j * dv + n];
            tmp[i * dv + n] = s + S[i * dv + n];
        }
    memcpy(R, tmp, sizeof(double) * (size_t)dk * dv);
}

/*
 * Ordered composition over chains ([ZH] 2.1, "left-multiply by T_C, then
 * add"): for each chain c and step j with id = pair_id[c][j] >= 0,
 * S_run[c] <- T[id] S_run[c] + S[id], per head.  id < 0 skips the step.
 * T_cache is [n_pair][H][d_k][d_k], or [n_pair][H] when t_scalar != 0.
 */
void oracle_compose(int32_t H, int32_t dk, int32_t dv, int32_t t_scalar,
                    int32_t n_chain, int32_t n_step, const int32_t *pair_id,
                    const double *T_cache, const double *S_cache, double *S_run)
{
    const int64_t n_unit = (int64_t)n_chain * H;
    const int64_t tsz = t_scalar ? 1 : (int64_t)dk * dk, ssz = (int64_t)dk * dv;
#pragma omp parallel
    {
        double *tmp = (double *)malloc(sizeof(double) * (size_t)ssz);
#pragma omp for schedule(dynamic, 1)
        for (int64_t unit = 0; unit < n_unit; ++unit) {
            const int c = (int)(unit / H), h = (int)(unit % H);
            double *R = S_run + unit * ssz;
            for (int j = 0; j < n_step; ++j) {
                const int id = pair_id[(int64_t)c * n_step + j];
                if (id < 0) continue;
                compose_one(dk, dv, t_scalar, T_cache + ((int64_t)id * H + h) * tsz,
                            S_cache + ((int64_t)id * H + h) * ssz, R, tmp);
            }
        }
        free(tmp);
    }
}

/*
 * Seam advance ([ZH] 2.2): for each chain c and step j, in order:
 *   1. if seam_start[c][j] >= 0, step the w tokens starting there from the
 *      running state, writing each token's output to out[c][j][i][h][:];
 *   2. if pair_id is given and pair_id[c][j] >= 0, compose with that pair.
 * out rows of steps without a seam are left untouched.
 */
void oracle_seam_advance(const ora_dims *d, int32_t n_chain, int32_t n_step,
                         int32_t w, const int64_t *seam_start, const double *q,
                         const double *k, const double *v, const double *g,
                         const double *beta, double scale, const int32_t *pair_id,
                         int32_t t_scalar, const double *T_cache,
                         const double *S_cache, double *S_run, double *out)
{
    const int H = d->n_heads, dk = d->d_k, dv = d->d_v;
    const int64_t n_unit = (int64_t)n_chain * H;
    const int64_t tsz = t_scalar ? 1 : (int64_t)dk * dk, ssz = (int64_t)dk * dv;
#pragma omp parallel
    {
        double *tmp = (double *)malloc(sizeof(double) * (size_t)ssz);
        double *u = (double *)malloc(sizeof(double) * (size_t)(dk > dv ? dk : dv));
#pragma omp for schedule(dynamic, 1)
        for (int64_t unit = 0; unit < n_unit; ++unit) {
            const int c = (int)(unit / H), h = (int)(unit % H);
            double *R = S_run + unit * ssz;
            for (int j = 0; j < n_step; ++j) {
                const int64_t cj = (int64_t)c * n_step + j;
                const int64_t s0 = seam_start[cj];
                if (s0 >= 0) {
                    for (int i = 0; i < w; ++i) {
                        apply_token(d, s0 + i, h, k, v, g, beta, R, dv, u);
                        token_output(d, s0 + i, h, q, scale, R,
                                     out + ((cj * w + i) * H + h) * (int64_t)dv);
                    }
                }
                if (pair_id && pair_id[cj] >= 0) {
                    const int id = pair_id[cj];
                    compose_one(dk, dv, t_scalar, T_cache + ((int64_t)id * H + h) * tsz,
                                S_cache + ((int64_t)id * H + h) * ssz, R, tmp);
                }
            }
        }
        free(u);
        free(tmp);
    }
}
