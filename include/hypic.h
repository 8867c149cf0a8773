/*
 * hypic.h -- C ABI of libhypic.so: the data-parallel hot path of HYPIC's
 * position-independent caching for linear-attention layers, on AMD Instinct
 * MI355X (gfx950).
 *
 * Sources (web pages retelling the HYPIC work; cited by short key):
 *   [ZH] "首 token 延迟降 3.25 倍！小红书联合北大、上交提出 HYPIC，让混合注意力
 *        大模型用上「位置无关缓存」" (nav.aitube.vip): section 2.1 (linear
 *        layers cache the segment transition operator), section 2.2 (seam
 *        windows), section 2.3 (segment parallelism).
 *   [ES] "Xiaohongshu, la Universidad de Pekín y la Universidad de Jiao Tong
 *        de Shanghai presentan HYPIC ..." (xix.ai): the paragraphs on the
 *        linear layers and on the seam windows.
 *
 * The method ([ZH] 2.1): a linear-attention head keeps a state S (d_k x d_v);
 * every token t applies its transition M_t (d_k x d_k) and adds a write term:
 *     S_t = M_t S_{t-1} + c_t k_t v_t^T.
 * For a segment C of tokens 1..L the cached pair is
 *     T_C    = M_L ... M_1                      (ordered product, later left)
 *     S(C|0) = state after C started from S = 0,
 * and any prefix composes exactly:  S(C1 C2) = T(C2) S(C1) + S(C2).
 *
 * Transition families (gate x delta):
 *     gate HEAD,  delta 0 : M_t = gamma_h I,                  c_t = 1   (RetNet-style)
 *     gate TOKEN, delta 1 : M_t = alpha_t (I - b_t k_t k_t^T), c_t = b_t (gated DeltaNet)
 *     gate DIAG,  delta 1 : M_t = diag(a_t)(I - b_t k_t k_t^T), c_t = b_t (KDA-style)
 *     gate DIAG,  delta 2 : M_t = (I - b_t k_t k_t^T)diag(a_t), c_t = b_t (KDA, gate first)
 *     gate TOKEN, delta 0 : M_t = alpha_t I,                 c_t = 1   (Mamba2-style)
 *     gate DIAG,  delta 0 : M_t = diag(a_t),                 c_t = 1   (GLA-style)
 * (DeltaNet is gate TOKEN, delta 1 with all g = 0.  For scalar gates delta 2,
 * the gate applied before the erase, is the same transition as delta 1.)
 * Gates are passed as log-gates g <= 0 (gamma = exp(g), alpha_t = exp(g_t),
 * a_t = exp(g_t) per key channel).
 *
 * Conventions for every entry point
 *   - All array arguments are DEVICE pointers owned by the caller; nothing is
 *     copied, retained or freed.  The library allocates no device memory (its one
 *     static device array, used only by hypic_seam_advance_noalloc, is described
 *     there).
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream) and returns once the kernels are enqueued.
 *   - Argument errors return HYPIC_E_INVALID before anything is launched;
 *     valid but unimplemented combinations return HYPIC_E_UNSUPPORTED; a failed
 *     launch returns HYPIC_E_DEVICE.  Faults while kernels run surface when the
 *     caller synchronises.  The library never aborts and never prints;
 *     hypic_last_error() gives a message for the last non-OK status of the
 *     calling thread.
 *   - Values the host cannot check are made safe on the device: token ranges
 *     are clamped to [0, n_tokens), pair ids outside [0, n_pair) skip their
 *     step, seam windows that do not fit in [0, n_tokens) are skipped.
 *   - Layouts are row-major.  Token arrays are packed over the prompt:
 *     k, q [n_tokens][H][d_k], v [n_tokens][H][d_v], beta [n_tokens][H],
 *     g [H] (HEAD, always fp32) | [n_tokens][H] (TOKEN) | [n_tokens][H][d_k] (DIAG).
 *     q, k, v, beta and token gates have dtype `in_dtype`.
 *     Pairs: S [n_pair][H][d_k][d_v] fp32; T by hypic_t_layout:
 *       DENSE  : fp32 [n_pair][H][d_k][d_k];
 *       SCALAR : fp32 [n_pair][H], T = t I (scalar gates without the delta rule);
 *       DIAG   : fp32 [n_pair][H][d_k], T = diag(t) (gate DIAG without the delta rule);
 *       SPLIT  : bf16 [n_pair][H][2][d_k*d_k], plane 0 = hi = bf16(T) and
 *                plane 1 = lo = bf16(T - hi), both round-to-nearest-even, so
 *                T = hi + lo to about 2^-16 relative.  Within a plane, entry
 *                (r, c) sits at ((r/16)*(d_k/8) + c/8)*128 + (r%16)*8 + c%8:
 *                16 x 8 blocks, row-major inside a block and across blocks.
 *                Same 4 bytes per entry as DENSE; it is the MFMA operand
 *                format of the composition kernels, which load it as is, one
 *                contiguous KiB per operand fragment (the layout to cache T
 *                in when it is only ever composed).
 *   - Outputs of concurrent calls must not alias each other.
 */
#ifndef HYPIC_H
#define HYPIC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HYPIC_ABI_VERSION 6

typedef enum {
    HYPIC_OK = 0,
    HYPIC_E_INVALID = 1,     /* bad argument; nothing was launched              */
    HYPIC_E_UNSUPPORTED = 2, /* valid combination this build does not implement  */
    HYPIC_E_DEVICE = 3       /* HIP error while launching                       */
} hypic_status;

typedef enum { HYPIC_GATE_HEAD = 0, HYPIC_GATE_TOKEN = 1, HYPIC_GATE_DIAG = 2 } hypic_gate;
typedef enum { HYPIC_F32 = 0, HYPIC_BF16 = 1 } hypic_dtype;
typedef enum { HYPIC_T_DENSE = 0, HYPIC_T_SCALAR = 1, HYPIC_T_SPLIT = 2, HYPIC_T_DIAG = 3 } hypic_t_layout;

typedef struct {
    int32_t n_heads;  /* H >= 1                                                  */
    int32_t d_k;      /* key dim: 16, 32, 64 or 128                             */
    int32_t d_v;      /* value dim: 16, 32, 64 or 128                           */
    int32_t gate;     /* hypic_gate                                             */
    int32_t delta;    /* 0: plain write; 1: delta-rule erase, then the gate, and
                         beta-weighted write; 2: as 1 with the gate first      */
    int32_t in_dtype; /* hypic_dtype of q, k, v, beta and token gates            */
    int32_t t_layout; /* hypic_t_layout of T (SCALAR: gate HEAD or TOKEN, delta 0;
                         DIAG: gate DIAG, delta 0)                              */
} hypic_dims;

/*
 * hypic_segment_build -- the one-time cost at a segment's first prefill
 * ([ZH] 2.1 and the overhead paragraph of the evaluation): for every segment i
 * and head h, start from T = I, S = 0 and apply the tokens
 * [seg_begin[i], seg_end[i]) in order, writing
 *     T_out[i][h] = T_C  and  S_out[i][h] = S(C|0).
 * Segments are independent and may overlap or leave gaps (e.g. seam windows
 * excluded from the cache); an empty range yields the identity pair (I, 0).
 *   seg_begin, seg_end : int64 [n_seg] token offsets into the packed arrays
 *   n_tokens           : length of the packed token arrays (ranges are clamped)
 *   beta               : ignored (may be NULL) when delta == 0
 *   T_out              : in the dims' t_layout; may be NULL to skip T (S only)
 *   workspace          : NULL, or device scratch of at least
 *                        hypic_build_workspace_bytes(dims, n_seg, n_tokens) bytes,
 *                        256-byte aligned, owned by the caller, contents overwritten;
 *                        concurrent calls need distinct workspaces.  With it, long
 *                        segments are built as pieces in parallel and the pieces'
 *                        pairs folded by the composition law ([ZH] 2.1 and the segment
 *                        parallelism of 2.3).  Gated delta rule: a segment of c > 16
 *                        64-token chunks is cut on chunk boundaries into ceil(c / 16)
 *                        near-equal pieces.  Without the delta rule (delta 0): every
 *                        segment of c chunks is cut into min(8, c) near-equal runs of
 *                        chunks, whose scalar or diagonal transitions make the fold an
 *                        elementwise weighted sum.  How a segment is cut depends on its
 *                        length only, so its pair does not depend on the other segments
 *                        of the call.  Without it (or where the query returns 0) every
 *                        segment is one serial chain.
 * Implemented:
 *   gate HEAD, TOKEN or DIAG, delta 0 : any d_k and d_v in {16, 32, 64, 128}, fp32 or
 *                                 bf16 inputs;
 *   gate TOKEN, delta 1 or 2    : d_k = 16, 32 or 64 (fp32 or bf16), 128 (bf16;
 *                                 fp32 at 128 would need 250 KiB of LDS);
 *   gate DIAG,  delta 1 or 2    : any d_k, bf16 inputs (d_k = 16 and 32 run on the
 *                                 d_k = 64 kernel with the key channels past d_k read
 *                                 as zeros);
 *   with the delta rule any d_v: the columns of S evolve independently (the
 *                                 erase and the gate act on its rows), so a state
 *                                 wider than d_k (d_v a multiple of d_k) is built as
 *                                 d_v / d_k blocks of d_k columns, one launch each, T
 *                                 with the first, and a narrower one in one launch
 *                                 whose missing value columns read as zeros and are not
 *                                 written; calls with d_v != d_k do not cut segments
 *                                 (the workspace is not used).
 * Other combinations return HYPIC_E_UNSUPPORTED.  For the delta-rule kernels
 * the state and values must stay within fp16 range (|entries| < 6e4): they are
 * fp16 operands of the matrix products (v itself with the scalar gate, beta * v
 * with the per-channel gate).  This is not checked (the call is asynchronous); an
 * operand beyond it is rounded to an infinity, never clamped to a finite value, so
 * the S of its (segment, head) comes out non-finite while T and the other
 * (segment, head) pairs are unaffected: S is either non-finite or accurate.  A
 * caller that cannot bound its values tests S for finite entries.
 */
hypic_status hypic_segment_build(const hypic_dims* dims, int32_t n_seg,
                                 const int64_t* seg_begin, const int64_t* seg_end,
                                 int64_t n_tokens, const void* k, const void* v,
                                 const void* g, const void* beta,
                                 void* T_out, float* S_out,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of build workspace that let hypic_segment_build cut long segments; 0 where it
 * would not (the workspace is then ignored).
 *   gate TOKEN with the delta rule, bf16 inputs, d in {64, 128}, n_tokens >= 1024: sized
 *     for segments that do not overlap, (2 d^2 4 bytes per head) per slot,
 *     floor(n_tokens / 1024) slots, plus the plan; a segment whose pieces do not fit is
 *     built uncut;
 *   without the delta rule, segments averaging at least 256 tokens (n_tokens >= 256 n_seg):
 *     8 pieces per (segment, head) of (d^2 + d) 4 bytes (diagonal gate; d^2 + 1 otherwise).
 *   other combinations: 0. */
size_t hypic_build_workspace_bytes(const hypic_dims* dims, int32_t n_seg, int64_t n_tokens);

/*
 * hypic_segment_prefill -- a segment's first (cold) prefill through the linear layer
 * with the pair built on the way ([ZH] 2.1: the pair is cached at the segment's first
 * prefill; each segment is prefilled in isolation, its state starting from zero): for
 * every segment i, head h and token t of [seg_begin[i], seg_end[i]),
 *     out[t][h][:] = S_t^T (scale * q_t),
 * S_t the state after token t (the first token starts from S = 0), plus the pair as
 * hypic_segment_build writes it (T_out may be NULL).  Rows of tokens outside the segments
 * are not written; segments must not overlap.  Segments are not cut (the outputs need
 * every token's prefix state).
 *   q     : [n_tokens][H][d_k], dtype in_dtype
 *   out   : fp32 [n_tokens][H][d_v]
 * Implemented: gate TOKEN, delta 1 or 2, bf16 inputs, d_k in {64, 128} and any d_v (as in
 * hypic_segment_build: column blocks of d_k, or one launch with zero-padded values below
 * d_k; output column n depends on state column n only); T layout DENSE or SPLIT.  Other combinations return
 * HYPIC_E_UNSUPPORTED.
 */
hypic_status hypic_segment_prefill(const hypic_dims* dims, int32_t n_seg,
                                   const int64_t* seg_begin, const int64_t* seg_end,
                                   int64_t n_tokens, const void* q, const void* k, const void* v,
                                   const void* g, const void* beta, float scale,
                                   void* T_out, float* S_out, float* out, void* stream);

/*
 * hypic_compose -- reuse of cached pairs ([ZH] 2.1: left-multiply by T_C,
 * then add): for every chain c, head h and step j = 0..n_step-1 in order,
 * with id = pair_id[c][j],
 *     S_run[c][h] <- T[id][h] S_run[c][h] + S[id][h]      (0 <= id < n_pair)
 * and nothing for other ids.  A chain is one request's running state in one
 * linear layer; several layers go in one call as separate chains whose ids
 * index that layer's part of the caches.
 *   pair_id : int32 [n_chain][n_step]
 *   T_cache : in the dims' t_layout (any of the four, any d_k and d_v)
 *   S_run   : fp32 [n_chain][H][d_k][d_v], read and written in place
 * Each chain is composed step after step.  For a few long chains, hypic_seam_advance with
 * no windows (every seam_start -1) composes the same pairs as a blocked scan in a caller
 * workspace (faster from about 50 steps on for one chain of 16 heads at d = 128).
 */
hypic_status hypic_compose(const hypic_dims* dims, int32_t n_chain, int32_t n_step,
                           const int32_t* pair_id, int32_t n_pair,
                           const void* T_cache, const float* S_cache,
                           float* S_run, void* stream);

/*
 * hypic_seam_advance -- reuse with seam windows ([ZH] 2.2): for every chain c,
 * head h and step j in order:
 *   1. if s = seam_start[c][j] >= 0 (and s + w <= n_tokens), step the w tokens
 *      s .. s+w-1 from the running state with their own transitions and
 *      writes, and emit each token's output
 *          out[c][j][i][h][:] = S_after_token^T (scale * q_{s+i})
 *      (output rows of steps without a seam are not written);
 *   2. if pair_id is not NULL and 0 <= pair_id[c][j] < n_pair, compose with
 *      that cached pair as in hypic_compose.
 * Internal segments cache tokens [start + w, end) and pass their first w
 * tokens here as the seam window; the final state equals the full recurrence.
 *   seam_start : int64 [n_chain][n_step], -1 = no seam at this step
 *   w          : 1..16 (the pages' default is 8)
 *   out        : fp32 [n_chain][n_step][w][H][d_v]
 *   workspace  : device scratch of hypic_seam_workspace_bytes(...) bytes,
 *                owned by the caller, 256-byte aligned; contents are
 *                overwritten; concurrent calls need distinct workspaces.
 *   T_cache    : t_layout DENSE or SPLIT
 * Implemented: gate TOKEN, delta 1 or 2, d_k and d_v in {16, 32, 64, 128}.  The columns of
 * the state, of the pairs' S, of the windows' values and of the outputs evolve
 * independently: a state wider than d_k advances in d_v / d_k blocks of d_k columns, one
 * after the other through the same workspace (sized for one block), a narrower one in one
 * pass whose column blocks end at its last column.
 */
hypic_status hypic_seam_advance(const hypic_dims* dims, int32_t n_chain, int32_t n_step,
                                int32_t w, const int64_t* seam_start, int64_t n_tokens,
                                const void* q, const void* k, const void* v,
                                const void* g, const void* beta, float scale,
                                const int32_t* pair_id, int32_t n_pair,
                                const void* T_cache, const float* S_cache,
                                float* S_run, float* out,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace hypic_seam_advance needs (0 on invalid dims). */
size_t hypic_seam_workspace_bytes(const hypic_dims* dims, int32_t n_chain, int32_t n_step,
                                  int32_t w);

/*
 * hypic_seam_advance_noalloc -- for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation, arguments and results as hypic_seam_advance, with the workspace taken from a
 * static device array of the library instead of the caller.
 *   - The array holds HYPIC_NOALLOC_SCRATCH_BYTES (128 MiB) on every device the library
 *     runs on, from its first use there until the process ends; a call whose
 *     hypic_seam_workspace_bytes exceeds that returns HYPIC_E_INVALID before any launch
 *     (e.g. 1 chain x 128 steps x 16 heads at d = 128 needs 107.5 MiB).
 *   - The device is the stream's (the current device for the NULL stream).  The call
 *     allocates nothing: no hipMalloc, hipFree or allocating library routine.
 *   - Every call on one device uses that device's one array, so calls that overlap on a
 *     device (other streams, other threads) race; serialise them.  The array keeps the last
 *     call's contents; nothing in it needs to start cleared.
 */
#define HYPIC_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
hypic_status hypic_seam_advance_noalloc(const hypic_dims* dims, int32_t n_chain, int32_t n_step,
                                        int32_t w, const int64_t* seam_start, int64_t n_tokens,
                                        const void* q, const void* k, const void* v,
                                        const void* g, const void* beta, float scale,
                                        const int32_t* pair_id, int32_t n_pair,
                                        const void* T_cache, const float* S_cache,
                                        float* S_run, float* out, void* stream);

/* Message for the last non-OK status returned on the calling thread ("" if none). */
const char* hypic_last_error(void);

/* HYPIC_ABI_VERSION of the loaded library. */
int32_t hypic_abi_version(void);

/*
 * Diagnostic, not part of the method: runs one wave that exercises the MFMA
 * lane layouts, the accumulator-to-operand lane shuffle and the global-to-LDS
 * direct loads the kernels rely on.  Reads 256 floats from the device buffer
 * `in`, writes 2112 floats to the device buffer `out` (layout documented in
 * the library source).  The test-suite recomputes the expected values.
 */
hypic_status hypic_selftest_layouts(const float* in, float* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* HYPIC_H */
