// hypic_kernels.h -- host-side launchers of the gfx950 kernels (internal to libhypic).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hypic {

// Seam-window arguments of the seam chain kernel (hypic_seam_advance).
struct SeamArgs {
    const int64_t* seam_start;  // [n_chain][n_step], -1 = none
    int64_t n_tokens;
    int w;
    int in_bf16;
    float scale;
    const void* q;
    const void* k;
    const void* ws;             // records of seam_prep (seam_layout.h)
    float* out;                 // [n_chain][n_step][w][H][ld]
    int ld = 0;                 // row length of S_cache, S_run and out: d_v of the caller's tensors,
                                // when they point at d columns of a wider state, or a narrower
                                // state's d_v < d (its missing columns are not computed) (0 = d)
    // blocked scan (nblk > 1): blocks of blk steps run at once (seam_chain.hip)
    int nblk = 1;
    int blk = 0;
    float* ox = nullptr;        // readouts of X at the windows: [n_chain][n_step][w][H][2 d_v]
    void* agg_T = nullptr;      // block aggregates, T as bf16 hi/lo planes [n_chain][nblk-1][H][2][d][d]
    float* agg_S = nullptr;     //                   S fp32 [n_chain][nblk-1][H][d][d]
};

// Launch plan of hypic_seam_advance and the byte offsets of its workspace parts:
// window records at 0, then (blocked scan only) the readouts, aggregates and the
// trail of block entry states.
struct SeamPlan {
    int nb;        // state columns per workgroup of the chain kernel
    int nblk;      // blocks of steps per chain (1: the plain chain)
    int blk;       // steps per block
    size_t ox_off, agg_t_off, agg_s_off, trail_off, bytes;
};

// compose.hip
// t_split: T as bf16 hi/lo planes [n_pair][H][2][dk][dk]; else fp32 [n_pair][H][dk][dk];
// S fp32 [n_pair][H][dk][dv].  pair_id NULL: step j of chain c applies pair c * n_step + j.
// trail (may be NULL): the state before each step, fp32 [n_chain][n_step][H][dk][dv].
// r_ld: row length of Srun when it holds dv columns of a wider state (0 = dv)
hipError_t compose_dense(int dk, int dv, int n_chain, int H, int n_step, const int32_t* pair_id, int n_pair,
                         const void* Tc, bool t_split, const float* Sc, float* Srun, float* trail,
                         hipStream_t st, int r_ld = 0);
// diag: T cached as fp32 [n_pair][H][dk] (T = diag(t)); else fp32 [n_pair][H] (T = t I)
hipError_t compose_scalar(int dk, int dv, bool diag, int n_chain, int H, int n_step, const int32_t* pair_id,
                          int n_pair, const float* Tc, const float* Sc, float* Srun, hipStream_t st);

// Build kernels: t_split writes T as bf16 hi/lo planes [n_seg][H][2][d][d].
// Items mode of the GDN build (out != NULL): the n_seg ranges are the plan's items, of
// which the first *n_items are live; item i writes its pair to slot out[i] of T_out /
// S_out when out[i] >= 0, else to slot -1 - out[i] of T_ws (bf16 hi/lo planes) / S_ws.
struct BuildItems {
    const int32_t* n_items = nullptr;
    const int32_t* out = nullptr;
    void* T_ws = nullptr;
    float* S_ws = nullptr;
};
// Per-token outputs of the GDN build (out != NULL; bf16 inputs, d 64 or 128, uncut):
// out[t][h][:] = S_t^T (scale q_t), S_t the state after token t from S = 0 at the
// segment's first token.
struct BuildOut {
    const void* q = nullptr;
    float scale = 0.f;
    float* out = nullptr;
};
// build_gdn.hip (scalar gate, delta rule)
// v_ld: row length of v and S_out when they are d-column blocks of a wider state (0 = d).
hipError_t build_gdn(int d, bool in_bf16, int n_seg, int H, const int64_t* sb, const int64_t* se,
                     int64_t n_tok, const void* k, const void* v, const void* g, const void* beta,
                     void* T_out, bool t_split, float* S_out, const BuildItems& items, const BuildOut& ob,
                     hipStream_t st, int v_ld = 0);

// build_split.hip: long segments built as pieces in parallel and folded by composition
// (GDN, d in {64, 128}).  Workspace bytes for (d, H, n_seg, n_tokens); 0 = never cut.
size_t split_workspace_bytes(int d, int H, int n_seg, int64_t n_tokens);
hipError_t build_gdn_split(int d, bool in_bf16, int n_seg, int H, const int64_t* sb, const int64_t* se,
                           int64_t n_tok, const void* k, const void* v, const void* g, const void* beta,
                           void* T_out, bool t_split, float* S_out, void* ws, hipStream_t st);

// build_kda.hip (per-channel gate, delta rule; bf16 inputs)
hipError_t build_kda(int d, bool in_bf16, bool gate_first, int n_seg, int H, const int64_t* sb, const int64_t* se, int64_t n_tok,
                     const void* k, const void* v, const void* g, const void* beta, void* T_out, bool t_split,
                     float* S_out, hipStream_t st, int v_ld = 0);

// build_decay.hip (gate: 0 head-constant, 1 per-token scalar, 2 per-channel; no erase);
// t_layout: 0 dense f32, 1 scalar, 2 dense bf16 hi/lo planes, 3 diagonal.  ws (may be NULL):
// decay_workspace_bytes(...) bytes; segments are then built as up to 8 pieces in parallel
// and the pieces composed.  The bytes are 0 where pieces would not pay.
size_t decay_workspace_bytes(int dk, int dv, int H, int n_seg, int64_t n_tokens, bool diag);
hipError_t build_decay(int dk, int dv, bool in_bf16, int gate, int n_seg, int H, const int64_t* sb,
                       const int64_t* se, int64_t n_tok, const void* k, const void* v, const void* g,
                       void* T_out, int t_layout, float* S_out, void* ws, hipStream_t st);

// seam.hip
// v_ld: row length of v when it points at d columns of wider values (0 = d)
hipError_t seam_prep(int d, int n_chain, int n_step, int H, const int64_t* seam_start, int64_t n_tokens,
                     int w, const void* q, const void* k, const void* v, const void* g, const void* beta,
                     bool in_bf16, float scale, void* ws, hipStream_t st, int v_ld = 0);
size_t seam_record_bytes(int d);

// seam_chain.hip (pair_id may be NULL: windows only)
// dv: the state's columns when fewer than d (0: d); the column blocks then end at its last column
SeamPlan seam_plan(int d, int n_chain, int H, int n_step, int w, int dv = 0);
hipError_t seam_chain(int d, int nb, int n_chain, int H, int n_step, const int32_t* pair_id, int n_pair,
                      const void* Tc, bool t_split, const float* Sc, float* Srun, const SeamArgs& sa,
                      hipStream_t st);
hipError_t seam_readout(int d, int n_chain, int H, int n_step, int nblk, int blk, int w,
                        const int64_t* seam_start, int64_t n_tokens, const float* ox, const float* trail,
                        float* out, hipStream_t st, int ld = 0);

// selftest.hip
hipError_t selftest_layouts(const float* in, float* out, hipStream_t st);

}  // namespace hypic
