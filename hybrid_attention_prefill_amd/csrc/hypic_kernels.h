// hypic_kernels.h -- host-side launchers of the gfx950 kernels (internal to libhypic).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hypic {

// compose.hip
hipError_t compose_dense(int d, int n_chain, int H, int n_step, const int32_t* pair_id, int n_pair,
                         const float* Tc, const float* Sc, float* Srun, hipStream_t st);
hipError_t compose_scalar(int dk, int dv, int n_chain, int H, int n_step, const int32_t* pair_id,
                          int n_pair, const float* Tc, const float* Sc, float* Srun, hipStream_t st);

// build_gdn.hip (scalar gate, delta rule)
hipError_t build_gdn(int d, bool in_bf16, int n_seg, int H, const int64_t* sb, const int64_t* se,
                     int64_t n_tok, const void* k, const void* v, const void* g, const void* beta,
                     float* T_out, float* S_out, hipStream_t st);

// build_decay.hip (scalar gate or head-constant decay, no erase)
hipError_t build_decay(int d, bool in_bf16, bool head_gate, int n_seg, int H, const int64_t* sb,
                       const int64_t* se, int64_t n_tok, const void* k, const void* v, const void* g,
                       float* T_out, int t_scalar, float* S_out, hipStream_t st);

// selftest.hip
hipError_t selftest_layouts(float* out, hipStream_t st);

}  // namespace hypic
