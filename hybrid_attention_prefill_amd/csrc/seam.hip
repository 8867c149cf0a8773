// seam.hip -- state-independent preparation of the seam windows.
//
// [ZH] (the Chinese HYPIC page), section 2.2: the first w tokens of every
// internal segment are kept out of the cache; at reuse the linear layers work
// out the window's own transition and state, advance the running state with
// it and send each window token's output to the attention layer above.
//
// For a window of w <= 16 tokens (padded to 16 with no-op tokens), with b the
// in-window cumulative log-gate and At = (I + Lt)^-1, Lt[t][s] = b_t k_t.k_s
// (s < t), everything that does not depend on the running state R is
//     Wt[t] = sum_s At[t][s] beta_s k_s                 (16 x d_k)
//     U[t]  = sum_s e^{b_t-b_s} At[t][s] beta_s v_s     (16 x d_v)
//     Mo[t][s] = scale e^{b_t-b_s} (q_t . k_s), s <= t  (16 x 16)
// and the chain kernel then needs only (design notes: chunk form, in-chunk
// outputs):
//     U' = U - diag(e^b) (Wt R)
//     O  = diag(e^b) (scale Q R) + Mo U'                 (window outputs)
//     R <- e^{b_w} R + K^T diag(e^{b_w - b}) U'          (state after the window)
// One workgroup per (chain, step, head) window, fp32 on the vector ALUs.
#include "hypic_device.h"
#include "hypic_kernels.h"
#include "seam_layout.h"

namespace hypic {

template <int D>
__global__ __launch_bounds__(256) void seam_prep_kernel(
    int n_cj, int H, const int64_t* __restrict__ seam_start, int64_t n_tokens, int w,
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const void* __restrict__ gl, const void* __restrict__ beta, int in_bf16, float scale,
    float* __restrict__ ws)
{
    constexpr int W = kSeamMaxW;
    __shared__ float Ks[W][D + 1], Vs[W][D + 1], Qs[W][D + 1];
    __shared__ float gs[W], bs[W], bt[W], Lt[W][W + 1], At[W][W + 1];

    const int rec = blockIdx.x;             // (cj, h)
    const int cj = rec / H, h = rec % H;
    const int tid = threadIdx.x;
    const int64_t s0 = seam_start[cj];
    if (s0 < 0 || s0 + w > n_tokens) return;  // uniform: no seam at this step

    auto ld = [&](const void* base, size_t e) -> float {
        return in_bf16 ? bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[e])
                       : reinterpret_cast<const float*>(base)[e];
    };
    for (int it = tid; it < W * D; it += 256) {
        const int t = it / D, ch = it % D;
        const bool ok = t < w;
        const size_t e = (size_t)(s0 + t) * H * D + (size_t)h * D + ch;
        Ks[t][ch] = ok ? ld(k, e) : 0.f;
        Vs[t][ch] = ok ? ld(v, e) : 0.f;
        Qs[t][ch] = ok ? scale * ld(q, e) : 0.f;
    }
    if (tid < W) {
        const bool ok = tid < w;
        const size_t e = (size_t)(s0 + tid) * H + h;
        gs[tid] = ok ? ld(gl, e) : 0.f;
        bt[tid] = ok ? ld(beta, e) : 0.f;
    }
    __syncthreads();
    float* rp = ws + (size_t)rec * SeamRec<D>::kFloats;
    if (tid == 0) {  // cumsum over the (<= 16) window tokens
        float acc = 0.f;
        for (int t = 0; t < W; ++t) { acc += gs[t]; bs[t] = acc; }
    }
    __syncthreads();
    {   // Lt and Mo: one (t, s) pair per thread
        const int t = tid / W, s = tid % W;
        float kk = 0.f, qk = 0.f;
        for (int ch = 0; ch < D; ++ch) {
            kk += Ks[t][ch] * Ks[s][ch];
            qk += Qs[t][ch] * Ks[s][ch];
        }
        Lt[t][s] = (s < t) ? bt[t] * kk : 0.f;
        rp[SeamRec<D>::kMo + t * W + s] = (s <= t) ? expf(bs[t] - bs[s]) * qk : 0.f;
        if (s == 0) {
            rp[SeamRec<D>::kEb + t] = expf(bs[t]);
            rp[SeamRec<D>::kEbw + t] = expf(bs[W - 1] - bs[t]);
        }
        if (tid == 0) rp[SeamRec<D>::kEbW] = expf(bs[W - 1]);
    }
    __syncthreads();
    if (tid < W) {  // At = (I + Lt)^-1, column `tid`, forward substitution
        float x[W];
#pragma unroll
        for (int r = 0; r < W; ++r) {
            float s = (r == tid) ? 1.f : 0.f;
#pragma unroll
            for (int c = 0; c < r; ++c) s -= Lt[r][c] * x[c];
            x[r] = s;
        }
#pragma unroll
        for (int r = 0; r < W; ++r) At[r][tid] = x[r];
    }
    __syncthreads();
    for (int it = tid; it < W * D; it += 256) {  // window keys, channel-major, for the state update
        const int ch = it / W, t = it % W;
        rp[SeamRec<D>::kKt + ch * W + t] = Ks[t][ch];
    }
    for (int it = tid; it < W * D; it += 256) {
        const int t = it / D, ch = it % D;
        float wk = 0.f, uv = 0.f;
        for (int s = 0; s <= t; ++s) {
            const float a = At[t][s] * bt[s];
            wk += a * Ks[s][ch];
            uv += a * expf(bs[t] - bs[s]) * Vs[s][ch];
        }
        rp[SeamRec<D>::kWt + t * D + ch] = wk;
        rp[SeamRec<D>::kU + t * D + ch] = uv;
    }
}

hipError_t seam_prep(int d, int n_chain, int n_step, int H, const int64_t* seam_start, int64_t n_tokens,
                     int w, const void* q, const void* k, const void* v, const void* g, const void* beta,
                     bool in_bf16, float scale, float* ws, hipStream_t st)
{
    const long long n_rec = (long long)n_chain * n_step * H;
    if (n_rec == 0) return hipSuccess;
#define HYPIC_CASE(D_)                                                                                       \
    if (d == D_) {                                                                                           \
        hipLaunchKernelGGL(seam_prep_kernel<D_>, dim3((unsigned)n_rec), dim3(256), 0, st, n_chain * n_step, \
                           H, seam_start, n_tokens, w, q, k, v, g, beta, (int)in_bf16, scale, ws);           \
        return hipGetLastError();                                                                            \
    }
    HYPIC_CASE(16) HYPIC_CASE(32) HYPIC_CASE(64) HYPIC_CASE(128)
#undef HYPIC_CASE
    return hipErrorNotSupported;
}

size_t seam_record_floats(int d)
{
    switch (d) {
    case 16: return SeamRec<16>::kFloats;
    case 32: return SeamRec<32>::kFloats;
    case 64: return SeamRec<64>::kFloats;
    case 128: return SeamRec<128>::kFloats;
    default: return 0;
    }
}

}  // namespace hypic
