// build_decay.hip -- segment build for transitions without the delta-rule erase:
// M_t = e^{g_t} I (g_t = log gamma_h for RetNet-style constant decay, or a
// per-token scalar log-gate as in Mamba2), write k_t v_t^T.  Here T_C = e^{sum g} I and
//     S(C|0) = sum_t e^{sum_{s>t} g_s} k_t v_t^T = K^T diag(w) V
// ([ZH] = the Chinese HYPIC page, section 2.1, which names RetNet among the
// decayed families whose segments need T_C and claims the whole linear-attention
// family).  For a constant decay gamma this is w_t = gamma^(L-1-t), the closed form.
// With a per-channel gate (GLA-style, M_t = diag(a_t)) the weights act on the key
// channels instead: S(C|0) = sum_t diag(e^{sum_{s>t} g_s}) k_t v_t^T and T_C =
// diag(e^{sum g}).
//
// Chunks of 64 tokens, in order: S <- e^{b_C} S + K^T diag(e^{b_C - b}) V with
// b the in-chunk cumulative log-gate, so every exponent is <= 0 (per channel:
// S <- diag(e^{b_C}) S + (e^{b_C - b} o K)^T V).  One
// workgroup (4 waves) per (segment, head); S tiles are dealt to waves and stay
// in fp32 MFMA accumulators.  The product runs on v_mfma_f32_16x16x32_bf16:
// the weighted V is split into bf16 hi + lo (bf16 keys are exact; fp32 keys
// are split too), keeping the fp32 exponent range for the tiny weights of
// fast-decaying heads.
#include "hypic_device.h"
#include "hypic_kernels.h"

namespace hypic {

namespace {
constexpr int CH = 64;
constexpr int LDT = CH + 8;

template <bool BF16>
__device__ __forceinline__ float ld1(const void* base, size_t e) {
    if constexpr (BF16) return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[e]);
    else return reinterpret_cast<const float*>(base)[e];
}
}  // namespace

template <int D, bool BF16, int GATE>
__global__ __launch_bounds__(256) void build_decay_kernel(
    int n_seg, int H, const int64_t* __restrict__ seg_begin, const int64_t* __restrict__ seg_end,
    int64_t n_tokens, const void* __restrict__ k, const void* __restrict__ v,
    const void* __restrict__ gl, void* __restrict__ T_out, int t_layout, float* __restrict__ S_out)
{
    constexpr bool DIAG = GATE == 2;       // per-channel gate: the weights move from V to K
    constexpr int RT = D / 16;
    constexpr int NT = RT * RT;            // output tiles
    constexpr int TW = (NT + 3) / 4;       // tiles per wave
    constexpr bool KSPLIT = !BF16 || DIAG; // keys need a lo plane (fp32, or weighted per channel)
    constexpr bool VSPLIT = !BF16 || !DIAG;
    __shared__ __attribute__((aligned(16))) uint16_t Kt[2][D][LDT];   // K^T (hi, lo); DIAG: weighted
    __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D][LDT];   // V^T (hi, lo); scalar: weighted
    __shared__ float gsh[CH], wsh[CH];
    __shared__ float gd[DIAG ? CH : 1][DIAG ? D + 1 : 1];   // DIAG: gates, then in-chunk cumulative sums
    __shared__ float bcd[DIAG ? D : 1], logd[DIAG ? D : 1];  // DIAG: chunk total and segment total per channel
    __shared__ float bCs;

    const int unit = blockIdx.x, seg = unit / H, h = unit % H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g4 = lane >> 4, n16 = lane & 15;
    int64_t beg = seg_begin[seg], end = seg_end[seg];
    beg = beg < 0 ? 0 : (beg > n_tokens ? n_tokens : beg);
    end = end < beg ? beg : (end > n_tokens ? n_tokens : end);

    f32x4 acc[TW];
#pragma unroll
    for (int i = 0; i < TW; ++i) acc[i] = zero4();
    float log_t = 0.f;
    const float ghead = GATE == 0 ? reinterpret_cast<const float*>(gl)[h] : 0.f;
    const size_t stride = (size_t)H * D;
    if constexpr (DIAG) {
        for (int ch = tid; ch < D; ch += 256) logd[ch] = 0.f;
    }

    for (int64_t c0 = beg; c0 < end; c0 += CH) {
        const int n = (int)((end - c0) < CH ? (end - c0) : CH);
        if constexpr (DIAG) {
            // per-channel gates, then the in-chunk inclusive cumulative sums b_t[ch] (one
            // channel per thread) and the chunk totals b_C[ch]
            for (int it = tid; it < CH * D; it += 256) {
                const int t = it / D, ch = it % D;
                gd[t][ch] = t < n ? ld1<BF16>(gl, (size_t)(c0 + t) * stride + (size_t)h * D + ch) : 0.f;
            }
            __syncthreads();
            for (int ch = tid; ch < D; ch += 256) {
                float x = 0.f;
                for (int t = 0; t < CH; ++t) {
                    x += gd[t][ch];
                    gd[t][ch] = x;
                }
                bcd[ch] = x;
                logd[ch] += x;
            }
        } else {
            if (tid < CH) {
                float gv = 0.f;
                if (tid < n) gv = GATE == 0 ? ghead : ld1<BF16>(gl, (size_t)(c0 + tid) * H + h);
                gsh[tid] = gv;
            }
            __syncthreads();
            if (wave == 0) {  // in-chunk inclusive cumsum; weight e^{b_C - b_t}
                float x = gsh[lane];
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const float y = __shfl_up(x, off, 64);
                    if (lane >= off) x += y;
                }
                const float bc = __shfl(x, 63, 64);
                wsh[lane] = lane < n ? expf(bc - x) : 0.f;
                if (lane == 0) bCs = bc;
            }
        }
        __syncthreads();
        for (int it = tid; it < CH * D; it += 256) {
            const int t = it / D, ch = it % D;  // consecutive threads: consecutive channels
            float kx = 0.f, vx = 0.f;
            if (t < n) {
                const size_t e = (size_t)(c0 + t) * stride + (size_t)h * D + ch;
                kx = ld1<BF16>(k, e);
                vx = ld1<BF16>(v, e);
                if constexpr (DIAG) kx *= expf(bcd[ch] - gd[t][ch]);   // key channel ch decays by e^{b_C - b_t}
                else vx *= wsh[t];
            }
            __bf16 kh, kl, vh, vl;
            split_bf16(kx, kh, kl);
            split_bf16(vx, vh, vl);
            Kt[0][ch][t] = bf16_bits(kh);
            Kt[1][ch][t] = bf16_bits(kl);
            Vt[0][ch][t] = bf16_bits(vh);
            Vt[1][ch][t] = bf16_bits(vl);
        }
        __syncthreads();
        const float ebc = DIAG ? 0.f : expf(bCs);
#pragma unroll
        for (int i = 0; i < TW; ++i) {
            const int tile = wave + 4 * i;
            if (tile >= NT) continue;
            const int mt = tile / RT, nt = tile % RT;  // key-channel tile, value-channel tile
            f32x4 a;
            if constexpr (DIAG) {   // row (key channel) m decays by e^{b_C[m]}
#pragma unroll
                for (int e = 0; e < 4; ++e) a[e] = acc[i][e] * expf(bcd[mt * 16 + 4 * g4 + e]);
            } else {
                a = acc[i] * ebc;
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 kh = *reinterpret_cast<const bf16x8*>(&Kt[0][mt * 16 + n16][ks * 32 + 8 * g4]);
                const bf16x8 vh = *reinterpret_cast<const bf16x8*>(&Vt[0][nt * 16 + n16][ks * 32 + 8 * g4]);
                a = mma_bf16(kh, vh, a);
                if constexpr (VSPLIT) {
                    const bf16x8 vl = *reinterpret_cast<const bf16x8*>(&Vt[1][nt * 16 + n16][ks * 32 + 8 * g4]);
                    a = mma_bf16(kh, vl, a);
                }
                if constexpr (KSPLIT) {
                    const bf16x8 kl = *reinterpret_cast<const bf16x8*>(&Kt[1][mt * 16 + n16][ks * 32 + 8 * g4]);
                    a = mma_bf16(kl, vh, a);
                }
            }
            acc[i] = a;
        }
        if constexpr (!DIAG) log_t += bCs;
        __syncthreads();
    }

    const size_t pair = (size_t)seg * H + h;
    float* S = S_out + pair * D * D;
#pragma unroll
    for (int i = 0; i < TW; ++i) {
        const int tile = wave + 4 * i;
        if (tile >= NT) continue;
        const int mt = tile / RT, nt = tile % RT;
#pragma unroll
        for (int e = 0; e < 4; ++e) S[(size_t)(mt * 16 + 4 * g4 + e) * D + nt * 16 + n16] = acc[i][e];
    }
    if (T_out) {
        if constexpr (DIAG) {
            if (t_layout == 3) {   // diagonal
                for (int ch = tid; ch < D; ch += 256) reinterpret_cast<float*>(T_out)[pair * D + ch] = expf(logd[ch]);
            } else {               // dense diag(t), fp32 or bf16 hi/lo planes
                for (int it = tid; it < D * D; it += 256)
                    put_t(T_out, t_layout == 2, pair, D, it / D, it % D, (it / D == it % D) ? expf(logd[it / D]) : 0.f);
            }
        } else {
            const float tval = expf(log_t);
            if (t_layout == 1) {   // scalar
                if (tid == 0) reinterpret_cast<float*>(T_out)[pair] = tval;
            } else {               // dense t I, fp32 or bf16 hi/lo planes
                for (int it = tid; it < D * D; it += 256)
                    put_t(T_out, t_layout == 2, pair, D, it / D, it % D, (it / D == it % D) ? tval : 0.f);
            }
        }
    }
}

template <int D, bool BF16, int GATE>
static hipError_t launch_decay(int n_seg, int H, const int64_t* sb, const int64_t* se, int64_t n_tok,
                               const void* k, const void* v, const void* g, void* T_out, int t_layout,
                               float* S_out, hipStream_t st)
{
    hipLaunchKernelGGL((build_decay_kernel<D, BF16, GATE>), dim3(n_seg * H), dim3(256), 0, st, n_seg, H,
                       sb, se, n_tok, k, v, g, T_out, t_layout, S_out);
    return hipGetLastError();
}

hipError_t build_decay(int d, bool in_bf16, int gate, int n_seg, int H, const int64_t* sb,
                       const int64_t* se, int64_t n_tok, const void* k, const void* v, const void* g,
                       void* T_out, int t_layout, float* S_out, hipStream_t st)
{
#define HYPIC_GATES(D_, B_)                                                                                  \
    if (gate == 0) return launch_decay<D_, B_, 0>(n_seg, H, sb, se, n_tok, k, v, g, T_out, t_layout, S_out, st); \
    if (gate == 1) return launch_decay<D_, B_, 1>(n_seg, H, sb, se, n_tok, k, v, g, T_out, t_layout, S_out, st); \
    return launch_decay<D_, B_, 2>(n_seg, H, sb, se, n_tok, k, v, g, T_out, t_layout, S_out, st);
#define HYPIC_CASE(D_)                    \
    if (d == D_) {                        \
        if (in_bf16) { HYPIC_GATES(D_, true) } \
        HYPIC_GATES(D_, false)            \
    }
    HYPIC_CASE(16) HYPIC_CASE(32) HYPIC_CASE(64) HYPIC_CASE(128)
#undef HYPIC_CASE
#undef HYPIC_GATES
    return hipErrorNotSupported;
}

}  // namespace hypic
