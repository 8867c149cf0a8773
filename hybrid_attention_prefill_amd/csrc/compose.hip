// compose.hip -- reuse of cached (T_C, S(C|0)) pairs along chains.
//
// The composition law of HYPIC ([ZH] = the Chinese HYPIC page, section 2.1):
// S(C1 C2) = T(C2) S(C1) + S(C2); on reuse the running state is left-multiplied
// by the cached T_C and the cached S(C|0) is added.  A chain is one request's
// running state in one linear layer, stepped through its cached segments.
//
// Dense T: one workgroup per (chain, head, block of NB state columns).  The
// product T S_run only couples rows, so column blocks are independent and every
// block needs all of T; the blocks of one (chain, head) are placed on the same
// XCD so T is fetched from HBM once and served to the others from L2.
// The running state stays in fp32 MFMA accumulators for the whole chain; each
// step it is re-split into bf16 hi + lo planes in LDS (the B operand), T is
// split the same way in registers (the A operand), and the product is taken as
// hi*hi + hi*lo + lo*hi on v_mfma_f32_16x16x32_bf16 (relative error ~2^-16,
// with fp32's exponent range, so tiny T entries are not flushed).
//
// With SEAM (hypic_seam_advance, [ZH] section 2.2) a step may first advance the
// state through its seam window using the state-independent window factors
// prepared by seam.hip: Y = Wt R and Z = scale Q R on MFMA, then the window
// outputs O = diag(e^b) Z + Mo U' and the rank-16 update
// R <- e^{b_w} R + K^T diag(e^{b_w-b}) U', U' = U - diag(e^b) Y.
#include "hypic_device.h"
#include "hypic_kernels.h"
#include "seam_layout.h"

namespace hypic {

template <int DK, int DV, int NB, bool SEAM>
__global__ __launch_bounds__(256) void compose_dense_kernel(
    int n_units, int H, int n_step, const int32_t* __restrict__ pair_id, int n_pair,
    const float* __restrict__ Tc, const float* __restrict__ Sc, float* __restrict__ Srun,
    SeamArgs sa)
{
    constexpr int NCB = DV / NB;
    constexpr int KP = DK < 32 ? 32 : DK;   // contraction length padded to the MFMA K
    constexpr int KS = KP / 32;
    constexpr int RT = DK / 16;             // 16-row tiles of the state
    constexpr int CT = NB / 16;             // 16-column tiles of the block
    constexpr int RTW = (RT + 3) / 4;       // row tiles per wave
    constexpr int LDB = KP + 8;             // LDS row length (16-bit units), padded
    __shared__ __attribute__((aligned(16))) uint16_t Rh[2][NB][LDB];
    __shared__ __attribute__((aligned(16))) uint16_t Rl[2][NB][LDB];
    // seam window: K^T (hi, lo; k = window token), U'' (hi, lo; k = window token),
    // Y and Z = scale Q R (fp32)
    constexpr int LDW = 32 + 8;
    constexpr int SW = SEAM ? 1 : 0;
    __shared__ __attribute__((aligned(16))) uint16_t Kw[2][SW ? DK : 1][LDW];
    __shared__ __attribute__((aligned(16))) uint16_t Uw[2][SW ? NB : 1][LDW];
    __shared__ float Ysh[SW ? kSeamMaxW : 1][NB + 1], Zsh[SW ? kSeamMaxW : 1][NB + 1];

    const UnitSlot us = xcd_unit_slot(blockIdx.x, NCB);
    if (us.unit >= n_units) return;
    const int c = us.unit / H, h = us.unit % H, cb = us.sub;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g4 = lane >> 4, n16 = lane & 15;

    if (KP > DK) {  // rows DK..KP-1 of the B operand stay zero
        for (int i = threadIdx.x; i < 2 * NB * LDB; i += blockDim.x) {
            (&Rh[0][0][0])[i] = 0;
            (&Rl[0][0][0])[i] = 0;
        }
    }
    if constexpr (SEAM) {  // window tokens 16..31 of the k = token operands stay zero
        for (int i = threadIdx.x; i < 2 * DK * LDW; i += blockDim.x) (&Kw[0][0][0])[i] = 0;
        for (int i = threadIdx.x; i < 2 * NB * LDW; i += blockDim.x) (&Uw[0][0][0])[i] = 0;
    }
    __syncthreads();

    float* Rg = Srun + ((size_t)c * H + h) * DK * DV + cb * NB;
    f32x4 acc[RTW][CT];
#pragma unroll
    for (int i = 0; i < RTW; ++i) {
        const int rt = wave + 4 * i;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            acc[i][ct] = zero4();
            if (rt < RT) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[i][ct][e] = Rg[(size_t)(rt * 16 + 4 * g4 + e) * DV + ct * 16 + n16];
            }
        }
    }

    auto store_split = [&](int buf) {
#pragma unroll
        for (int i = 0; i < RTW; ++i) {
            const int rt = wave + 4 * i;
            if (rt >= RT) continue;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                unsigned h0, h1, l0, l1;
                pack_bf16_split(acc[i][ct], h0, h1, l0, l1);
                const int col = ct * 16 + n16, row = rt * 16 + 4 * g4;
                *reinterpret_cast<u32x2*>(&Rh[buf][col][row]) = u32x2{h0, h1};
                *reinterpret_cast<u32x2*>(&Rl[buf][col][row]) = u32x2{l0, l1};
            }
        }
    };
    store_split(0);
    __syncthreads();

    // ---- one seam window (SEAM only): reads R from planes `buf`, leaves the
    // advanced state in the accumulators and in planes buf ^ 1.
    auto seam_step = [&](size_t cj, int64_t s0, int buf) {
        const float* rec = sa.ws + (cj * H + h) * SeamRec<DK>::kFloats;
        const size_t tok_base = (size_t)s0 * H * DK + (size_t)h * DK;
        auto ldin = [&](const void* base, size_t e) -> float {
            return sa.in_bf16 ? bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[e])
                              : reinterpret_cast<const float*>(base)[e];
        };
        // stage K^T of the window (k = token), split into bf16 hi + lo
        for (int it = threadIdx.x; it < kSeamMaxW * DK; it += blockDim.x) {
            const int t = it / DK, ch = it % DK;
            const float x = t < sa.w ? ldin(sa.k, tok_base + (size_t)t * H * DK + ch) : 0.f;
            __bf16 hi, lo;
            split_bf16(x, hi, lo);
            Kw[0][ch][t] = bf16_bits(hi);
            Kw[1][ch][t] = bf16_bits(lo);
        }
        // Y = Wt R (tile x < CT) and Z = scale Q R (tile x >= CT), 16 x NB each
        for (int x = wave; x < 2 * CT; x += 4) {
            const bool isz = x >= CT;
            const int ct = isz ? x - CT : x;
            f32x4 p = zero4();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int k0 = ks * 32 + 8 * g4;
                float a[8];
                if (k0 < DK) {
                    if (!isz) {
                        const f32x4* src = reinterpret_cast<const f32x4*>(rec + SeamRec<DK>::kWt + n16 * DK + k0);
                        const f32x4 x0 = src[0], x1 = src[1];
#pragma unroll
                        for (int e = 0; e < 4; ++e) { a[e] = x0[e]; a[4 + e] = x1[e]; }
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            a[e] = n16 < sa.w ? sa.scale * ldin(sa.q, tok_base + (size_t)n16 * H * DK + k0 + e) : 0.f;
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) a[e] = 0.f;
                }
                bf16x8 ah, al;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    __bf16 hi, lo;
                    split_bf16(a[e], hi, lo);
                    ah[e] = hi;
                    al[e] = lo;
                }
                const bf16x8 bh = *reinterpret_cast<const bf16x8*>(&Rh[buf][ct * 16 + n16][ks * 32 + 8 * g4]);
                const bf16x8 bl = *reinterpret_cast<const bf16x8*>(&Rl[buf][ct * 16 + n16][ks * 32 + 8 * g4]);
                p = mma_bf16(ah, bh, p);
                p = mma_bf16(ah, bl, p);
                p = mma_bf16(al, bh, p);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (isz) Zsh[4 * g4 + e][ct * 16 + n16] = p[e];
                else Ysh[4 * g4 + e][ct * 16 + n16] = p[e];
            }
        }
        __syncthreads();
        // window outputs and U'' = diag(e^{b_w - b}) U'  (k = token operand)
        const float* eb = rec + SeamRec<DK>::kEb;
        const float* ebw = rec + SeamRec<DK>::kEbw;
        const float* Mo = rec + SeamRec<DK>::kMo;
        const float* Ur = rec + SeamRec<DK>::kU;
        for (int it = threadIdx.x; it < kSeamMaxW * NB; it += blockDim.x) {
            const int t = it / NB, n = it % NB;
            const int col = cb * NB + n;
            float o = eb[t] * Zsh[t][n];
            for (int s = 0; s <= t; ++s) o += Mo[t * kSeamMaxW + s] * (Ur[s * DV + col] - eb[s] * Ysh[s][n]);
            if (t < sa.w) sa.out[((cj * sa.w + t) * H + h) * DV + col] = o;
            const float u2 = ebw[t] * (Ur[t * DV + col] - eb[t] * Ysh[t][n]);
            __bf16 hi, lo;
            split_bf16(u2, hi, lo);
            Uw[0][n][t] = bf16_bits(hi);
            Uw[1][n][t] = bf16_bits(lo);
        }
        __syncthreads();
        // R <- e^{b_w} R + K^T U''
        const float ebW = rec[SeamRec<DK>::kEbW];
#pragma unroll
        for (int i = 0; i < RTW; ++i) {
            const int rt = wave + 4 * i;
            if (rt >= RT) continue;
            const bf16x8 kh = *reinterpret_cast<const bf16x8*>(&Kw[0][rt * 16 + n16][8 * g4]);
            const bf16x8 kl = *reinterpret_cast<const bf16x8*>(&Kw[1][rt * 16 + n16][8 * g4]);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                const bf16x8 uh = *reinterpret_cast<const bf16x8*>(&Uw[0][ct * 16 + n16][8 * g4]);
                const bf16x8 ul = *reinterpret_cast<const bf16x8*>(&Uw[1][ct * 16 + n16][8 * g4]);
                f32x4 a = acc[i][ct] * ebW;
                a = mma_bf16(kh, uh, a);
                a = mma_bf16(kh, ul, a);
                a = mma_bf16(kl, uh, a);
                acc[i][ct] = a;
            }
        }
        store_split(buf ^ 1);
        __syncthreads();
    };

    int cur = 0;
    const int32_t* ids = pair_id ? pair_id + (size_t)c * n_step : nullptr;
    for (int j = 0; j < n_step; ++j) {
        if constexpr (SEAM) {
            const size_t cj = (size_t)c * n_step + j;
            const int64_t s0 = sa.seam_start[cj];
            if (s0 >= 0 && s0 + sa.w <= sa.n_tokens) {  // uniform over the workgroup
                seam_step(cj, s0, cur);
                cur ^= 1;
            }
        }
        const int id = ids ? ids[j] : -1;
        if ((unsigned)id >= (unsigned)n_pair) continue;  // uniform over the workgroup
        const float* T = Tc + ((size_t)id * H + h) * DK * DK;
        const float* S = Sc + ((size_t)id * H + h) * DK * DV + cb * NB;

        f32x4 p[RTW][CT];
#pragma unroll
        for (int i = 0; i < RTW; ++i)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) p[i][ct] = zero4();

#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            bf16x8 bh[CT], bl[CT];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                bh[ct] = *reinterpret_cast<const bf16x8*>(&Rh[cur][ct * 16 + n16][ks * 32 + 8 * g4]);
                bl[ct] = *reinterpret_cast<const bf16x8*>(&Rl[cur][ct * 16 + n16][ks * 32 + 8 * g4]);
            }
#pragma unroll
            for (int i = 0; i < RTW; ++i) {
                const int rt = wave + 4 * i;
                if (rt >= RT) continue;
                const int k0 = ks * 32 + 8 * g4;
                float a[8];
                if (k0 < DK) {
                    const f32x4* src = reinterpret_cast<const f32x4*>(T + (size_t)(rt * 16 + n16) * DK + k0);
                    const f32x4 x0 = src[0], x1 = src[1];
#pragma unroll
                    for (int e = 0; e < 4; ++e) { a[e] = x0[e]; a[4 + e] = x1[e]; }
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) a[e] = 0.f;
                }
                bf16x8 ah, al;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    __bf16 hi, lo;
                    split_bf16(a[e], hi, lo);
                    ah[e] = hi;
                    al[e] = lo;
                }
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    p[i][ct] = mma_bf16(ah, bh[ct], p[i][ct]);
                    p[i][ct] = mma_bf16(ah, bl[ct], p[i][ct]);
                    p[i][ct] = mma_bf16(al, bh[ct], p[i][ct]);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < RTW; ++i) {
            const int rt = wave + 4 * i;
            if (rt >= RT) continue;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[i][ct][e] = p[i][ct][e] + S[(size_t)(rt * 16 + 4 * g4 + e) * DV + ct * 16 + n16];
        }
        store_split(cur ^ 1);
        __syncthreads();
        cur ^= 1;
    }

#pragma unroll
    for (int i = 0; i < RTW; ++i) {
        const int rt = wave + 4 * i;
        if (rt >= RT) continue;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                Rg[(size_t)(rt * 16 + 4 * g4 + e) * DV + ct * 16 + n16] = acc[i][ct][e];
    }
}

// Scalar T (constant-decay families cache T_C = gamma^L I as one number):
// S_run <- t S_run + S, elementwise; 4 consecutive state entries per thread.
__global__ __launch_bounds__(256) void compose_scalar_kernel(
    int n_chain, int H, int DKV, int n_step, const int32_t* __restrict__ pair_id, int n_pair,
    const float* __restrict__ Tc, const float* __restrict__ Sc, float* __restrict__ Srun)
{
    const int per_unit = DKV / 4;  // float4 groups per (chain, head)
    const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long total = (long long)n_chain * H * per_unit;
    if (gid >= total) return;
    const int q = (int)(gid % per_unit);
    const long long unit = gid / per_unit;
    const int c = (int)(unit / H), h = (int)(unit % H);
    f32x4* R = reinterpret_cast<f32x4*>(Srun + unit * (long long)DKV) + q;
    f32x4 r = *R;
    const int32_t* ids = pair_id + (size_t)c * n_step;
    for (int j = 0; j < n_step; ++j) {
        const int id = ids[j];
        if ((unsigned)id >= (unsigned)n_pair) continue;
        const float t = Tc[(size_t)id * H + h];
        const f32x4 s = reinterpret_cast<const f32x4*>(Sc + ((size_t)id * H + h) * DKV)[q];
        r = t * r + s;
    }
    *R = r;
}

// ---------------------------------------------------------------- launchers
static constexpr int KP_OF(int dk) { return dk < 32 ? 32 : dk; }

template <int DK, int DV, int NB>
static hipError_t launch_dense(int n_chain, int H, int n_step, const int32_t* pair_id, int n_pair,
                               const float* Tc, const float* Sc, float* Srun, const SeamArgs* sa,
                               hipStream_t st)
{
    const int n_units = n_chain * H;
    const int grid = xcd_grid_size(n_units, DV / NB);
    if (sa) {
        // the seam path's extra LDS does not fit beside a full-width 128-column block
        if constexpr (NB * KP_OF(DK) <= 64 * 128)
            hipLaunchKernelGGL((compose_dense_kernel<DK, DV, NB, true>), dim3(grid), dim3(256), 0, st,
                               n_units, H, n_step, pair_id, n_pair, Tc, Sc, Srun, *sa);
        else
            return hipErrorInvalidValue;
    } else
        hipLaunchKernelGGL((compose_dense_kernel<DK, DV, NB, false>), dim3(grid), dim3(256), 0, st,
                           n_units, H, n_step, pair_id, n_pair, Tc, Sc, Srun, SeamArgs{});
    return hipGetLastError();
}

// Column-block width: enough workgroups to cover the CUs when there are few
// chains (one long request), full width when there are many.
static int pick_nb(long long n_units, int dv)
{
    int nb = dv;
    while (nb > 16 && n_units * (dv / nb) < 1024) nb /= 2;
    return nb;
}

hipError_t compose_dense(int d, int n_chain, int H, int n_step, const int32_t* pair_id, int n_pair,
                         const float* Tc, const float* Sc, float* Srun, const SeamArgs* sa, hipStream_t st)
{
    int nb = pick_nb((long long)n_chain * H, d);
    if (sa && nb > 64) nb = 64;
#define HYPIC_CASE(D_, NB_) \
    if (d == D_ && nb == NB_) return launch_dense<D_, D_, NB_>(n_chain, H, n_step, pair_id, n_pair, Tc, Sc, Srun, sa, st);
    HYPIC_CASE(16, 16)
    HYPIC_CASE(32, 32) HYPIC_CASE(32, 16)
    HYPIC_CASE(64, 64) HYPIC_CASE(64, 32) HYPIC_CASE(64, 16)
    HYPIC_CASE(128, 128) HYPIC_CASE(128, 64) HYPIC_CASE(128, 32) HYPIC_CASE(128, 16)
#undef HYPIC_CASE
    return hipErrorInvalidValue;
}

hipError_t compose_scalar(int dk, int dv, int n_chain, int H, int n_step, const int32_t* pair_id,
                          int n_pair, const float* Tc, const float* Sc, float* Srun, hipStream_t st)
{
    const long long total = (long long)n_chain * H * (dk * dv / 4);
    const int grid = (int)((total + 255) / 256);
    hipLaunchKernelGGL(compose_scalar_kernel, dim3(grid), dim3(256), 0, st, n_chain, H, dk * dv,
                       n_step, pair_id, n_pair, Tc, Sc, Srun);
    return hipGetLastError();
}

}  // namespace hypic
