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
#include "build_common.h"

namespace hypic {
using bld::FragB;
using bld::dpair_to_fragb;

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
    constexpr int LDW = 32 + 8;
    constexpr int SW = SEAM ? 1 : 0;
    constexpr int W16 = kSeamMaxW;
    static_assert(!SEAM || CT <= 4, "seam epilogue: one wave per column tile");
    __shared__ __attribute__((aligned(16))) uint16_t Rh[2][NB][LDB];   // R, bf16 hi, [column][row]
    __shared__ __attribute__((aligned(16))) uint16_t Rl[2][NB][LDB];   // R, bf16 lo
    __shared__ __attribute__((aligned(16))) uint16_t Uh[SW ? NB : 1][LDW];   // U'' hi, [column][token]
    __shared__ __attribute__((aligned(16))) uint16_t Ul[SW ? NB : 1][LDW];

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
    if constexpr (SEAM) {  // window tokens 16..31 of the k = token operand stay zero
        for (int i = threadIdx.x; i < NB * LDW; i += blockDim.x) {
            (&Uh[0][0])[i] = 0;
            (&Ul[0][0])[i] = 0;
        }
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

    auto ldin8 = [&](const void* base, size_t e, float* out) {
        if (sa.in_bf16) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(base) + e);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                out[2 * x] = __uint_as_float(w[x] << 16);
                out[2 * x + 1] = __uint_as_float(w[x] & 0xFFFF0000u);
            }
        } else {
            const f32x4* p = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(base) + e);
            const f32x4 a = p[0], b = p[1];
#pragma unroll
            for (int x = 0; x < 4; ++x) { out[x] = a[x]; out[4 + x] = b[x]; }
        }
    };
    auto ld8f = [&](const float* p, float* out) {
        const f32x4 a = reinterpret_cast<const f32x4*>(p)[0], b = reinterpret_cast<const f32x4*>(p)[1];
#pragma unroll
        for (int x = 0; x < 4; ++x) { out[x] = a[x]; out[4 + x] = b[x]; }
    };
    auto split8 = [&](const float* a, bf16x8& hi, bf16x8& lo) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            __bf16 x, y;
            split_bf16(a[e], x, y);
            hi[e] = x;
            lo[e] = y;
        }
    };

    // ---- what a step's first products read (T rows, window Wt and q rows): loaded one step ahead.
    // The rest of a step's inputs (S block, window factors and keys) is loaded when the step
    // starts; its latency overlaps the step's MFMAs.
    struct Step {
        int id;          // pair index, or -1
        int64_t s0;      // seam window start, or -1
        float ta[RTW][KS][8];      // T rows of this wave (A operand)
        float wt[SW ? KS : 1][8];  // Wt row (A operand), waves < CT
        float qa[SW ? KS : 1][8];  // scale * q row (A operand), waves < CT
    };
    const int32_t* ids = pair_id ? pair_id + (size_t)c * n_step : nullptr;
    auto load_step = [&](int j, Step& st) {
        st.id = ids ? ids[j] : -1;
        if ((unsigned)st.id >= (unsigned)n_pair) st.id = -1;
        st.s0 = -1;
        if constexpr (SEAM) {
            const int64_t s0 = sa.seam_start[(size_t)c * n_step + j];
            if (s0 >= 0 && s0 + sa.w <= sa.n_tokens) st.s0 = s0;
        }
        if (st.id >= 0) {
            const float* T = Tc + ((size_t)st.id * H + h) * DK * DK;
#pragma unroll
            for (int i = 0; i < RTW; ++i) {
                const int rt = wave + 4 * i;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int k0 = ks * 32 + 8 * g4;
                    if (rt < RT && k0 < DK) ld8f(T + (size_t)(rt * 16 + n16) * DK + k0, st.ta[i][ks]);
                    else
#pragma unroll
                        for (int e = 0; e < 8; ++e) st.ta[i][ks][e] = 0.f;
                }
            }
        }
        if constexpr (SEAM) {
            if (st.s0 >= 0 && wave < CT) {
                const size_t cj = (size_t)c * n_step + j;
                const float* rec = sa.ws + (cj * H + h) * SeamRec<DK>::kFloats;
                const size_t tok = (size_t)(st.s0 + n16) * H * DK + (size_t)h * DK;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int k0 = ks * 32 + 8 * g4;
                    if (k0 < DK) {
                        ld8f(rec + SeamRec<DK>::kWt + n16 * DK + k0, st.wt[ks]);
                        if (n16 < sa.w) {
                            ldin8(sa.q, tok + k0, st.qa[ks]);
#pragma unroll
                            for (int e = 0; e < 8; ++e) st.qa[ks][e] *= sa.scale;
                        } else {
#pragma unroll
                            for (int e = 0; e < 8; ++e) st.qa[ks][e] = 0.f;
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e) { st.wt[ks][e] = 0.f; st.qa[ks][e] = 0.f; }
                    }
                }
            }
        }
    };

    // ---- R <- T R + S on the planes `buf` (result in the accumulators)
    auto compose_step = [&](const Step& st, int buf) {
        const float* S = Sc + ((size_t)st.id * H + h) * DK * DV + cb * NB;
#pragma unroll
        for (int i = 0; i < RTW; ++i) {
            const int rt = wave + 4 * i;
            if (rt >= RT) continue;
            float sv[CT][4];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) sv[ct][e] = S[(size_t)(rt * 16 + 4 * g4 + e) * DV + ct * 16 + n16];
            f32x4 p[CT];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) p[ct] = zero4();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                bf16x8 ah, al;
                split8(st.ta[i][ks], ah, al);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    const bf16x8 bh = *reinterpret_cast<const bf16x8*>(&Rh[buf][ct * 16 + n16][ks * 32 + 8 * g4]);
                    const bf16x8 bl = *reinterpret_cast<const bf16x8*>(&Rl[buf][ct * 16 + n16][ks * 32 + 8 * g4]);
                    p[ct] = mma_bf16(ah, bh, p[ct]);
                    p[ct] = mma_bf16(ah, bl, p[ct]);
                    p[ct] = mma_bf16(al, bh, p[ct]);
                }
            }
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][ct][e] = p[ct][e] + sv[ct][e];
        }
    };

    // ---- one seam window on the planes `buf`: outputs, then R <- e^{b_w} R + K^T U''
    auto seam_step = [&](const Step& st, int buf, size_t cj) {
        const float* rec = sa.ws + (cj * H + h) * SeamRec<DK>::kFloats;
        const float ebW = rec[SeamRec<DK>::kEbW];
        float kt[RTW][8];   // window K^T rows of this wave (A operand, k = token)
#pragma unroll
        for (int i = 0; i < RTW; ++i) {
            const int rt = wave + 4 * i;
            if (rt < RT && g4 < 2) ld8f(rec + SeamRec<DK>::kKt + (rt * 16 + n16) * W16 + 8 * g4, kt[i]);
            else
#pragma unroll
                for (int e = 0; e < 8; ++e) kt[i][e] = 0.f;
        }
        if (wave < CT) {
            const int ct = wave;
            float mo[8], ur[4], eb[4], ebw[4];
            if (g4 < 2) ld8f(rec + SeamRec<DK>::kMo + n16 * W16 + 8 * g4, mo);
            else
#pragma unroll
                for (int e = 0; e < 8; ++e) mo[e] = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 4 * g4 + e;
                ur[e] = rec[SeamRec<DK>::kU + t * DV + cb * NB + ct * 16 + n16];
                eb[e] = rec[SeamRec<DK>::kEb + t];
                ebw[e] = rec[SeamRec<DK>::kEbw + t];
            }
            f32x4 y = zero4(), z = zero4();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 bh = *reinterpret_cast<const bf16x8*>(&Rh[buf][ct * 16 + n16][ks * 32 + 8 * g4]);
                const bf16x8 bl = *reinterpret_cast<const bf16x8*>(&Rl[buf][ct * 16 + n16][ks * 32 + 8 * g4]);
                bf16x8 ah, al;
                split8(st.wt[ks], ah, al);
                y = mma_bf16(ah, bh, y);
                y = mma_bf16(ah, bl, y);
                y = mma_bf16(al, bh, y);
                split8(st.qa[ks], ah, al);
                z = mma_bf16(ah, bh, z);
                z = mma_bf16(ah, bl, z);
                z = mma_bf16(al, bh, z);
            }
            f32x4 u;   // U' = U - diag(e^b) Y, rows t = 4 g4 + e
#pragma unroll
            for (int e = 0; e < 4; ++e) u[e] = ur[e] - eb[e] * y[e];
            // O = diag(e^b) Z + Mo U'  (U' as the B operand, tokens 16..31 zero)
            const FragB ub = dpair_to_fragb(u, zero4());
            bf16x8 mh, ml;
            split8(mo, mh, ml);
            f32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = eb[e] * z[e];
            o = mma_bf16(mh, ub.h, o);
            o = mma_bf16(mh, ub.l, o);
            o = mma_bf16(ml, ub.h, o);
            const int col = cb * NB + ct * 16 + n16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 4 * g4 + e;
                if (t < sa.w) sa.out[((cj * sa.w + t) * H + h) * DV + col] = o[e];
            }
            f32x4 u2;
#pragma unroll
            for (int e = 0; e < 4; ++e) u2[e] = ebw[e] * u[e];
            unsigned h0, h1, l0, l1;
            pack_bf16_split(u2, h0, h1, l0, l1);
            *reinterpret_cast<u32x2*>(&Uh[ct * 16 + n16][4 * g4]) = u32x2{h0, h1};
            *reinterpret_cast<u32x2*>(&Ul[ct * 16 + n16][4 * g4]) = u32x2{l0, l1};
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < RTW; ++i) {
            const int rt = wave + 4 * i;
            if (rt >= RT) continue;
            bf16x8 kh, kl;
            split8(kt[i], kh, kl);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                const bf16x8 uh = *reinterpret_cast<const bf16x8*>(&Uh[ct * 16 + n16][8 * g4]);
                const bf16x8 ul = *reinterpret_cast<const bf16x8*>(&Ul[ct * 16 + n16][8 * g4]);
                f32x4 a = acc[i][ct] * ebW;
                a = mma_bf16(kh, uh, a);
                a = mma_bf16(kh, ul, a);
                a = mma_bf16(kl, uh, a);
                acc[i][ct] = a;
            }
        }
    };

    int cur = 0;
    Step st_cur;
    if (n_step > 0) load_step(0, st_cur);
    for (int j = 0; j < n_step; ++j) {
        Step st_nxt;
        if (j + 1 < n_step) load_step(j + 1, st_nxt);
        if constexpr (SEAM) {
            if (st_cur.s0 >= 0) {  // uniform over the workgroup
                seam_step(st_cur, cur, (size_t)c * n_step + j);
                store_split(cur ^ 1);
                __syncthreads();
                cur ^= 1;
            }
        }
        if (st_cur.id >= 0) {  // uniform over the workgroup
            compose_step(st_cur, cur);
            store_split(cur ^ 1);
            __syncthreads();
            cur ^= 1;
        }
        if (j + 1 < n_step) st_cur = st_nxt;
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
