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
// step it is re-split into bf16 hi + lo planes in LDS (the B operand).  T is the
// A operand, as bf16 hi + lo planes: cached that way by the build kernels (T layout
// SPLIT, loaded as is) or split in registers from fp32.  The product is taken as
// hi*hi + hi*lo + lo*hi on v_mfma_f32_16x16x32_bf16 (relative error ~2^-16, with
// fp32's exponent range, so tiny T entries are not flushed).
// (hypic_seam_advance, which also steps seam windows, runs seam_chain.hip.)
#include "hypic_device.h"
#include "hypic_kernels.h"

namespace hypic {

// s_waitcnt immediate (gfx9 encoding) that waits for every outstanding vector-memory
// operation and every LDS access: vmcnt = 0, expcnt = 7 (unconstrained), lgkmcnt = 0.
constexpr unsigned kWaitVmcnt0 = 0x0070;
constexpr int kRing = 512, kRingFill = 256;   // LDS ring of per-step pair ids

// waves per workgroup: one 16-row tile of the state per wave at d_k = 128
constexpr int chain_waves(int dk) { return dk >= 128 ? 8 : 4; }

// TS: T cached as bf16 hi/lo planes ([n_pair][H][2][DK][DK], hypic_t_layout SPLIT),
// fed to the MFMA units as loaded; otherwise fp32 T, split in registers.
template <int DK, int DV, int NB, bool TS>
__global__ __launch_bounds__(64 * chain_waves(DK)) void compose_dense_kernel(
    int n_units, int H, int n_step, const int32_t* __restrict__ pair_id, int n_pair,
    const void* __restrict__ Tc, const float* __restrict__ Sc, float* __restrict__ Srun, float* __restrict__ trail)
{
    constexpr int NCB = DV / NB;
    constexpr int KP = DK < 32 ? 32 : DK;   // contraction length padded to the MFMA K
    constexpr int KS = KP / 32;
    constexpr int RT = DK / 16;             // 16-row tiles of the state
    constexpr int CT = NB / 16;             // 16-column tiles of the block
    constexpr int NW = chain_waves(DK);
    constexpr int RTW = (RT + NW - 1) / NW; // row tiles per wave
    constexpr int LDB = KP + 8;             // LDS row length (16-bit units), padded
    __shared__ __attribute__((aligned(16))) uint16_t Rh[2][NB][LDB];   // R, bf16 hi, [column][row]
    __shared__ __attribute__((aligned(16))) uint16_t Rl[2][NB][LDB];   // R, bf16 lo
    __shared__ int ring_id[kRing];

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
    __syncthreads();

    float* Rg = Srun + ((size_t)c * H + h) * DK * DV + cb * NB;
    f32x4 acc[RTW][CT];
#pragma unroll
    for (int i = 0; i < RTW; ++i) {
        const int rt = wave + NW * i;
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
            const int rt = wave + NW * i;
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
    auto rfrag = [&](const uint16_t (*P)[LDB], int col, int k0) -> bf16x8 {
        return *reinterpret_cast<const bf16x8*>(&P[col][k0]);
    };

    // ---- everything a step reads besides the running state, loaded one step ahead into
    // one of two register sets (the loop is unrolled by two, so the sets never get copied)
    struct Step {
        int id;                                        // pair index, or -1
        u32x4 th[TS ? RTW : 1][TS ? KS : 1];           // T rows of this wave, bf16 hi (A operand)
        u32x4 tl[TS ? RTW : 1][TS ? KS : 1];           //                      bf16 lo
        float ta[TS ? 1 : RTW][TS ? 1 : KS][8];        // T rows, fp32
        float sv[RTW][CT][4];                          // S block (D layout)
    };
    // without an id array, step j of chain c applies pair c * n_step + j
    const int32_t* ids = pair_id ? pair_id + (size_t)c * n_step : nullptr;
    // Pair ids go through an LDS ring of 512 steps, filled 256 steps ahead, so the per-step
    // lookups are LDS reads and never wait on the vector-memory counter.
    auto fill_ring = [&](int base) {   // steps [base, base + 256)
        for (int x = threadIdx.x; x < kRingFill; x += blockDim.x) {
            const int j = base + x;
            ring_id[j & (kRing - 1)] = j < n_step ? (ids ? ids[j] : c * n_step + j) : -1;
        }
    };
    // the state before step j, when the caller keeps the trail
    auto put_trail = [&](int j) {
        if (!trail) return;
        float* Tr = trail + (((size_t)c * n_step + j) * H + h) * DK * DV + cb * NB;
#pragma unroll
        for (int i = 0; i < RTW; ++i) {
            const int rt = wave + NW * i;
            if (rt >= RT) continue;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    Tr[(size_t)(rt * 16 + 4 * g4 + e) * DV + ct * 16 + n16] = acc[i][ct][e];
        }
    };
    auto read_id = [&](int j) -> int { return ring_id[j & (kRing - 1)]; };
    // The loads below are unconditional within a step that has a pair (addresses clamped
    // into the pair; lanes and waves outside the tile are masked where the values are
    // used): a load whose result is selected or copied right away makes the compiler wait
    // for it, and with the in-order vector-memory counter that would wait for the whole
    // prefetch.
    auto load_step = [&](int id, Step& st) {
        id = __builtin_amdgcn_readfirstlane((unsigned)id < (unsigned)n_pair ? id : -1);
        st.id = id;
        if (id >= 0) {
            const float* S = Sc + ((size_t)id * H + h) * DK * DV + cb * NB;
#pragma unroll
            for (int i = 0; i < RTW; ++i) {
                const int rt = (RTW * NW == RT) ? wave + NW * i : min(wave + NW * i, RT - 1);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int k0 = KP == DK ? ks * 32 + 8 * g4 : min(ks * 32 + 8 * g4, DK - 8);
                    if constexpr (TS) {   // fragment-ordered planes: the wave reads 1 KiB contiguous
                        const uint16_t* T = reinterpret_cast<const uint16_t*>(Tc) + ((size_t)id * H + h) * 2 * DK * DK;
                        const int e = frag_off(rt * 16 + n16, k0, DK);
                        st.th[i][ks] = *reinterpret_cast<const u32x4*>(T + e);
                        st.tl[i][ks] = *reinterpret_cast<const u32x4*>(T + DK * DK + e);
                    } else {
                        ld8f(reinterpret_cast<const float*>(Tc) + ((size_t)id * H + h) * DK * DK +
                             (size_t)(rt * 16 + n16) * DK + k0, st.ta[i][ks]);
                    }
                }
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        st.sv[i][ct][e] = S[(size_t)(rt * 16 + 4 * g4 + e) * DV + ct * 16 + n16];
            }
        }
    };

    // ---- R <- T R + S on the planes `buf` (result in the accumulators); the three
    // products hi*hi, hi*lo, lo*hi go to separate accumulators (shorter dependency chains)
    auto compose_step = [&](const Step& st, int buf) {
#pragma unroll
        for (int i = 0; i < RTW; ++i) {
            const int rt = wave + NW * i;
            if (rt >= RT) continue;
            // separate accumulators only where the column tiles give too little independent work
            constexpr int NA = CT >= 4 ? 1 : 3;
            f32x4 p0[CT], p1[NA == 3 ? CT : 1], p2[NA == 3 ? CT : 1];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                p0[ct] = f32x4{st.sv[i][ct][0], st.sv[i][ct][1], st.sv[i][ct][2], st.sv[i][ct][3]};
                if constexpr (NA == 3) {
                    p1[ct] = zero4();
                    p2[ct] = zero4();
                }
            }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                bf16x8 ah, al;
                if constexpr (TS) {
                    ah = as_frag<bf16x8>(st.th[i][ks]);
                    al = as_frag<bf16x8>(st.tl[i][ks]);
                } else {
                    split8(st.ta[i][ks], ah, al);
                }
                if (KP > DK && ks * 32 + 8 * g4 >= DK) {   // columns past d_k (the loads were clamped)
                    ah = as_frag<bf16x8>(u32x4{0, 0, 0, 0});
                    al = ah;
                }
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    const bf16x8 bh = rfrag(Rh[buf], ct * 16 + n16, ks * 32 + 8 * g4);
                    const bf16x8 bl = rfrag(Rl[buf], ct * 16 + n16, ks * 32 + 8 * g4);
                    p0[ct] = mma_bf16(ah, bh, p0[ct]);
                    if constexpr (NA == 3) {
                        p1[ct] = mma_bf16(ah, bl, p1[ct]);
                        p2[ct] = mma_bf16(al, bh, p2[ct]);
                    } else {
                        p0[ct] = mma_bf16(ah, bl, p0[ct]);
                        p0[ct] = mma_bf16(al, bh, p0[ct]);
                    }
                }
            }
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                if constexpr (NA == 3) acc[i][ct] = p0[ct] + (p1[ct] + p2[ct]);
                else acc[i][ct] = p0[ct];
            }
        }
    };

    int cur = 0;
    auto run_step = [&](const Step& st) {
        if (st.id >= 0) {  // uniform over the workgroup
            compose_step(st, cur);
            store_split(cur ^ 1);
            lds_barrier();
            cur ^= 1;
        }
    };

    fill_ring(0);
    fill_ring(kRingFill);
    lds_barrier();
    Step sA, sB;
    int id1 = read_id(1);
    load_step(read_id(0), sA);
    // Every load of step j was issued a whole step earlier: wait for all of them once, at the
    // top of the step, then issue step j+1's loads.  (Using a value right after its load
    // would make the in-order vector-memory counter drain the prefetch as well.)
    for (int j = 0; j < n_step; j += 2) {
        // step j from sA; prefetch step j+1 into sB; id of step j+2
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        if (j > 0 && (j & (kRingFill - 1)) == 0) {  // steps j+256 .. j+511 replace steps j-256 .. j-1
            // Waves meet only at steps that have a pair, so after a run of skipped steps a
            // wave may still have to read the id of step j-1 (slot (j+255) & 511): every wave
            // gets here before any of them refills.
            lds_barrier();
            fill_ring(j + kRingFill);
            lds_barrier();
        }
        const int id2 = read_id(j + 2);
        if (j + 1 < n_step) load_step(id1, sB);
        put_trail(j);
        run_step(sA);
        if (j + 1 >= n_step) break;
        // step j+1 from sB; prefetch step j+2 into sA; id of step j+3
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        id1 = read_id(j + 3);
        if (j + 2 < n_step) load_step(id2, sA);
        put_trail(j + 1);
        run_step(sB);
    }

#pragma unroll
    for (int i = 0; i < RTW; ++i) {
        const int rt = wave + NW * i;
        if (rt >= RT) continue;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                Rg[(size_t)(rt * 16 + 4 * g4 + e) * DV + ct * 16 + n16] = acc[i][ct][e];
    }
}

// Scalar or diagonal T (gates without the delta rule cache T_C = t I as one number per
// (pair, head), or T_C = diag(t) for the per-channel gate): S_run <- T S_run + S is
// elementwise, S_run[r][c] <- t_r S_run[r][c] + S[r][c]; 4 consecutive state entries
// (one row) per thread.
template <bool DIAG>
__global__ __launch_bounds__(256) void compose_scalar_kernel(
    int n_chain, int H, int DK, int DV, int n_step, const int32_t* __restrict__ pair_id, int n_pair,
    const float* __restrict__ Tc, const float* __restrict__ Sc, float* __restrict__ Srun)
{
    const int per_unit = DK * DV / 4;  // float4 groups per (chain, head)
    const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long total = (long long)n_chain * H * per_unit;
    if (gid >= total) return;
    const int q = (int)(gid % per_unit);
    const int row = 4 * q / DV;
    const long long unit = gid / per_unit;
    const int c = (int)(unit / H), h = (int)(unit % H);
    f32x4* R = reinterpret_cast<f32x4*>(Srun + unit * (long long)(DK * DV)) + q;
    f32x4 r = *R;
    const int32_t* ids = pair_id + (size_t)c * n_step;
    // groups of 8 steps: the ids first, then every T and S of the group, then the updates
    // (the loads of a group are in flight together instead of one dependent pair per step)
    constexpr int G = 8;
    for (int j0 = 0; j0 < n_step; j0 += G) {
        int id[G];
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const int x = j0 + i < n_step ? ids[j0 + i] : -1;
            id[i] = (unsigned)x < (unsigned)n_pair ? x : -1;
        }
        float t[G];
        f32x4 sv[G];
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const size_t p = (size_t)(id[i] < 0 ? 0 : id[i]) * H + h;   // a skipped step reads pair 0, unused
            t[i] = n_pair > 0 ? (DIAG ? Tc[p * DK + row] : Tc[p]) : 1.f;
            sv[i] = n_pair > 0 ? reinterpret_cast<const f32x4*>(Sc + p * DK * DV)[q] : zero4();
        }
#pragma unroll
        for (int i = 0; i < G; ++i)
            if (id[i] >= 0) r = t[i] * r + sv[i];
    }
    *R = r;
}

// ---------------------------------------------------------------- launchers
template <int DK, int DV, int NB, bool TS>
static hipError_t launch_dense(int n_chain, int H, int n_step, const int32_t* pair_id, int n_pair,
                               const void* Tc, const float* Sc, float* Srun, float* trail, hipStream_t st)
{
    const int n_units = n_chain * H;
    const int grid = xcd_grid_size(n_units, DV / NB);
    hipLaunchKernelGGL((compose_dense_kernel<DK, DV, NB, TS>), dim3(grid), dim3(64 * chain_waves(DK)), 0, st,
                       n_units, H, n_step, pair_id, n_pair, Tc, Sc, Srun, trail);
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
                         const void* Tc, bool t_split, const float* Sc, float* Srun, float* trail,
                         hipStream_t st)
{
    const int nb = pick_nb((long long)n_chain * H, d);
#define HYPIC_CASE(D_, NB_)                                                                                   \
    if (d == D_ && nb == NB_)                                                                                 \
        return t_split                                                                                        \
                   ? launch_dense<D_, D_, NB_, true>(n_chain, H, n_step, pair_id, n_pair, Tc, Sc, Srun, trail, st) \
                   : launch_dense<D_, D_, NB_, false>(n_chain, H, n_step, pair_id, n_pair, Tc, Sc, Srun, trail, st);
    HYPIC_CASE(16, 16)
    HYPIC_CASE(32, 32) HYPIC_CASE(32, 16)
    HYPIC_CASE(64, 64) HYPIC_CASE(64, 32) HYPIC_CASE(64, 16)
    HYPIC_CASE(128, 128) HYPIC_CASE(128, 64) HYPIC_CASE(128, 32) HYPIC_CASE(128, 16)
#undef HYPIC_CASE
    return hipErrorInvalidValue;
}

hipError_t compose_scalar(int dk, int dv, bool diag, int n_chain, int H, int n_step, const int32_t* pair_id,
                          int n_pair, const float* Tc, const float* Sc, float* Srun, hipStream_t st)
{
    const long long total = (long long)n_chain * H * (dk * dv / 4);
    const int grid = (int)((total + 255) / 256);
    if (diag)
        hipLaunchKernelGGL(compose_scalar_kernel<true>, dim3(grid), dim3(256), 0, st, n_chain, H, dk, dv,
                           n_step, pair_id, n_pair, Tc, Sc, Srun);
    else
        hipLaunchKernelGGL(compose_scalar_kernel<false>, dim3(grid), dim3(256), 0, st, n_chain, H, dk, dv,
                           n_step, pair_id, n_pair, Tc, Sc, Srun);
    return hipGetLastError();
}

}  // namespace hypic
