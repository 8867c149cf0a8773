// seam_chain.hip -- a request's running state stepped through its seam windows and
// cached pairs (hypic_seam_advance).
//
// Per step j of a chain ([ZH] = the Chinese HYPIC page, sections 2.1 and 2.2): if the
// step has a seam window, its w tokens are run on the running state R with their fresh
// inputs and emit their outputs; then the cached pair (T_j, S_j) of the rest of the
// segment is applied.  With the state-independent window factors prepared by seam.hip
// (Wt, U, Mo and the decays e^b, e^{b_w-b}, e^{b_w}) the window is the chunk form of the
// gated delta rule:
//     U'  = U - diag(e^b) (Wt R),        U'' = diag(e^{b_w - b}) U'
//     O   = scale diag(e^b) (Q R) + Mo U'                  (window outputs)
//     R_w = e^{b_w} R + K^T U''                            (state after the window)
// and the step ends with T_j R_w + S_j.  The kernel folds the two:
//     R_{j+1} = e^{b_w} (T_j R) + P_j U'' + S_j,     P_j = T_j K^T  (d_k x 16),
// so a step takes two products from R -- T_j R on the row waves, Wt R on the window
// wave, side by side -- and one rank-16 product once U'' is known: two workgroup
// barriers per step.  P_j depends only on cached and window data; the row waves form
// it while the window wave works out U''.
//
// One workgroup per (chain, head, 16-column block of the state): d_k/16 row waves (one
// 16-row tile of the state each; the state stays in fp32 accumulators) plus one window
// wave.  Blocks of one (chain, head) are placed on one XCD so T_j is fetched from HBM
// once and served to the others from L2.  Operands are bf16 hi/lo pairs and every
// product is taken as hi*hi + hi*lo + lo*hi (relative error ~2^-16 per step, fp32
// exponent range).  Data movement: each row wave loads T_{j+1} and S_{j+1} into
// registers during step j; at the top of step j the window wave fetches the window
// factors of step j+2 into one of three LDS stages (global->LDS direct loads), before
// the row waves' loads fill the queue.
#include "hypic_device.h"
#include "hypic_kernels.h"
#include "seam_layout.h"

namespace hypic {

namespace {

constexpr unsigned kWaitAll = 0x0070;           // s_waitcnt: vmcnt = 0, lgkmcnt = 0
constexpr int kRing = 512, kRingFill = 256;     // LDS ring of per-step pair ids / seam starts
constexpr int kStages = 3;                      // window factors are fetched two steps ahead

// B fragment of the identity for k-block ks and columns r0 .. r0+15: lane (g, n) holds
// rows 32 ks + 8 g + j (j = 0..7) of column r0 + n, as bf16.
__device__ __forceinline__ u32x4 ident_bfrag(int r0, int ks, int g4, int n16)
{
    const int d = r0 + n16 - (ks * 32 + 8 * g4);
    unsigned w[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) w[x] = (d == 2 * x ? 0x3F80u : 0u) | (d == 2 * x + 1 ? 0x3F800000u : 0u);
    return u32x4{w[0], w[1], w[2], w[3]};
}

// hi / lo B fragments of a 16 x 16 D tile used as the k = 0..15 half of a 32-deep k-block
__device__ __forceinline__ void dtile_bfrags(const f32x4& d, bf16x8& hi, bf16x8& lo)
{
    unsigned h0, h1, l0, l1;
    pack_bf16_split(d, h0, h1, l0, l1);
    hi = as_frag<bf16x8>(dtiles_to_bfrag(h0, h1, 0u, 0u));
    lo = as_frag<bf16x8>(dtiles_to_bfrag(l0, l1, 0u, 0u));
}

}  // namespace

template <int DK, bool TS>
__global__ __launch_bounds__(64 * (DK / 16 + 1)) void seam_chain_kernel(
    int n_units, int H, int n_step, const int32_t* __restrict__ pair_id, int n_pair,
    const void* __restrict__ Tc, const float* __restrict__ Sc, float* __restrict__ Srun, SeamArgs sa)
{
    constexpr int DV = DK;
    constexpr int NR = DK / 16;                 // row waves
    constexpr int KP = DK < 32 ? 32 : DK;       // contraction length padded to the MFMA K
    constexpr int KS = KP / 32;
    constexpr int LDB = KP + 8;                 // LDS row of the R planes (16-bit units), padded
    constexpr int NCB = DV / 16;
    // record offsets as kernel-scope constants (used inside lambdas)
    constexpr int kRecW = SeamRec<DK>::kW, kRecQ = SeamRec<DK>::kQ, kRecK = SeamRec<DK>::kK;
    constexpr int kRecM = SeamRec<DK>::kM, kRecU = SeamRec<DK>::kU, kRecEbL = SeamRec<DK>::kEbL;
    constexpr int kRecEbwL = SeamRec<DK>::kEbwL, kRecEbW = SeamRec<DK>::kEbW;
    constexpr int kPlaneWD = SeamRec<DK>::kPlaneWD, kPlaneM = SeamRec<DK>::kPlaneM;
    constexpr int kRecBytes = SeamRec<DK>::kBytes;

    __shared__ __attribute__((aligned(16))) uint16_t Rh[16][LDB];   // R, bf16 hi, [column][row]
    __shared__ __attribute__((aligned(16))) uint16_t Rl[16][LDB];   // R, bf16 lo
    __shared__ __attribute__((aligned(16))) u32x4 Uf[2][64];        // U'' B fragment hi / lo, lane order
    __shared__ int ring_id[kRing];
    __shared__ int64_t ring_s0[kRing];
    // window factors, fragment / lane ordered as fetched (lane l's 16 bytes at 16 l)
    __shared__ __attribute__((aligned(16))) u32x4 sk[kStages][KS][2][64];   // K (token-major) hi / lo
    __shared__ __attribute__((aligned(16))) u32x4 sw[kStages][KS][2][64];   // Wt hi / lo
    __shared__ __attribute__((aligned(16))) u32x4 sq[kStages][KS][2][64];   // q hi / lo
    __shared__ __attribute__((aligned(16))) u32x4 sm[kStages][2][64];       // Mo hi / lo
    __shared__ __attribute__((aligned(16))) f32x4 su[kStages][3][64];       // U block, e^{b_w-b}, e^b
    __shared__ float sebw[kStages][64];                                     // e^{b_w}

    const UnitSlot us = xcd_unit_slot(blockIdx.x, NCB);
    if (us.unit >= n_units) return;
    const int c = us.unit / H, h = us.unit % H, cb = us.sub;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool win = wave == NR;                // the window wave
    const int rt = win ? 0 : wave;              // a row wave's 16-row tile
    const int g4 = lane >> 4, n16 = lane & 15;
    const bool f32in = !sa.in_bf16;


    float* Rg = Srun + ((size_t)c * H + h) * DK * DV + cb * 16;
    f32x4 acc = zero4();   // row waves: rows rt*16 + 4 g4 + e, column n16 of the block
    auto store_split = [&]() {
        unsigned h0, h1, l0, l1;
        pack_bf16_split(acc, h0, h1, l0, l1);
        *reinterpret_cast<u32x2*>(&Rh[n16][rt * 16 + 4 * g4]) = u32x2{h0, h1};
        *reinterpret_cast<u32x2*>(&Rl[n16][rt * 16 + 4 * g4]) = u32x2{l0, l1};
    };

    const int32_t* ids = pair_id ? pair_id + (size_t)c * n_step : nullptr;
    const int64_t* seams = sa.seam_start + (size_t)c * n_step;
    auto fill_ring = [&](int base) {   // steps [base, base + 256)
        for (int x = threadIdx.x; x < kRingFill; x += blockDim.x) {
            const int j = base + x;
            ring_id[j & (kRing - 1)] = (j < n_step && ids) ? ids[j] : -1;
            ring_s0[j & (kRing - 1)] = j < n_step ? seams[j] : -1;
        }
    };
    // validated, wave-uniform pair id and seam start of step j
    auto read_id = [&](int j) -> int {
        const int id = ring_id[j & (kRing - 1)];
        return __builtin_amdgcn_readfirstlane((unsigned)id < (unsigned)n_pair ? id : -1);
    };
    auto read_s0 = [&](int j) -> int64_t {
        int64_t s0 = ring_s0[j & (kRing - 1)];
        s0 = (s0 >= 0 && s0 + sa.w <= sa.n_tokens) ? s0 : -1;
        return (int64_t)(((uint64_t)__builtin_amdgcn_readfirstlane((unsigned)((uint64_t)s0 >> 32)) << 32) |
                         (uint64_t)__builtin_amdgcn_readfirstlane((unsigned)(uint64_t)s0));
    };
    for (int i = threadIdx.x; i < 16 * LDB; i += blockDim.x) {   // rows DK..KP-1 stay zero
        (&Rh[0][0])[i] = 0;
        (&Rl[0][0])[i] = 0;
    }
    fill_ring(0);
    fill_ring(kRingFill);
    __syncthreads();
    if (!win) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = Rg[(size_t)(rt * 16 + 4 * g4 + e) * DV + n16];
        store_split();
    }

    // ---- row waves: T_j rows (A operand; as B operand of P^T = K T^T) and the S_j tile
    struct Step {
        u32x4 th[TS ? KS : 1], tl[TS ? KS : 1];   // bf16 hi / lo planes, fragment order
        float ta[TS ? 1 : KS][8];                 // fp32 rows
        float sv[4];
    };
    auto load_rows = [&](int id, Step& st) {
        if (id < 0) return;   // uniform
        const float* S = Sc + ((size_t)id * H + h) * DK * DV + cb * 16;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int k0 = KP == DK ? ks * 32 + 8 * g4 : min(ks * 32 + 8 * g4, DK - 8);   // clamped; zeroed at use
            if constexpr (TS) {   // the wave reads 1 KiB contiguous per plane and k-block
                const uint16_t* T = reinterpret_cast<const uint16_t*>(Tc) + ((size_t)id * H + h) * 2 * DK * DK;
                const int e = frag_off(rt * 16 + n16, k0, DK);
                st.th[ks] = *reinterpret_cast<const u32x4*>(T + e);
                st.tl[ks] = *reinterpret_cast<const u32x4*>(T + DK * DK + e);
            } else {
                const float* T = reinterpret_cast<const float*>(Tc) + ((size_t)id * H + h) * DK * DK +
                                 (size_t)(rt * 16 + n16) * DK + k0;
                const f32x4 a = reinterpret_cast<const f32x4*>(T)[0], b = reinterpret_cast<const f32x4*>(T)[1];
#pragma unroll
                for (int x = 0; x < 4; ++x) { st.ta[ks][x] = a[x]; st.ta[ks][4 + x] = b[x]; }
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) st.sv[e] = S[(size_t)(rt * 16 + 4 * g4 + e) * DV + n16];
    };
    auto t_frags = [&](const Step& st, int ks, bf16x8& ah, bf16x8& al) {
        if constexpr (TS) {
            ah = as_frag<bf16x8>(st.th[ks]);
            al = as_frag<bf16x8>(st.tl[ks]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                __bf16 x, y;
                split_bf16(st.ta[ks][e], x, y);
                ah[e] = x;
                al[e] = y;
            }
        }
        if (KP > DK && ks * 32 + 8 * g4 >= DK) {   // columns past d_k (the loads were clamped)
            ah = as_frag<bf16x8>(u32x4{0, 0, 0, 0});
            al = ah;
        }
    };

    // ---- window wave: window factors of step j into stage j % 3 (global->LDS direct loads)
    auto fetch_window = [&](int j) {
        if (j >= n_step) return;
        const int64_t s0 = read_s0(j);
        if (s0 < 0) return;   // uniform
        const int s = j % kStages;
        const unsigned char* rec =
            reinterpret_cast<const unsigned char*>(sa.ws) + (((size_t)c * n_step + j) * H + h) * kRecBytes;
        auto item = [&](const unsigned char* src, void* slot, bool on, int size = 16) {
            if (on) {
                if (size == 16)
                    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)slot, 16, 0, 0);
                else
                    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)slot, 4, 0, 0);
            }
        };
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int k0 = (ks * 32 + 8 * g4) < DK ? ks * 32 + 8 * g4 : 0;   // past DK: B rows are zero
            const int off = frag_off(n16, k0, DK) * 2;
#pragma unroll
            for (int p = 0; p < 2; ++p) {   // bf16 inputs have no lo part of k and q
                item(rec + kRecW + p * kPlaneWD + off, &sw[s][ks][p][0], true);
                item(rec + kRecK + p * kPlaneWD + off, &sk[s][ks][p][0], p == 0 || f32in);
                item(rec + kRecQ + p * kPlaneWD + off, &sq[s][ks][p][0], p == 0 || f32in);
            }
        }
#pragma unroll
        for (int p = 0; p < 2; ++p)   // lanes g4 >= 2 fetch a duplicate (zeroed at use)
            item(rec + kRecM + p * kPlaneM + frag_off(n16, 8 * (g4 & 1), 16) * 2, &sm[s][p][0], true);
        item(rec + kRecU + (cb * 64 + lane) * 16, &su[s][0][0], true);
        item(rec + kRecEbwL + lane * 16, &su[s][1][0], true);
        item(rec + kRecEbL + lane * 16, &su[s][2][0], true);
        item(rec + kRecEbW, &sebw[s][0], true, 4);
    };

    Step sA, sB;
    if (win) {
        fetch_window(0);
        fetch_window(1);
        __builtin_amdgcn_s_waitcnt(kWaitAll);
    } else {
        load_rows(read_id(0), sA);
    }
    lds_barrier();

    const u32x4 z4 = u32x4{0, 0, 0, 0};
    // The window wave and the row waves run separate loops (no register state is shared,
    // so neither carries the other's live values); each step both pass the same barriers.
    auto ring_refill = [&](int j) {
        if (j > 0 && (j & (kRingFill - 1)) == 0) {   // steps j+256 .. j+511 replace j-256 .. j-1
            fill_ring(j + kRingFill);
            lds_barrier();
        }
    };
    if (win) {
        __builtin_amdgcn_s_setprio(2);   // the window products are on the critical path of a step
        for (int j = 0; j < n_step; ++j) {
            ring_refill(j);
            const int64_t s0 = read_s0(j);
            const int s = j % kStages;
            // the factors of step j+1 (fetched during step j-1) and the output stores of
            // step j-1 are complete; fetch those of step j+2 before this step's products
            __builtin_amdgcn_s_waitcnt(kWaitAll);
            fetch_window(j + 2);
            if (s0 >= 0) {
                // Y = Wt R and Z = Q R (three / two accumulators), U' = U - diag(e^b) Y,
                // U'' = diag(e^{b_w-b}) U'
                bf16x8 rh[KS], rl[KS], wh[KS], wl[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    rh[ks] = *reinterpret_cast<const bf16x8*>(&Rh[n16][ks * 32 + 8 * g4]);
                    rl[ks] = *reinterpret_cast<const bf16x8*>(&Rl[n16][ks * 32 + 8 * g4]);
                    wh[ks] = as_frag<bf16x8>(sw[s][ks][0][lane]);
                    wl[ks] = as_frag<bf16x8>(sw[s][ks][1][lane]);
                }
                f32x4 y0 = zero4(), y1 = zero4(), y2 = zero4();
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    y0 = mma_bf16(wh[ks], rh[ks], y0);
                    y1 = mma_bf16(wh[ks], rl[ks], y1);
                    y2 = mma_bf16(wl[ks], rh[ks], y2);
                }
                const f32x4 y = y0 + (y1 + y2);
                const f32x4 u = su[s][0][lane], ebwb = su[s][1][lane], eb = su[s][2][lane];
                f32x4 u1, u2;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    u1[e] = u[e] - eb[e] * y[e];
                    u2[e] = ebwb[e] * u1[e];
                }
                bf16x8 u2h, u2l;
                dtile_bfrags(u2, u2h, u2l);
                Uf[0][lane] = __builtin_bit_cast(u32x4, u2h);
                Uf[1][lane] = __builtin_bit_cast(u32x4, u2l);
                lds_barrier();   // U'' visible to the row waves
                // outputs O = scale diag(e^b) (Q R) + Mo U'  (the padded window rows of q are zero)
                f32x4 z0 = zero4(), z1 = zero4();
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const bf16x8 qh = as_frag<bf16x8>(sq[s][ks][0][lane]);
                    z0 = mma_bf16(qh, rh[ks], z0);
                    z1 = mma_bf16(qh, rl[ks], z1);
                    if (f32in) z1 = mma_bf16(as_frag<bf16x8>(sq[s][ks][1][lane]), rh[ks], z1);
                }
                bf16x8 u1h, u1l;
                dtile_bfrags(u1, u1h, u1l);
                f32x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = sa.scale * eb[e] * (z0[e] + z1[e]);
                const bf16x8 mh = as_frag<bf16x8>(g4 < 2 ? sm[s][0][lane] : z4);
                const bf16x8 ml = as_frag<bf16x8>(g4 < 2 ? sm[s][1][lane] : z4);
                o = mma_bf16(mh, u1h, o);
                o = mma_bf16(mh, u1l, o);
                o = mma_bf16(ml, u1h, o);
                const size_t cj = (size_t)c * n_step + j;
                const int col = cb * 16 + n16;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 4 * g4 + e;
                    if (t < sa.w) sa.out[((cj * sa.w + t) * H + h) * DV + col] = o[e];
                }
            } else {
                lds_barrier();
            }
            lds_barrier();   // R_{j+1}
        }
        __builtin_amdgcn_s_waitcnt(kWaitAll);
        return;
    }

    // ---- row waves.  T_j / S_j in `cur` (loaded a step earlier), T_{j+1} / S_{j+1} into `nxt`.
    auto step = [&](int j, const Step& cur, Step& nxt) {
        ring_refill(j);
        const int id = read_id(j);
        const int64_t s0 = read_s0(j);
        const bool pair = id >= 0, seam = s0 >= 0;
        const int s = j % kStages;
        __builtin_amdgcn_s_waitcnt(kWaitAll);   // T_j, S_j
        f32x4 a = acc;
        bf16x8 ph, pl;
        if (pair) {   // T_j R, three accumulators
            f32x4 t0 = zero4(), t1 = zero4(), t2 = zero4();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                bf16x8 ah, al;
                t_frags(cur, ks, ah, al);
                const bf16x8 bh = *reinterpret_cast<const bf16x8*>(&Rh[n16][ks * 32 + 8 * g4]);
                const bf16x8 bl = *reinterpret_cast<const bf16x8*>(&Rl[n16][ks * 32 + 8 * g4]);
                t0 = mma_bf16(ah, bh, t0);
                t1 = mma_bf16(ah, bl, t1);
                t2 = mma_bf16(al, bh, t2);
            }
            a = t0 + (t1 + t2);
        }
        if (seam) {   // P^T = K T_j^T (K I^T without a pair), then the A fragments of P
            f32x4 p0 = zero4(), p1 = zero4();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                bf16x8 bh, bl;
                if (pair) {
                    t_frags(cur, ks, bh, bl);
                } else {
                    bh = as_frag<bf16x8>(ident_bfrag(rt * 16, ks, g4, n16));
                    bl = as_frag<bf16x8>(z4);
                }
                const bf16x8 kh = as_frag<bf16x8>(sk[s][ks][0][lane]);
                p0 = mma_bf16(kh, bh, p0);
                p1 = mma_bf16(kh, bl, p1);
                if (f32in) p1 = mma_bf16(as_frag<bf16x8>(sk[s][ks][1][lane]), bh, p1);
            }
            dtile_bfrags(p0 + p1, ph, pl);
            a = a * sebw[s][lane];
        }
        if (pair) {
#pragma unroll
            for (int e = 0; e < 4; ++e) a[e] += cur.sv[e];
        }
        // T_{j+1}, S_{j+1}: in flight across the rest of this step
        if (j + 1 < n_step) load_rows(read_id(j + 1), nxt);
        lds_barrier();   // U'' from the window wave
        if (seam) {
            const bf16x8 uh = as_frag<bf16x8>(Uf[0][lane]);
            const bf16x8 ul = as_frag<bf16x8>(Uf[1][lane]);
            a = mma_bf16(ph, uh, a);
            a = mma_bf16(ph, ul, a);
            a = mma_bf16(pl, uh, a);
        }
        acc = a;
        store_split();
        lds_barrier();   // R_{j+1} planes
    };

    for (int j = 0; j < n_step; j += 2) {
        step(j, sA, sB);
        if (j + 1 >= n_step) break;
        step(j + 1, sB, sA);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) Rg[(size_t)(rt * 16 + 4 * g4 + e) * DV + n16] = acc[e];
}

template <int DK, bool TS>
static hipError_t launch_seam_chain(int n_chain, int H, int n_step, const int32_t* pair_id, int n_pair,
                                    const void* Tc, const float* Sc, float* Srun, const SeamArgs& sa,
                                    hipStream_t st)
{
    const int n_units = n_chain * H;
    const int grid = xcd_grid_size(n_units, DK / 16);
    hipLaunchKernelGGL((seam_chain_kernel<DK, TS>), dim3(grid), dim3(64 * (DK / 16 + 1)), 0, st, n_units, H,
                       n_step, pair_id, n_pair, Tc, Sc, Srun, sa);
    return hipGetLastError();
}

hipError_t seam_chain(int d, int n_chain, int H, int n_step, const int32_t* pair_id, int n_pair,
                      const void* Tc, bool t_split, const float* Sc, float* Srun, const SeamArgs& sa,
                      hipStream_t st)
{
#define HYPIC_CASE(D_)                                                                                       \
    if (d == D_)                                                                                             \
        return t_split ? launch_seam_chain<D_, true>(n_chain, H, n_step, pair_id, n_pair, Tc, Sc, Srun, sa, st) \
                       : launch_seam_chain<D_, false>(n_chain, H, n_step, pair_id, n_pair, Tc, Sc, Srun, sa, st);
    HYPIC_CASE(16) HYPIC_CASE(32) HYPIC_CASE(64) HYPIC_CASE(128)
#undef HYPIC_CASE
    return hipErrorNotSupported;
}

}  // namespace hypic
