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
// waves, side by side -- and one rank-16 product once U'' is known: two workgroup
// barriers per step.  P_j depends only on cached and window data; the row waves form
// it while the window waves work out U''.
//
// Every step is affine in R (R -> A_j R + B_j) and its outputs are an affine readout of
// the R it starts from (O_j = G_j R + H_j), so a long chain is also run as a blocked
// scan (the composition law applied to whole runs of steps):
//   1. this kernel runs every block of steps at once.  Block 0 starts from the chain's
//      running state and is the plain chain.  Block b >= 1 carries the augmented state
//      X = [Tx | Sx] (d_k x 2 d_v), from [I | 0]: the transition columns take the
//      window and the product with T_j but no U and no S_j.  At each window it writes
//      the readout of X (G_j Tx and G_j Sx + H_j: the same formula as the outputs) and
//      at the end the block's aggregate pair (Tx as bf16 hi/lo planes, Sx in fp32);
//   2. compose.hip composes the aggregates in order and keeps the state entering each
//      block;
//   3. seam_readout_kernel turns each readout into outputs, O_j = (G_j Tx) R_in + (G_j Sx + H_j).
// The block count is chosen so that the workgroups of phase 1 fit the GPU in one round.
//
// One workgroup per (chain, block, head, NB-column block of the state): d_k/16 row
// waves (one 16-row tile of the state each, NB/16 column tiles; the state stays in fp32
// accumulators) plus NB/16 window waves (one column tile each).  The column blocks of one (chain, block, head),
// transition and state halves alike, are placed on one XCD so T_j is fetched from HBM
// once and served to the others from L2.  Operands are bf16 hi/lo pairs and every
// product is taken as hi*hi + hi*lo + lo*hi (relative error ~2^-16 per step, fp32
// exponent range).  Data movement: each row wave loads T_{j+1} and S_{j+1} into the
// registers of T_j and S_j during step j, each k-block of T right after step j's products
// have read it; at the top of step j the first window wave fetches the window factors of
// step j+2 into one of three LDS stages (global->LDS direct loads), before the row waves'
// loads fill the queue.
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

template <int DK, bool TS, int NB>
__global__ __launch_bounds__(64 * (DK / 16 + NB / 16)) void seam_chain_kernel(
    int n_units, int H, int n_step, const int32_t* __restrict__ pair_id, int n_pair,
    const void* __restrict__ Tc, const float* __restrict__ Sc, float* __restrict__ Srun, SeamArgs sa)
{
    constexpr int DV = DK;
    constexpr int NR = DK / 16;                 // row waves
    constexpr int KP = DK < 32 ? 32 : DK;       // contraction length padded to the MFMA K
    constexpr int KS = KP / 32;
    constexpr int LDB = KP + 8;                 // LDS row of the R planes (16-bit units), padded
    constexpr int NCB = DV / NB;                // column blocks of the state
    constexpr int CT = NB / 16;                 // 16-column tiles of a block
    // record offsets as kernel-scope constants (used inside lambdas)
    constexpr int kRecW = SeamRec<DK>::kW, kRecQ = SeamRec<DK>::kQ, kRecK = SeamRec<DK>::kK;
    constexpr int kRecM = SeamRec<DK>::kM, kRecU = SeamRec<DK>::kU, kRecEbL = SeamRec<DK>::kEbL;
    constexpr int kRecEbwL = SeamRec<DK>::kEbwL, kRecEbW = SeamRec<DK>::kEbW;
    constexpr int kPlaneWD = SeamRec<DK>::kPlaneWD, kPlaneM = SeamRec<DK>::kPlaneM;
    constexpr int kRecBytes = SeamRec<DK>::kBytes;

    __shared__ __attribute__((aligned(16))) uint16_t Rh[NB][LDB];   // R, bf16 hi, [column][row]
    __shared__ __attribute__((aligned(16))) uint16_t Rl[NB][LDB];   // R, bf16 lo
    __shared__ __attribute__((aligned(16))) u32x4 Uf[CT][2][64];    // U'' B fragments hi / lo, lane order
    __shared__ int ring_id[kRing];
    __shared__ int64_t ring_s0[kRing];
    // window factors, fragment / lane ordered as fetched (lane l's 16 bytes at 16 l)
    __shared__ __attribute__((aligned(16))) u32x4 sk[kStages][KS][2][64];   // K (token-major) hi / lo
    __shared__ __attribute__((aligned(16))) u32x4 sw[kStages][KS][2][64];   // Wt hi / lo
    __shared__ __attribute__((aligned(16))) u32x4 sq[kStages][KS][2][64];   // q hi / lo
    __shared__ __attribute__((aligned(16))) u32x4 sm[kStages][2][64];       // Mo hi / lo
    __shared__ __attribute__((aligned(16))) f32x4 su[kStages][CT + 2][64];  // U tiles, e^{b_w-b}, e^b
    __shared__ float sebw[kStages][64];                                     // e^{b_w}
    __shared__ int zflag[2];   // transition columns: some entry of X nonzero after step j (slot j & 1)

    // ---- unit: (chain c, block b, head h); sub-block: a column block of the state, or
    // in blocks b >= 1 one of the transition half (sub < NCB) or of the state half
    const int nblk = sa.nblk;
    int unit, sub;
    if (nblk > 1) {
        // all transition-column workgroups are dispatched before the state-column ones
        // (they end early once their columns vanish); the sub-blocks of a unit share an XCD
        const int xcd = blockIdx.x & 7, li = blockIdx.x >> 3, ng = (n_units + 7) / 8;
        const int part = li / (ng * NCB), rem = li % (ng * NCB);
        unit = (rem / NCB) * 8 + xcd;
        sub = part * NCB + rem % NCB;
    } else {
        const UnitSlot us = xcd_unit_slot(blockIdx.x, NCB);
        unit = us.unit;
        sub = us.sub;
    }
    if (unit >= n_units) return;
    const int h = unit % H, cbk = unit / H;
    const int b = cbk % nblk, c = cbk / nblk;
    if (b == 0 && sub < NCB && nblk > 1) return;   // block 0 has state columns only (uniform)
    const bool tcol = b > 0 && sub < NCB;          // transition columns of X
    const int cb = sub % NCB;
    // a state narrower than DV (sa.ld < DV, a multiple of NB): its missing column blocks have
    // no work (the transition columns are all needed)
    if (!tcol && sa.ld < DV && cb * NB >= sa.ld) return;
    const int j0 = b * sa.blk, j1 = min(n_step, j0 + sa.blk);
    const size_t agg = (size_t)c * (nblk - 1) + (b - 1);   // aggregate slot of block b >= 1

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool win = wave >= NR;                // a window wave
    const int wct = win ? wave - NR : 0;        // a window wave's column tile
    const int rt = win ? 0 : wave;              // a row wave's 16-row tile
    const int g4 = lane >> 4, n16 = lane & 15;
    const bool f32in = !sa.in_bf16;

    // S_run, the pairs' S and the outputs have rows of sa.ld values (DV unless they hold DV
    // columns of a wider state); the workspace parts (readouts, aggregates) have rows of DV
    const int ld = sa.ld;
    float* Rg = Srun + ((size_t)c * H + h) * DK * ld + cb * NB;
    f32x4 acc[CT];   // row waves: rows rt*16 + 4 g4 + e, column ct*16 + n16 of the block
    auto store_split = [&]() {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            unsigned h0, h1, l0, l1;
            pack_bf16_split(acc[ct], h0, h1, l0, l1);
            *reinterpret_cast<u32x2*>(&Rh[ct * 16 + n16][rt * 16 + 4 * g4]) = u32x2{h0, h1};
            *reinterpret_cast<u32x2*>(&Rl[ct * 16 + n16][rt * 16 + 4 * g4]) = u32x2{l0, l1};
        }
    };

    const int32_t* ids = pair_id ? pair_id + (size_t)c * n_step : nullptr;
    const int64_t* seams = sa.seam_start + (size_t)c * n_step;
    auto fill_ring = [&](int base) {   // steps [base, base + 256)
        for (int x = threadIdx.x; x < kRingFill; x += blockDim.x) {
            const int j = base + x;
            ring_id[j & (kRing - 1)] = (j < j1 && ids) ? ids[j] : -1;
            ring_s0[j & (kRing - 1)] = j < j1 ? seams[j] : -1;
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
    for (int i = threadIdx.x; i < NB * LDB; i += blockDim.x) {   // rows DK..KP-1 stay zero
        (&Rh[0][0])[i] = 0;
        (&Rl[0][0])[i] = 0;
    }
    fill_ring(j0);
    fill_ring(j0 + kRingFill);
    if (threadIdx.x == 0) zflag[0] = zflag[1] = 0;
    __syncthreads();
    if (!win) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = rt * 16 + 4 * g4 + e, col = cb * NB + ct * 16 + n16;
                acc[ct][e] = b == 0 ? Rg[(size_t)row * ld + ct * 16 + n16] : (tcol && row == col ? 1.f : 0.f);
            }
        store_split();
    }

    // ---- row waves: T_j rows (A operand; as B operand of P^T = K T^T) and the S_j block
    struct Step {
        u32x4 th[TS ? KS : 1], tl[TS ? KS : 1];   // bf16 hi / lo planes, fragment order
        float ta[TS ? 1 : KS][8];                 // fp32 rows
        float sv[CT][4];
    };
    // k-block ks of this wave's rows of T_id, and this workgroup's block of S_id
    auto load_t = [&](int id, int ks, Step& st) {
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
    };
    auto load_s = [&](int id, Step& st) {
        if (!tcol) {   // uniform; the transition columns add no S
            const float* S = Sc + ((size_t)id * H + h) * DK * ld + cb * NB;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) st.sv[ct][e] = S[(size_t)(rt * 16 + 4 * g4 + e) * ld + ct * 16 + n16];
        }
    };
    auto load_rows = [&](int id, Step& st) {
        if (id < 0) return;   // uniform
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) load_t(id, ks, st);
        load_s(id, st);
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

    // ---- first window wave: window factors of step j into stage j % 3 (global->LDS direct loads)
    auto fetch_window = [&](int j) {
        if (j >= j1) return;
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
        // rows past the window (tokens w .. 15) are neither written by the preparation nor
        // fetched: their lanes' slots were zeroed once, at the start
        const bool row_on = n16 < sa.w;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int k0 = (ks * 32 + 8 * g4) < DK ? ks * 32 + 8 * g4 : 0;   // past DK: B rows are zero
            const int off = frag_off(n16, k0, DK) * 2;
#pragma unroll
            for (int p = 0; p < 2; ++p) {   // bf16 inputs have no lo part of k and q
                item(rec + kRecW + p * kPlaneWD + off, &sw[s][ks][p][0], row_on);
                item(rec + kRecK + p * kPlaneWD + off, &sk[s][ks][p][0], (p == 0 || f32in) && row_on);
                item(rec + kRecQ + p * kPlaneWD + off, &sq[s][ks][p][0], (p == 0 || f32in) && row_on);
            }
        }
#pragma unroll
        for (int p = 0; p < 2; ++p)   // lanes g4 >= 2 fetch a duplicate (zeroed at use)
            item(rec + kRecM + p * kPlaneM + frag_off(n16, 8 * (g4 & 1), 16) * 2, &sm[s][p][0], row_on);
        if (!tcol) {   // the transition columns take no U (lane (g4, n16): rows 4 g4 .. 4 g4 + 3)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
                item(rec + kRecU + ((cb * CT + ct) * 64 + lane) * 16, &su[s][ct][0], 4 * g4 < sa.w);
        }
        item(rec + kRecEbwL + lane * 16, &su[s][CT][0], true);
        item(rec + kRecEbL + lane * 16, &su[s][CT + 1][0], true);
        item(rec + kRecEbW, &sebw[s][0], true, 4);
    };

    // One register set: every use of step j's T and S precedes the loads of step j+1.
    Step st;
    if (win) {
        if (wct == 0) {
            // the slots of rows past the window, which no fetch writes, hold zeros
#pragma unroll
            for (int s = 0; s < kStages; ++s) {
                if (n16 >= sa.w) {
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                        for (int p = 0; p < 2; ++p)
                            sw[s][ks][p][lane] = sk[s][ks][p][lane] = sq[s][ks][p][lane] = u32x4{0, 0, 0, 0};
#pragma unroll
                    for (int p = 0; p < 2; ++p) sm[s][p][lane] = u32x4{0, 0, 0, 0};
                }
                if (4 * g4 >= sa.w) {
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) su[s][ct][lane] = zero4();
                }
            }
            fetch_window(j0);
            fetch_window(j0 + 1);
            __builtin_amdgcn_s_waitcnt(kWaitAll);
        }
    } else {
        load_rows(read_id(j0), st);
    }
    lds_barrier();

    const u32x4 z4 = u32x4{0, 0, 0, 0};
    // The window waves and the row waves run separate loops (no register state is shared,
    // so neither carries the other's live values); each step all pass the same barriers.
    auto ring_refill = [&](int j) {
        if (j > j0 && ((j - j0) & (kRingFill - 1)) == 0) {   // steps j+256 .. j+511 replace j-256 .. j-1
            fill_ring(j + kRingFill);
            lds_barrier();
        }
    };
    if (win) {
        // window wave wct: the window products of column tile wct; window wave 0 also
        // fetches every stage's factors
        __builtin_amdgcn_s_setprio(2);   // the window products are on the critical path of a step
        const int ct = wct;
        const int col = cb * NB + ct * 16 + n16;
        for (int j = j0; j < j1; ++j) {
            ring_refill(j);
            if (tcol && j > j0 && zflag[(j - 1) & 1] == 0) {
                // the transition columns are exactly zero and stay zero: so do their readouts
                for (int jj = j; jj < j1; ++jj) {
                    if (read_s0(jj) < 0) continue;
                    const size_t cj = (size_t)c * n_step + jj;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int t = 4 * g4 + e;
                        if (t < sa.w) sa.ox[((cj * sa.w + t) * H + h) * 2 * DV + col] = 0.f;
                    }
                }
                break;
            }
            const int64_t s0 = read_s0(j);
            const int s = j % kStages;
            // the factors of step j+1 (fetched during step j-1) and the output stores of
            // step j-1 are complete; fetch those of step j+2 before this step's products
            __builtin_amdgcn_s_waitcnt(kWaitAll);
            if (wct == 0) fetch_window(j + 2);
            if (s0 >= 0) {
                // Y = Wt R and Z = Q R, U' = U - diag(e^b) Y, U'' = diag(e^{b_w-b}) U' (before
                // the first barrier: the row waves overwrite the R planes after it)
                const f32x4 ebwb = su[s][CT][lane], eb = su[s][CT + 1][lane];
                f32x4 y0 = zero4(), y1 = zero4(), y2 = zero4(), z0 = zero4(), z1 = zero4();
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const bf16x8 rh = *reinterpret_cast<const bf16x8*>(&Rh[ct * 16 + n16][ks * 32 + 8 * g4]);
                    const bf16x8 rl = *reinterpret_cast<const bf16x8*>(&Rl[ct * 16 + n16][ks * 32 + 8 * g4]);
                    const bf16x8 wh = as_frag<bf16x8>(sw[s][ks][0][lane]);
                    const bf16x8 wl = as_frag<bf16x8>(sw[s][ks][1][lane]);
                    const bf16x8 qh = as_frag<bf16x8>(sq[s][ks][0][lane]);
                    y0 = mma_bf16(wh, rh, y0);
                    y1 = mma_bf16(wh, rl, y1);
                    y2 = mma_bf16(wl, rh, y2);
                    z0 = mma_bf16(qh, rh, z0);
                    z1 = mma_bf16(qh, rl, z1);
                    if (f32in) z1 = mma_bf16(as_frag<bf16x8>(sq[s][ks][1][lane]), rh, z1);
                }
                const f32x4 y = y0 + (y1 + y2);
                const f32x4 z = z0 + z1;
                const f32x4 u = tcol ? zero4() : su[s][ct][lane];
                f32x4 u1, u2;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    u1[e] = u[e] - eb[e] * y[e];
                    u2[e] = ebwb[e] * u1[e];
                }
                bf16x8 u2h, u2l;
                dtile_bfrags(u2, u2h, u2l);
                Uf[ct][0][lane] = __builtin_bit_cast(u32x4, u2h);
                Uf[ct][1][lane] = __builtin_bit_cast(u32x4, u2l);
                lds_barrier();   // U'' visible to the row waves
                if (tcol && wct == 0 && lane == 0) zflag[(j + 1) & 1] = 0;   // every wave has read it
                // outputs O = scale diag(e^b) (Q R) + Mo U'  (the padded window rows of q are zero);
                // in blocks b >= 1 the readout of X (transition half, then state half)
                const bf16x8 mh = as_frag<bf16x8>(g4 < 2 ? sm[s][0][lane] : z4);
                const bf16x8 ml = as_frag<bf16x8>(g4 < 2 ? sm[s][1][lane] : z4);
                const size_t cj = (size_t)c * n_step + j;
                bf16x8 u1h, u1l;
                dtile_bfrags(u1, u1h, u1l);
                f32x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = sa.scale * eb[e] * z[e];
                o = mma_bf16(mh, u1h, o);
                o = mma_bf16(mh, u1l, o);
                o = mma_bf16(ml, u1h, o);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 4 * g4 + e;
                    if (t < sa.w) {
                        if (b == 0)
                            sa.out[((cj * sa.w + t) * H + h) * ld + col] = o[e];
                        else
                            sa.ox[((cj * sa.w + t) * H + h) * 2 * DV + (tcol ? 0 : DV) + col] = o[e];
                    }
                }
            } else {
                lds_barrier();
                if (tcol && wct == 0 && lane == 0) zflag[(j + 1) & 1] = 0;
            }
            lds_barrier();   // R_{j+1}
        }
        __builtin_amdgcn_s_waitcnt(kWaitAll);
        return;
    }

    // ---- row waves.  T_j / S_j in `cur` (loaded a step earlier); T_{j+1} / S_{j+1} into `nxt`
    // (the same registers) once the products of step j have read them.
    auto step = [&](int j, const Step& cur, Step& nxt) -> bool {
        ring_refill(j);
        if (tcol && j > j0 && zflag[(j - 1) & 1] == 0) return false;   // X is zero (uniform)
        const int id = read_id(j);
        const int64_t s0 = read_s0(j);
        const bool pair = id >= 0, seam = s0 >= 0;
        const int s = j % kStages;
        __builtin_amdgcn_s_waitcnt(kWaitAll);   // T_j, S_j
        const int idn = j + 1 < j1 ? read_id(j + 1) : -1;
        f32x4 a[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) a[ct] = acc[ct];
        // per k-block of T_j: P^T = K T_j^T (K I^T without a pair) and T_j R, then the loads
        // of the same k-block of T_{j+1} into the registers just read (so the next step's
        // loads are in flight from the start of this one); three accumulators for T_j R
        // where one tile gives too little independent work
        constexpr int NA = CT >= 4 ? 1 : 3;
        f32x4 t0[CT], t1[NA == 3 ? CT : 1], t2[NA == 3 ? CT : 1];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            t0[ct] = zero4();
            if constexpr (NA == 3) {
                t1[ct] = zero4();
                t2[ct] = zero4();
            }
        }
        f32x4 p0 = zero4(), p1 = zero4();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            bf16x8 ah, al;
            if (pair) {
                t_frags(cur, ks, ah, al);
            } else {
                ah = as_frag<bf16x8>(ident_bfrag(rt * 16, ks, g4, n16));
                al = as_frag<bf16x8>(z4);
            }
            if (seam) {
                const bf16x8 kh = as_frag<bf16x8>(sk[s][ks][0][lane]);
                p0 = mma_bf16(kh, ah, p0);
                p1 = mma_bf16(kh, al, p1);
                if (f32in) p1 = mma_bf16(as_frag<bf16x8>(sk[s][ks][1][lane]), ah, p1);
            }
            if (pair) {
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    const bf16x8 bh = *reinterpret_cast<const bf16x8*>(&Rh[ct * 16 + n16][ks * 32 + 8 * g4]);
                    const bf16x8 bl = *reinterpret_cast<const bf16x8*>(&Rl[ct * 16 + n16][ks * 32 + 8 * g4]);
                    t0[ct] = mma_bf16(ah, bh, t0[ct]);
                    if constexpr (NA == 3) {
                        t1[ct] = mma_bf16(ah, bl, t1[ct]);
                        t2[ct] = mma_bf16(al, bh, t2[ct]);
                    } else {
                        t0[ct] = mma_bf16(ah, bl, t0[ct]);
                        t0[ct] = mma_bf16(al, bh, t0[ct]);
                    }
                }
            }
            if (idn >= 0) load_t(idn, ks, nxt);   // uniform
        }
        if (pair) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                if constexpr (NA == 3) a[ct] = t0[ct] + (t1[ct] + t2[ct]);
                else a[ct] = t0[ct];
            }
        }
        bf16x8 ph, pl;
        if (seam) {   // the A fragments of P
            dtile_bfrags(p0 + p1, ph, pl);
            const float ebw = sebw[s][lane];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) a[ct] = a[ct] * ebw;
        }
        if (pair && !tcol) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) a[ct][e] += cur.sv[ct][e];
        }
        if (idn >= 0) load_s(idn, nxt);   // S_{j+1}: in flight across the rest of this step
        lds_barrier();   // U'' from the window waves
        if (seam) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                const bf16x8 uh = as_frag<bf16x8>(Uf[ct][0][lane]);
                const bf16x8 ul = as_frag<bf16x8>(Uf[ct][1][lane]);
                a[ct] = mma_bf16(ph, uh, a[ct]);
                a[ct] = mma_bf16(ph, ul, a[ct]);
                a[ct] = mma_bf16(pl, uh, a[ct]);
            }
        }
        bool nz = false;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            acc[ct] = a[ct];
#pragma unroll
            for (int e = 0; e < 4; ++e) nz |= a[ct][e] != 0.f;
        }
        store_split();
        if (tcol && nz) zflag[j & 1] = 1;
        lds_barrier();   // R_{j+1} planes
        return true;
    };

    for (int j = j0; j < j1; ++j)
        if (!step(j, st, st)) break;
    __builtin_amdgcn_s_waitcnt(kWaitAll);   // loads of a step not taken
    if (b == 0) {   // the chain's running state
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) Rg[(size_t)(rt * 16 + 4 * g4 + e) * ld + ct * 16 + n16] = acc[ct][e];
    } else if (tcol) {   // the block's aggregate transition, bf16 hi/lo planes
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                put_t(sa.agg_T, true, agg * H + h, DK, rt * 16 + 4 * g4 + e, cb * NB + ct * 16 + n16, acc[ct][e]);
    } else {   // the block's aggregate state
        float* Sa = sa.agg_S + (agg * H + h) * DK * DV + cb * NB;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) Sa[(size_t)(rt * 16 + 4 * g4 + e) * DV + ct * 16 + n16] = acc[ct][e];
    }
}

// ---- phase 3 of the blocked scan: window outputs from the readouts of X.  One workgroup
// (8 waves) per (chain, block b >= 1, head, group of 8 windows): R_in, the state entering
// the block (fp32), is split into bf16 hi/lo planes in LDS ([column][row], the B operand),
// then each wave forms the outputs of one window:
//     out_j = Gx_j R_in + Hx_j,   Gx_j = readout of the transition half, Hx_j = of the state half.
template <int DK>
__global__ __launch_bounds__(512) void seam_readout_kernel(
    int n_chain, int H, int n_step, int nblk, int blk, int w, const int64_t* __restrict__ seam_start,
    int64_t n_tokens, const float* __restrict__ ox, const float* __restrict__ trail, float* __restrict__ out,
    int ld)
{
    // ld: row length of the outputs (DV unless they hold DV columns of wider ones)
    constexpr int DV = DK;
    constexpr int KP = DK < 32 ? 32 : DK;
    constexpr int KS = KP / 32;
    constexpr int LDB = KP + 8;
    constexpr int NT = DV / 16;                  // column tiles
    __shared__ __attribute__((aligned(16))) uint16_t Rh[DV][LDB];
    __shared__ __attribute__((aligned(16))) uint16_t Rl[DV][LDB];
    // unit: (chain, block b >= 1, head, group of 8 windows); one window per wave
    const int ngrp = (blk + 7) / 8;
    const int unit = blockIdx.x / ngrp, grp = blockIdx.x % ngrp;
    const int h = unit % H, cbk = unit / H;
    const int b = 1 + cbk % (nblk - 1), c = cbk / (nblk - 1);
    if (c >= n_chain) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g4 = lane >> 4, n16 = lane & 15;
    const float* R = trail + (((size_t)c * (nblk - 1) + (b - 1)) * H + h) * DK * DV;
    const int j = b * blk + grp * 8 + wave;
    const bool live = grp * 8 + wave < blk && j < n_step;
    const size_t cj = (size_t)c * n_step + (live ? j : 0);
    const int64_t s0 = live ? seam_start[cj] : -1;
    const bool has = live && s0 >= 0 && s0 + w <= n_tokens;   // a window at this step (uniform)
    // this wave's readout rows first (they do not depend on R_in): A fragments of the
    // transition half (row t = n16, k = 32 ks + 8 g4 + 0..7) and the state half (the
    // accumulators' initial values)
    f32x4 a0[KS], a1[KS], hx[NT];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int k0 = ks * 32 + 8 * g4;
        a0[ks] = a1[ks] = zero4();
        if (has && n16 < w && k0 < DK) {
            const f32x4* p = reinterpret_cast<const f32x4*>(ox + ((cj * w + n16) * H + h) * 2 * DV + k0);
            a0[ks] = p[0];
            a1[ks] = p[1];
        }
    }
#pragma unroll
    for (int ct = 0; ct < NT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = 4 * g4 + e;
            hx[ct][e] = has && t < w ? ox[((cj * w + t) * H + h) * 2 * DV + DV + ct * 16 + n16] : 0.f;
        }
    {   // R_in: item = (4 rows, 1 column), columns fastest across lanes (coalesced loads), written
        // as 4-row runs of a column row of the planes; every load of the thread issued first
        constexpr int NI = (KP / 4) * DV, PER = (NI + 511) / 512;
        float r4[PER][4];
#pragma unroll
        for (int x = 0; x < PER; ++x) {
            const int i = threadIdx.x + 512 * x, col = i % DV, k0 = 4 * (i / DV);
#pragma unroll
            for (int e = 0; e < 4; ++e) r4[x][e] = (i < NI && k0 + e < DK) ? R[(size_t)(k0 + e) * DV + col] : 0.f;
        }
#pragma unroll
        for (int x = 0; x < PER; ++x) {
            const int i = threadIdx.x + 512 * x, col = i % DV, k0 = 4 * (i / DV);
            if (i >= NI) continue;
            unsigned hh[2], ll[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                hh[e] = cvt2_bf16(r4[x][2 * e], r4[x][2 * e + 1]);
                const f32x2 hv = bf16x2_to_f32(hh[e]);
                ll[e] = cvt2_bf16(r4[x][2 * e] - hv.x, r4[x][2 * e + 1] - hv.y);
            }
            *reinterpret_cast<u32x2*>(&Rh[col][k0]) = u32x2{hh[0], hh[1]};
            *reinterpret_cast<u32x2*>(&Rl[col][k0]) = u32x2{ll[0], ll[1]};
        }
    }
    __syncthreads();
    if (!has) return;
    {
        bf16x8 ah[KS], al[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                __bf16 hi, lo;
                split_bf16(x < 4 ? a0[ks][x] : a1[ks][x - 4], hi, lo);
                ah[ks][x] = hi;
                al[ks][x] = lo;
            }
        }
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
            const int col = ct * 16 + n16;
            f32x4 o0 = hx[ct], o1 = zero4(), o2 = zero4();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 bh = *reinterpret_cast<const bf16x8*>(&Rh[col][ks * 32 + 8 * g4]);
                const bf16x8 bl = *reinterpret_cast<const bf16x8*>(&Rl[col][ks * 32 + 8 * g4]);
                o0 = mma_bf16(ah[ks], bh, o0);
                o1 = mma_bf16(ah[ks], bl, o1);
                o2 = mma_bf16(al[ks], bh, o2);
            }
            const f32x4 o = o0 + (o1 + o2);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 4 * g4 + e;
                if (t < w && col < ld) out[((cj * w + t) * H + h) * ld + col] = o[e];
            }
        }
    }
}

// ---------------------------------------------------------------- host side

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

SeamPlan seam_plan(int d, int n_chain, int H, int n_step, int w, int dv)
{
    SeamPlan p;
    const long long units16 = (long long)n_chain * H * (d / 16);
    if (units16 <= 256 && n_step < 16) {   // few short chains: the narrowest blocks, one pass
        p.nb = 16;
        p.nblk = 1;
    } else {
        // every block has d/nb state-column workgroups per (chain, head), which about fill
        // the CUs at one workgroup each; blocks >= 1 add as many transition-column
        // workgroups, dispatched first, which end early where the transitions vanish
        p.nb = d < 64 ? d : 64;
        const long long units = (long long)n_chain * H * (d / p.nb);
        long long nblk = units >= 256 ? 1 : 256 / units;
        nblk = nblk < n_step / 4 ? nblk : n_step / 4;        // at least 4 steps per block
        p.nblk = nblk < 2 ? 1 : (int)nblk;
    }
    if (dv > 0 && dv < d && dv % p.nb != 0) p.nb = 16;   // column blocks that end at a narrower state's last column
    p.blk = p.nblk > 1 ? (n_step + p.nblk - 1) / p.nblk : n_step;
    if (p.nblk > 1) p.nblk = (n_step + p.blk - 1) / p.blk;
    const size_t n_rec = (size_t)n_chain * n_step * H;
    size_t off = align256(n_rec * seam_record_bytes(d));
    p.ox_off = p.agg_t_off = p.agg_s_off = p.trail_off = off;
    if (p.nblk > 1) {
        const size_t n_agg = (size_t)n_chain * (p.nblk - 1) * H;
        p.ox_off = off;
        off = align256(off + n_rec * w * 2 * d * sizeof(float));
        p.agg_t_off = off;
        off = align256(off + n_agg * 2 * d * d * sizeof(uint16_t));
        p.agg_s_off = off;
        off = align256(off + n_agg * d * d * sizeof(float));
        p.trail_off = off;
        off = align256(off + n_agg * d * d * sizeof(float));
    }
    p.bytes = off;
    return p;
}

template <int DK, bool TS, int NB>
static hipError_t launch_seam_chain(int n_chain, int H, int n_step, const int32_t* pair_id, int n_pair,
                                    const void* Tc, const float* Sc, float* Srun, const SeamArgs& sa,
                                    hipStream_t st)
{
    const int n_units = n_chain * sa.nblk * H;
    const int nsub = (sa.nblk > 1 ? 2 : 1) * (DK / NB);
    const int grid = xcd_grid_size(n_units, nsub);
    hipLaunchKernelGGL((seam_chain_kernel<DK, TS, NB>), dim3(grid), dim3(64 * (DK / 16 + NB / 16)), 0, st, n_units, H,
                       n_step, pair_id, n_pair, Tc, Sc, Srun, sa);
    return hipGetLastError();
}

hipError_t seam_chain(int d, int nb, int n_chain, int H, int n_step, const int32_t* pair_id, int n_pair,
                      const void* Tc, bool t_split, const float* Sc, float* Srun, const SeamArgs& sa_in,
                      hipStream_t st)
{
    SeamArgs sa = sa_in;
    if (sa.ld == 0) sa.ld = d;
#define HYPIC_CASE(D_, NB_)                                                                                     \
    if (d == D_ && nb == NB_)                                                                                   \
        return t_split ? launch_seam_chain<D_, true, NB_>(n_chain, H, n_step, pair_id, n_pair, Tc, Sc, Srun, sa, st) \
                       : launch_seam_chain<D_, false, NB_>(n_chain, H, n_step, pair_id, n_pair, Tc, Sc, Srun, sa, st);
    HYPIC_CASE(16, 16) HYPIC_CASE(32, 16) HYPIC_CASE(32, 32) HYPIC_CASE(64, 16) HYPIC_CASE(64, 64)
    HYPIC_CASE(128, 16) HYPIC_CASE(128, 64)
#undef HYPIC_CASE
    return hipErrorNotSupported;
}

hipError_t seam_readout(int d, int n_chain, int H, int n_step, int nblk, int blk, int w,
                        const int64_t* seam_start, int64_t n_tokens, const float* ox, const float* trail,
                        float* out, hipStream_t st, int ld)
{
    if (ld == 0) ld = d;
    const long long grid = (long long)n_chain * (nblk - 1) * H * ((blk + 7) / 8);
    if (nblk < 2 || grid <= 0) return hipSuccess;
#define HYPIC_CASE(D_)                                                                                   \
    if (d == D_) {                                                                                       \
        hipLaunchKernelGGL(seam_readout_kernel<D_>, dim3((unsigned)grid), dim3(512), 0, st, n_chain, H, \
                           n_step, nblk, blk, w, seam_start, n_tokens, ox, trail, out, ld);              \
        return hipGetLastError();                                                                        \
    }
    HYPIC_CASE(16) HYPIC_CASE(32) HYPIC_CASE(64) HYPIC_CASE(128)
#undef HYPIC_CASE
    return hipErrorNotSupported;
}

}  // namespace hypic
