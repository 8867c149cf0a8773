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
// column blocks of the full-width composition (4 x this waves per workgroup; one column
// block, 4 waves, measured 28% slower at the 64-request reuse plan: one wave per SIMD
// leaves the loads and LDS reads of a step exposed)
constexpr int kWideCB = 2;

// waves per workgroup: one 16-row tile of the state per wave at d_k = 128
constexpr int chain_waves(int dk) { return dk >= 128 ? 8 : 4; }

// TS: T cached as bf16 hi/lo planes ([n_pair][H][2][DK][DK], hypic_t_layout SPLIT),
// fed to the MFMA units as loaded; otherwise fp32 T, split in registers.
template <int DK, int DV, int NB, bool TS>
__global__ __launch_bounds__(64 * chain_waves(DK)) void compose_dense_kernel(
    int n_units, int H, int n_step, const int32_t* __restrict__ pair_id, int n_pair,
    const void* __restrict__ Tc, const float* __restrict__ Sc, float* __restrict__ Srun, float* __restrict__ trail,
    int r_ld)
{
    // r_ld: row length of the running states ([chain][H][DK][r_ld]; DV unless Srun points at DV
    // columns of a wider state)
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
    if (r_ld < DV && cb * NB >= r_ld) return;   // past the columns of a narrower running state (a multiple of NB)
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g4 = lane >> 4, n16 = lane & 15;

    if (KP > DK) {  // rows DK..KP-1 of the B operand stay zero
        for (int i = threadIdx.x; i < 2 * NB * LDB; i += blockDim.x) {
            (&Rh[0][0][0])[i] = 0;
            (&Rl[0][0][0])[i] = 0;
        }
    }
    __syncthreads();

    float* Rg = Srun + ((size_t)c * H + h) * DK * r_ld + cb * NB;
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
                    acc[i][ct][e] = Rg[(size_t)(rt * 16 + 4 * g4 + e) * r_ld + ct * 16 + n16];
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
                Rg[(size_t)(rt * 16 + 4 * g4 + e) * r_ld + ct * 16 + n16] = acc[i][ct][e];
    }
}

// Full width at d_k = d_v = 128 (many chains: one workgroup per (chain, head) holding all
// 128 state columns).  The 8 waves split the state 4 x 2: wave w owns rows 32 (w >> 1) ..
// +31 and columns 64 (w & 1) .. +63, a 2 x 4 block of 16 x 16 accumulator tiles, so per
// step a wave reads 2 A fragments of T per k-block (from global memory, SPLIT planes as is
// or fp32 split in registers) and 4 B fragments of the running state's planes from LDS:
// 256 KiB of LDS operand reads per step instead of the 512 KiB of one 16-row tile per wave
// with all columns.  The pair ids go through an LDS ring that holds the valid ids only
// (compacted as each block of 256 steps is read), so every iteration is a real step and
// the next step's T and S are always loaded: T_{j+1} k-block by k-block into the registers
// that step j's products of that k-block have just read, S_{j+1} once step j's first
// products have read S_j as their accumulator input.  Nothing is loaded conditionally, so
// the register sets are never merged or copied.
template <bool TS, int CB>
__global__ __launch_bounds__(256 * CB) void compose_wide_kernel(
    int n_units, int H, int n_step, const int32_t* __restrict__ pair_id, int n_pair,
    const void* __restrict__ Tc, const float* __restrict__ Sc, float* __restrict__ Srun)
{
    // planes [column][row] with a row stride of 66 dwords: the B-fragment reads (16 bytes,
    // 8-byte aligned on odd columns) and the 8-byte split stores are both free of bank
    // conflicts at this stride (measured; 68 and 64 dwords conflict on both)
    constexpr int D = 128, LDB = D + 4, KS = D / 32;
    constexpr int CT = 8 / CB;   // column tiles per wave
    __shared__ __attribute__((aligned(16))) uint16_t Rh[2][D][LDB];   // R, bf16 hi, [column][row]
    __shared__ __attribute__((aligned(16))) uint16_t Rl[2][D][LDB];   // R, bf16 lo
    __shared__ int ring_id[kRing];                                     // valid pair ids, in step order
    __shared__ int wave_cnt[8];

    // Units in head-major order (u = h n_chain + c), each XCD a contiguous eighth of them:
    // the workgroups an XCD runs at one time are consecutive chains of one head, and chains
    // of one layer are consecutive, so they all read the pairs of one (layer, head) -- 64
    // pairs x 128 KiB for the 64-segment cache, about twice that XCD's L2 -- instead of
    // several heads' pairs each.
    const int per_xcd = (n_units + 7) / 8;
    const int li = blockIdx.x >> 3;
    const int u = (blockIdx.x & 7) * per_xcd + li;
    if (li >= per_xcd || u >= n_units) return;
    const int n_chain = n_units / H;
    const int h = u / n_chain, c = u % n_chain;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g4 = lane >> 4, n16 = lane & 15;
    const int rt0 = 2 * (wave / CB), ct0 = CT * (wave % CB);   // first row / column tile of the block

    float* Rg = Srun + ((size_t)c * H + h) * D * D;
    f32x4 acc[2][CT];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                acc[i][ct][e] = Rg[(size_t)((rt0 + i) * 16 + 4 * g4 + e) * D + (ct0 + ct) * 16 + n16];

    auto store_split = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                unsigned h0, h1, l0, l1;
                pack_bf16_split(acc[i][ct], h0, h1, l0, l1);
                const int col = (ct0 + ct) * 16 + n16, row = (rt0 + i) * 16 + 4 * g4;
                *reinterpret_cast<u32x2*>(&Rh[buf][col][row]) = u32x2{h0, h1};
                *reinterpret_cast<u32x2*>(&Rl[buf][col][row]) = u32x2{l0, l1};
            }
    };
    store_split(0);

    // ---- the ring: steps are read 256 at a time; the valid ids of a block are appended at
    // wpos (ballot + popcount prefix within each wave, wave totals through LDS).  Positions
    // are uniform counters; the loop consumes at rpos and refills before it runs dry.
    const int32_t* ids = pair_id ? pair_id + (size_t)c * n_step : nullptr;
    int wpos = 0, rpos = 0, next_raw = 0;
    auto fill_block = [&]() {
        int id = -1;
        if (threadIdx.x < kRingFill) {
            const int j = next_raw + threadIdx.x;
            if (j < n_step) {
                const int x = ids ? ids[j] : c * n_step + j;
                id = (unsigned)x < (unsigned)n_pair ? x : -1;
            }
        }
        const unsigned long long m = __ballot(id >= 0);
        const int pre = __popcll(m & ((1ull << lane) - 1ull));
        if (lane == 0) wave_cnt[wave] = __popcll(m);
        lds_barrier();
        int base = wpos, tot = 0;
#pragma unroll
        for (int w = 0; w < kRingFill / 64; ++w) {
            const int n = wave_cnt[w];
            base += w < wave ? n : 0;
            tot += n;
        }
        if (id >= 0) ring_id[(base + pre) & (kRing - 1)] = id;
        lds_barrier();   // the ring entries are visible; wave_cnt is read before the next block
        wpos += __builtin_amdgcn_readfirstlane(tot);
        next_raw += kRingFill;
    };
    // at least the current step and the one after it in the ring (or every step read)
    auto ensure = [&]() {
        while (wpos < rpos + 2 && next_raw < n_step) fill_block();
    };
    auto ring = [&](int pos) -> int { return __builtin_amdgcn_readfirstlane(ring_id[pos & (kRing - 1)]); };

    // registers of one step: this wave's A fragments of T and its block of S
    u32x4 th[2][KS], tl[2][KS];   // SPLIT: bf16 hi / lo planes as loaded
    float ta[TS ? 1 : 2][TS ? 1 : KS][8];
    float sv[2][CT][4];
    auto load_t = [&](int id, int ks) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int row = (rt0 + i) * 16 + n16, k0 = ks * 32 + 8 * g4;
            if constexpr (TS) {   // fragment-ordered planes: 1 KiB contiguous per fragment
                const uint16_t* T = reinterpret_cast<const uint16_t*>(Tc) + ((size_t)id * H + h) * 2 * D * D;
                const int e = frag_off(row, k0, D);
                th[i][ks] = *reinterpret_cast<const u32x4*>(T + e);
                tl[i][ks] = *reinterpret_cast<const u32x4*>(T + D * D + e);
            } else {
                const f32x4* p = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(Tc) +
                                                                 ((size_t)id * H + h) * D * D + (size_t)row * D + k0);
                const f32x4 a = p[0], b = p[1];
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    ta[i][ks][x] = a[x];
                    ta[i][ks][4 + x] = b[x];
                }
            }
        }
    };
    auto load_s = [&](int id) {
        const float* S = Sc + ((size_t)id * H + h) * D * D;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sv[i][ct][e] = S[(size_t)((rt0 + i) * 16 + 4 * g4 + e) * D + (ct0 + ct) * 16 + n16];
    };
    auto a_frags = [&](int i, int ks, bf16x8& ah, bf16x8& al) {
        if constexpr (TS) {
            ah = as_frag<bf16x8>(th[i][ks]);
            al = as_frag<bf16x8>(tl[i][ks]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                __bf16 x, y;
                split_bf16(ta[i][ks][e], x, y);
                ah[e] = x;
                al[e] = y;
            }
        }
    };

    ensure();
    if (wpos > 0) {
        const int id0 = ring(0);
        load_s(id0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) load_t(id0, ks);
    }
    int cur = 0;
    while (rpos < wpos) {
        // R <- T R + S on the planes `cur`: hi*hi + hi*lo + lo*hi into the accumulators, which
        // start from S; the next step's id is in the ring (or there is none: then this step's
        // own pair is fetched again, unused).  Per k-block the three products go out product by
        // product over the 8 tiles, so consecutive products feed different accumulators (a
        // dependent product waits for the previous one's result); the next k-block's B
        // fragments are read from LDS before this block's products.
        const int idn = rpos + 1 < wpos ? ring(rpos + 1) : ring(rpos);
        bf16x8 bh[2][CT], bl[2][CT];
        auto read_b = [&](int ks, int slot) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                const int col = (ct0 + ct) * 16 + n16, k0 = ks * 32 + 8 * g4;
                bh[slot][ct] = *reinterpret_cast<const bf16x8*>(&Rh[cur][col][k0]);
                bl[slot][ct] = *reinterpret_cast<const bf16x8*>(&Rl[cur][col][k0]);
            }
        };
        read_b(0, 0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int sl = ks & 1;
            if (ks + 1 < KS) read_b(ks + 1, sl ^ 1);
            bf16x8 ah[2], al[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) a_frags(i, ks, ah[i], al[i]);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const f32x4 a0 = ks == 0 ? f32x4{sv[i][ct][0], sv[i][ct][1], sv[i][ct][2], sv[i][ct][3]} : acc[i][ct];
                    acc[i][ct] = mma_bf16(ah[i], bh[sl][ct], a0);
                }
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int i = 0; i < 2; ++i) acc[i][ct] = mma_bf16(ah[i], bl[sl][ct], acc[i][ct]);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int i = 0; i < 2; ++i) acc[i][ct] = mma_bf16(al[i], bh[sl][ct], acc[i][ct]);
            if (ks == 0) load_s(idn);
            load_t(idn, ks);
            // keep the k-blocks in order (the scheduler would otherwise hoist every block's
            // LDS reads to the top of the step and run out of registers)
            if (ks + 1 < KS) __builtin_amdgcn_sched_barrier(0);
        }
        store_split(cur ^ 1);
        lds_barrier();
        cur ^= 1;
        ++rpos;
        ensure();
    }

#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                Rg[(size_t)((rt0 + i) * 16 + 4 * g4 + e) * D + (ct0 + ct) * 16 + n16] = acc[i][ct][e];
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
                               const void* Tc, const float* Sc, float* Srun, float* trail, hipStream_t st, int r_ld)
{
    const int n_units = n_chain * H;
    const int grid = xcd_grid_size(n_units, DV / NB);
    hipLaunchKernelGGL((compose_dense_kernel<DK, DV, NB, TS>), dim3(grid), dim3(64 * chain_waves(DK)), 0, st,
                       n_units, H, n_step, pair_id, n_pair, Tc, Sc, Srun, trail, r_ld ? r_ld : DV);
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

hipError_t compose_dense(int dk, int dv, int n_chain, int H, int n_step, const int32_t* pair_id, int n_pair,
                         const void* Tc, bool t_split, const float* Sc, float* Srun, float* trail,
                         hipStream_t st, int r_ld)
{
    if (dk != dv) {   // rectangular states: 16-column blocks
#define HYPIC_RECT(DK_, DV_)                                                                                   \
    if (dk == DK_ && dv == DV_)                                                                                \
        return t_split ? launch_dense<DK_, DV_, 16, true>(n_chain, H, n_step, pair_id, n_pair, Tc, Sc, Srun, trail, st, r_ld) \
                       : launch_dense<DK_, DV_, 16, false>(n_chain, H, n_step, pair_id, n_pair, Tc, Sc, Srun, trail, st, r_ld);
        HYPIC_RECT(16, 32) HYPIC_RECT(16, 64) HYPIC_RECT(16, 128)
        HYPIC_RECT(32, 16) HYPIC_RECT(32, 64) HYPIC_RECT(32, 128)
        HYPIC_RECT(64, 16) HYPIC_RECT(64, 32) HYPIC_RECT(64, 128)
        HYPIC_RECT(128, 16) HYPIC_RECT(128, 32) HYPIC_RECT(128, 64)
#undef HYPIC_RECT
        return hipErrorInvalidValue;
    }
    const int d = dk;
    int nb = pick_nb((long long)n_chain * H, d);
    while (r_ld > 0 && r_ld < dv && r_ld % nb != 0) nb /= 2;   // blocks that end at a narrower state's last column
    if (d == 128 && nb == 128 && trail == nullptr && (r_ld == 0 || r_ld == dv)) {
        const int n_units = n_chain * H;
        const int grid = (n_units + 7) / 8 * 8;
        if (t_split)
            hipLaunchKernelGGL((compose_wide_kernel<true, kWideCB>), dim3(grid), dim3(256 * kWideCB), 0, st, n_units,
                               H, n_step, pair_id, n_pair, Tc, Sc, Srun);
        else
            hipLaunchKernelGGL((compose_wide_kernel<false, kWideCB>), dim3(grid), dim3(256 * kWideCB), 0, st,
                               n_units, H, n_step, pair_id, n_pair, Tc, Sc, Srun);
        return hipGetLastError();
    }
#define HYPIC_CASE(D_, NB_)                                                                                   \
    if (d == D_ && nb == NB_)                                                                                 \
        return t_split                                                                                        \
                   ? launch_dense<D_, D_, NB_, true>(n_chain, H, n_step, pair_id, n_pair, Tc, Sc, Srun, trail, st, r_ld) \
                   : launch_dense<D_, D_, NB_, false>(n_chain, H, n_step, pair_id, n_pair, Tc, Sc, Srun, trail, st, r_ld);
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
