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

// s_waitcnt immediate (gfx9 encoding) that waits for every outstanding vector-memory
// load (including global->LDS direct loads) and every LDS access: vmcnt = 0,
// expcnt = 7 (unconstrained), lgkmcnt = 0.
constexpr unsigned kWaitVmcnt0 = 0x0070;   // also lgkmcnt = 0: LDS reads of the stage being refilled are done
constexpr int kRing = 512, kRingFill = 256;   // LDS ring of per-step pair ids / seam starts
using bld::dpair_to_fragb;

// waves per workgroup: one 16-row tile of the state per wave for plain composition at
// d_k = 128; the seam variant keeps four (its window factors need the register room)
constexpr int chain_waves(int dk, bool seam) { return (dk >= 128 && !seam) ? 8 : 4; }

template <int DK, int DV, int NB, bool SEAM>
__global__ __launch_bounds__(64 * chain_waves(DK, SEAM)) void compose_dense_kernel(
    int n_units, int H, int n_step, const int32_t* __restrict__ pair_id, int n_pair,
    const float* __restrict__ Tc, const float* __restrict__ Sc, float* __restrict__ Srun,
    SeamArgs sa)
{
    constexpr int NCB = DV / NB;
    constexpr int KP = DK < 32 ? 32 : DK;   // contraction length padded to the MFMA K
    constexpr int KS = KP / 32;
    constexpr int RT = DK / 16;             // 16-row tiles of the state
    constexpr int CT = NB / 16;             // 16-column tiles of the block
    constexpr int NW = chain_waves(DK, SEAM);
    constexpr int RTW = (RT + NW - 1) / NW; // row tiles per wave
    constexpr int LDB = KP + 8;             // LDS row length (16-bit units), padded
    constexpr int LDW = 32 + 8;
    constexpr int SW = SEAM ? 1 : 0;
    constexpr int W16 = kSeamMaxW;
    static_assert(!SEAM || CT == 1, "seam path: one 16-column tile per workgroup");
    constexpr bool PF_S = RTW * CT * 4 <= 16;   // prefetch the S block too when it is small
    // tile ct's Y = Wt R (state path) runs on wave ct, its Z = scale Q R (outputs) on wave CT + ct
    __shared__ __attribute__((aligned(16))) uint16_t Rh[2][NB][LDB];   // R, bf16 hi, [column][row]
    __shared__ __attribute__((aligned(16))) uint16_t Rl[2][NB][LDB];   // R, bf16 lo
    __shared__ __attribute__((aligned(16))) uint16_t Uh[SW ? 2 : 1][SW ? NB : 1][LDW];  // [U'' | U'] hi, [col][token]
    __shared__ __attribute__((aligned(16))) uint16_t Ul[SW ? 2 : 1][SW ? NB : 1][LDW];
    __shared__ int ring_id[kRing];
    __shared__ int64_t ring_s0[SW ? kRing : 1];
    // Seam window factors of the next step, fetched by global->LDS direct loads into
    // wave-private regions (two stages).  Each lane reads back exactly the bytes it
    // fetched (lane l's 16 or 4 bytes land at offset 16 l or 4 l of a 1 KiB or 256 B slot).
    //   per wave: Kt slots [RTW][2] (all waves), ebW slot
    //   wave 0 (Y): Wt slots [KS][2], U and e^{b_w-b} dword slots [8], e^b dword slots [4]
    //   wave 1 (Z): q slots [KS][2], Mo slots [2], e^b dword slots [4]
    constexpr int KT_SLOTS = SW ? RTW * 2 : 1;
    __shared__ __attribute__((aligned(16))) f32x4 st_kt[SW ? 2 : 1][SW ? NW : 1][KT_SLOTS][64];
    __shared__ __attribute__((aligned(16))) f32x4 st_xa[SW ? 2 : 1][SW ? 2 : 1][SW ? KS * 2 : 1][64];
    __shared__ __attribute__((aligned(16))) float st_yz[SW ? 2 : 1][SW ? 2 : 1][SW ? 8 : 1][64];
    __shared__ __attribute__((aligned(16))) float st_eb[SW ? 2 : 1][SW ? 2 : 1][SW ? 4 : 1][64];
    __shared__ __attribute__((aligned(16))) float st_ebw[SW ? 2 : 1][SW ? NW : 1][64];

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
        for (int i = threadIdx.x; i < 2 * NB * LDW; i += blockDim.x) {
            (&Uh[0][0][0])[i] = 0;
            (&Ul[0][0][0])[i] = 0;
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
    auto zero8 = [&](float* a) {
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = 0.f;
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

    // ---- everything a step reads besides the running state, loaded one step ahead into
    // one of two register sets (the loop is unrolled by two, so the sets never get copied)
    struct Step {
        int id;                    // pair index, or -1
        int64_t s0;                // seam window start, or -1
        float ta[RTW][KS][8];      // T rows of this wave (A operand)
        float sv[PF_S ? RTW : 1][PF_S ? CT : 1][4];  // S block (D layout), when prefetched
    };
    const int32_t* ids = pair_id ? pair_id + (size_t)c * n_step : nullptr;
    const int64_t* seams = SEAM ? sa.seam_start + (size_t)c * n_step : nullptr;
    // Pair ids and seam starts go through an LDS ring of 512 steps, filled 256 steps ahead, so
    // the per-step lookups are LDS reads and never wait on the vector-memory counter.
    auto fill_ring = [&](int base) {   // steps [base, base + 256)
        for (int x = threadIdx.x; x < kRingFill; x += blockDim.x) {
            const int j = base + x;
            ring_id[j & (kRing - 1)] = (j < n_step && ids) ? ids[j] : -1;
            if constexpr (SEAM) ring_s0[j & (kRing - 1)] = j < n_step ? seams[j] : -1;
        }
    };
    auto read_id = [&](int j) -> int { return ring_id[j & (kRing - 1)]; };
    auto read_s0 = [&](int j) -> int64_t {
        if constexpr (!SEAM) return -1;
        return ring_s0[j & (kRing - 1)];
    };
    auto load_step = [&](int j, int id, int64_t s0, Step& st) {
        id = (unsigned)id < (unsigned)n_pair ? id : -1;
        if constexpr (SEAM) s0 = (s0 >= 0 && s0 + sa.w <= sa.n_tokens) ? s0 : -1;
        st.id = id;
        st.s0 = s0;
        if (id >= 0) {
            const float* T = Tc + ((size_t)id * H + h) * DK * DK;
            const float* S = Sc + ((size_t)id * H + h) * DK * DV + cb * NB;
#pragma unroll
            for (int i = 0; i < RTW; ++i) {
                const int rt = wave + NW * i;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int k0 = ks * 32 + 8 * g4;
                    if (rt < RT && k0 < DK) ld8f(T + (size_t)(rt * 16 + n16) * DK + k0, st.ta[i][ks]);
                    else zero8(st.ta[i][ks]);
                }
                if constexpr (PF_S) {
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            st.sv[i][ct][e] = rt < RT ? S[(size_t)(rt * 16 + 4 * g4 + e) * DV + ct * 16 + n16] : 0.f;
                }
            }
        }
        if constexpr (SEAM) {
            if (s0 >= 0) {
                const int sg = j & 1;
                const size_t cj = (size_t)c * n_step + j;
                const float* rec = sa.ws + (cj * H + h) * SeamRec<DK>::kFloats;
                auto dma16 = [&](const void* src, void* slot) {
                    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)slot, 16, 0, 0);
                };
                auto dma4 = [&](const void* src, void* slot) {
                    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)slot, 4, 0, 0);
                };
                const int gk = g4 & 1;   // lanes g4 >= 2 fetch a duplicate (ignored), keeping addresses valid
#pragma unroll
                for (int i = 0; i < RTW; ++i) {
                    const int rt = (wave + NW * i) < RT ? wave + NW * i : 0;
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf)
                        dma16(rec + SeamRec<DK>::kKt + (rt * 16 + n16) * W16 + 8 * gk + 4 * hf, &st_kt[sg][wave][2 * i + hf][0]);
                }
                dma4(rec + SeamRec<DK>::kEbW, &st_ebw[sg][wave][0]);
                if (wave < 2) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) dma4(rec + SeamRec<DK>::kEb + 4 * g4 + e, &st_eb[sg][wave][e][0]);
                }
                if (wave == 0) {   // Y wave: Wt rows, U block, e^{b_w - b}
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const int k0 = (ks * 32 + 8 * g4) < DK ? ks * 32 + 8 * g4 : 0;
#pragma unroll
                        for (int hf = 0; hf < 2; ++hf)
                            dma16(rec + SeamRec<DK>::kWt + n16 * DK + k0 + 4 * hf, &st_xa[sg][0][2 * ks + hf][0]);
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        dma4(rec + SeamRec<DK>::kU + (4 * g4 + e) * DV + cb * NB + n16, &st_yz[sg][0][e][0]);
                        dma4(rec + SeamRec<DK>::kEbw + 4 * g4 + e, &st_yz[sg][0][4 + e][0]);
                    }
                } else if (wave == 1) {   // Z wave: q rows (raw bits), Mo row
                    const int tq = n16 < sa.w ? n16 : sa.w - 1;   // rows past the window are masked at use
                    const size_t tok = (size_t)(s0 + tq) * H * DK + (size_t)h * DK;
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const int k0 = (ks * 32 + 8 * g4) < DK ? ks * 32 + 8 * g4 : 0;
                        if (sa.in_bf16) {
                            dma16(reinterpret_cast<const uint16_t*>(sa.q) + tok + k0, &st_xa[sg][1][2 * ks][0]);
                        } else {
#pragma unroll
                            for (int hf = 0; hf < 2; ++hf)
                                dma16(reinterpret_cast<const float*>(sa.q) + tok + k0 + 4 * hf, &st_xa[sg][1][2 * ks + hf][0]);
                        }
                    }
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf)
                        dma16(rec + SeamRec<DK>::kMo + n16 * W16 + 8 * gk + 4 * hf, &st_yz[sg][1][4 * hf][0]);
                }
            }
        }
    };

    // ---- R <- T R + S on the planes `buf` (result in the accumulators)
    auto compose_step = [&](const Step& st, int buf) {
        const float* S = Sc + ((size_t)st.id * H + h) * DK * DV + cb * NB;
#pragma unroll
        for (int i = 0; i < RTW; ++i) {
            const int rt = wave + NW * i;
            if (rt >= RT) continue;
            float sv[CT][4];   // S block: prefetched, or loaded now (its latency overlaps the MFMAs)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sv[ct][e] = PF_S ? st.sv[PF_S ? i : 0][PF_S ? ct : 0][e]
                                     : S[(size_t)(rt * 16 + 4 * g4 + e) * DV + ct * 16 + n16];
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

    // product of an A-operand row set (8 floats per k-step) with column tile ct of R (planes buf)
    auto rowprod = [&](const float (*a)[8], int ct, int buf) -> f32x4 {
        f32x4 y = zero4();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 bh = *reinterpret_cast<const bf16x8*>(&Rh[buf][ct * 16 + n16][ks * 32 + 8 * g4]);
            const bf16x8 bl = *reinterpret_cast<const bf16x8*>(&Rl[buf][ct * 16 + n16][ks * 32 + 8 * g4]);
            bf16x8 ah, al;
            split8(a[ks], ah, al);
            y = mma_bf16(ah, bh, y);
            y = mma_bf16(ah, bl, y);
            y = mma_bf16(al, bh, y);
        }
        return y;
    };

    // ---- one seam window on the planes `buf`: R <- e^{b_w} R + K^T U'' and the window outputs.
    // The window factors come from the LDS stage `sg` this wave's direct loads filled.
    auto stage16 = [&](const f32x4* slot, float* out4) {
        const f32x4 v = slot[lane];
#pragma unroll
        for (int x = 0; x < 4; ++x) out4[x] = v[x];
    };
    auto seam_step = [&](const Step& st, int buf, size_t cj, int sg) {
        f32x4 z = zero4();
        const bool zw = wave == 1;
        float eb[4];
        if (wave < 2) {
#pragma unroll
            for (int e = 0; e < 4; ++e) eb[e] = st_eb[sg][wave][e][lane];
        }
        if (wave == 0) {  // state path: Y = Wt R, U' = U - diag(e^b) Y, U'' = diag(e^{b_w - b}) U'
            float xa[KS][8];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                stage16(&st_xa[sg][0][2 * ks][0], xa[ks]);
                stage16(&st_xa[sg][0][2 * ks + 1][0], xa[ks] + 4);
            }
            const f32x4 y = rowprod(xa, 0, buf);
            f32x4 u, u2;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                u[e] = st_yz[sg][0][e][lane] - eb[e] * y[e];
                u2[e] = st_yz[sg][0][4 + e][lane] * u[e];
            }
            unsigned h0, h1, l0, l1;
            pack_bf16_split(u2, h0, h1, l0, l1);
            *reinterpret_cast<u32x2*>(&Uh[0][n16][4 * g4]) = u32x2{h0, h1};
            *reinterpret_cast<u32x2*>(&Ul[0][n16][4 * g4]) = u32x2{l0, l1};
            pack_bf16_split(u, h0, h1, l0, l1);
            *reinterpret_cast<u32x2*>(&Uh[1][n16][4 * g4]) = u32x2{h0, h1};
            *reinterpret_cast<u32x2*>(&Ul[1][n16][4 * g4]) = u32x2{l0, l1};
        } else if (zw) {  // Z = scale Q R for the outputs (rows past the window are zero)
            float qa[KS][8];
            const float msk = n16 < sa.w ? sa.scale : 0.f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (sa.in_bf16) {
                    float w4[4];
                    stage16(&st_xa[sg][1][2 * ks][0], w4);
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        const unsigned wv = __float_as_uint(w4[x]);
                        qa[ks][2 * x] = msk * __uint_as_float(wv << 16);
                        qa[ks][2 * x + 1] = msk * __uint_as_float(wv & 0xFFFF0000u);
                    }
                } else {
                    stage16(&st_xa[sg][1][2 * ks][0], qa[ks]);
                    stage16(&st_xa[sg][1][2 * ks + 1][0], qa[ks] + 4);
#pragma unroll
                    for (int x = 0; x < 8; ++x) qa[ks][x] *= msk;
                }
            }
            z = rowprod(qa, 0, buf);
        }
        lds_barrier();
        // state: R <- e^{b_w} R + K^T U''
        const float ebW = st_ebw[sg][wave][lane];
#pragma unroll
        for (int i = 0; i < RTW; ++i) {
            const int rt = wave + NW * i;
            if (rt >= RT) continue;
            float kt[8];
            stage16(&st_kt[sg][wave][2 * i][0], kt);
            stage16(&st_kt[sg][wave][2 * i + 1][0], kt + 4);
            if (g4 >= 2) zero8(kt);   // window tokens 16..31 do not exist
            bf16x8 kh, kl;
            split8(kt, kh, kl);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                const bf16x8 uh = *reinterpret_cast<const bf16x8*>(&Uh[0][ct * 16 + n16][8 * g4]);
                const bf16x8 ul = *reinterpret_cast<const bf16x8*>(&Ul[0][ct * 16 + n16][8 * g4]);
                f32x4 a = acc[i][ct] * ebW;
                a = mma_bf16(kh, uh, a);
                a = mma_bf16(kh, ul, a);
                a = mma_bf16(kl, uh, a);
                acc[i][ct] = a;
            }
        }
        // outputs: O = diag(e^b) Z + Mo U'   (off the state's critical path)
        if (zw) {
            float mo[8];
            stage16(reinterpret_cast<const f32x4*>(&st_yz[sg][1][0][0]), mo);   // two 16-byte loads
            stage16(reinterpret_cast<const f32x4*>(&st_yz[sg][1][4][0]), mo + 4);
            if (g4 >= 2) zero8(mo);
            bf16x8 mh, ml;
            split8(mo, mh, ml);
            const bf16x8 uh = *reinterpret_cast<const bf16x8*>(&Uh[1][n16][8 * g4]);
            const bf16x8 ul = *reinterpret_cast<const bf16x8*>(&Ul[1][n16][8 * g4]);
            f32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = eb[e] * z[e];
            o = mma_bf16(mh, uh, o);
            o = mma_bf16(mh, ul, o);
            o = mma_bf16(ml, uh, o);
            const int col = cb * NB + n16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 4 * g4 + e;
                if (t < sa.w) sa.out[((cj * sa.w + t) * H + h) * DV + col] = o[e];
            }
        }
    };

    int cur = 0;
    auto run_step = [&](int j, const Step& st) {
        if constexpr (SEAM) {
            if (st.s0 >= 0) {  // uniform over the workgroup
                seam_step(st, cur, (size_t)c * n_step + j, j & 1);
                store_split(cur ^ 1);
                lds_barrier();
                cur ^= 1;
            }
        }
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
    int64_t s1 = read_s0(1);
    load_step(0, read_id(0), read_s0(0), sA);
    // Every load of step j was issued a whole step earlier: wait for all of them once, at the
    // top of the step, then issue step j+1's loads.  (Using a value right after its load would
    // make the in-order vector-memory counter drain the prefetch as well.)
    for (int j = 0; j < n_step; j += 2) {
        // step j from sA; prefetch step j+1 into sB; ids of step j+2
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        if (j > 0 && (j & (kRingFill - 1)) == 0) {  // steps j+256 .. j+511 replace steps j-256 .. j-1
            fill_ring(j + kRingFill);
            lds_barrier();
        }
        const int id2 = read_id(j + 2);
        const int64_t s2 = read_s0(j + 2);
        if (j + 1 < n_step) load_step(j + 1, id1, s1, sB);
        run_step(j, sA);
        if (j + 1 >= n_step) break;
        // step j+1 from sB; prefetch step j+2 into sA; ids of step j+3
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        id1 = read_id(j + 3);
        s1 = read_s0(j + 3);
        if (j + 2 < n_step) load_step(j + 2, id2, s2, sA);
        run_step(j + 1, sB);
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
        // the seam epilogue needs a Y wave and a Z wave per 16-column tile
        if constexpr (NB == 16)
            hipLaunchKernelGGL((compose_dense_kernel<DK, DV, NB, true>), dim3(grid), dim3(64 * chain_waves(DK, true)), 0, st,
                               n_units, H, n_step, pair_id, n_pair, Tc, Sc, Srun, *sa);
        else
            return hipErrorInvalidValue;
    } else
        hipLaunchKernelGGL((compose_dense_kernel<DK, DV, NB, false>), dim3(grid), dim3(64 * chain_waves(DK, false)), 0, st,
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
    if (sa) nb = 16;   // the seam path works on 16-column blocks
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
