// build_gdn.hip -- segment build (T_C, S(C|0)) for the scalar-gated delta rule.
//
// Per token: S_t = alpha_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T.  The
// cached pair of a segment is T_C = M_L..M_1 and S(C|0) ([ZH] = the Chinese
// HYPIC page, section 2.1: the segment operator is the ordered product of the
// token transitions, and both quantities depend on the segment's own tokens).
//
// Chunked form (C = 64 tokens; derivation in the design notes).  Inside a
// chunk let b_t = g_1 + .. + g_t (log-gates), D = diag(e^{b_t}), and
//     Lt[t][s] = b_t (k_t . k_s) for s < t,   At = (I + Lt)^-1   (undecayed)
//     Wt = At diag(b) K,   U = D At D^-1 diag(b) V,   A = D At D^-1
// (A[t][s] = e^{b_t - b_s} At[t][s] has only non-positive exponents).  Then
//     S <- e^{b_C} S + K^T diag(e^{b_C - b}) (U - D Wt S)
//     H <- H - K^T (Wt H),      T_C = e^{sum of all g} H
// where H is the undecayed transition product, so the T columns never
// underflow the 16-bit MFMA operands however strong the decay; the decay of T
// is one fp32 scale at the end.
//
// One workgroup (8 waves) per (segment, head).  The augmented state X = [H | S]
// (d x 2d, fp32) lives in MFMA accumulators, 16-column tiles dealt to waves;
// every product runs on v_mfma_f32_16x16x32_f16 with fp32 accumulation:
// K K^T, Wt, U, Y = Wt X and X += K^T R.  X and R reach the B operand without
// LDS through two cross-lane swaps.  The 64x64 triangular inverse is blocked
// 16x16: diagonal blocks by forward substitution (fp32), the rest with
// v_mfma_f32_16x16x4_f32.  Operands are fp16 (one rounding, NSPLIT = 1) for
// bf16 inputs, or fp16 hi + lo with three products (NSPLIT = 2) for fp32 inputs.
#include "hypic_device.h"
#include "hypic_kernels.h"
#include "build_common.h"

namespace hypic {

namespace {
using namespace bld;

constexpr int CH = 64;       // chunk length
constexpr int LDT = CH + 8;  // padded LDS row for token-indexed rows (16-bit units)
constexpr int LDF = CH + 1;  // padded LDS row for fp32 64x64 matrices

template <int D, int NSPLIT>
struct alignas(16) GdnSmem {
    static constexpr int KP = D < 32 ? 32 : D;  // channel contraction padded to 32
    static constexpr int LDK = KP + 8;
    uint16_t Kr[NSPLIT][CH][LDK];  // K, token-major (channels >= D are zero)
    uint16_t Kt[NSPLIT][D][LDT];   // K^T, channel-major
    uint16_t Vt[NSPLIT][D][LDT];   // V^T, channel-major
    uint16_t Ap[NSPLIT][CH][LDT];  // At diag(beta)
    uint16_t Ad[NSPLIT][CH][LDT];  // A diag(beta)
    uint16_t Wt[NSPLIT][CH][LDK];  // Wt, token-major (channels >= D are zero)
    float F1[CH][LDF];             // Lt (strictly lower)
    float F2[CH][LDF];             // At
    float F3[32][33];              // inverse scratch
    float gate[CH], beta[CH], b[CH], eb[CH], ebr[CH];
    float bC;
};

// Inverse of I + Lt (64x64 unit lower triangular, Lt in F1) into F2.
template <typename SM>
__device__ void tri_inverse(SM& sm, int wave, int lane) {
    // (1) the four 16x16 diagonal blocks, one column per lane
    if (wave < 4 && lane < 16) {
        const int o = wave * 16, j = lane;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float s = (r == j) ? 1.f : 0.f;
#pragma unroll
            for (int q = 0; q < r; ++q) s -= sm.F1[o + r][o + q] * x[q];
            x[r] = s;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sm.F2[o + r][o + j] = x[r];
    }
    __syncthreads();
    // (2) blocks (1,0) and (3,2):  A_ij = -D_i L_ij D_j
    if (wave < 2) {
        const int i = 2 * wave + 1, j = 2 * wave;
        f32x4 p = mm16_f32(&sm.F1[i * 16][j * 16], LDF, &sm.F2[j * 16][j * 16], LDF, lane);
        float* tmp = &sm.F3[wave * 16][0];
        st16_f32(tmp, 33, p, lane, 1.f);
    }
    __syncthreads();
    if (wave < 2) {
        const int i = 2 * wave + 1, j = 2 * wave;
        f32x4 q = mm16_f32(&sm.F2[i * 16][i * 16], LDF, &sm.F3[wave * 16][0], 33, lane);
        st16_f32(&sm.F2[i * 16][j * 16], LDF, q, lane, -1.f);
    }
    __syncthreads();
    // (3) lower-left 32x32 block: -E1 Lt[2:4, 0:2] E0 with E0, E1 the 32x32 inverses
    if (wave < 4) {
        const int r = 2 + (wave >> 1), cc = wave & 1;
        f32x4 p = mm16_f32(&sm.F1[r * 16][cc * 16], LDF, &sm.F2[cc * 16][cc * 16], LDF, lane);
        if (cc == 0) {
            const f32x4 p2 = mm16_f32(&sm.F1[r * 16][16], LDF, &sm.F2[16][0], LDF, lane);
            p += p2;
        }
        st16_f32(&sm.F3[(r - 2) * 16][cc * 16], 33, p, lane, 1.f);
    }
    __syncthreads();
    if (wave < 4) {
        const int r = 2 + (wave >> 1), cc = wave & 1;
        f32x4 q = mm16_f32(&sm.F2[r * 16][r * 16], LDF, &sm.F3[(r - 2) * 16][cc * 16], 33, lane);
        if (r == 3) {
            const f32x4 q2 = mm16_f32(&sm.F2[48][32], LDF, &sm.F3[0][cc * 16], 33, lane);
            q += q2;
        }
        st16_f32(&sm.F2[r * 16][cc * 16], LDF, q, lane, -1.f);
    }
    __syncthreads();
}

}  // namespace

template <int D, int NSPLIT, bool BF16>
__global__ __launch_bounds__(512) void build_gdn_kernel(
    int n_seg, int H, const int64_t* __restrict__ seg_begin, const int64_t* __restrict__ seg_end,
    int64_t n_tokens, const void* __restrict__ k, const void* __restrict__ v,
    const void* __restrict__ gl, const void* __restrict__ beta, void* __restrict__ T_out, int t_split,
    float* __restrict__ S_out)
{
    using SM = GdnSmem<D, NSPLIT>;
    constexpr int KP = SM::KP;
    constexpr int KSD = KP / 32;            // k-steps over channels
    constexpr int RT = D / 16;              // row tiles of X
    constexpr int NCT = 2 * RT;             // column tiles of X = [H | S]
    constexpr int CTW = (NCT + 7) / 8;      // column tiles per wave
    __shared__ SM sm;

    const int unit = blockIdx.x;
    const int seg = unit / H, h = unit % H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g4 = lane >> 4, n16 = lane & 15;

    int64_t beg = seg_begin[seg], end = seg_end[seg];
    beg = beg < 0 ? 0 : (beg > n_tokens ? n_tokens : beg);
    end = end < beg ? beg : (end > n_tokens ? n_tokens : end);

    // zero the channel padding of Kr / Wt once (D < 32 only)
    if (KP > D) {
        for (int i = tid; i < NSPLIT * CH * SM::LDK; i += 512) {
            (&sm.Kr[0][0][0])[i] = 0;
            (&sm.Wt[0][0][0])[i] = 0;
        }
    }

    // X tiles owned by this wave: column tile ct = wave + 8*c; X[rt][c] (D layout)
    f32x4 X[RT][CTW];
#pragma unroll
    for (int c = 0; c < CTW; ++c) {
        const int ct = wave + 8 * c;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            X[rt][c] = zero4();
            if (ct < RT) {  // H starts as the identity
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    X[rt][c][e] = (rt * 16 + 4 * g4 + e == ct * 16 + n16) ? 1.f : 0.f;
            }
        }
    }
    float log_s = 0.f;  // log of the scalar decay factored out of T

    const size_t tok_stride = (size_t)H * D;
    for (int64_t c0 = beg; c0 < end; c0 += CH) {
        const int n = (int)((end - c0) < CH ? (end - c0) : CH);
        // ---- 1. stage the chunk: K, V (16-bit planes, both orientations), gates
        for (int it = tid; it < CH * (D / 8); it += 512) {
            const int t = it / (D / 8), cg = it % (D / 8);
            float kx[8], vx[8];
            if (t < n) {
                const size_t e = (size_t)(c0 + t) * tok_stride + (size_t)h * D + cg * 8;
                load8<BF16>(k, e, kx);
                load8<BF16>(v, e, vx);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) { kx[e] = 0.f; vx[e] = 0.f; }
            }
            uint16_t kh[8], kl[8], vh[8], vl[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                put16<NSPLIT>(&kh[e], &kl[e], kx[e]);
                put16<NSPLIT>(&vh[e], &vl[e], vx[e]);
            }
            *reinterpret_cast<u32x4*>(&sm.Kr[0][t][cg * 8]) =
                u32x4{pack2(kh[0], kh[1]), pack2(kh[2], kh[3]), pack2(kh[4], kh[5]), pack2(kh[6], kh[7])};
            if constexpr (NSPLIT == 2)
                *reinterpret_cast<u32x4*>(&sm.Kr[1][t][cg * 8]) =
                    u32x4{pack2(kl[0], kl[1]), pack2(kl[2], kl[3]), pack2(kl[4], kl[5]), pack2(kl[6], kl[7])};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                sm.Kt[0][cg * 8 + e][t] = kh[e];
                sm.Vt[0][cg * 8 + e][t] = vh[e];
                if constexpr (NSPLIT == 2) {
                    sm.Kt[1][cg * 8 + e][t] = kl[e];
                    sm.Vt[1][cg * 8 + e][t] = vl[e];
                }
            }
        }
        if (tid < CH) {
            const bool ok = tid < n;
            const size_t e = (size_t)(c0 + tid) * H + h;
            sm.gate[tid] = ok ? load1<BF16>(gl, e) : 0.f;
            sm.beta[tid] = ok ? load1<BF16>(beta, e) : 0.f;
        }
        __syncthreads();

        // ---- 2. gate cumsum (wave 0, one token per lane) and Lt = tril(b K K^T, -1)
        if (wave == 0) {
            float x = sm.gate[lane];
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(x, off, 64);
                if (lane >= off) x += y;
            }
            const float bc = __shfl(x, 63, 64);
            sm.b[lane] = x;
            sm.eb[lane] = expf(x);
            sm.ebr[lane] = expf(bc - x);
            if (lane == 0) sm.bC = bc;
        }
        for (int tile = wave; tile < 10; tile += 8) {
            // lower-triangular 16x16 tiles (ti >= tj) of the 64x64 Gram matrix
            const int ti = tile < 1 ? 0 : tile < 3 ? 1 : tile < 6 ? 2 : 3;
            const int tj = tile - ti * (ti + 1) / 2;
            f32x4 gacc = zero4();
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) {
                const Frag<NSPLIT> a = frag_at<NSPLIT>(sm.Kr, ti * 16 + n16, ks * 32 + 8 * g4);
                const Frag<NSPLIT> bb = frag_at<NSPLIT>(sm.Kr, tj * 16 + n16, ks * 32 + 8 * g4);
                gacc = mma<NSPLIT>(a, bb, gacc);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = ti * 16 + 4 * g4 + e, s = tj * 16 + n16;
                sm.F1[t][s] = (s < t) ? sm.beta[t] * gacc[e] : 0.f;
            }
        }
        __syncthreads();

        // ---- 3. At = (I + Lt)^-1
        tri_inverse(sm, wave, lane);

        // ---- 4. Ap = At diag(beta), Ad = A diag(beta) with A[t][s] = e^{b_t - b_s} At[t][s]
        for (int it = tid; it < CH * CH; it += 512) {
            const int t = it / CH, s = it % CH;
            float ap = 0.f, ad = 0.f;
            if (s <= t) {
                const float a = sm.F2[t][s] * sm.beta[s];
                ap = a;
                ad = a * expf(sm.b[t] - sm.b[s]);
            }
            put16<NSPLIT>(&sm.Ap[0][t][s], &sm.Ap[NSPLIT - 1][t][s], ap);
            put16<NSPLIT>(&sm.Ad[0][t][s], &sm.Ad[NSPLIT - 1][t][s], ad);
        }
        __syncthreads();

        // ---- 5. Wt^T = K^T Ap^T (written token-major into Wt), and U for own S tiles
        for (int tile = wave; tile < RT * 4; tile += 8) {
            const int mt = tile / 4, nt = tile % 4;  // channel tile, token tile
            f32x4 acc = zero4();
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const Frag<NSPLIT> a = frag_at<NSPLIT>(sm.Kt, mt * 16 + n16, ks * 32 + 8 * g4);
                const Frag<NSPLIT> bb = frag_at<NSPLIT>(sm.Ap, nt * 16 + n16, ks * 32 + 8 * g4);
                acc = mma<NSPLIT>(a, bb, acc);
            }
            // lane holds Wt[token nt*16+n16][channels mt*16+4*g4 .. +3]
            uint16_t hh[4], ll[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) put16<NSPLIT>(&hh[e], &ll[e], acc[e]);
            *reinterpret_cast<u32x2*>(&sm.Wt[0][nt * 16 + n16][mt * 16 + 4 * g4]) =
                u32x2{pack2(hh[0], hh[1]), pack2(hh[2], hh[3])};
            if constexpr (NSPLIT == 2)
                *reinterpret_cast<u32x2*>(&sm.Wt[1][nt * 16 + n16][mt * 16 + 4 * g4]) =
                    u32x2{pack2(ll[0], ll[1]), pack2(ll[2], ll[3])};
        }
        f32x4 U[4][CTW];
#pragma unroll
        for (int c = 0; c < CTW; ++c) {
            const int ct = wave + 8 * c;
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                U[tt][c] = zero4();
                if (ct >= RT && ct < NCT) {
                    const int vt = ct - RT;  // value-channel tile
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        const Frag<NSPLIT> a = frag_at<NSPLIT>(sm.Ad, tt * 16 + n16, ks * 32 + 8 * g4);
                        const Frag<NSPLIT> bb = frag_at<NSPLIT>(sm.Vt, vt * 16 + n16, ks * 32 + 8 * g4);
                        U[tt][c] = mma<NSPLIT>(a, bb, U[tt][c]);
                    }
                }
            }
        }
        __syncthreads();

        // ---- 6..8. per owned column tile: Y = Wt X, R, X += K^T R
        const float bC = sm.bC;
        const float ebC = expf(bC);
#pragma unroll
        for (int c = 0; c < CTW; ++c) {
            const int ct = wave + 8 * c;
            if (ct >= NCT) continue;
            const bool is_s = ct >= RT;
            // X column tile as B fragments (k = X rows)
            Frag<NSPLIT> xb[KSD];
#pragma unroll
            for (int kb = 0; kb < KSD; ++kb) {
                const f32x4 d0 = X[2 * kb][c];
                const f32x4 d1 = (2 * kb + 1 < RT) ? X[2 * kb + 1 < RT ? 2 * kb + 1 : 0][c] : zero4();
                xb[kb] = dpair_to_frag<NSPLIT>(d0, d1);
            }
            f32x4 R[4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                f32x4 y = zero4();
#pragma unroll
                for (int kb = 0; kb < KSD; ++kb) {
                    const Frag<NSPLIT> a = frag_at<NSPLIT>(sm.Wt, tt * 16 + n16, kb * 32 + 8 * g4);
                    y = mma<NSPLIT>(a, xb[kb], y);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = tt * 16 + 4 * g4 + e;
                    R[tt][e] = is_s ? sm.ebr[t] * (U[tt][c][e] - sm.eb[t] * y[e]) : -y[e];
                }
            }
            Frag<NSPLIT> rb[2];
            rb[0] = dpair_to_frag<NSPLIT>(R[0], R[1]);
            rb[1] = dpair_to_frag<NSPLIT>(R[2], R[3]);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                f32x4 acc = is_s ? X[rt][c] * ebC : X[rt][c];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const Frag<NSPLIT> a = frag_at<NSPLIT>(sm.Kt, rt * 16 + n16, kb * 32 + 8 * g4);
                    acc = mma<NSPLIT>(a, rb[kb], acc);
                }
                X[rt][c] = acc;
            }
        }
        log_s += bC;
        __syncthreads();
    }

    // ---- emit T_C = e^{log_s} H and S(C|0)
    const float tscale = expf(log_s);
    const size_t pair = (size_t)seg * H + h;
#pragma unroll
    for (int c = 0; c < CTW; ++c) {
        const int ct = wave + 8 * c;
        if (ct >= NCT) continue;
        const bool is_s = ct >= RT;
        if (!is_s && T_out == nullptr) continue;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = rt * 16 + 4 * g4 + e;
                if (is_s) S_out[pair * D * D + (size_t)row * D + (ct - RT) * 16 + n16] = X[rt][c][e];
                else put_t(T_out, t_split, pair, D, row, ct * 16 + n16, tscale * X[rt][c][e]);
            }
    }
}

template <int D, int NSPLIT, bool BF16>
static hipError_t launch_gdn(int n_seg, int H, const int64_t* sb, const int64_t* se, int64_t n_tok,
                             const void* k, const void* v, const void* g, const void* beta,
                             void* T_out, bool t_split, float* S_out, hipStream_t st)
{
    hipLaunchKernelGGL((build_gdn_kernel<D, NSPLIT, BF16>), dim3(n_seg * H), dim3(512), 0, st, n_seg,
                       H, sb, se, n_tok, k, v, g, beta, T_out, (int)t_split, S_out);
    return hipGetLastError();
}

hipError_t build_gdn(int d, bool in_bf16, int n_seg, int H, const int64_t* sb, const int64_t* se,
                     int64_t n_tok, const void* k, const void* v, const void* g, const void* beta,
                     void* T_out, bool t_split, float* S_out, hipStream_t st)
{
    if (d == 128 && in_bf16) return launch_gdn<128, 1, true>(n_seg, H, sb, se, n_tok, k, v, g, beta, T_out, t_split, S_out, st);
    if (d == 64 && in_bf16) return launch_gdn<64, 1, true>(n_seg, H, sb, se, n_tok, k, v, g, beta, T_out, t_split, S_out, st);
    if (d == 16 && !in_bf16) return launch_gdn<16, 2, false>(n_seg, H, sb, se, n_tok, k, v, g, beta, T_out, t_split, S_out, st);
    if (d == 16 && in_bf16) return launch_gdn<16, 1, true>(n_seg, H, sb, se, n_tok, k, v, g, beta, T_out, t_split, S_out, st);
    return hipErrorNotSupported;
}

}  // namespace hypic
