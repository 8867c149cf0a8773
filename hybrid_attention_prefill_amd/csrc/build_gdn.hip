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
//
// Data movement: the next chunk's k, v, gates and betas are loaded into
// registers while the current chunk is processed (raw bits, unconditional
// loads of clamped token rows); staging converts them and writes K token-major
// and K^T, V^T channel-major through 4 x 8 register transposes.  Every LDS
// operand matrix is kept in fragment order (frag_off), so each MFMA operand
// fragment is one contiguous, conflict-free 1 KiB read; a wave reads each A
// fragment once for all of its column tiles.
#include "hypic_device.h"
#include "hypic_kernels.h"
#include "build_common.h"

namespace hypic {

namespace {
using namespace bld;

constexpr int CH = 64;       // chunk length
constexpr float kLog2e = 1.4426950408889634f;
constexpr int LDF = CH + 1;  // padded LDS row for fp32 64x64 matrices

template <int D, int NSPLIT>
struct alignas(16) GdnSmem {
    static constexpr int KP = D < 32 ? 32 : D;  // channel contraction padded to 32
    uint16_t Kr[NSPLIT][CH * KP];  // K, rows = tokens, cols = channels (>= D zero)
    uint16_t Kt[NSPLIT][D * CH];   // K^T, rows = channels, cols = tokens
    uint16_t Vt[NSPLIT][D * CH];   // V^T, rows = channels, cols = tokens
    uint16_t Ap[NSPLIT][CH * CH];  // At diag(beta)
    uint16_t Ad[NSPLIT][CH * CH];  // A diag(beta)
    uint16_t Wt[NSPLIT][CH * KP];  // Wt, rows = tokens, cols = channels (>= D zero)
    float F1[CH][LDF];             // Lt (strictly lower)
    float F2[CH][LDF];             // At
    float F3[32][33];              // inverse scratch
    float gate[CH], beta[CH], b[CH], eb[CH], ebr[CH];   // b in log2 units
    float bC;
};

// LDS operand planes are fragment-ordered (frag_off) with the 16-byte chunks XOR-swizzled:
// chunk c is stored at c ^ ((c >> 4 ^ c >> 7) & 7).  The swizzle permutes chunks within
// aligned groups of 8, so a fragment read stays one 1 KiB block read conflict-free, while
// the staging stores (token rows, channel rows, 8 lanes on 8 different rows) spread over
// the banks instead of landing on one.
__device__ __forceinline__ int swz(int off) {
    const int c = off >> 3;
    return ((c ^ (((c >> 4) ^ (c >> 7)) & 7)) << 3) | (off & 7);
}
__device__ __forceinline__ int lds_off(int row, int col, int ncols) { return swz(frag_off(row, col, ncols)); }

// A-operand fragment (row tile rt, k-block ks) of a [rows][ncols] plane: lane l gets
// row rt*16 + l%16, columns ks*32 + 8(l/16) .. +7.  Fragment F = rt*(ncols/32) + ks is
// chunks 64F .. 64F+63; for those the swizzle reduces to l -> l ^ (l >> 4) ^ K_F with
// K_F = 4(F & 1) ^ ((F >> 1) & 7), so with lx = l ^ (l >> 4) per thread every read is a
// lane offset from 8 fixed values plus an immediate.
template <int NCOLS>
__device__ __forceinline__ f16x8 lds_frag(const uint16_t* P, int rt, int ks, int lx) {
    const int F = rt * (NCOLS / 32) + ks;
    const int K = ((F & 1) << 2) ^ ((F >> 1) & 7);
    return *reinterpret_cast<const f16x8*>(P + F * 512 + 8 * (lx ^ K));
}
template <int NSPLIT, int NCOLS, typename Arr>
__device__ __forceinline__ Frag<NSPLIT> frag_of(const Arr& a, int rt, int ks, int lx) {
    Frag<NSPLIT> f;
    f.h = lds_frag<NCOLS>(a[0], rt, ks, lx);
    if constexpr (NSPLIT == 2) f.l = lds_frag<NCOLS>(a[1], rt, ks, lx);
    return f;
}

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

// 16-bit operand bits of x (NSPLIT 1: fp16; NSPLIT 2: fp16 hi and lo)
template <int NSPLIT>
__device__ __forceinline__ void to16(float x, uint16_t& hi, uint16_t& lo) {
    if constexpr (NSPLIT == 1) {
        hi = f16_bits((_Float16)x);
        lo = 0;
    } else {
        _Float16 a, b;
        split_f16(x, a, b);
        hi = f16_bits(a);
        lo = f16_bits(b);
    }
}

// An empty asm that "modifies" x: values derived from it inside a loop body are
// recomputed each iteration instead of being hoisted (and then spilled) by the compiler.
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

__device__ __forceinline__ u32x4 pack8(const uint16_t* x) {
    return u32x4{pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]), pack2(x[6], x[7])};
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
    constexpr int CB = D / 8;               // 8-channel blocks per token
    constexpr int NBLK = (CH / 4) * CB;     // 4-token x 8-channel blocks per matrix
    constexpr int WPR = BF16 ? 1 : 2;       // 16-byte words per 8 channels of one token
    static_assert(2 * NBLK <= 512, "one block per thread");
    __shared__ SM sm;

    const int unit = blockIdx.x;
    const int seg = unit / H, h = unit % H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g4 = lane >> 4, n16 = lane & 15;
    // column tile ct = wave + 8 c of X is an S tile (ct >= RT); known at compile time when
    // the H and S tiles split evenly over the 8 waves
    auto s_tile = [&](int c) -> bool { return RT % 8 == 0 ? c * 8 >= RT : wave + 8 * c >= RT; };
    auto own_tile = [&](int c) -> bool { return NCT % 8 == 0 || wave + 8 * c < NCT; };

    int64_t beg = seg_begin[seg], end = seg_end[seg];
    beg = beg < 0 ? 0 : (beg > n_tokens ? n_tokens : beg);
    end = end < beg ? beg : (end > n_tokens ? n_tokens : end);

    // zero the channel padding of Kr / Wt once (D < 32 only)
    if (KP > D) {
        for (int i = tid; i < NSPLIT * CH * KP; i += 512) {
            (&sm.Kr[0][0])[i] = 0;
            (&sm.Wt[0][0])[i] = 0;
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

    // ---- next-chunk prefetch: thread -> (matrix K or V, 4-token block tb, 8-channel block cb)
    const bool has_blk = tid < 2 * NBLK;
    const int blk = has_blk ? tid : 0;
    const bool blk_v = blk >= NBLK;
    const int tb0 = (blk % NBLK) / CB, cb0 = (blk % NBLK) % CB;
    const void* blk_src = blk_v ? v : k;
    const size_t tok_stride = (size_t)H * D;
    u32x4 raw[4][WPR];            // 4 token rows x 8 channels, raw input bits
    uint32_t graw = 0, braw = 0;  // gate and beta of token `lane` (wave 0), raw bits
    auto prefetch = [&](int64_t c0) {
        // rows past the segment are clamped into it (masked when staged); the loads are
        // unconditional so that nothing waits for them before the next chunk's staging
        const int tb = opaque(tb0), cb = opaque(cb0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            int64_t t = c0 + tb * 4 + r;
            t = t < end ? t : end - 1;
            const size_t e = (size_t)t * tok_stride + (size_t)h * D + cb * 8;
            if constexpr (BF16) {
                raw[r][0] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(blk_src) + e);
            } else {
                const u32x4* p = reinterpret_cast<const u32x4*>(reinterpret_cast<const float*>(blk_src) + e);
                raw[r][0] = p[0];
                raw[r][WPR - 1] = p[1];
            }
        }
        int64_t t = c0 + lane;
        t = t < end ? t : end - 1;
        const size_t e = (size_t)t * H + h;
        if constexpr (BF16) {
            graw = reinterpret_cast<const uint16_t*>(gl)[e];
            braw = reinterpret_cast<const uint16_t*>(beta)[e];
        } else {
            graw = reinterpret_cast<const uint32_t*>(gl)[e];
            braw = reinterpret_cast<const uint32_t*>(beta)[e];
        }
    };
    auto raw_val = [&](int r, int c) -> float {   // channel c (0..7) of row r
        if constexpr (BF16) {
            const uint32_t w = raw[r][0][c >> 1];
            return __uint_as_float((c & 1) ? (w & 0xFFFF0000u) : (w << 16));
        } else {
            return __uint_as_float(raw[r][c >> 2][c & 3]);
        }
    };
    auto raw1 = [&](uint32_t x) -> float { return BF16 ? __uint_as_float(x << 16) : __uint_as_float(x); };

    if (beg < end) prefetch(beg);

    for (int64_t c0 = beg; c0 < end; c0 += CH) {
        const int n = (int)((end - c0) < CH ? (end - c0) : CH);
        // lane-derived indices, recomputed per chunk (cheap) rather than kept live across it
        const int lane_c = opaque(lane);
        const int g4 = lane_c >> 4, n16 = lane_c & 15, lx = lane_c ^ g4;
        const int tb = opaque(tb0), cb = opaque(cb0);
        // ---- 1. stage the chunk: K token-major, K^T and V^T channel-major (16-bit), gates
        if (has_blk) {
            // masked values of the 4 x 8 block; rows past the segment are zero
            float f[4][8];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool live = tb * 4 + r < n;
#pragma unroll
                for (int c = 0; c < 8; ++c) f[r][c] = live ? raw_val(r, c) : 0.f;
            }
            uint16_t(*dst)[D * CH] = blk_v ? sm.Vt : sm.Kt;
            if constexpr (NSPLIT == 1 && BF16) {
                // bf16 values are exact in fp16 (inside its range): round-toward-zero packing is exact
                auto pk = [](float a, float b) -> unsigned {
                    return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(a, b));
                };
                if (!blk_v) {   // K rows (8 channels of one token = 16 contiguous bytes)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        *reinterpret_cast<u32x4*>(&sm.Kr[0][lds_off(tb * 4 + r, cb * 8, KP)]) =
                            u32x4{pk(f[r][0], f[r][1]), pk(f[r][2], f[r][3]), pk(f[r][4], f[r][5]), pk(f[r][6], f[r][7])};
                }
                // transposed: one channel row, 4 consecutive tokens = 8 contiguous bytes
#pragma unroll
                for (int c = 0; c < 8; ++c)
                    *reinterpret_cast<u32x2*>(&dst[0][lds_off(cb * 8 + c, tb * 4, CH)]) =
                        u32x2{pk(f[0][c], f[1][c]), pk(f[2][c], f[3][c])};
            } else {
                uint16_t hb[4][8], lb[4][8];   // [token][channel]
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int c = 0; c < 8; ++c) to16<NSPLIT>(f[r][c], hb[r][c], lb[r][c]);
                if (!blk_v) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int off = lds_off(tb * 4 + r, cb * 8, KP);
                        *reinterpret_cast<u32x4*>(&sm.Kr[0][off]) = pack8(hb[r]);
                        if constexpr (NSPLIT == 2) *reinterpret_cast<u32x4*>(&sm.Kr[1][off]) = pack8(lb[r]);
                    }
                }
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const int off = lds_off(cb * 8 + c, tb * 4, CH);
                    *reinterpret_cast<u32x2*>(&dst[0][off]) = u32x2{pack2(hb[0][c], hb[1][c]), pack2(hb[2][c], hb[3][c])};
                    if constexpr (NSPLIT == 2)
                        *reinterpret_cast<u32x2*>(&dst[1][off]) = u32x2{pack2(lb[0][c], lb[1][c]), pack2(lb[2][c], lb[3][c])};
                }
            }
        }
        if (wave == 0) {
            const bool ok = lane < n;
            sm.gate[lane] = ok ? raw1(graw) : 0.f;
            sm.beta[lane] = ok ? raw1(braw) : 0.f;
        }
        // the next chunk's loads fly during this chunk
        if (c0 + CH < end) prefetch(c0 + CH);
        __syncthreads();

        // ---- 2. gate cumsum (wave 0, one token per lane) and Lt = tril(b K K^T, -1)
        if (wave == 0) {
            float x = sm.gate[lane];
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(x, off, 64);
                if (lane >= off) x += y;
            }
            // decay factors through v_exp_f32 (2^x) on log2-scaled sums; b is kept in log2 units
            const float bc = __shfl(x, 63, 64);
            const float x2 = x * kLog2e, bc2 = bc * kLog2e;
            sm.b[lane] = x2;
            sm.eb[lane] = __builtin_amdgcn_exp2f(x2);
            sm.ebr[lane] = __builtin_amdgcn_exp2f(bc2 - x2);
            if (lane == 0) sm.bC = bc;
        }
        for (int tile = wave; tile < 10; tile += 8) {
            // lower-triangular 16x16 tiles (ti >= tj) of the 64x64 Gram matrix
            const int ti = tile < 1 ? 0 : tile < 3 ? 1 : tile < 6 ? 2 : 3;
            const int tj = tile - ti * (ti + 1) / 2;
            f32x4 gacc = zero4();
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) {
                const Frag<NSPLIT> a = frag_of<NSPLIT, KP>(sm.Kr, ti, ks, lx);
                const Frag<NSPLIT> bb = frag_of<NSPLIT, KP>(sm.Kr, tj, ks, lx);   // K^T as B = rows of K
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

        // ---- 4. Ap = At diag(beta), Ad = A diag(beta) with A[t][s] = e^{b_t - b_s} At[t][s];
        // one token row t and 8 consecutive s per thread (16-byte stores)
        {
            const int t = tid >> 3, s0 = (tid & 7) * 8;
            uint16_t ph[8], pl[8], dh[8], dl[8];
            const float bt = sm.b[t];
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                const int s = s0 + x;
                float ap = 0.f, ad = 0.f;
                if (s <= t) {
                    ap = sm.F2[t][s] * sm.beta[s];
                    ad = ap * __builtin_amdgcn_exp2f(bt - sm.b[s]);   // e^{b_t - b_s}, exponent <= 0
                }
                to16<NSPLIT>(ap, ph[x], pl[x]);
                to16<NSPLIT>(ad, dh[x], dl[x]);
            }
            const int off = lds_off(t, s0, CH);
            *reinterpret_cast<u32x4*>(&sm.Ap[0][off]) = pack8(ph);
            *reinterpret_cast<u32x4*>(&sm.Ad[0][off]) = pack8(dh);
            if constexpr (NSPLIT == 2) {
                *reinterpret_cast<u32x4*>(&sm.Ap[1][off]) = pack8(pl);
                *reinterpret_cast<u32x4*>(&sm.Ad[1][off]) = pack8(dl);
            }
        }
        __syncthreads();

        // ---- 5. Wt^T = K^T Ap^T (written token-major into Wt), and U for own S tiles
        for (int tile = wave; tile < RT * 4; tile += 8) {
            const int mt = tile / 4, nt = tile % 4;  // channel tile, token tile
            f32x4 acc = zero4();
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const Frag<NSPLIT> a = frag_of<NSPLIT, CH>(sm.Kt, mt, ks, lx);
                const Frag<NSPLIT> bb = frag_of<NSPLIT, CH>(sm.Ap, nt, ks, lx);   // Ap^T as B = rows of Ap
                acc = mma<NSPLIT>(a, bb, acc);
            }
            // lane holds Wt[token nt*16+n16][channels mt*16+4*g4 .. +3]
            uint16_t hh[4], ll[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) to16<NSPLIT>(acc[e], hh[e], ll[e]);
            const int off = lds_off(nt * 16 + n16, mt * 16 + 4 * g4, KP);
            *reinterpret_cast<u32x2*>(&sm.Wt[0][off]) = u32x2{pack2(hh[0], hh[1]), pack2(hh[2], hh[3])};
            if constexpr (NSPLIT == 2)
                *reinterpret_cast<u32x2*>(&sm.Wt[1][off]) = u32x2{pack2(ll[0], ll[1]), pack2(ll[2], ll[3])};
        }
        f32x4 U[4][CTW];
#pragma unroll
        for (int c = 0; c < CTW; ++c) {
            const int ct = wave + 8 * c;
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                U[tt][c] = zero4();
                if (s_tile(c) && ct < NCT) {
                    const int vt = ct - RT;  // value-channel tile
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        const Frag<NSPLIT> a = frag_of<NSPLIT, CH>(sm.Ad, tt, ks, lx);
                        const Frag<NSPLIT> bb = frag_of<NSPLIT, CH>(sm.Vt, vt, ks, lx);   // V as B = rows of V^T
                        U[tt][c] = mma<NSPLIT>(a, bb, U[tt][c]);
                    }
                }
            }
        }
        __syncthreads();

        // ---- 6..8. Y = Wt X, R, X += K^T R for all owned column tiles at once (each A
        // fragment is read once per wave)
        const float bC = sm.bC;
        const float ebC = __builtin_amdgcn_exp2f(bC * kLog2e);
        if (wave < NCT) {
            f32x4 R[4][CTW];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                for (int c = 0; c < CTW; ++c) R[tt][c] = zero4();
#pragma unroll
            for (int kb = 0; kb < KSD; ++kb) {
                Frag<NSPLIT> xb[CTW];   // rows 32 kb .. 32 kb + 31 of the X column tiles as B fragments
#pragma unroll
                for (int c = 0; c < CTW; ++c) {
                    const f32x4 d0 = X[2 * kb][c];
                    const f32x4 d1 = (2 * kb + 1 < RT) ? X[2 * kb + 1 < RT ? 2 * kb + 1 : 0][c] : zero4();
                    xb[c] = dpair_to_frag<NSPLIT>(d0, d1);
                }
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    const Frag<NSPLIT> a = frag_of<NSPLIT, KP>(sm.Wt, tt, kb, lx);
#pragma unroll
                    for (int c = 0; c < CTW; ++c)
                        if (own_tile(c)) R[tt][c] = mma<NSPLIT>(a, xb[c], R[tt][c]);
                }
            }
            Frag<NSPLIT> rb[2][CTW];
#pragma unroll
            for (int c = 0; c < CTW; ++c) {
                const bool is_s = s_tile(c);
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int t = tt * 16 + 4 * g4 + e;
                        R[tt][c][e] = is_s ? sm.ebr[t] * (U[tt][c][e] - sm.eb[t] * R[tt][c][e]) : -R[tt][c][e];
                    }
                rb[0][c] = dpair_to_frag<NSPLIT>(R[0][c], R[1][c]);
                rb[1][c] = dpair_to_frag<NSPLIT>(R[2][c], R[3][c]);
                if (is_s) {
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) X[rt][c] *= ebC;
                }
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const Frag<NSPLIT> a = frag_of<NSPLIT, CH>(sm.Kt, rt, kb, lx);
#pragma unroll
                    for (int c = 0; c < CTW; ++c)
                        if (own_tile(c)) X[rt][c] = mma<NSPLIT>(a, rb[kb][c], X[rt][c]);
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
