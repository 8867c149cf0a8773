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
// where H is the undecayed transition product, so the decay never pushes the T
// columns out of the 16-bit MFMA operands' range; the decay of T is one fp32
// scale at the end.  The erase alone still shrinks H over long segments, so H
// is renormalised by powers of two between chunks (exponent kept apart).
//
// One workgroup (8 waves) per (segment, head).  The augmented state X = [H | S]
// (d x 2d, fp32) lives in MFMA accumulators, 16-column tiles dealt to waves;
// the chunk products run on v_mfma_f32_16x16x32_f16 with fp32 accumulation:
// K K^T, Wt, U, Y = Wt X and X += K^T R.  X and R reach the B operand without
// LDS through two cross-lane swaps.  Operands are fp16 (one rounding, NSPLIT = 1)
// for bf16 inputs, or fp16 hi + lo with three products (NSPLIT = 2) for fp32
// inputs.  The 64 x 64 triangular system is blocked 16 x 16: each diagonal block
// is inverted as the product (I + N)(I + N^2)(I + N^4)(I + N^8), N = -Lt_ii, on
// v_mfma_f32_16x16x16_f16 with hi / lo operands.  Without per-token outputs the
// chunks are pipelined (two steps per chunk, described at the loop): the inverse
// At diag(b) is formed explicitly from the blocks and Wt, U are dense products
// with it.  With outputs, Wt and U come from block forward substitution.
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

// K^T and V^T come in KTB buffers (by chunk parity), the betas, log-decays and decay
// factors in RB (by chunk index modulo RB)
template <int D, int NSPLIT, int KTB, int RB>
struct alignas(16) GdnSmem {
    static constexpr int KP = D < 32 ? 32 : D;  // channel contraction padded to 32
    uint16_t Kr[NSPLIT][CH * KP];  // K, rows = tokens, cols = channels (>= D zero)
    uint16_t Kt[KTB][NSPLIT][D * CH];   // K^T, rows = channels, cols = tokens
    uint16_t Vt[KTB][NSPLIT][D * CH];   // V^T, rows = channels, cols = tokens
    uint16_t Wt[NSPLIT][CH * KP];  // -Wt, rows = tokens, cols = channels (>= D zero)
    // block forward substitution operands: A fragments of v_mfma_f32_16x16x16_f16 (lane
    // 16 g + r holds row r, columns 4 g .. 4 g + 3), fp16 hi / lo planes
    uint16_t Ln[2][6][256];        // -Lt_ij for the blocks j < i (index i (i - 1) / 2 + j)
    uint16_t Lnd[2][6][256];       // the same with the decay: -e^{b_t - b_s} Lt
    uint16_t Dv[2][4][256];        // (I + Lt_ii)^-1, diagonal block i
    uint16_t Dvd[2][4][256];       // the same with the decay e^{b_t - b_s}
    float Sd[4][16][20];           // per diagonal block: (I + Lt_ii)^-1 (fp32)
    float beta[RB][CH];
    float lb[RB][CH], eb[RB][CH], ebr[RB][CH];   // b_t (log2 units), e^{b_t}, e^{b_C - b_t}
    float bC[RB];
    float hmax[2][8];              // per wave: max |H| after a chunk's update (by chunk parity)
};

// The chunk's inverse with the betas folded in, Ab = (I + Lt)^-1 diag(b), and its decayed
// form D Ab D^-1, as A-operand planes of v_mfma_f32_16x16x32_f16 (fp16 hi / lo): fragment
// f = (row tile, 32-token k-step) for the six pairs (0,0) (1,0) (2,0) (2,1) (3,0) (3,1)
// that hold the lower triangle; lane l holds row l % 16, columns 8 (l / 16) .. + 7.  The
// blocks above the diagonal inside them, (0,1) and (2,3), stay zero.
template <bool ON>
struct alignas(16) GdnInvSmem {
    uint16_t Ab[2][2][6][512];   // [plain, decayed][hi, lo][fragment][lane * 8 + j]
};
template <>
struct alignas(16) GdnInvSmem<false> {
    uint16_t Ab[1][1][1][8];
};
__device__ __forceinline__ int ab_frag(int rt, int ks) { return rt < 2 ? rt : 2 * rt - 2 + ks; }

template <int J>
struct IntC {
    static constexpr int value = J;
};

// LDS of the per-token outputs (OUT): q of this or the next chunk as loaded (bf16,
// token-major, direct global->LDS), q of this chunk as an fp16 operand plane like Kr, and the masked
// product M = scale (Q K^T o e^{b_t - b_s}, s <= t) as an fp16 operand plane.
template <int D>
struct alignas(16) GdnOutSmem {
    static constexpr int KP = D < 32 ? 32 : D;
    uint16_t Qraw[2][CH * D];      // by chunk parity
    uint16_t Qr[1][CH * KP];
    uint16_t Mq[1][CH * CH];
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

// a lane's value moved by a DPP control (lanes without a source, or outside row_mask, get 0)
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_move(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWS, 0xf, true));
}
// Inclusive sum over the 64 lanes of a wave on DPP: shifts by 1, 2, 4, 8 inside each row of
// 16 lanes, then the last lane of row r added to the rows above it (row_bcast:15, :31).
__device__ __forceinline__ float wave_inclusive_sum(float x) {
    x += dpp_move<0x111, 0xf>(x);   // row_shr:1
    x += dpp_move<0x112, 0xf>(x);   // row_shr:2
    x += dpp_move<0x114, 0xf>(x);   // row_shr:4
    x += dpp_move<0x118, 0xf>(x);   // row_shr:8
    x += dpp_move<0x142, 0xa>(x);   // row_bcast:15 into rows 1, 3
    x += dpp_move<0x143, 0xc>(x);   // row_bcast:31 into rows 2, 3
    return x;
}

__device__ __forceinline__ u32x4 pack8(const uint16_t* x) {
    return u32x4{pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]), pack2(x[6], x[7])};
}

}  // namespace

template <int D, int NSPLIT, bool BF16, bool WANT_T, bool OUT, bool NW>
__global__ __launch_bounds__(512) void build_gdn_kernel(
    int n_seg, int H, const int64_t* __restrict__ seg_begin, const int64_t* __restrict__ seg_end,
    int64_t n_tokens, const void* __restrict__ k, const void* __restrict__ v,
    const void* __restrict__ gl, const void* __restrict__ beta, void* __restrict__ T_out, int t_split,
    float* __restrict__ S_out, int v_ld, BuildItems items, BuildOut ob)
{
    // v_ld: the row length of v ([n_tokens][H][v_ld]) and of S_out ([pair][D][v_ld]); v and
    // S_out point at this call's D columns (D columns of a wider state, built one block at a
    // time: the columns of S evolve independently).  With v_ld < D (NW, narrow values) the
    // values have only v_ld columns: the rest are read as zeros and those columns of S are not
    // written.
    const int v_cols = NW ? v_ld : D;
    // Without outputs the chunks are pipelined (two steps per chunk, see the loop below);
    // with outputs they run one after the other, in four steps.
    constexpr bool PIPE = !OUT;
    using SM = GdnSmem<D, NSPLIT, PIPE ? 2 : 1, PIPE ? 3 : 1>;
    static_assert(!OUT || (NSPLIT == 1 && BF16 && D >= 64), "outputs: bf16 inputs, d 64 or 128");
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
    __shared__ GdnOutSmem<OUT ? D : 16> so_;   // used only with OUT
    auto& so = so_;
    __shared__ GdnInvSmem<PIPE> si;

    const int unit = blockIdx.x;
    const int seg = unit / H, h = unit % H;
    // items mode: range `seg` of the plan is a segment or a piece of one; its pair goes to
    // the caller's slot out >= 0 or to workspace slot -1 - out (T as bf16 hi/lo planes)
    int64_t beg = seg_begin[seg], end = seg_end[seg];
    int out = seg;
    int s_ld = v_ld;   // row length of the S destination (workspace slots are D x D)
    int s_cols = v_cols;
    if (items.out) {
        // the item's fields are read before the live-item check (the arrays hold n_seg
        // entries), so the loads go out together
        const int n_live = *items.n_items;
        out = items.out[seg];
        if (seg >= n_live) return;
        if (out < 0) {
            T_out = items.T_ws;
            t_split = 1;
            S_out = items.S_ws;
            s_ld = D;
            s_cols = D;
            out = -1 - out;
        }
    }
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g4 = lane >> 4, n16 = lane & 15;
    // column tiles of X owned by this wave: ct = tile(c) = wave + 8 c, c < CTW; ct >= RT is
    // an S tile, known at compile time when the H and S tiles split evenly over the 8 waves
    // (two tiles per wave: one of each kind, which balances the state update's work)
    auto tile = [&](int c) -> int { return wave + 8 * c; };
    auto s_tile = [&](int c) -> bool { return RT % 8 == 0 ? c * 8 >= RT : tile(c) >= RT; };
    auto own_tile = [&](int c) -> bool { return NCT % 8 == 0 || tile(c) < NCT; };

    // WANT_T false (T not requested): only the S columns of X are advanced (the Wt solve
    // is shared by both)
    auto upd_tile = [&](int c) -> bool { return own_tile(c) && (WANT_T || s_tile(c)); };
    beg = beg < 0 ? 0 : (beg > n_tokens ? n_tokens : beg);
    end = end < beg ? beg : (end > n_tokens ? n_tokens : end);

    // the blocks above the diagonal inside the inverse planes: lanes 32..63 of fragments 0, 3
    if constexpr (PIPE) {
        for (int i = tid; i < 2 * 2 * 2 * 256; i += 512) {
            const int pl = i >> 9, f = ((i >> 8) & 1) ? 3 : 0;
            (&si.Ab[0][0][0][0])[pl * 6 * 512 + f * 512 + 256 + (i & 255)] = 0;
        }
    }
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
        const int ct = tile(c);
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
    int h2 = 0;         // power of two factored out of H: T_C = e^{log_s} 2^{h2} H

    // ---- next-chunk prefetch: thread -> (matrix K or V, 4-token block tb, 8-channel block cb)
    const bool has_blk = tid < 2 * NBLK;
    const int blk = has_blk ? tid : 0;
    const bool blk_v = blk >= NBLK;
    const int tb0 = (blk % NBLK) / CB, cb0 = (blk % NBLK) % CB;
    const void* blk_src = blk_v ? v : k;
    // row length of this thread's matrix: K blocks d, V blocks v_ld (uniform per wave where the
    // V blocks fill whole waves, so it is kept in a scalar register there)
    const int blk_ld = (NBLK % 64 == 0) ? __builtin_amdgcn_readfirstlane(blk_v ? v_ld : D) : (blk_v ? v_ld : D);
    // V blocks past the value columns (v_ld < D) load column block 0 and are not staged: their
    // rows of the V^T planes keep the zeros written at the start
    const bool blk_zero = NW && blk_v && cb0 * 8 >= v_cols;
    u32x4 raw[4][WPR];            // 4 token rows x 8 channels, raw input bits
    uint32_t graw = 0, braw = 0;  // gate and beta of token `lane` (wave 0), raw bits
    auto prefetch = [&](int64_t c0) {
        // rows past the segment are clamped into it (masked when staged); the loads are
        // unconditional so that nothing waits for them before the next chunk's staging
        const int tb = opaque(tb0), cb = blk_zero ? 0 : opaque(cb0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            int64_t t = c0 + tb * 4 + r;
            t = t < end ? t : end - 1;
            const size_t e = ((size_t)t * H + h) * blk_ld + cb * 8;
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

    // q of a chunk, global -> LDS direct (16 bytes per lane, token-major; rows past the
    // segment are clamped into it and masked when converted)
    auto fetch_q = [&](int64_t c0, int buf) {
        if constexpr (OUT) {
            constexpr int NQ = CH * D / 8;   // 16-byte pieces
#pragma unroll
            for (int r = 0; r < NQ / 512; ++r) {
                const int m = r * 512 + wave * 64 + lane;
                int64_t t = c0 + m / (D / 8);
                t = t < end ? t : end - 1;
                const uint16_t* src = reinterpret_cast<const uint16_t*>(ob.q) + (t * H + h) * D + (m % (D / 8)) * 8;
                __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(so.Qraw[buf] + (r * 512 + wave * 64) * 8),
                                                 16, 0, 0);
            }
        }
    };

    // ---- staging of a chunk of n_s tokens from the prefetched registers, in two parts:
    // (a) K token-major, betas and log-decays into ring slot rb; (b) K^T and V^T channel-major
    // into buffer kbuf (16-bit operands).
    // Rows past the segment (the last chunk's) hold copies of its last row, finite values:
    // their betas are staged as zero, so their rows and columns of Ab are zero (Lt has zero
    // rows there and (I + Lt)^-1 diag(b) zero columns), and with them their rows of Wt, U and
    // R: they enter no product with a nonzero weight and need no zeroing.
    auto stage_rows = [&](float (&f)[4][8]) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < 8; ++c) f[r][c] = raw_val(r, c);
    };
    // bf16 values are exact in fp16 inside its range; round-to-nearest packing (one
    // instruction on this chip) turns a value beyond it into an infinity, not the largest
    // finite fp16 that round-toward-zero would give, so the overflow shows in the results
    auto pk = [](float a, float b) -> unsigned { return cvt2_f16(a, b); };
    // bf16 inputs: the transposed words are packed in part (a), with the rows, and written
    // in part (b) (they take the prefetch registers' place in between)
    u32x2 tw[8];
    auto pack_t = [&](int n_s) {   // the transposed words alone (before a part (b) without (a))
        if constexpr (NSPLIT == 1 && BF16) {
            if (has_blk) {
                float f[4][8];
                stage_rows(f);
#pragma unroll
                for (int c = 0; c < 8; ++c) tw[c] = u32x2{pk(f[0][c], f[1][c]), pk(f[2][c], f[3][c])};
            }
        }
    };
    auto stage_a = [&](int n_s, int rb) {
        const int tb = opaque(tb0), cb = opaque(cb0);
        if constexpr (NSPLIT == 1 && BF16) {
            if (has_blk) {
                float f[4][8];
                stage_rows(f);
#pragma unroll
                for (int c = 0; c < 8; ++c) tw[c] = u32x2{pk(f[0][c], f[1][c]), pk(f[2][c], f[3][c])};
                if (!blk_v) {   // K rows (8 channels of one token = 16 contiguous bytes)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        *reinterpret_cast<u32x4*>(&sm.Kr[0][lds_off(tb * 4 + r, cb * 8, KP)]) =
                            u32x4{pk(f[r][0], f[r][1]), pk(f[r][2], f[r][3]), pk(f[r][4], f[r][5]), pk(f[r][6], f[r][7])};
                }
            }
        } else if (has_blk && !blk_v) {   // K rows (8 channels of one token = 16 contiguous bytes)
            float f[4][8];
            stage_rows(f);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int off = lds_off(tb * 4 + r, cb * 8, KP);
                if constexpr (NSPLIT == 1 && BF16) {
                    *reinterpret_cast<u32x4*>(&sm.Kr[0][off]) =
                        u32x4{pk(f[r][0], f[r][1]), pk(f[r][2], f[r][3]), pk(f[r][4], f[r][5]), pk(f[r][6], f[r][7])};
                } else {
                    uint16_t hb[8], lw[8];
#pragma unroll
                    for (int c = 0; c < 8; ++c) to16<NSPLIT>(f[r][c], hb[c], lw[c]);
                    *reinterpret_cast<u32x4*>(&sm.Kr[0][off]) = pack8(hb);
                    if constexpr (NSPLIT == 2) *reinterpret_cast<u32x4*>(&sm.Kr[1][off]) = pack8(lw);
                }
            }
        }
        if (wave == 7) {
            // betas, and the log-decays b_t = g_1 + .. + g_t of the chunk (inclusive scan over
            // the lanes, one token each) with the decay factors of the state update (v_exp_f32)
            const bool ok = lane < n_s;
            sm.beta[rb][lane] = ok ? raw1(braw) : 0.f;
            const float x = wave_inclusive_sum(ok ? raw1(graw) : 0.f);
            const float bc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
            const float b2 = x * kLog2e;
            sm.lb[rb][lane] = b2;
            sm.eb[rb][lane] = __builtin_amdgcn_exp2f(b2);
            sm.ebr[rb][lane] = __builtin_amdgcn_exp2f(bc * kLog2e - b2);
            if (lane == 0) sm.bC[rb] = bc;
        }
    };
    auto stage_b = [&](int n_s, int kbuf) {
        const int tb = opaque(tb0), cb = opaque(cb0);
        if (has_blk && !blk_zero) {   // transposed: one channel row, 4 consecutive tokens = 8 contiguous bytes
            uint16_t(*dst)[D * CH] = blk_v ? sm.Vt[kbuf] : sm.Kt[kbuf];
            float f[4][8];
            if constexpr (!(NSPLIT == 1 && BF16)) stage_rows(f);
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const int off = lds_off(cb * 8 + c, tb * 4, CH);
                if constexpr (NSPLIT == 1 && BF16) {
                    *reinterpret_cast<u32x2*>(&dst[0][off]) = tw[c];
                } else {
                    uint16_t hb[4], lw[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) to16<NSPLIT>(f[r][c], hb[r], lw[r]);
                    *reinterpret_cast<u32x2*>(&dst[0][off]) = u32x2{pack2(hb[0], hb[1]), pack2(hb[2], hb[3])};
                    if constexpr (NSPLIT == 2)
                        *reinterpret_cast<u32x2*>(&dst[1][off]) = u32x2{pack2(lw[0], lw[1]), pack2(lw[2], lw[3])};
                }
            }
        }
    };

    if (beg < end) {
        fetch_q(beg, 0);
        if (beg + CH < end) fetch_q(beg + CH, 1);
        prefetch(beg);
    }
    if (NW) {   // value channels past v_ld: zero rows of the V^T planes, never staged
        uint32_t* z = reinterpret_cast<uint32_t*>(&sm.Vt[0][0][0]);
        for (int i = tid; i < (int)(sizeof(sm.Vt) / 4); i += 512) z[i] = 0u;
    }
    if constexpr (OUT) {
        // the output products read M in 32-column blocks: of the tiles above the diagonal,
        // (0, 1) and (2, 3) fall inside one and stay zero (the others are never read)
        for (int i = tid; i < 512; i += 512) {
            const int ti = i < 256 ? 0 : 2, r = (i & 255) >> 4, c = i & 15;
            so.Mq[0][lds_off(16 * ti + r, 16 * (ti + 1) + c, CH)] = 0;
        }
        // the first chunk's q is in LDS before it is staged
        __builtin_amdgcn_s_waitcnt(0x0070);
        __syncthreads();
    }

    // lane-derived indices are recomputed in each phase (cheap) rather than kept live
    // across it.  Buffers of parity `par` hold the chunk's K^T, V^T, gates, betas and
    // decay factors.
    f32x4 U[4][CTW];   // the solved value block of this wave's S tiles (phase 3 -> phase 4)

    // 16 x 16 x 16 product with fp16 hi / lo operands (three products; lo x lo dropped)
    auto mma16 = [](const u32x2& ah, const u32x2& al, const u32x2& bh, const u32x2& bl, f32x4 c) {
        c = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, ah), __builtin_bit_cast(f16x4, bh), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, ah), __builtin_bit_cast(f16x4, bl), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, al), __builtin_bit_cast(f16x4, bh), c, 0, 0, 0);
        return c;
    };
    // a 16 x 16 block in the accumulator layout as fp16 hi / lo operand bits: the B operand of
    // v_mfma_f32_16x16x16_f16, or the A operand of the transposed block
    struct Hl16 {
        u32x2 h, l;
    };
    auto hl16 = [](const f32x4& x) {
        unsigned a, b, c, d;
        pack_f16_split(x, a, b, c, d);
        return Hl16{u32x2{a, b}, u32x2{c, d}};
    };
    auto mm16 = [&](const Hl16& a, const Hl16& b) { return mma16(a.h, a.l, b.h, b.l, zero4()); };

    // ---- 2. Gram blocks Lt = tril(b K K^T, -1) of the chunk at c0: the diagonal 16 x 16
    // blocks are inverted by waves 0..3, the off-diagonal blocks stored negated (fp16 hi / lo
    // operand planes, plain and decayed)
    auto phase_gram = [&](int64_t c0, int rb) {
        const int lane_c = opaque(lane);
        const int g4 = lane_c >> 4, n16 = lane_c & 15, lx = lane_c ^ g4;
        const float* const lb = sm.lb[rb];
        auto gram = [&](int ti, int tj) -> f32x4 {   // lane (g, n): G[16 ti + 4g + e][16 tj + n]
            f32x4 gacc = zero4();
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) {
                const Frag<NSPLIT> a = frag_of<NSPLIT, KP>(sm.Kr, ti, ks, lx);
                const Frag<NSPLIT> bb = frag_of<NSPLIT, KP>(sm.Kr, tj, ks, lx);   // K^T as B = rows of K
                gacc = mma<NSPLIT>(a, bb, gacc);
            }
            return gacc;
        };
        // M = scale (Q K^T o e^{b_t - b_s}), s <= t, as an fp16 operand plane, tile by tile:
        // tile idx = 0..9 is (ti, tj), tj <= ti, row-major over the lower triangle of 16 x 16
        // tiles (the tiles above it are zero or never read).
        auto mq_tile = [&](int idx) {
            if constexpr (OUT) {
                const int ti = idx < 1 ? 0 : idx < 3 ? 1 : idx < 6 ? 2 : 3;
                const int tj = idx - (ti * (ti + 1)) / 2;
                f32x4 m = zero4();
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks) {
                    const Frag<1> a = frag_of<1, KP>(so.Qr, ti, ks, lx);
                    const Frag<1> bb = frag_of<1, KP>(sm.Kr, tj, ks, lx);
                    m = mma<1>(a, bb, m);
                }
                const float bs = lb[16 * tj + n16];
                const f32x4 bt = *reinterpret_cast<const f32x4*>(&lb[16 * ti + 4 * g4]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 16 * ti + 4 * g4 + e;
                    const float x = (16 * tj + n16 <= t) ? ob.scale * m[e] * __builtin_amdgcn_exp2f(bt[e] - bs) : 0.f;
                    so.Mq[0][lds_off(t, 16 * tj + n16, CH)] = f16_bits((_Float16)x);
                }
            }
        };
        if (wave < 4) {
            // (I + Lt_ii)^-1 = (I - N)^-1 with N = -Lt_ii strictly lower (N^16 = 0):
            //   (I - N)^-1 = P1 (I + N^4)(I + N^8),   P1 = (I + N)(I + N^2) = I + N + N^2 + N^3
            // as 16 x 16 products on MFMA (hi / lo operands), formed transposed (Y^T = (I +
            // N^8)^T (I + N^4)^T P1^T) with each identity term as the product's fp32
            // accumulator input.  A product's A operand is the accumulator layout of the
            // transposed factor, so N and N^T are carried along; N^T comes from the same
            // Gram block (it is symmetric).
            const int i = wave;
            const f32x4 gacc = gram(i, i);
            const f32x4 bet = *reinterpret_cast<const f32x4*>(&sm.beta[rb][16 * i + 4 * g4]);
            const float bn = sm.beta[rb][16 * i + n16];
            f32x4 nd, nt;   // N[4g + e][n], N^T[4g + e][n]
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * g4 + e;
                nd[e] = n16 < r ? -bet[e] * gacc[e] : 0.f;
                nt[e] = r < n16 ? -bn * gacc[e] : 0.f;
            }
            const Hl16 n1 = hl16(nd), n1t = hl16(nt);
            const f32x4 n2 = mm16(n1t, n1), n2t = mm16(n1, n1t);                    // N^2, (N^2)^T
            const Hl16 q2 = hl16(n2), q2t = hl16(n2t);
            f32x4 c1;   // I + N^T + (N^2)^T
#pragma unroll
            for (int e = 0; e < 4; ++e) c1[e] = nt[e] + n2t[e] + ((4 * g4 + e == n16) ? 1.f : 0.f);
            const f32x4 n4 = mm16(q2t, q2), n4t = mm16(q2, q2t);                    // N^4, (N^4)^T
            const f32x4 p1t = mma16(q2.h, q2.l, n1t.h, n1t.l, c1);                  // P1^T = c1 + (N^2)^T N^T
            const Hl16 q4 = hl16(n4), q4t = hl16(n4t), r1t = hl16(p1t);
            const f32x4 n8 = mm16(q4t, q4);                                         // N^8
            const f32x4 p2t = mma16(q4.h, q4.l, r1t.h, r1t.l, p1t);                 // (P1 (I + N^4))^T
            const Hl16 q8 = hl16(n8), r2t = hl16(p2t);
            const f32x4 yt = mma16(q8.h, q8.l, r2t.h, r2t.l, p2t);                  // the inverse, transposed
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.Sd[i][n16][4 * g4 + e] = yt[e];   // row-major (fp32)
            // A fragment (lane (g, n): row n, columns 4g .. 4g+3) = accumulator layout of the
            // transpose; the decayed block has the factors e^{b_t - b_s}, t >= s
            const float bt = lb[16 * i + n16];
            const f32x4 bs = *reinterpret_cast<const f32x4*>(&lb[16 * i + 4 * g4]);
            f32x4 dd;
#pragma unroll
            for (int x = 0; x < 4; ++x) dd[x] = 4 * g4 + x <= n16 ? yt[x] * __builtin_amdgcn_exp2f(bt - bs[x]) : 0.f;
            const Hl16 dv = hl16(yt), dvd = hl16(dd);
            *reinterpret_cast<u32x2*>(&sm.Dv[0][i][lane * 4]) = dv.h;
            *reinterpret_cast<u32x2*>(&sm.Dv[1][i][lane * 4]) = dv.l;
            *reinterpret_cast<u32x2*>(&sm.Dvd[0][i][lane * 4]) = dvd.h;
            *reinterpret_cast<u32x2*>(&sm.Dvd[1][i][lane * 4]) = dvd.l;
        }
        // off-diagonal blocks k = (1,0) (2,0) (2,1) (3,0) (3,1) (3,2): waves 4..7 take k = 0..3,
        // waves 2, 3 k = 4, 5.  The transposed Gram block G_ji = K_j K_i^T has, in the
        // accumulator layout, the A-operand layout of Lt_ij (lane (g, n): row n, columns 4g..)
        {
            const int k = wave >= 4 ? wave - 4 : (wave >= 2 ? wave + 2 : -1);
            if (k >= 0) {
                const int ti = k < 1 ? 1 : k < 3 ? 2 : 3;
                const int tj = k - (ti * (ti - 1)) / 2;
                const f32x4 gacc = gram(tj, ti);
                const float bn = sm.beta[rb][16 * ti + n16];
                const float bt = lb[16 * ti + n16];
                const f32x4 bs = *reinterpret_cast<const f32x4*>(&lb[16 * tj + 4 * g4]);
                f32x4 l, ld;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    l[e] = -bn * gacc[e];
                    ld[e] = l[e] * __builtin_amdgcn_exp2f(bt - bs[e]);
                }
                const Hl16 lq = hl16(l), lqd = hl16(ld);
                *reinterpret_cast<u32x2*>(&sm.Ln[0][k][lane * 4]) = lq.h;
                *reinterpret_cast<u32x2*>(&sm.Ln[1][k][lane * 4]) = lq.l;
                *reinterpret_cast<u32x2*>(&sm.Lnd[0][k][lane * 4]) = lqd.h;
                *reinterpret_cast<u32x2*>(&sm.Lnd[1][k][lane * 4]) = lqd.l;
            }
        }
        if (wave >= 4) {
            if constexpr (OUT) {   // the masked Q K^T tiles: waves 4, 5: 0, 4 | 1, 5; waves 6, 7: 2, 6, 8 | 3, 7, 9
                mq_tile(wave - 4);
                mq_tile(wave);
                if (wave >= 6) mq_tile(wave + 2);
            }
        }
    };

    // ---- 3. forward substitution (Wt to LDS, U to registers); the chunks one after the other
    auto phase_solve = [&](int par) {
        const int lane_c = opaque(lane);
        const int g4 = lane_c >> 4, n16 = lane_c & 15, lx = lane_c ^ g4;
        // ---- 3. block forward substitution, one chain per owned column tile (no barriers):
        //   Wt_i = (I + Lt_ii)^-1 (diag(beta) K_i - sum_{j<i} Lt_ij Wt_j)       (H tiles: channel tile)
        //   U_i  = the same with the decayed blocks and diag(beta) V_i           (S tiles: value tile)
        // on v_mfma_f32_16x16x16_f16 with fp16 hi/lo operands (three products): its B operand
        // has the accumulator's lane layout, so a solved block feeds the next products as
        // packed, without cross-lane moves.  Wt goes to LDS for every wave's Y = Wt X; U stays
        // in this wave's registers for its S tile.
        {
            // the chains of this wave's tiles advance block by block together, so the
            // latency of one chain's step overlaps the other's
            u32x2 xh[3][CTW], xl[3][CTW];   // solved blocks 0..2 as packed B operands (hi / lo)
            f32x4 sol[4][CTW];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int c = 0; c < CTW; ++c) {
                    if (!own_tile(c)) continue;
                    const bool is_s = s_tile(c);
                    const int q = is_s ? tile(c) - RT : tile(c);   // channel / value tile
                    const uint16_t(*rhs_src)[D * CH] = is_s ? sm.Vt[par] : sm.Kt[par];
                    // right-hand side diag(beta) K_i (or V_i): lane (g, n) = rows 16i + 4g + e, column 16q + n
                    f32x4 acc;
                    {
                        const int off = lds_off(16 * q + n16, 16 * i + 4 * g4, CH);
                        const u32x2 hw = *reinterpret_cast<const u32x2*>(&rhs_src[0][off]);
                        f32x2 v0 = f16x2_to_f32(hw[0]), v1 = f16x2_to_f32(hw[1]);
                        if constexpr (NSPLIT == 2) {
                            const u32x2 lw = *reinterpret_cast<const u32x2*>(&rhs_src[1][off]);
                            v0 += f16x2_to_f32(lw[0]);
                            v1 += f16x2_to_f32(lw[1]);
                        }
                        const f32x4 bt = *reinterpret_cast<const f32x4*>(&sm.beta[par][16 * i + 4 * g4]);
                        acc = f32x4{bt[0] * v0.x, bt[1] * v0.y, bt[2] * v1.x, bt[3] * v1.y};
                    }
                    // - sum_{j<i} Lt_ij X_j
#pragma unroll
                    for (int j = 0; j < i; ++j) {
                        const int kb = i * (i - 1) / 2 + j;
                        const uint16_t(*L)[6][256] = is_s ? sm.Lnd : sm.Ln;
                        const u32x2 ah = *reinterpret_cast<const u32x2*>(&L[0][kb][lane * 4]);
                        const u32x2 al = *reinterpret_cast<const u32x2*>(&L[1][kb][lane * 4]);
                        acc = mma16(ah, al, xh[j][c], xl[j][c], acc);
                    }
                    // X_i = (I + Lt_ii)^-1 acc
                    const uint16_t(*Dm)[4][256] = is_s ? sm.Dvd : sm.Dv;
                    const u32x2 dh = *reinterpret_cast<const u32x2*>(&Dm[0][i][lane * 4]);
                    const u32x2 dl = *reinterpret_cast<const u32x2*>(&Dm[1][i][lane * 4]);
                    unsigned b0, b1, b2, b3;
                    pack_f16_split(acc, b0, b1, b2, b3);
                    sol[i][c] = mma16(dh, dl, u32x2{b0, b1}, u32x2{b2, b3}, zero4());
                    if (i < 3) {
                        pack_f16_split(sol[i][c], b0, b1, b2, b3);
                        xh[i][c] = u32x2{b0, b1};
                        xl[i][c] = u32x2{b2, b3};
                    }
                }
            }
#pragma unroll
            for (int c = 0; c < CTW; ++c) {
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) U[tt][c] = zero4();
                if (!own_tile(c)) continue;
                if (s_tile(c)) {
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) U[tt][c] = sol[tt][c];
                } else {   // -Wt rows 16i + 4g + e, channel 16q + n, token-major
                    const int q = tile(c);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int off = lds_off(16 * i + 4 * g4 + e, 16 * q + n16, KP);
                            uint16_t h, lo;
                            to16<NSPLIT>(-sol[i][c][e], h, lo);
                            sm.Wt[0][off] = h;
                            if constexpr (NSPLIT == 2) sm.Wt[1][off] = lo;
                        }
                }
            }
        }
    };

    // ---- 4. the state update of the chunk at c0 (n tokens; K^T in buffer kpar, decay
    // factors in ring slot rs)
    // The erase alone contracts H (token by token in the direction of k_t), so over long
    // segments with weak decay its entries fall towards fp16's subnormal range, where they
    // lose precision and then flush to zero as MFMA operands.  After every update each wave
    // posts the largest |H| of its tiles; before the next update, once the largest over the
    // workgroup is below 1/4, H is scaled by the power of two that brings it into [1/2, 1)
    // (exact) and the exponent is kept in h2.
    auto h_renorm = [&](int slot) {
        if constexpr (WANT_T) {
            float mm = 0.f;
#pragma unroll
            for (int w = 0; w < 8; ++w) mm = fmaxf(mm, sm.hmax[slot][w]);
            if (mm > 0.f && mm < 0.25f) {
                int em;
                frexpf(mm, &em);
                const float sc = ldexpf(1.f, -em);
#pragma unroll
                for (int c = 0; c < CTW; ++c)
                    if (own_tile(c) && !s_tile(c))
#pragma unroll
                        for (int rt = 0; rt < RT; ++rt) X[rt][c] *= sc;
                h2 += em;
            }
        }
    };
    auto h_post = [&](int slot) {
        if constexpr (WANT_T) {
            float m = 0.f;
#pragma unroll
            for (int c = 0; c < CTW; ++c)
                if (own_tile(c) && !s_tile(c))
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                        for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(X[rt][c][e]));
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
            if (lane == 0) sm.hmax[slot][wave] = m;
        }
    };

    auto phase_update = [&](int64_t c0, int n, int kpar, int rs, int slot) {
        // slot: parity of the chunk's index in the segment (renormalisation records)
        if (c0 != beg) h_renorm(slot ^ 1);
        // pipelined, the fragment reads' lane offsets (lx ^ K, eight values) stay live
        // across the loop; with outputs (no registers to spare) they are recomputed
        int lane_c = lane;
        if constexpr (!PIPE) lane_c = opaque(lane);
        const int g4 = lane_c >> 4, n16 = lane_c & 15, lx = lane_c ^ g4;
        // ---- 6..8. Y = Wt X, R, X += K^T R for all owned column tiles at once (each A
        // fragment is read once per wave)
        const float bC = sm.bC[rs];
        const float ebC = __builtin_amdgcn_exp2f(bC * kLog2e);
        if (wave < NCT) {
            f32x4 R[4][CTW];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                for (int c = 0; c < CTW; ++c) R[tt][c] = zero4();
            f32x4 P[OUT ? 4 : 1];   // Q S_0 for this wave's S tile (OUT)
#pragma unroll
            for (int tt = 0; tt < (OUT ? 4 : 1); ++tt) P[tt] = zero4();
#pragma unroll
            for (int kb = 0; kb < KSD; ++kb) {
                Frag<NSPLIT> xb[CTW];   // rows 32 kb .. 32 kb + 31 of the X column tiles as B fragments
#pragma unroll
                for (int c = 0; c < CTW; ++c) {
                    if (!upd_tile(c)) continue;
                    const f32x4 d0 = X[2 * kb][c];
                    const f32x4 d1 = (2 * kb + 1 < RT) ? X[2 * kb + 1 < RT ? 2 * kb + 1 : 0][c] : zero4();
                    xb[c] = dpair_to_frag<NSPLIT>(d0, d1);
                }
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    const Frag<NSPLIT> a = frag_of<NSPLIT, KP>(sm.Wt, tt, kb, lx);
#pragma unroll
                    for (int c = 0; c < CTW; ++c)
                        if (upd_tile(c)) R[tt][c] = mma<NSPLIT>(a, xb[c], R[tt][c]);
                }
                if constexpr (OUT) {
#pragma unroll
                    for (int c = 0; c < CTW; ++c) {
                        if (!own_tile(c) || !s_tile(c)) continue;
#pragma unroll
                        for (int tt = 0; tt < 4; ++tt)
                            P[tt] = mma<1>(frag_of<1, KP>(so.Qr, tt, kb, lx), xb[c], P[tt]);
                    }
                }
            }
            Frag<NSPLIT> rb[2][CTW];
#pragma unroll
            for (int c = 0; c < CTW; ++c) {
                if (!upd_tile(c)) continue;
                const bool is_s = s_tile(c);
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int t = tt * 16 + 4 * g4 + e;
                        // the plane holds -Wt, so R = -Wt X already for the H tiles
                        if (is_s) {   // new values U' = U - diag(e^b) Wt S_0; R = diag(e^{b_C - b}) U'
                            const float up = U[tt][c][e] + sm.eb[rs][t] * R[tt][c][e];
                            U[tt][c][e] = up;
                            R[tt][c][e] = sm.ebr[rs][t] * up;
                        }
                    }
                rb[0][c] = dpair_to_frag<NSPLIT>(R[0][c], R[1][c]);
                rb[1][c] = dpair_to_frag<NSPLIT>(R[2][c], R[3][c]);
                if constexpr (OUT) {
                    if (is_s) {   // o_t = scale e^{b_t} (Q S_0)_t + (M U')_t for the tile's 16 value columns
                        const Frag<1> ub0 = dpair_to_frag<1>(U[0][c], U[1][c]);
                        const Frag<1> ub1 = dpair_to_frag<1>(U[2][c], U[3][c]);
                        const int vq = tile(c) - RT;
#pragma unroll
                        for (int tt = 0; tt < 4; ++tt) {
                            f32x4 o;
                            const f32x4 ebt = *reinterpret_cast<const f32x4*>(&sm.eb[rs][tt * 16 + 4 * g4]);
#pragma unroll
                            for (int e = 0; e < 4; ++e) o[e] = ob.scale * ebt[e] * P[tt][e];
                            o = mma<1>(frag_of<1, CH>(so.Mq, tt, 0, lx), ub0, o);
                            if (tt >= 2) o = mma<1>(frag_of<1, CH>(so.Mq, tt, 1, lx), ub1, o);
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const int t = tt * 16 + 4 * g4 + e;
                                if (t < n && (!NW || vq * 16 + n16 < v_cols))
                                    ob.out[((size_t)(c0 + t) * H + h) * v_ld + vq * 16 + n16] = o[e];
                            }
                        }
                    }
                }
                if (is_s) {
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) X[rt][c] *= ebC;
                }
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int kbk = 0; kbk < 2; ++kbk) {
                    const Frag<NSPLIT> a = frag_of<NSPLIT, CH>(sm.Kt[kpar], rt, kbk, lx);
#pragma unroll
                    for (int c = 0; c < CTW; ++c)
                        if (upd_tile(c)) X[rt][c] = mma<NSPLIT>(a, rb[kbk][c], X[rt][c]);
                }
        }
        log_s += bC;
        h_post(slot);
    };

    // ---- 3a. the inverse blocks Ab_ij (i >= j) of the chunk whose Gram blocks are in LDS
    // (betas in ring slot rb), block column j = wave / 2 of the plain (even waves) or decayed
    // (odd waves) inverse:
    //   Ab_jj = (I + Lt_jj)^-1 diag(b_j),   Ab_ij = (I + Lt_ii)^-1 sum_{j <= k < i} (-Lt_ik) Ab_kj
    // on v_mfma_f32_16x16x16_f16 with hi / lo operands, whose B operand has the accumulator's
    // lane layout; each block goes to the inverse planes as soon as it is known
    auto phase_ainv = [&](int rb) {
        if constexpr (PIPE) {
            const int lane_c = opaque(lane);
            const int g4 = lane_c >> 4, n16 = lane_c & 15;
            const int v = wave & 1;
            const uint16_t(*const Lm)[6][256] = v ? sm.Lnd : sm.Ln;
            const uint16_t(*const Dm)[4][256] = v ? sm.Dvd : sm.Dv;
            auto chain = [&](auto jc) {
                constexpr int j = decltype(jc)::value;
                auto put_block = [&](int i, const Hl16& z) {   // D layout (hi / lo pairs) -> A fragment entries
                    // row 4g + e of the block: A lane 4g + e + 16 (col / 8), entry col % 8
                    const int f = ab_frag(i, j >> 1), col = 16 * (j & 1) + n16;
                    const int idx = (4 * g4 + 16 * (col >> 3)) * 8 + (col & 7);
                    uint16_t* const ph = &si.Ab[v][0][f][idx];
                    uint16_t* const pl = &si.Ab[v][1][f][idx];
                    ph[0] = (uint16_t)z.h[0];
                    ph[8] = (uint16_t)(z.h[0] >> 16);
                    ph[16] = (uint16_t)z.h[1];
                    ph[24] = (uint16_t)(z.h[1] >> 16);
                    pl[0] = (uint16_t)z.l[0];
                    pl[8] = (uint16_t)(z.l[0] >> 16);
                    pl[16] = (uint16_t)z.l[1];
                    pl[24] = (uint16_t)(z.l[1] >> 16);
                };
                // Ab_jj from the fp32 diagonal inverse (decayed: times e^{b_t - b_s}, t >= s)
                f32x4 z;
                {
                    const float* const lbr = sm.lb[rb];
                    const float bs = lbr[16 * j + n16], bet = sm.beta[rb][16 * j + n16];
                    const f32x4 bt = *reinterpret_cast<const f32x4*>(&lbr[16 * j + 4 * g4]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * g4 + e;
                        float d = sm.Sd[j][r][n16];
                        if (v) d = n16 <= r ? d * __builtin_amdgcn_exp2f(bt[e] - bs) : 0.f;
                        z[e] = d * bet;
                    }
                }
                Hl16 zs[4];   // Ab_kj (k = j .. 3) as hi / lo pairs: the B operands of the chain
                zs[j] = hl16(z);
                put_block(j, zs[j]);
                // right-looking: as soon as Ab_kj is known, its terms of every later block go
                // out together (independent products), then the next block is finished; each
                // block's terms still accumulate in the order k = j, j + 1, ..
                f32x4 acc[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = zero4();
#pragma unroll
                for (int k = j; k < 3; ++k) {
#pragma unroll
                    for (int i = k + 1; i < 4; ++i) {
                        const int kb = i * (i - 1) / 2 + k;
                        const u32x2 ah = *reinterpret_cast<const u32x2*>(&Lm[0][kb][lane * 4]);
                        const u32x2 al = *reinterpret_cast<const u32x2*>(&Lm[1][kb][lane * 4]);
                        acc[i] = mma16(ah, al, zs[k].h, zs[k].l, acc[i]);
                    }
                    const int i = k + 1;
                    unsigned b0, b1, b2, b3;
                    pack_f16_split(acc[i], b0, b1, b2, b3);
                    const u32x2 dh = *reinterpret_cast<const u32x2*>(&Dm[0][i][lane * 4]);
                    const u32x2 dl = *reinterpret_cast<const u32x2*>(&Dm[1][i][lane * 4]);
                    zs[i] = hl16(mma16(dh, dl, u32x2{b0, b1}, u32x2{b2, b3}, zero4()));
                    put_block(i, zs[i]);
                }
            };
            switch (wave >> 1) {
                case 0: chain(IntC<0>{}); break;
                case 1: chain(IntC<1>{}); break;
                case 2: chain(IntC<2>{}); break;
                default: chain(IntC<3>{}); break;
            }
        }
    };

    // ---- 3b. Wt = Ab K and U = (D Ab D^-1) V for this wave's column tiles, as dense products
    // over the lower triangle (K, V exact in fp16 for bf16 inputs: two products per step);
    // K^T, V^T in buffer kpar.  Wt goes to LDS, U stays in registers.
    auto phase_dsolve = [&](int kpar) {
        if constexpr (PIPE) {
            const int lane_c = opaque(lane);
            const int g4 = lane_c >> 4, n16 = lane_c & 15, lx = lane_c ^ g4;
#pragma unroll
            for (int c = 0; c < CTW; ++c) {
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) U[tt][c] = zero4();
                if (!own_tile(c)) continue;
                const bool is_s = s_tile(c);
                const int q = is_s ? tile(c) - RT : tile(c);   // value / channel tile
                const int v = is_s ? 1 : 0;
                const uint16_t(*src)[D * CH] = is_s ? sm.Vt[kpar] : sm.Kt[kpar];
                const Frag<NSPLIT> kf[2] = {frag_of<NSPLIT, CH>(src, q, 0, lx), frag_of<NSPLIT, CH>(src, q, 1, lx)};
                // the six fragment pairs are read together, then the products go out in an
                // order where consecutive ones feed different accumulators
                f16x8 ah[6], al[6];
#pragma unroll
                for (int f = 0; f < 6; ++f) {
                    ah[f] = *reinterpret_cast<const f16x8*>(&si.Ab[v][0][f][lane * 8]);
                    al[f] = *reinterpret_cast<const f16x8*>(&si.Ab[v][1][f][lane * 8]);
                }
                f32x4 acc[4];
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) acc[tt] = zero4();
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                    for (int tt = 2 * ks; tt < 4; ++tt) acc[tt] = mma_f16(ah[ab_frag(tt, ks)], kf[ks].h, acc[tt]);
#pragma unroll
                    for (int tt = 2 * ks; tt < 4; ++tt) acc[tt] = mma_f16(al[ab_frag(tt, ks)], kf[ks].h, acc[tt]);
                    if constexpr (NSPLIT == 2) {
#pragma unroll
                        for (int tt = 2 * ks; tt < 4; ++tt) acc[tt] = mma_f16(ah[ab_frag(tt, ks)], kf[ks].l, acc[tt]);
                    }
                }
                if (is_s) {
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) U[tt][c] = acc[tt];
                } else {   // -Wt rows 16 tt + 4 g + e, channel 16 q + n, token-major
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int off = lds_off(16 * tt + 4 * g4 + e, 16 * q + n16, KP);
                            uint16_t h, lo;
                            to16<NSPLIT>(-acc[tt][e], h, lo);
                            sm.Wt[0][off] = h;
                            if constexpr (NSPLIT == 2) sm.Wt[1][off] = lo;
                        }
                }
            }
        }
    };

    auto chunk_len = [&](int64_t c0) -> int { return (int)((end - c0) < CH ? (end - c0) : CH); };
    if constexpr (PIPE) {
        // Chunk i's state update needs its Wt and U; nothing else in a chunk depends on the
        // state.  So the chunks are pipelined, two steps per chunk, one barrier after each:
        //   1: update(i), inverse(i + 1), stage K rows, betas, log-decays of i + 2
        //   2: dense solve(i + 1), Gram blocks(i + 2), stage K^T, V^T of i + 2
        // The state-independent parts fill the SIMD time that the state update leaves.
        // K^T and V^T are double-buffered (chunk parity), the per-token scalars kept for three
        // chunks (index modulo 3); Kr, Wt, the Gram blocks and the inverse planes are single.
        const int nch = (int)((end - beg + CH - 1) / CH);
        if (nch > 0) {   // prologue: chunk 0 up to its dense solve, chunk 1 up to its Gram blocks
            stage_a(chunk_len(beg), 0);
            stage_b(chunk_len(beg), 0);
            if (nch > 1) prefetch(beg + CH);
            __syncthreads();
            phase_gram(beg, 0);
            if (nch > 1) {
                pack_t(chunk_len(beg + CH));
                stage_b(chunk_len(beg + CH), 1);
            }
            __syncthreads();
            phase_ainv(0);
            if (nch > 1) {
                stage_a(chunk_len(beg + CH), 1);
                if (nch > 2) prefetch(beg + 2 * CH);
            }
            __syncthreads();
            phase_dsolve(0);
            if (nch > 1) phase_gram(beg + CH, 1);
            __syncthreads();
        }
        for (int ci = 0; ci < nch; ++ci) {
            const int64_t c0 = beg + (int64_t)ci * CH;
            phase_update(c0, chunk_len(c0), ci & 1, ci % 3, ci & 1);
            if (ci + 1 < nch) phase_ainv((ci + 1) % 3);
            if (ci + 2 < nch) stage_a(chunk_len(c0 + 2 * CH), (ci + 2) % 3);
            __syncthreads();
            if (ci + 1 < nch) {
                phase_dsolve((ci + 1) & 1);
                if (ci + 2 < nch) {
                    phase_gram(c0 + 2 * CH, (ci + 2) % 3);
                    stage_b(chunk_len(c0 + 2 * CH), ci & 1);
                    if (ci + 3 < nch) prefetch(c0 + 3 * CH);
                }
                __syncthreads();
            }
        }
    } else {
        for (int64_t c0 = beg; c0 < end; c0 += CH) {
            const int n = chunk_len(c0);
            const int tb = opaque(tb0), cb = opaque(cb0);
            const int qbuf = (int)(((c0 - beg) / CH) & 1);
            if constexpr (OUT) {
                if (has_blk && blk_v) {   // q block (tb, cb) to the fp16 plane Qr; rows past the segment zeroed
                    auto pk = [](float a, float b) -> unsigned { return cvt2_f16(a, b); };
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int t = tb * 4 + r;
                        u32x4 w = *reinterpret_cast<const u32x4*>(&so.Qraw[qbuf][t * D + cb * 8]);
                        if (t >= n) w = u32x4{0u, 0u, 0u, 0u};
                        u32x4 o;
#pragma unroll
                        for (int x = 0; x < 4; ++x)
                            o[x] = pk(__uint_as_float(w[x] << 16), __uint_as_float(w[x] & 0xFFFF0000u));
                        *reinterpret_cast<u32x4*>(&so.Qr[0][lds_off(t, cb * 8, KP)]) = o;
                    }
                }
            }
            stage_a(n, 0);
            stage_b(n, 0);
            // the next chunk's loads fly during this chunk
            if (c0 + CH < end) prefetch(c0 + CH);
            __syncthreads();
            phase_gram(c0, 0);
            __syncthreads();
            phase_solve(0);
            // q goes two chunks ahead: wait for everything in flight -- the next chunk's q (sent
            // at this point of the previous chunk), its k, v, g, beta (sent at the end of staging)
            // and the previous chunk's output stores -- then send q of the chunk after next into
            // the buffer this chunk's q was converted from
            if constexpr (OUT) {
                __builtin_amdgcn_s_waitcnt(0x0070);
                if (c0 + 2 * CH < end) fetch_q(c0 + 2 * CH, qbuf);
            }
            __syncthreads();
            phase_update(c0, n, 0, 0, qbuf);
            __syncthreads();
        }
    }

    // ---- emit T_C = e^{log_s} 2^{h2} H and S(C|0)
    const float tscale = ldexpf(expf(log_s), h2);
    const size_t pair = (size_t)out * H + h;
#pragma unroll
    for (int c = 0; c < CTW; ++c) {
        const int ct = tile(c);
        if (ct >= NCT) continue;
        const bool is_s = ct >= RT;
        if (!is_s && T_out == nullptr) continue;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = rt * 16 + 4 * g4 + e;
                if (is_s) {
                    if (!NW || (ct - RT) * 16 + n16 < s_cols)
                        S_out[pair * D * s_ld + (size_t)row * s_ld + (ct - RT) * 16 + n16] = X[rt][c][e];
                }
                else put_t(T_out, t_split, pair, D, row, ct * 16 + n16, tscale * X[rt][c][e]);
            }
    }

}

template <int D, int NSPLIT, bool BF16, bool OUT, bool NW>
static hipError_t launch_gdn_nw(int n_seg, int H, const int64_t* sb, const int64_t* se, int64_t n_tok,
                                const void* k, const void* v, const void* g, const void* beta,
                                void* T_out, bool t_split, float* S_out, int v_ld, const BuildItems& items,
                                const BuildOut& ob, hipStream_t st)
{
    // pieces of cut segments always produce T (the fold needs it)
    if (T_out != nullptr || items.out != nullptr)
        hipLaunchKernelGGL((build_gdn_kernel<D, NSPLIT, BF16, true, OUT, NW>), dim3(n_seg * H), dim3(512), 0, st,
                           n_seg, H, sb, se, n_tok, k, v, g, beta, T_out, (int)t_split, S_out, v_ld, items, ob);
    else
        hipLaunchKernelGGL((build_gdn_kernel<D, NSPLIT, BF16, false, OUT, NW>), dim3(n_seg * H), dim3(512), 0, st,
                           n_seg, H, sb, se, n_tok, k, v, g, beta, T_out, (int)t_split, S_out, v_ld, items, ob);
    return hipGetLastError();
}

template <int D, int NSPLIT, bool BF16, bool OUT>
static hipError_t launch_gdn(int n_seg, int H, const int64_t* sb, const int64_t* se, int64_t n_tok,
                             const void* k, const void* v, const void* g, const void* beta,
                             void* T_out, bool t_split, float* S_out, int v_ld, const BuildItems& items,
                             const BuildOut& ob, hipStream_t st)
{
    return v_ld < D ? launch_gdn_nw<D, NSPLIT, BF16, OUT, true>(n_seg, H, sb, se, n_tok, k, v, g, beta, T_out,
                                                              t_split, S_out, v_ld, items, ob, st)
                    : launch_gdn_nw<D, NSPLIT, BF16, OUT, false>(n_seg, H, sb, se, n_tok, k, v, g, beta, T_out,
                                                               t_split, S_out, v_ld, items, ob, st);
}

hipError_t build_gdn(int d, bool in_bf16, int n_seg, int H, const int64_t* sb, const int64_t* se,
                     int64_t n_tok, const void* k, const void* v, const void* g, const void* beta,
                     void* T_out, bool t_split, float* S_out, const BuildItems& items, const BuildOut& ob,
                     hipStream_t st, int v_ld)
{
    const bool out = ob.out != nullptr;
    if (v_ld == 0) v_ld = d;
#define HYPIC_GDN(D_, NS_, BF_, OUT_)                                                                     \
    if (d == D_ && in_bf16 == BF_ && out == OUT_)                                                         \
        return launch_gdn<D_, NS_, BF_, OUT_>(n_seg, H, sb, se, n_tok, k, v, g, beta, T_out, t_split, S_out, \
                                              v_ld, items, ob, st);
    HYPIC_GDN(128, 1, true, false)
    HYPIC_GDN(128, 1, true, true)
    HYPIC_GDN(64, 1, true, false)
    HYPIC_GDN(64, 1, true, true)
    HYPIC_GDN(16, 2, false, false)
    HYPIC_GDN(16, 1, true, false)
    HYPIC_GDN(32, 1, true, false)
    HYPIC_GDN(32, 2, false, false)
    HYPIC_GDN(64, 2, false, false)
#undef HYPIC_GDN
    return hipErrorNotSupported;
}

}  // namespace hypic
