// build_kda.hip -- segment build (T_C, S(C|0)) for the per-channel (diagonal)
// gate with the delta rule, in either order of gate and erase:
//     M_t = diag(a_t) (I - b_t k_t k_t^T)   (gate after the erase), or
//     M_t = (I - b_t k_t k_t^T) diag(a_t)   (gate before the erase, GF),
//     S_t = M_t S_{t-1} + b_t k_t v_t^T,
// a_t = e^{g_t} per key channel.  The cached pair is T_C = M_L..M_1 and S(C|0)
// ([ZH] = the Chinese HYPIC page, section 2.1, which names KDA among the
// families the transition operator covers without fixing the order).
//
// Chunked form (C = 32; derivation in the design notes).  In the coordinates
// Z_t = Gamma_t^-1 S_t (Gamma_t = diag of the inclusive cumulative gate) a token
// is Z <- Z - b e_t (f_t^T Z) + b w_t v_t^T with write vector w_t = Gamma_t^-1 k_t
// and erase vectors e_t = G^-1 k_t, f_t = G k_t, where G = Gamma_{t-1} when the
// gate follows the erase and G = Gamma_t when it comes first.  Per key channel
// let i_t be the inclusive in-chunk cumulative log-gate (the write vector's) and
// c_t the erase vectors' one: the exclusive sum (c_0 = 0) for the first order,
// c_t = i_t for GF; b_C is the chunk total.  With
//     Lp[t][s] = b_t sum_c k_t k_s e^{c_t - c_s},  L'[t][s] = sum_c k_t k_s e^{c_t - i_s}  (s < t)
//     A = (I + Lp)^-1,  W = A diag(b) (e^{c} o K),  U = A diag(b) L' diag(b) V
//     Kh = e^{b_C - c} o K,  Kh' = e^{b_C - i} o K
// the augmented state X = [T | S] advances as
//     X <- diag(e^{b_C}) X - Kh^T (W X) + [0 | Kh'^T diag(b) V - Kh^T U].
// Every exponential has a non-positive exponent except inside the decay-weighted
// Gram matrices, which are factored per 16-token row block I around
// rho_I = c_{16 I}: left e^{c_t - rho_I} <= 1 and right e^{rho_I - c_s}, which is
// <= 1 off the diagonal block and bounded by one 16-token block's decay on it.
// Those two Gram matrices, W (while T is live) and every product of the T columns use
// bf16 hi + lo operands (three products on v_mfma_f32_16x16x32_bf16, fp32 range): with
// strong per-channel decay the decayed rows of W and Kh leave fp16's range while T is
// still far above the floor.  The S columns use fp16 operands with fp32
// accumulation on v_mfma_f32_16x16x32_f16 (their small entries are negligible
// next to the fresh writes).  The T columns are renormalised by a power of two
// each chunk (a per-channel decay cannot be factored out as one scalar), and
// once every T entry is below 2^-120 they are dropped: T_C = 0 is then within
// the comparison floor and stays so, since the transitions do not expand
// (log-gates <= 0, 0 <= b ||k||^2 <= 2).
//
// One workgroup (8 waves) per (segment, head); X in MFMA accumulators, two
// 16-column tiles per wave (one of T, one of S at d = 128).  bf16 inputs.
#include "hypic_device.h"
#include "hypic_kernels.h"
#include "build_common.h"

namespace hypic {

namespace {

template <int V>
struct IntConst {
    static constexpr int value = V;
};
using namespace bld;

constexpr float kLog2e = 1.4426950408889634f;
// 2^x on the transcendental unit (v_exp_f32): log-gates are carried in log2 units, so each
// decay factor is one instruction
__device__ __forceinline__ float exp2_raw(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr int CK = 32;        // chunk length
constexpr int LDT = CK + 8;   // token-indexed 16-bit rows
constexpr int LDF = CK + 4;   // fp32 32x32 matrices (16-byte aligned rows)

template <int D>
struct alignas(16) KdaSmem {
    uint16_t Kb[CK][D];            // K (bf16 bits), token-major, loaded global -> LDS directly
    float Ag[CK + 1][D + 4];       // exclusive cumulative log2-gate per channel; row t+1 inclusive, row CK = b_C
    float beta[2][CK];             // beta per token, by chunk parity
    float eBC[D];                  // e^{b_C} per channel (the chunk's decay of the state rows)
    float F1[CK][LDF];             // Lp (strictly lower, beta folded); its diagonal blocks then inverted in place
    float F1p[CK][LDF];            // L'
    union {
        uint16_t RmT[2][D][LDT];   // (e^{a} o K)^T, bf16 hi / lo
        struct {                   // the next chunk's v and log-gates (bf16 bits), loaded global -> LDS
            uint16_t Vr[CK * D];   // directly, 8 channels of one token per staging item, item-major
            uint16_t Gr[CK * D];
        } nx;
    } rv;
    union {
        uint16_t KhTb[2][D][LDT];  // Kh^T, bf16 hi / lo (T columns)
        struct {                   // once T is dropped: the next chunk's v and log-gates, loaded
            uint16_t Vr[CK * D];   // during the Gram phase (item-major, as below)
            uint16_t Gr[CK * D];
        } nx;
    } kt;
    uint16_t KhT[D][LDT];          // Kh^T
    uint16_t KhpT[D][LDT];         // Kh'^T
    uint16_t bVT[D][LDT];          // (diag(b) V)^T
    union {
        struct {                       // phases 3-5
            uint16_t ApB[2][CK][LDT];      // A diag(b), bf16 hi / lo
            uint16_t WpB[2][CK][D + 8];    // W, token-major, bf16 hi / lo (T columns)
            uint16_t Ap[CK][LDT];          // A diag(b)
            uint16_t Lpb[CK][LDT];         // L' (fp16)
            uint16_t Z1T[D][LDT];          // (L' diag(b) V)^T
            uint16_t Wp[CK][D + 8];        // W, token-major (S columns)
        } p;
        struct {                       // phase 2: operands of the decay-weighted Gram products
            uint16_t GL[2][CK][D + 8];     // k_t e^{c_t - rho}, bf16 hi / lo, token-major
            uint16_t GR[2][CK][D + 8];     // k_s e^{rho - c_s}            (Lp)
            uint16_t GR1[2][CK][D + 8];    // k_s e^{rho - i_s}            (L'; the gate-first order reuses GR)
        } g;
    } u;
    float red2[2][8];              // per wave: max |T| after a chunk's update (by chunk parity)
    float bmx[2][4];               // per staging wave: the largest chunk log2-decay b_C it staged (by chunk parity)
};

__device__ __forceinline__ float bf(uint16_t b) { return bf16_bits_to_f32(b); }

// inv16_t (the transposed (I - N)^-1 by the four-factor product) with single fp16 operands:
// one product per factor instead of three
__device__ __forceinline__ f32x4 inv16_t1(const f32x4& nd, const f32x4& nt, int g4, int n16) {
    auto h = [](const f32x4& x) { return __builtin_bit_cast(f16x4, u32x2{cvt2_f16(x[0], x[1]), cvt2_f16(x[2], x[3])}); };
    auto mm = [](f16x4 a, f16x4 b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0); };
    const f16x4 n1 = h(nd), n1t = h(nt);
    const f32x4 n2 = mm(n1t, n1, zero4()), n2t = mm(n1, n1t, zero4());     // N^2, (N^2)^T
    const f16x4 q2 = h(n2), q2t = h(n2t);
    f32x4 c1;   // I + N^T + (N^2)^T
#pragma unroll
    for (int e = 0; e < 4; ++e) c1[e] = nt[e] + n2t[e] + ((4 * g4 + e == opaque(n16)) ? 1.f : 0.f);   // (formed here, not kept)
    const f32x4 n4 = mm(q2t, q2, zero4()), n4t = mm(q2, q2t, zero4());     // N^4, (N^4)^T
    const f32x4 p1t = mm(q2, n1t, c1);                                      // P1^T = c1 + (N^2)^T N^T
    const f16x4 q4 = h(n4), q4t = h(n4t), r1t = h(p1t);
    const f32x4 n8 = mm(q4t, q4, zero4());                                  // N^8
    const f32x4 p2t = mm(q4, r1t, p1t);                                     // (P1 (I + N^4))^T
    return mm(h(n8), h(p2t), p2t);
}

// The channel-major key planes ((e^{a} o K)^T, Kh^T, Kh'^T; [D][LDT] 16-bit) hold row r's
// 16-byte token chunk q at chunk q ^ ((r >> 3) & 3): the operand pass stores 4 tokens of a
// channel pair per lane with rows two apart across the lanes, which without the swizzle fall on
// 8 of the 32 banks (4-way conflicts; 2-way with it, by a bank model), while the 16-byte
// fragment reads of 16 consecutive rows stay conflict-free.
__device__ __forceinline__ int kswz(int row, int t) { return (((t >> 3) ^ ((row >> 3) & 3)) << 3) | (t & 7); }

// fp16 operand fragment: 8 consecutive values at (row, col) of a row-major LDS matrix.
__device__ __forceinline__ Frag<1> f16frag(const uint16_t* base, int ld, int row, int col) {
    Frag<1> f;
    f.h = *reinterpret_cast<const f16x8*>(base + row * ld + col);
    return f;
}

}  // namespace

template <int D, bool GF, bool NW, bool NK>
__global__ __launch_bounds__(512) void build_kda_kernel(
    int n_seg, int H, const int64_t* __restrict__ seg_begin, const int64_t* __restrict__ seg_end,
    int64_t n_tokens, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ gl, const uint16_t* __restrict__ beta, void* __restrict__ T_out,
    int t_split, float* __restrict__ S_out, int v_ld, int k_d)
{
    // v_ld: the row length of v ([n_tokens][H][v_ld]) and of S_out ([pair][D][v_ld]); v and
    // S_out point at this call's D columns (D columns of a wider state, built one block at a
    // time: the columns of S evolve independently).  With v_ld < D (NW, narrow values) the
    // values have only v_ld columns: the rest are read as zeros and those columns of S are not
    // written.
    const int v_cols = NW ? v_ld : D;
    // k_d: with NK (narrow keys, d_k = k_d < D) the keys and log-gates have k_d channels; the
    // kernel runs at D with the other channels read as zeros (key 0, log-gate 0: they take no
    // part, and the rows and columns of T past k_d stay those of the identity), and T and S
    // are written for their first k_d rows (T also for its first k_d columns) only
    const int k_ld = NK ? k_d : D;
    using SM = KdaSmem<D>;
    constexpr int RT = D / 16;
    constexpr int NCT = 2 * RT;
    constexpr int CTW = (NCT + 7) / 8;
    constexpr int KSD = D / 32;
    static_assert(D % 32 == 0, "d must be a multiple of 32");
    constexpr int E1 = GF ? 1 : 0;   // row of Ag holding the erase vectors' cumulative gate of token 0
    __shared__ SM sm;

    const int unit = blockIdx.x;
    const int seg = unit / H, h = unit % H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g4 = lane >> 4, n16 = lane & 15;
    int64_t beg = seg_begin[seg], end = seg_end[seg];
    beg = beg < 0 ? 0 : (beg > n_tokens ? n_tokens : beg);
    end = end < beg ? beg : (end > n_tokens ? n_tokens : end);

    // Column tiles of X = [T | S]: waves 0-3 own CTW S tiles each, waves 4-7 CTW T tiles each,
    // so every A fragment of the update feeds CTW products, and each SIMD (waves w and w + 4)
    // holds one wave of each kind.
    static_assert(NCT == 8 * CTW, "the column tiles split evenly over the eight waves");
    const bool s_wave = wave < 4;
    const int tile0 = (s_wave ? RT : 0) + (wave & 3) * CTW;   // first owned column tile
    f32x4 X[RT][CTW];
#pragma unroll
    for (int c = 0; c < CTW; ++c) {
        const int ct = tile0 + c;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            X[rt][c] = zero4();
            if (!s_wave) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    X[rt][c][e] = (rt * 16 + 4 * g4 + e == ct * 16 + n16) ? 1.f : 0.f;
            }
        }
    }
    int log2s = 0;       // T = 2^log2s * X_T
    bool t_live = true;  // false once every T entry is below 2^-120

    const size_t tok_stride = (size_t)H * k_ld;
    // A chunk's k, log-gates and v are loaded global -> LDS directly, one chunk ahead, in 1-KiB
    // pieces (16 bytes per lane): K token-major into Kb; v and the log-gates item-major, staging
    // item i (channel group i / CK, token i % CK) in piece i / 64, so a thread that stages an
    // item its own wave loaded needs no barrier first.  Rows past the segment are read clamped
    // to its last token (finite values) and masked where they are consumed: their log-gates
    // count as zero and their betas are zero, which takes them out of every product.
    //   - While T is live the S waves (52 products per chunk in the update against the T
    //     waves' 96) stage: wave w loads pieces w, w + 4, ... of every plane at the start of the
    //     update (v and the log-gates over RmT, read last before it) and stages its items at
    //     the top of the next chunk: a 32-lane scan of each item's 8 gates, v times beta to
    //     registers.
    //   - Once T is dropped the T waves, idle in the update, stage during it, so the next chunk
    //     starts staged: they load the same pieces in the Gram phase, after their Gram tile
    //     (into the T-only Kh^T planes; K into Kb, read last by the operand pass), stage them
    //     the same way after the update but put v times beta back over v as fp16, and copy
    //     that to (diag(b) V)^T at the top of the next chunk.
    constexpr int NPC = CK * D * 2 / 1024;   // 1-KiB pieces of a chunk's [CK][D] bf16 plane
    static_assert(NPC % 4 == 0 && NPC <= 8 && CK * (D / 8) <= 512, "pieces and items spread evenly");
    static_assert(sizeof(sm.rv.nx) <= sizeof(sm.rv.RmT) && sizeof(sm.kt.nx) <= sizeof(sm.kt.KhTb),
                  "v and log-gates fit over RmT and over the Kh^T planes");
    constexpr int IPT = NPC / 4;             // items per S-wave thread
    const int vt = lane % CK;                // token of this thread's staging items
    uint16_t braw = 0;   // beta of token vt of the chunk being fetched
    // piece pc of chunk c0n: token-major (K) or item-major (v, log-gates); ts and ho are the
    // source's token stride and head offset, cols its channels (an item past them loads
    // channel group 0, and is zeroed where staged)
    auto dma = [&](int64_t c0n, const uint16_t* src, uint16_t* dst, int pc, bool item_major, size_t ts, int ho,
                   int cols) {
        // chunk base (uniform, 64-bit) + row offset below 32 tokens (32-bit); rows past the
        // segment clamped to its last token
        const int last = (end - 1 - c0n) < CK - 1 ? (int)(end - 1 - c0n) : CK - 1;
        const int ln = opaque(lane);           // (recomputed here rather than kept live)
        const int e = pc * 512 + ln * 8;       // token-major: element e of the plane
        const int i = pc * 64 + ln;            // item-major: item i
        const int cg = ((NW || NK) && (i / CK) * 8 >= cols) ? 0 : (i / CK) * 8;
        const int ch = (NK && e % D >= cols) ? 0 : e % D;
        const unsigned off = item_major ? (unsigned)min(i % CK, last) * (unsigned)ts + (unsigned)cg
                                        : (unsigned)min(e / D, last) * (unsigned)ts + (unsigned)ch;
        // (the address is a local: as a call inside the builtin's arguments it stops the host
        // pass from emitting the kernel's launch stub)
        const uint16_t* ps = src + (size_t)c0n * ts + (size_t)ho + off;
        __builtin_amdgcn_global_load_lds(ps, (__attribute__((address_space(3))) void*)(dst + pc * 512), 16, 0, 0);
    };
    auto load_beta = [&](int64_t c0n) {
        const int last = (end - 1 - c0n) < CK - 1 ? (int)(end - 1 - c0n) : CK - 1;
        braw = beta[(size_t)(c0n + min(vt, last)) * H + h];
    };
    auto fetch = [&](int64_t c0n, uint16_t* vr, uint16_t* gr) {   // pieces (wave & 3) + 4 r of every plane
#pragma unroll 1   // (unrolled, the addresses of every piece are formed at once: spills)
        for (int r = 0; r < IPT; ++r) {
            const int pc = (wave & 3) + 4 * r;
            dma(c0n, k, &sm.Kb[0][0], pc, false, tok_stride, h * k_ld, k_ld);
            dma(c0n, v, vr, pc, true, (size_t)H * v_ld, h * v_ld, v_cols);
            dma(c0n, gl, gr, pc, true, tok_stride, h * k_ld, k_ld);
        }
        load_beta(c0n);
    };
    auto wait_vm0 = []() {   // s_waitcnt vmcnt(0): this wave's loads have landed
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0x0070);
        asm volatile("" ::: "memory");
    };
    // Staging (this wave's loads landed): for each of the thread's items (wave & 3) * 64 + lane
    // + 256 r, v times beta to registers (vx, written to (diag(b) V)^T past the chunk's first
    // barrier) or back over v as fp16 (to_lds), and the inclusive cumulative log2-gate of its 8
    // channels over the chunk by a 32-lane scan (the item's token is its lane within the
    // half-wave) to Ag; beta to LDS (by chunk parity: a chunk reads its own until its
    // off-diagonal phase).  Rows past the segment are masked by bits (a select on the loaded
    // values compiles to branches around each conversion).
    auto stage = [&](uint16_t* vr, const uint16_t* gr, int nn, float (&vx)[IPT][8], bool to_lds, int bpar) {
        const unsigned lm = vt < nn ? 0xFFFFFFFFu : 0u;
        float bm = -3.0e38f;   // largest b_C over this thread's channels (lanes of token CK - 1)
        const float bt = __uint_as_float(((unsigned)braw << 16) & lm);
        // inclusive scan over the 32 lanes of each half-wave: within rows of 16 lanes by row
        // shifts (lanes shifted in from outside the row read 0), then row 1 (3) adds the total
        // of row 0 (2) by row_bcast:15
        auto dpp_add = [](float a, auto ctrl, auto rmask) {
            return a + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, a),
                                                   decltype(ctrl)::value, decltype(rmask)::value, 0xf, true));
        };
#pragma unroll
        for (int r = 0; r < IPT; ++r) {
            const int i = (wave & 3) * 64 + lane + 256 * r, vcg = i / CK;
            const u32x4 vw = *reinterpret_cast<const u32x4*>(&vr[i * 8]);
            u32x4 gw = *reinterpret_cast<const u32x4*>(&gr[i * 8]);
            if constexpr (NK) {   // log-gates of the channels past k_d: 0 (bit masks, no branch)
                const unsigned gm = vcg * 8 < k_ld ? ~0u : 0u;
#pragma unroll
                for (int e = 0; e < 4; ++e) gw[e] &= gm;
            }
            float x[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                vx[r][2 * e] = bt * __uint_as_float(vw[e] << 16);
                vx[r][2 * e + 1] = bt * __uint_as_float(vw[e] & 0xFFFF0000u);
                x[2 * e] = __uint_as_float((gw[e] << 16) & lm) * kLog2e;
                x[2 * e + 1] = __uint_as_float(gw[e] & 0xFFFF0000u & lm) * kLog2e;
            }
            // step-major over the 8 channels, so that consecutive DPP operations are independent
            // (channel-major, each step waits on the previous one's result)
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = dpp_add(x[e], IntConst<0x111>{}, IntConst<0xf>{});   // row_shr:1
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = dpp_add(x[e], IntConst<0x112>{}, IntConst<0xf>{});   // row_shr:2
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = dpp_add(x[e], IntConst<0x114>{}, IntConst<0xf>{});   // row_shr:4
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = dpp_add(x[e], IntConst<0x118>{}, IntConst<0xf>{});   // row_shr:8
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = dpp_add(x[e], IntConst<0x142>{}, IntConst<0xa>{});   // row_bcast:15 into rows 1, 3
            *reinterpret_cast<f32x4*>(&sm.Ag[vt + 1][vcg * 8]) = f32x4{x[0], x[1], x[2], x[3]};
            *reinterpret_cast<f32x4*>(&sm.Ag[vt + 1][vcg * 8 + 4]) = f32x4{x[4], x[5], x[6], x[7]};
            if (vcg == 0) sm.beta[bpar][vt] = bt;
#pragma unroll
            for (int e = 0; e < 8; ++e) bm = fmaxf(bm, (NK && vcg * 8 >= k_ld) ? -3.0e38f : x[e]);   // (real channels only)
            if (to_lds)
                *reinterpret_cast<u32x4*>(&vr[i * 8]) =
                    u32x4{cvt2_f16(vx[r][0], vx[r][1]), cvt2_f16(vx[r][2], vx[r][3]),
                          cvt2_f16(vx[r][4], vx[r][5]), cvt2_f16(vx[r][6], vx[r][7])};
        }
        // lanes 31 and 63 hold token CK - 1: their cumulative values are the chunk totals
        const float b31 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bm), 31));
        const float b63 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bm), 63));
        if (lane == 0) sm.bmx[bpar][wave & 3] = fmaxf(b31, b63);
    };
    bool staged = false;   // the chunk at hand was staged by the T waves during the previous chunk
    if (beg < end && wave < 4) fetch(beg, sm.rv.nx.Vr, sm.rv.nx.Gr);
    for (int c = tid; c < D; c += 512) sm.Ag[0][c] = 0.f;   // row 0 (exclusive gate of token 0) stays zero
    if (NW) {   // value channels past v_ld: zero rows of (diag(b) V)^T (token columns)
        for (int i = v_cols * LDT + tid; i < D * LDT; i += 512) (&sm.bVT[0][0])[i] = 0;
    }
    static_assert(LDT >= CK + 8, "padding columns of the token-indexed rows");
    for (int64_t c0 = beg; c0 < end; c0 += CK) {
        const int n = (int)((end - c0) < CK ? (end - c0) : CK);
        const int par = (int)(((c0 - beg) / CK) & 1);   // chunk parity (betas, renormalisation records)
        // ---- 1. staging.  Before the chunk's first barrier it writes only what the previous
        // chunk last read before its own final barrier (Ag, betas of this parity): other waves
        // may still be in the previous chunk's state update, which reads (diag(b) V)^T and
        // e^{b_C}, so those are written after the barrier.
        float vx[IPT][8];
        if (!staged && wave < 4) {
            wait_vm0();
            stage(sm.rv.nx.Vr, sm.rv.nx.Gr, n, vx, false, par);
        }
        lds_barrier();
        // (diag(b) V)^T, fp16 (first read in the W and Z1 phase), by the staging waves for
        // their items: from registers, or, when staged during the previous chunk, from the fp16
        // values over v
        // Value channels past v_ld keep the zero rows written at the start: their items write
        // to the rows' padding columns instead (CK .. LDT-1, which no fragment reads), so the
        // stores need no branch.
        auto put_bvt = [&](int r, const uint16_t (&hv)[8]) {
            const int vcg = ((wave & 3) * 64 + lane + 256 * r) / CK;
            const int col = (NW && vcg * 8 >= v_cols) ? CK + (vt & 7) : vt;
#pragma unroll
            for (int e = 0; e < 8; ++e) sm.bVT[vcg * 8 + e][col] = hv[e];
        };
        if (staged) {
            if (wave >= 4) {
#pragma unroll
                for (int r = 0; r < IPT; ++r) {
                    const int i = (wave & 3) * 64 + lane + 256 * r;
                    const u32x4 w4 = *reinterpret_cast<const u32x4*>(&sm.kt.nx.Vr[i * 8]);
                    uint16_t hv[8];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        hv[2 * e] = (uint16_t)(w4[e] & 0xFFFFu);
                        hv[2 * e + 1] = (uint16_t)(w4[e] >> 16);
                    }
                    put_bvt(r, hv);
                }
            }
        } else if (wave < 4) {
#pragma unroll
            for (int r = 0; r < IPT; ++r) {
                uint16_t hv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) hv[e] = f16_bits((_Float16)vx[r][e]);
                put_bvt(r, hv);
            }
        }

        // ---- 2a. renormalisation of the T columns by a power of two when they have become
        // small, from the largest |T| each wave posted after the previous chunk's update (read
        // past this chunk's first barrier); the factor tsc is applied with e^{b_C} in the update,
        // so no branch rewrites the state registers.  Once every T entry is below 2^-120 the T
        // columns are dropped (no longer updated; written as zeros).  One chunk of delay is
        // safe: a chunk decays T by at most e^{-32 max|g|}, far inside fp32.
        float tsc = 1.f;
        if (c0 != beg && t_live) {
            float mm = 0.f;
#pragma unroll
            for (int w = 0; w < 8; ++w) mm = fmaxf(mm, sm.red2[par ^ 1][w]);
            int em = 0;
            if (mm > 0.f) frexpf(mm, &em);
            if (mm == 0.f || log2s + em < -120) {   // T is below the floor for good
                t_live = false;
            } else if (mm < 0x1p-16f) {
                tsc = ldexpf(1.f, -em);
                log2s += em;
            }
        }

        // Once T is dropped, a chunk whose decay factors e^{b_C} are all below 2^-8 carries
        // the state into its update only through terms of that relative size (the decayed
        // state and its erase); the Gram matrices then matter only through the chunk's own
        // erase of its fresh writes (a few per cent of them), and their operands are single
        // bf16 values instead of hi / lo pairs (errors ~2^-9 of those few per cent).
        bool strong = false;
        if (!t_live) {
            strong = fmaxf(fmaxf(sm.bmx[par][0], sm.bmx[par][1]), fmaxf(sm.bmx[par][2], sm.bmx[par][3])) < -8.f;
        }
        const bool stage_next = !t_live && c0 + CK < end;   // the T waves stage the next chunk

        // ---- 2. operands of the decay-weighted Gram matrices and the decay-scaled keys, in one
        // pass (all waves; item = 4 tokens x 2 channels, channel pair fastest across lanes).
        // With one reference rho = c_16 per channel (the second 16-token block's first gate),
        // the Gram operands are k e^{c - rho}, k e^{rho - c} and k e^{rho - i} (i the inclusive
        // gate): every factor is <= 1 except on a diagonal block, where it is bounded by one
        // block's decay, and rho cancels in the products.  The key operands follow from the same
        // factors and two per-channel constants: e^{a} o k = (k e^{c - rho}) e^{rho},
        // Kh = (k e^{rho - c}) e^{b_C - rho}, Kh' = (k e^{rho - i}) e^{b_C - rho}; and e^{rho - i_t}
        // = e^{rho - c_{t+1}} is the next token's e^{rho - c}, so a 4-token item takes 11
        // exponentials per channel instead of 24.  Gram operands go token-major (4-byte stores of
        // the channel pair), key operands channel-major (8-byte stores of the 4 tokens).
        // The pass is instantiated once per precision mode (LIVE: T is live; LO: Gram operands
        // as hi / lo pairs), so that each form is straight-line code: a uniform branch per
        // store kept every exponential next to its store, one dependent chain at a time.
        auto operand_pass = [&](auto live_c, auto lo_c) {
            constexpr bool LIVE = decltype(live_c)::value != 0, LO = decltype(lo_c)::value != 0;
            constexpr int NCP = D / 2;                 // channel pairs
            static_assert((CK / 4) * NCP <= 512, "one item per thread");
            if (tid < (CK / 4) * NCP) {
                const int c = 2 * (tid % NCP), t0 = 4 * (tid / NCP);
                const unsigned km = (!NK || c < k_ld) ? ~0u : 0u;   // keys of the channels past k_d: 0
                float kx[4][2], A[5][2], eg[4][2], er[5][2];
                float P[2], Q[2];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const unsigned kw = *reinterpret_cast<const unsigned*>(&sm.Kb[t0 + i][c]);
                    kx[i][0] = __uint_as_float((kw << 16) & km);
                    kx[i][1] = __uint_as_float(kw & 0xFFFF0000u & km);
                }
                // A[r] = the erase vectors' cumulative gate of token t0 + r (c_t; i_t = c_{t+1}
                // when the gate comes first); A[4] is the next token's
#pragma unroll
                for (int r = 0; r < 5; ++r) {
                    const f32x2 a2 = *reinterpret_cast<const f32x2*>(&sm.Ag[t0 + r + E1 < CK ? t0 + r + E1 : CK][c]);
                    A[r][0] = a2.x;
                    A[r][1] = a2.y;
                }
                const f32x2 rho2 = *reinterpret_cast<const f32x2*>(&sm.Ag[16 + E1][c]);
                const f32x2 bc2 = *reinterpret_cast<const f32x2*>(&sm.Ag[CK][c]);
                const float rho[2] = {rho2.x, rho2.y}, bc[2] = {bc2.x, bc2.y};
#pragma unroll
                for (int j = 0; j < 2; ++j) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) eg[i][j] = exp2_raw(A[i][j] - rho[j]);
#pragma unroll
                    for (int i = 0; i < 5; ++i) er[i][j] = (E1 && i == 4) ? 0.f : exp2_raw(rho[j] - A[i][j]);
                    P[j] = exp2_raw(rho[j]);
                    Q[j] = exp2_raw(bc[j] - rho[j]);
                }
                // e^{rho - i_t}: the next token's e^{rho - c} (gate after the erase); e^{rho - c_t}
                // itself when the gate comes first (i = c for the erase vectors then)
                auto er1 = [&](int i, int j) { return E1 ? er[i][j] : er[i + 1][j]; };
                // Gram operands, token-major
                auto put_tok = [&](uint16_t (*Pl)[CK][D + 8], int t, float x0, float x1) {
                    const unsigned hw = cvt2_bf16(x0, x1);
                    *reinterpret_cast<unsigned*>(&Pl[0][t][c]) = hw;
                    if constexpr (LO) {
                        const f32x2 hv = bf16x2_to_f32(hw);
                        *reinterpret_cast<unsigned*>(&Pl[1][t][c]) = cvt2_bf16(x0 - hv.x, x1 - hv.y);
                    }
                };
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    put_tok(sm.u.g.GL, t0 + i, kx[i][0] * eg[i][0], kx[i][1] * eg[i][1]);
                    put_tok(sm.u.g.GR, t0 + i, kx[i][0] * er[i][0], kx[i][1] * er[i][1]);
                    if (!E1) put_tok(sm.u.g.GR1, t0 + i, kx[i][0] * er1(i, 0), kx[i][1] * er1(i, 1));
                }
                // key operands, channel-major: 4 consecutive tokens of one channel per store, at
                // the swizzled column of rows c and c + 1 (the same for both)
                const int tsw = kswz(opaque(c), t0);
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    float rm[4], kh[4], kp[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        rm[i] = kx[i][j] * eg[i][j] * P[j];
                        kh[i] = kx[i][j] * er[i][j] * Q[j];
                        kp[i] = kx[i][j] * er1(i, j) * Q[j];
                    }
                    if constexpr (LIVE) {   // (e^{a} o K)^T as bf16 hi / lo (W feeds the T columns)
                        unsigned rh[2], rl[2];
#pragma unroll
                        for (int p2 = 0; p2 < 2; ++p2) {
                            rh[p2] = cvt2_bf16(rm[2 * p2], rm[2 * p2 + 1]);
                            const f32x2 hv = bf16x2_to_f32(rh[p2]);
                            rl[p2] = cvt2_bf16(rm[2 * p2] - hv.x, rm[2 * p2 + 1] - hv.y);
                        }
                        *reinterpret_cast<u32x2*>(&sm.rv.RmT[0][c + j][tsw]) = u32x2{rh[0], rh[1]};
                        *reinterpret_cast<u32x2*>(&sm.rv.RmT[1][c + j][tsw]) = u32x2{rl[0], rl[1]};
                    } else {        // fp16, in plane 0 (W feeds only the fp16 S products)
                        *reinterpret_cast<u32x2*>(&sm.rv.RmT[0][c + j][tsw]) =
                            u32x2{cvt2_f16(rm[0], rm[1]), cvt2_f16(rm[2], rm[3])};
                    }
                    *reinterpret_cast<u32x2*>(&sm.KhT[c + j][tsw]) = u32x2{cvt2_f16(kh[0], kh[1]), cvt2_f16(kh[2], kh[3])};
                    *reinterpret_cast<u32x2*>(&sm.KhpT[c + j][tsw]) = u32x2{cvt2_f16(kp[0], kp[1]), cvt2_f16(kp[2], kp[3])};
                    if constexpr (LIVE) {
                        unsigned khh[2], khl[2];
#pragma unroll
                        for (int p2 = 0; p2 < 2; ++p2) {
                            khh[p2] = cvt2_bf16(kh[2 * p2], kh[2 * p2 + 1]);
                            const f32x2 hv = bf16x2_to_f32(khh[p2]);
                            khl[p2] = cvt2_bf16(kh[2 * p2] - hv.x, kh[2 * p2 + 1] - hv.y);
                        }
                        *reinterpret_cast<u32x2*>(&sm.kt.KhTb[0][c + j][tsw]) = u32x2{khh[0], khh[1]};
                        *reinterpret_cast<u32x2*>(&sm.kt.KhTb[1][c + j][tsw]) = u32x2{khl[0], khl[1]};
                    }
                }
                if (t0 == 0) {   // e^{b_C} (wave 0)
                    sm.eBC[c] = exp2_raw(bc[0]);
                    sm.eBC[c + 1] = exp2_raw(bc[1]);
                }
            }
        };
        if (t_live) operand_pass(IntConst<1>{}, IntConst<1>{});
        else if (!strong) operand_pass(IntConst<0>{}, IntConst<1>{});
        else operand_pass(IntConst<0>{}, IntConst<0>{});
        lds_barrier();
        // the six Gram tiles Lp (waves 0-2) and L' (waves 3-5), bf16 hi + lo
        if (wave < 6) {
            const bool lp = wave < 3;
            const int tile = lp ? wave : wave - 3;
            const int I = tile == 0 ? 0 : 1, J = tile == 2 ? 1 : 0;
            const int t = 16 * I + n16, s = 16 * J + n16;
            const uint16_t(*R)[CK][D + 8] = (lp || E1) ? sm.u.g.GR : sm.u.g.GR1;
            f32x4 acc = zero4();
            if (strong) {   // single bf16 operands
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks) {
                    const int c = ks * 32 + 8 * g4;
                    acc = mma_bf16(*reinterpret_cast<const bf16x8*>(&sm.u.g.GL[0][t][c]),
                                   *reinterpret_cast<const bf16x8*>(&R[0][s][c]), acc);
                }
            } else {
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks) {
                    const int c = ks * 32 + 8 * g4;
                    const bf16x8 ah = *reinterpret_cast<const bf16x8*>(&sm.u.g.GL[0][t][c]);
                    const bf16x8 al = *reinterpret_cast<const bf16x8*>(&sm.u.g.GL[1][t][c]);
                    const bf16x8 bh = *reinterpret_cast<const bf16x8*>(&R[0][s][c]);
                    const bf16x8 bl = *reinterpret_cast<const bf16x8*>(&R[1][s][c]);
                    acc = mma_bf16(ah, bh, acc);
                    acc = mma_bf16(ah, bl, acc);
                    acc = mma_bf16(al, bh, acc);
                }
            }
            f32x4 nd;   // -Lp in the accumulator layout (waves 0 and 2: a diagonal block)
            // (the destination and the beta factor selected per wave, so the stores need no branch)
            float(*F)[LDF] = lp ? sm.F1 : sm.F1p;
            const f32x4 b4 = *reinterpret_cast<const f32x4*>(&sm.beta[par][16 * I + 4 * g4]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int tt = 16 * I + 4 * g4 + e, ss = 16 * J + n16;
                const float x = ss < tt ? (lp ? b4[e] : 1.f) * acc[e] : 0.f;
                nd[e] = -x;
                F[tt][ss] = x;
            }
            if (lp && I == J) {
                // D_I = (I + Lp_II)^-1 on MFMA in this wave (no barrier; single fp16 products in
                // the chunks whose Gram operands are single bf16 values): N^T read back from the
                // block just written (one wave's LDS accesses complete in order), the inverse
                // written over the block (row n16: Y[n16][4 g4 .. 4 g4 + 3] = the transposed
                // result's accumulator entries)
                const int o = 16 * I;
                asm volatile("" ::: "memory");
                const f32x4 lt = *reinterpret_cast<const f32x4*>(&sm.F1[o + n16][o + 4 * g4]);
                const f32x4 yt = strong ? inv16_t1(nd, -lt, g4, n16) : inv16_t(nd, -lt, g4, n16);
                asm volatile("" ::: "memory");
                *reinterpret_cast<f32x4*>(&sm.F1[o + n16][o + 4 * g4]) = yt;
            }
        }
        if (stage_next && wave >= 4) fetch(c0 + CK, sm.kt.nx.Vr, sm.kt.nx.Gr);   // (waves 4, 5 after their Gram tile)
        lds_barrier();

        // ---- 3. A = (I + Lp)^-1 to the operand planes of A diag(b) (fp16, and bf16 hi + lo):
        // wave 0 forms A10 = -D1 (L10 D0) and converts it from its accumulators, while the other
        // threads convert the diagonal blocks D0, D1 (in F1, inverted above) and L' to fp16
        // (the bf16 hi / lo planes only while T is live: then W is formed in bf16 hi / lo)
        auto put_ap = [&](int t, int s_, float a, auto live_c) {   // a = A[t][s] b_s
            sm.u.p.Ap[t][s_] = f16_bits((_Float16)a);
            if constexpr (decltype(live_c)::value != 0) put_bf16_split(&sm.u.p.ApB[0][t][s_], &sm.u.p.ApB[1][t][s_], a);
        };
        if (wave == 0) {
            // F = L10 D0 in MFMA accumulators (lane (g4, n16) holds rows 4 g4 .. 4 g4 + 3 of
            // column n16), then -D1 F with the contraction index of k-step kb taken as
            // 4 g4 + kb, so that F's accumulators are the B operand as they stand
            const f32x4 f = mm16_f32(&sm.F1[16][0], LDF, &sm.F1[0][0], LDF, lane);
            f32x4 acc = zero4();
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                acc = mma_f32(sm.F1[16 + n16][16 + 4 * g4 + kb], f[kb], acc);
            const float bn = sm.beta[par][n16];
            if (t_live) {
#pragma unroll
                for (int i = 0; i < 4; ++i) put_ap(16 + 4 * g4 + i, n16, -acc[i] * bn, IntConst<1>{});
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) put_ap(16 + 4 * g4 + i, n16, -acc[i] * bn, IntConst<0>{});
            }
        }
        // the other blocks in row pieces of 4: threads 64 .. 64 + CK * CK / 4 - 1, one piece each
        // (instantiated with and without the bf16 hi / lo planes, so each form is straight-line)
        static_assert(64 + CK * CK / 4 <= 512 && LDF % 4 == 0 && LDT % 4 == 0, "one row piece per thread");
        auto convert = [&](auto live_c) {
            constexpr bool LIVE = decltype(live_c)::value != 0;
            const int q = opaque(tid) - 64, t = q / (CK / 4), s0 = 4 * (q % (CK / 4));   // (addresses formed here)
            // L' to fp16 (row-major); the block above the diagonal is never computed
            const f32x4 l = *reinterpret_cast<const f32x4*>(&sm.F1p[t][s0]);
            *reinterpret_cast<u32x2*>(&sm.u.p.Lpb[t][s0]) =
                u32x2{cvt2_f16(s0 < t ? l[0] : 0.f, s0 + 1 < t ? l[1] : 0.f),
                      cvt2_f16(s0 + 2 < t ? l[2] : 0.f, s0 + 3 < t ? l[3] : 0.f)};
            if (!(t >= 16 && s0 < 16)) {   // (A10: wave 0)
                const f32x4 f = *reinterpret_cast<const f32x4*>(&sm.F1[t][s0]);
                const f32x4 b = *reinterpret_cast<const f32x4*>(&sm.beta[par][s0]);
                float a[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) a[e] = s0 + e <= t ? f[e] * b[e] : 0.f;
                *reinterpret_cast<u32x2*>(&sm.u.p.Ap[t][s0]) = u32x2{cvt2_f16(a[0], a[1]), cvt2_f16(a[2], a[3])};
                if constexpr (LIVE) {
                    uint16_t hi[4], lo[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) put_bf16_split(&hi[e], &lo[e], a[e]);
                    *reinterpret_cast<u32x2*>(&sm.u.p.ApB[0][t][s0]) = u32x2{pack2(hi[0], hi[1]), pack2(hi[2], hi[3])};
                    *reinterpret_cast<u32x2*>(&sm.u.p.ApB[1][t][s0]) = u32x2{pack2(lo[0], lo[1]), pack2(lo[2], lo[3])};
                }
            }
        };
        if (tid >= 64 && tid < 64 + CK * CK / 4) {
            if (t_live) convert(IntConst<1>{});
            else convert(IntConst<0>{});
        }
        lds_barrier();

        // ---- 4. W^T = Rm^T Ap^T (-> W token-major) and Z1^T = (bV)^T L'^T: wave w takes tiles
        // w, w + 8, ... of each (channel tile t / 2, token tile t % 2, so one token tile per
        // wave and one shared B fragment); every fragment is read before the first product.
        // W takes bf16 hi / lo operands while T is live, fp16 ones once only S is updated (it is
        // then rounded to fp16 for the S products either way; rows that decay below fp16's range
        // enter only erase terms of the carried state that are as small).
        {
            constexpr int TPW = RT * 2 / 8;   // W (and Z1) tiles per wave
            static_assert((RT * 2) % 8 == 0, "tiles spread evenly over the waves");
            const int nt = wave % 2;
            const Frag<1> zb = f16frag(&sm.u.p.Lpb[0][0], LDT, nt * 16 + n16, 8 * g4);
            Frag<1> za[TPW];
#pragma unroll
            for (int c = 0; c < TPW; ++c) za[c] = f16frag(&sm.bVT[0][0], LDT, ((wave + 8 * c) / 2) * 16 + n16, 8 * g4);
            f32x4 wacc[TPW], zacc[TPW];
            // swizzled fragment column of rows 16 mt + n16, mt = wave / 2 + 4 c (the same for every c)
            const int rcol = kswz((wave / 2) * 16 + opaque(n16), 8 * g4);
            if (t_live) {
                const FragB wb = fragb_at(&sm.u.p.ApB[0][0][0], &sm.u.p.ApB[1][0][0], LDT, nt * 16 + n16, 8 * g4);
                FragB wa[TPW];
#pragma unroll
                for (int c = 0; c < TPW; ++c)
                    wa[c] = fragb_at(&sm.rv.RmT[0][0][0], &sm.rv.RmT[1][0][0], LDT, ((wave + 8 * c) / 2) * 16 + n16, rcol);
#pragma unroll
                for (int c = 0; c < TPW; ++c) wacc[c] = mma3(wa[c], wb, zero4());
#pragma unroll
                for (int c = 0; c < TPW; ++c) {   // W as bf16 hi / lo (T columns)
                    const int row = nt * 16 + n16, col = ((wave + 8 * c) / 2) * 16 + 4 * g4;
                    uint16_t bh[4], bl[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) put_bf16_split(&bh[e], &bl[e], wacc[c][e]);
                    *reinterpret_cast<u32x2*>(&sm.u.p.WpB[0][row][col]) = u32x2{pack2(bh[0], bh[1]), pack2(bh[2], bh[3])};
                    *reinterpret_cast<u32x2*>(&sm.u.p.WpB[1][row][col]) = u32x2{pack2(bl[0], bl[1]), pack2(bl[2], bl[3])};
                }
            } else {
                const Frag<1> wb = f16frag(&sm.u.p.Ap[0][0], LDT, nt * 16 + n16, 8 * g4);
                Frag<1> wa[TPW];
#pragma unroll
                for (int c = 0; c < TPW; ++c) wa[c] = f16frag(&sm.rv.RmT[0][0][0], LDT, ((wave + 8 * c) / 2) * 16 + n16, rcol);
#pragma unroll
                for (int c = 0; c < TPW; ++c) wacc[c] = mma<1>(wa[c], wb, zero4());
            }
#pragma unroll
            for (int c = 0; c < TPW; ++c) zacc[c] = mma<1>(za[c], zb, zero4());
#pragma unroll
            for (int c = 0; c < TPW; ++c) {
                const int mt = (wave + 8 * c) / 2;
                const f32x4 acc = wacc[c];
                const int row = nt * 16 + n16, col = mt * 16 + 4 * g4;
                *reinterpret_cast<u32x2*>(&sm.u.p.Wp[row][col]) = u32x2{cvt2_f16(acc[0], acc[1]), cvt2_f16(acc[2], acc[3])};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sm.u.p.Z1T[mt * 16 + 4 * g4 + e][nt * 16 + n16] = f16_bits((_Float16)zacc[c][e]);
            }
        }
        lds_barrier();

        if (t_live && c0 + CK < end && wave < 4)   // Kb and RmT are not read again in this chunk
            fetch(c0 + CK, sm.rv.nx.Vr, sm.rv.nx.Gr);
        // fragment column of the swizzled key planes for rows 16 rt + n16: kswz gives chunk
        // g4 ^ ((2 rt + n16 / 8) & 3), one of two values by the parity of rt
        const int kcol0 = 8 * (g4 ^ (n16 >> 3)), kcol1 = kcol0 ^ 16;
        // ---- 5. update of the owned column tiles: Y = W X, R = -(Y [+ U]),
        // X <- e^{b_C} X + Kh^T R [+ Kh'^T bV].  The k-blocks of X are converted to B fragments
        // as they are used; each A fragment is read once for all CTW tiles.
        if (s_wave) {   // S columns: fp16 operands
            const int vt0 = (wave & 3) * CTW;   // first owned value tile
            f32x4 Y[CTW][2];
            {   // U = Ap Z1 as the products' initial value
                const Frag<1> a0 = f16frag(&sm.u.p.Ap[0][0], LDT, n16, 8 * g4);
                const Frag<1> a1 = f16frag(&sm.u.p.Ap[0][0], LDT, 16 + n16, 8 * g4);
#pragma unroll
                for (int c = 0; c < CTW; ++c) {
                    const Frag<1> b = f16frag(&sm.u.p.Z1T[0][0], LDT, (vt0 + c) * 16 + n16, 8 * g4);
                    Y[c][0] = mma<1>(a0, b, zero4());
                    Y[c][1] = mma<1>(a1, b, zero4());
                }
            }
#pragma unroll
            for (int kb = 0; kb < KSD; ++kb) {
                const Frag<1> a0 = f16frag(&sm.u.p.Wp[0][0], D + 8, n16, kb * 32 + 8 * g4);
                const Frag<1> a1 = f16frag(&sm.u.p.Wp[0][0], D + 8, 16 + n16, kb * 32 + 8 * g4);
#pragma unroll
                for (int c = 0; c < CTW; ++c) {
                    const Frag<1> xb = dpair_to_frag<1>(X[2 * kb][c], X[2 * kb + 1][c]);
                    Y[c][0] = mma<1>(a0, xb, Y[c][0]);
                    Y[c][1] = mma<1>(a1, xb, Y[c][1]);
                }
            }
            Frag<1> rb[CTW], vb[CTW];
#pragma unroll
            for (int c = 0; c < CTW; ++c) {
                rb[c] = dpair_to_frag<1>(-Y[c][0], -Y[c][1]);
                vb[c] = f16frag(&sm.bVT[0][0], LDT, (vt0 + c) * 16 + n16, 8 * g4);
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const f32x4 eb = *reinterpret_cast<const f32x4*>(&sm.eBC[rt * 16 + 4 * g4]);
                const Frag<1> a = f16frag(&sm.KhT[0][0], LDT, rt * 16 + n16, (rt & 1) ? kcol1 : kcol0);
                const Frag<1> a2 = f16frag(&sm.KhpT[0][0], LDT, rt * 16 + n16, (rt & 1) ? kcol1 : kcol0);
#pragma unroll
                for (int c = 0; c < CTW; ++c) {
                    f32x4 acc;
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[e] = X[rt][c][e] * eb[e];
                    acc = mma<1>(a, rb[c], acc);
                    X[rt][c] = mma<1>(a2, vb[c], acc);
                }
            }
        } else if (t_live) {   // T columns: bf16 hi + lo products
            f32x4 Y[CTW][2];
#pragma unroll
            for (int c = 0; c < CTW; ++c) Y[c][0] = Y[c][1] = zero4();
#pragma unroll
            for (int kb = 0; kb < KSD; ++kb) {
                const FragB a0 = fragb_at(&sm.u.p.WpB[0][0][0], &sm.u.p.WpB[1][0][0], D + 8, n16, kb * 32 + 8 * g4);
                const FragB a1 = fragb_at(&sm.u.p.WpB[0][0][0], &sm.u.p.WpB[1][0][0], D + 8, 16 + n16, kb * 32 + 8 * g4);
#pragma unroll
                for (int c = 0; c < CTW; ++c) {
                    const FragB xb = dpair_to_fragb(X[2 * kb][c], X[2 * kb + 1][c]);
                    Y[c][0] = mma3(a0, xb, Y[c][0]);
                    Y[c][1] = mma3(a1, xb, Y[c][1]);
                }
            }
            FragB rb[CTW];
#pragma unroll
            for (int c = 0; c < CTW; ++c) rb[c] = dpair_to_fragb(Y[c][0] * -tsc, Y[c][1] * -tsc);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const f32x4 eb = *reinterpret_cast<const f32x4*>(&sm.eBC[rt * 16 + 4 * g4]) * tsc;
                const FragB a = fragb_at(&sm.kt.KhTb[0][0][0], &sm.kt.KhTb[1][0][0], LDT, rt * 16 + n16, (rt & 1) ? kcol1 : kcol0);
#pragma unroll
                for (int c = 0; c < CTW; ++c) {
                    f32x4 acc;
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[e] = X[rt][c][e] * eb[e];
                    X[rt][c] = mma3(a, rb[c], acc);
                }
            }
        }
        // ---- 6. post this wave's largest |T| for the next chunk's renormalisation (no barrier:
        // the next chunk's staging writes nothing this update reads, and its barriers come
        // before the read); the S waves post 0
        float m = 0.f;
        if (!s_wave && t_live) {
#pragma unroll
            for (int c = 0; c < CTW; ++c)
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {   // (NK: the real block of T only; the rest is the identity's)
                        if (!NK || (rt * 16 + 4 * g4 + e < k_ld && (tile0 + c) * 16 + n16 < k_ld))
                            m = fmaxf(m, fabsf(X[rt][c][e]));
                    }
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
        }
        if (lane == 0) sm.red2[par][wave] = m;
        if (stage_next && !s_wave) {   // T waves, idle in the update: stage the next chunk
            const int64_t c1 = c0 + CK;
            float vx1[IPT][8];
            wait_vm0();
            stage(sm.kt.nx.Vr, sm.kt.nx.Gr, (int)((end - c1) < CK ? (end - c1) : CK), vx1, true, par ^ 1);
        }
        staged = stage_next;
    }

    const size_t pair = (size_t)seg * H + h;
    if (!s_wave && T_out == nullptr) return;
#pragma unroll
    for (int c = 0; c < CTW; ++c) {
        const int ct = tile0 + c;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = rt * 16 + 4 * g4 + e;
                if (s_wave) {
                    if ((!NW || (ct - RT) * 16 + n16 < v_cols) && (!NK || row < k_ld))
                        S_out[pair * k_ld * v_ld + (size_t)row * v_ld + (ct - RT) * 16 + n16] = X[rt][c][e];
                }
                else if (!NK || (row < k_ld && ct * 16 + n16 < k_ld))
                    put_t(T_out, t_split, pair, k_ld, row, ct * 16 + n16, t_live ? ldexpf(X[rt][c][e], log2s) : 0.f);
            }
    }
}

hipError_t build_kda(int d, bool in_bf16, bool gate_first, int n_seg, int H, const int64_t* sb, const int64_t* se, int64_t n_tok,
                     const void* k, const void* v, const void* g, const void* beta, void* T_out, bool t_split,
                     float* S_out, hipStream_t st, int v_ld)
{
    if (v_ld == 0) v_ld = d;
    // d_k = 16 or 32: the D = 64 kernel with the key channels past d_k read as zeros
    const int k_d = d;
    const bool nk = d < 64;
    if (nk) d = 64;
    if (!in_bf16) return hipErrorNotSupported;
    const uint16_t *k16 = static_cast<const uint16_t*>(k), *v16 = static_cast<const uint16_t*>(v),
                   *g16 = static_cast<const uint16_t*>(g), *b16 = static_cast<const uint16_t*>(beta);
#define HYPIC_KDA_NW(DD, GFV, NKV)                                                                              \
    if (v_ld < DD)                                                                                               \
        hipLaunchKernelGGL((build_kda_kernel<DD, GFV, true, NKV>), dim3(n_seg * H), dim3(512), 0, st, n_seg, H,    \
                           sb, se, n_tok, k16, v16, g16, b16, T_out, (int)t_split, S_out, v_ld, k_d);            \
    else                                                                                                         \
        hipLaunchKernelGGL((build_kda_kernel<DD, GFV, false, NKV>), dim3(n_seg * H), dim3(512), 0, st, n_seg, H,   \
                           sb, se, n_tok, k16, v16, g16, b16, T_out, (int)t_split, S_out, v_ld, k_d);
#define HYPIC_KDA(DD, GFV)                                                                                      \
    if (d == DD && gate_first == GFV) {                                                                          \
        if (DD == 64 && nk) {                                                                                    \
            HYPIC_KDA_NW(64, GFV, true)                                                                          \
        } else {                                                                                                 \
            HYPIC_KDA_NW(DD, GFV, false)                                                                         \
        }                                                                                                        \
        return hipGetLastError();                                                                                \
    }
    HYPIC_KDA(128, false)
    HYPIC_KDA(128, true)
    HYPIC_KDA(64, false)
    HYPIC_KDA(64, true)
#undef HYPIC_KDA
#undef HYPIC_KDA_NW
    return hipErrorNotSupported;
}

}  // namespace hypic
