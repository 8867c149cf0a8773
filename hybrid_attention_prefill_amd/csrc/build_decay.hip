// build_decay.hip -- segment build for transitions without the delta-rule erase:
// M_t = e^{g_t} I (g_t = log gamma_h for RetNet-style constant decay, or a
// per-token scalar log-gate as in Mamba2), write k_t v_t^T.  Here T_C = e^{sum g} I and
//     S(C|0) = sum_t e^{sum_{s>t} g_s} k_t v_t^T = K^T diag(w) V
// ([ZH] = the Chinese HYPIC page, section 2.1, which names RetNet among the
// decayed families whose segments need T_C and claims the whole linear-attention
// family).  For a constant decay gamma this is w_t = gamma^(L-1-t), the closed form.
// With a per-channel gate (GLA-style, M_t = diag(a_t)) the weights act on the key
// channels instead: S(C|0) = sum_t diag(e^{sum_{s>t} g_s}) k_t v_t^T and T_C =
// diag(e^{sum g}).
//
// Chunks of 64 tokens, in order: S <- e^{b_C} S + K^T diag(e^{b_C - b}) V with
// b the in-chunk cumulative log-gate, so every exponent is <= 0 (per channel:
// S <- diag(e^{b_C}) S + (e^{b_C - b} o K)^T V).  One
// workgroup (4 waves) per (segment, head); S tiles are dealt to waves and stay
// in fp32 MFMA accumulators.  The product runs on v_mfma_f32_16x16x32_bf16:
// the weighted V is split into bf16 hi + lo (bf16 keys are exact; fp32 keys
// are split too), keeping the fp32 exponent range for the tiny weights of
// fast-decaying heads.
//
// With a workspace, a segment is cut into up to 8 runs of whole chunks built in parallel
// (one workgroup each) and composed by decay_fold_kernel: without the erase every piece's
// transition is a scalar (or diagonal), so the composition law ([ZH] section 2.1) is an
// elementwise weighted sum.
#include "hypic_device.h"
#include "hypic_kernels.h"

namespace hypic {

namespace {
constexpr int CH = 64;
constexpr int LDT = CH + 8;

// Pieces of a segment (decay builds with a workspace): the segment's ceil(L / 64) chunks
// are cut into min(8, chunks) near-equal runs of whole chunks.  How a segment is cut
// depends on its length only.
constexpr int kMaxPieces = 8;
struct PieceRange { int64_t beg, end; int n_pieces; };
__host__ __device__ inline PieceRange piece_range(int64_t beg, int64_t end, int p) {
    const int64_t chunks = (end - beg + CH - 1) / CH;
    const int np = (int)(chunks < kMaxPieces ? chunks : kMaxPieces);
    PieceRange r{beg, beg, np};
    if (p < np) {
        const int64_t c0 = chunks * p / np, c1 = chunks * (p + 1) / np;
        r.beg = beg + c0 * CH;
        r.end = beg + c1 * CH < end ? beg + c1 * CH : end;
    }
    return r;
}
// workspace: piece states [n_seg][H][8][DK][DV] fp32, then piece log-decays [n_seg][H][8][DK]
// (one value per piece for scalar gates)
__host__ __device__ inline size_t piece_log_offset(int n_seg, int H, int DK, int DV) {
    return (size_t)n_seg * H * kMaxPieces * DK * DV;
}

// 8 consecutive values at element e (zeros when !on; the address is not formed then)
template <bool BF16>
__device__ __forceinline__ void load8(const void* base, size_t e, bool on, float* x) {
    if constexpr (BF16) {
        u32x4 w = u32x4{0u, 0u, 0u, 0u};
        if (on) w = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(base) + e);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(w[i] << 16);
            x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    } else {
        f32x4 a = zero4(), b = zero4();
        if (on) {
            const f32x4* p = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(base) + e);
            a = p[0];
            b = p[1];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) { x[i] = a[i]; x[4 + i] = b[i]; }
    }
}

template <bool BF16>
__device__ __forceinline__ float ld1(const void* base, size_t e) {
    if constexpr (BF16) return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[e]);
    else return reinterpret_cast<const float*>(base)[e];
}
}  // namespace

template <int DK, int DV, bool BF16, int GATE, bool PIECES>
__global__ __launch_bounds__(256) void build_decay_kernel(
    int n_seg, int H, const int64_t* __restrict__ seg_begin, const int64_t* __restrict__ seg_end,
    int64_t n_tokens, const void* __restrict__ k, const void* __restrict__ v,
    const void* __restrict__ gl, void* __restrict__ T_out, int t_layout, float* __restrict__ S_out,
    float* __restrict__ piece_ws)
{
    constexpr bool DIAG = GATE == 2;       // per-channel gate: the weights move from V to K
    constexpr int RTK = DK / 16, RTV = DV / 16;
    constexpr int NT = RTK * RTV;          // output tiles
    constexpr int TW = (NT + 3) / 4;       // tiles per wave
    constexpr int CGK = DK / 8, CGV = DV / 8;   // 8-channel groups per token
    constexpr int CG = CGK > CGV ? CGK : CGV;
    constexpr int NIT = (CH * CGK + 255) / 256;   // gate staging items per thread
    constexpr bool KSPLIT = !BF16 || DIAG; // keys need a lo plane (fp32, or weighted per channel)
    constexpr bool VSPLIT = !BF16 || !DIAG;
    __shared__ __attribute__((aligned(16))) uint16_t Kt[2][DK][LDT];  // K^T (hi, lo); DIAG: weighted
    __shared__ __attribute__((aligned(16))) uint16_t Vt[2][DV][LDT];  // V^T (hi, lo); scalar: weighted
    __shared__ float gsh[CH], wsh[CH];
    __shared__ float gd[DIAG ? CH : 1][DIAG ? DK + 1 : 1];   // DIAG: gates, then in-chunk cumulative sums
    __shared__ float bcd[DIAG ? DK : 1], logd[DIAG ? DK : 1];  // DIAG: chunk total and segment total per key channel
    __shared__ float bCs;

    // PIECES: one workgroup per (segment, head, piece); the piece's pair goes to the
    // workspace and decay_fold_kernel composes the pieces
    const int piece = PIECES ? blockIdx.x % kMaxPieces : 0;
    const int unit = PIECES ? blockIdx.x / kMaxPieces : blockIdx.x, seg = unit / H, h = unit % H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g4 = lane >> 4, n16 = lane & 15;
    int64_t beg = seg_begin[seg], end = seg_end[seg];
    beg = beg < 0 ? 0 : (beg > n_tokens ? n_tokens : beg);
    end = end < beg ? beg : (end > n_tokens ? n_tokens : end);
    if constexpr (PIECES) {
        const PieceRange pr = piece_range(beg, end, piece);
        if (pr.n_pieces <= piece) return;   // uniform: the segment has fewer pieces
        beg = pr.beg;
        end = pr.end;
    }

    f32x4 acc[TW];
#pragma unroll
    for (int i = 0; i < TW; ++i) acc[i] = zero4();
    float log_t = 0.f;
    const float ghead = GATE == 0 ? reinterpret_cast<const float*>(gl)[h] : 0.f;
    const size_t stride_k = (size_t)H * DK, stride_v = (size_t)H * DV;
    if constexpr (DIAG) {
        for (int ch = tid; ch < DK; ch += 256) logd[ch] = 0.f;
    }

    for (int64_t c0 = beg; c0 < end; c0 += CH) {
        const int n = (int)((end - c0) < CH ? (end - c0) : CH);
        if constexpr (DIAG) {
            // per-channel gates, then the in-chunk inclusive cumulative sums b_t[ch] (one
            // channel per thread) and the chunk totals b_C[ch]
            {   // 8 channels of one token per item, every load of the thread issued first
                float gx[NIT][8];
#pragma unroll
                for (int r = 0; r < NIT; ++r) {
                    const int it = tid + 256 * r, t = it / CGK, c8 = (it % CGK) * 8;
                    load8<BF16>(gl, (size_t)(c0 + t) * stride_k + (size_t)h * DK + c8, it < CH * CGK && t < n, gx[r]);
                }
#pragma unroll
                for (int r = 0; r < NIT; ++r) {
                    const int it = tid + 256 * r, t = it / CGK, c8 = (it % CGK) * 8;
                    if (it < CH * CGK)
#pragma unroll
                        for (int e = 0; e < 8; ++e) gd[t][c8 + e] = gx[r][e];
                }
            }
            __syncthreads();
            for (int ch = tid; ch < DK; ch += 256) {
                float x = 0.f;
                for (int t = 0; t < CH; ++t) {
                    x += gd[t][ch];
                    gd[t][ch] = x;
                }
                bcd[ch] = x;
                logd[ch] += x;
            }
        } else {
            if (tid < CH) {
                float gv = 0.f;
                if (tid < n) gv = GATE == 0 ? ghead : ld1<BF16>(gl, (size_t)(c0 + tid) * H + h);
                gsh[tid] = gv;
            }
            __syncthreads();
            if (wave == 0) {  // in-chunk inclusive cumsum; weight e^{b_C - b_t}
                float x = gsh[lane];
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const float y = __shfl_up(x, off, 64);
                    if (lane >= off) x += y;
                }
                const float bc = __shfl(x, 63, 64);
                wsh[lane] = lane < n ? expf(bc - x) : 0.f;
                if (lane == 0) bCs = bc;
            }
        }
        __syncthreads();
        {   // item: 4 tokens x 8 channels (4 loads of 8 key and 8 value channels), written as
            // 4-token runs of 8 channel rows of K^T and V^T; the token block is fastest across lanes,
            // so the runs of one row from 16 lanes are contiguous.  With d_k != d_v the items past
            // the smaller dimension load and write only the other.
            constexpr int NTB = CH / 4, NI = NTB * CG;
            for (int it = tid; it < NI; it += 256) {
                const int tb = it % NTB, c8 = (it / NTB) * 8;
                const bool hk = c8 < DK, hv = c8 < DV;
                float kx[4][8], vx[4][8];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 4 * tb + r;
                    load8<BF16>(k, (size_t)(c0 + t) * stride_k + (size_t)h * DK + c8, hk && t < n, kx[r]);
                    load8<BF16>(v, (size_t)(c0 + t) * stride_v + (size_t)h * DV + c8, hv && t < n, vx[r]);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 4 * tb + r;
                    if (t < n) {
#pragma unroll
                        for (int x = 0; x < 8; ++x) {
                            if constexpr (DIAG) {   // channel decays by e^{b_C - b_t}
                                if (hk) kx[r][x] *= expf(bcd[c8 + x] - gd[t][c8 + x]);
                            } else {
                                vx[r][x] *= wsh[t];
                            }
                        }
                    }
                }
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    unsigned kh[2], kl[2], vh[2], vl[2];
#pragma unroll
                    for (int r = 0; r < 2; ++r) {
                        kh[r] = cvt2_bf16(kx[2 * r][x], kx[2 * r + 1][x]);
                        const f32x2 kf = bf16x2_to_f32(kh[r]);
                        kl[r] = cvt2_bf16(kx[2 * r][x] - kf.x, kx[2 * r + 1][x] - kf.y);
                        vh[r] = cvt2_bf16(vx[2 * r][x], vx[2 * r + 1][x]);
                        const f32x2 vf = bf16x2_to_f32(vh[r]);
                        vl[r] = cvt2_bf16(vx[2 * r][x] - vf.x, vx[2 * r + 1][x] - vf.y);
                    }
                    if (hk) {
                        *reinterpret_cast<u32x2*>(&Kt[0][c8 + x][4 * tb]) = u32x2{kh[0], kh[1]};
                        *reinterpret_cast<u32x2*>(&Kt[1][c8 + x][4 * tb]) = u32x2{kl[0], kl[1]};
                    }
                    if (hv) {
                        *reinterpret_cast<u32x2*>(&Vt[0][c8 + x][4 * tb]) = u32x2{vh[0], vh[1]};
                        *reinterpret_cast<u32x2*>(&Vt[1][c8 + x][4 * tb]) = u32x2{vl[0], vl[1]};
                    }
                }
            }
        }
        __syncthreads();
        const float ebc = DIAG ? 0.f : expf(bCs);
#pragma unroll
        for (int i = 0; i < TW; ++i) {
            const int tile = wave + 4 * i;
            if (tile >= NT) continue;
            const int mt = tile / RTV, nt = tile % RTV;  // key-channel tile, value-channel tile
            f32x4 a;
            if constexpr (DIAG) {   // row (key channel) m decays by e^{b_C[m]}
#pragma unroll
                for (int e = 0; e < 4; ++e) a[e] = acc[i][e] * expf(bcd[mt * 16 + 4 * g4 + e]);
            } else {
                a = acc[i] * ebc;
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 kh = *reinterpret_cast<const bf16x8*>(&Kt[0][mt * 16 + n16][ks * 32 + 8 * g4]);
                const bf16x8 vh = *reinterpret_cast<const bf16x8*>(&Vt[0][nt * 16 + n16][ks * 32 + 8 * g4]);
                a = mma_bf16(kh, vh, a);
                if constexpr (VSPLIT) {
                    const bf16x8 vl = *reinterpret_cast<const bf16x8*>(&Vt[1][nt * 16 + n16][ks * 32 + 8 * g4]);
                    a = mma_bf16(kh, vl, a);
                }
                if constexpr (KSPLIT) {
                    const bf16x8 kl = *reinterpret_cast<const bf16x8*>(&Kt[1][mt * 16 + n16][ks * 32 + 8 * g4]);
                    a = mma_bf16(kl, vh, a);
                }
            }
            acc[i] = a;
        }
        if constexpr (!DIAG) log_t += bCs;
        __syncthreads();
    }

    const size_t pair = (size_t)seg * H + h;
    const size_t slot = PIECES ? pair * kMaxPieces + piece : pair;
    float* S = (PIECES ? piece_ws : S_out) + slot * DK * DV;
#pragma unroll
    for (int i = 0; i < TW; ++i) {
        const int tile = wave + 4 * i;
        if (tile >= NT) continue;
        const int mt = tile / RTV, nt = tile % RTV;
#pragma unroll
        for (int e = 0; e < 4; ++e) S[(size_t)(mt * 16 + 4 * g4 + e) * DV + nt * 16 + n16] = acc[i][e];
    }
    if constexpr (PIECES) {   // the piece's log-decay (per key channel for the diagonal gate)
        float* L = piece_ws + piece_log_offset(n_seg, H, DK, DV) + slot * (DIAG ? DK : 1);
        if constexpr (DIAG) {
            for (int ch = tid; ch < DK; ch += 256) L[ch] = logd[ch];
        } else {
            if (tid == 0) L[0] = log_t;
        }
        return;
    }
    if (T_out) {
        if constexpr (DIAG) {
            if (t_layout == 3) {   // diagonal
                for (int ch = tid; ch < DK; ch += 256) reinterpret_cast<float*>(T_out)[pair * DK + ch] = expf(logd[ch]);
            } else {               // dense diag(t), fp32 or bf16 hi/lo planes
                for (int it = tid; it < DK * DK; it += 256)
                    put_t(T_out, t_layout == 2, pair, DK, it / DK, it % DK, (it / DK == it % DK) ? expf(logd[it / DK]) : 0.f);
            }
        } else {
            const float tval = expf(log_t);
            if (t_layout == 1) {   // scalar
                if (tid == 0) reinterpret_cast<float*>(T_out)[pair] = tval;
            } else {               // dense t I, fp32 or bf16 hi/lo planes
                for (int it = tid; it < DK * DK; it += 256)
                    put_t(T_out, t_layout == 2, pair, DK, it / DK, it % DK, (it / DK == it % DK) ? tval : 0.f);
            }
        }
    }
}

// Composition of a segment's pieces, in order: S = sum_p (prod_{q > p} t_q) S_p and
// T = prod_p t_p, with t_p = e^{(log-decay of piece p)} a scalar, or per key channel (row of S)
// for the diagonal gate.  One workgroup per (segment, head); 4 consecutive entries of one row per
// thread and step.  A segment without tokens gets the identity pair.
template <int DK, int DV, bool DIAG>
__global__ __launch_bounds__(256) void decay_fold_kernel(int n_seg, int H, const int64_t* __restrict__ seg_begin,
                                                         const int64_t* __restrict__ seg_end, int64_t n_tokens,
                                                         const float* __restrict__ piece_ws, void* __restrict__ T_out,
                                                         int t_layout, float* __restrict__ S_out)
{
    const int unit = blockIdx.x, seg = unit / H, h = unit % H;
    const int tid = threadIdx.x;
    int64_t beg = seg_begin[seg], end = seg_end[seg];
    beg = beg < 0 ? 0 : (beg > n_tokens ? n_tokens : beg);
    end = end < beg ? beg : (end > n_tokens ? n_tokens : end);
    const int np = piece_range(beg, end, 0).n_pieces;
    const size_t pair = (size_t)seg * H + h;
    const float* Lg = piece_ws + piece_log_offset(n_seg, H, DK, DV) + pair * kMaxPieces * (DIAG ? DK : 1);
    const f32x4* Sp = reinterpret_cast<const f32x4*>(piece_ws + pair * kMaxPieces * DK * DV);
    f32x4* S = reinterpret_cast<f32x4*>(S_out + pair * DK * DV);
    constexpr int NQ = DK * DV / 4;
    // weight of piece p for row r: e^{log-decay of the pieces after p} (one row for scalar T)
    __shared__ float wt[kMaxPieces][DIAG ? DK : 1];
    for (int r = tid; r < (DIAG ? DK : 1); r += 256) {
        float l[kMaxPieces];
#pragma unroll
        for (int p = 0; p < kMaxPieces; ++p) l[p] = p < np ? Lg[p * (DIAG ? DK : 1) + r] : 0.f;
        float lsum = 0.f;
#pragma unroll
        for (int p = kMaxPieces - 1; p >= 0; --p) {
            wt[p][r] = __expf(lsum);
            lsum += l[p];
        }
    }
    __syncthreads();
    for (int q = tid; q < NQ; q += 256) {
        const int row = DIAG ? 4 * q / DV : 0;   // key channel of the 4 entries
        f32x4 sp[kMaxPieces];
#pragma unroll
        for (int p = 0; p < kMaxPieces; ++p) sp[p] = p < np ? Sp[(size_t)p * NQ + q] : zero4();
        f32x4 x = zero4();
#pragma unroll
        for (int p = kMaxPieces - 1; p >= 0; --p)
            if (p < np) x = x + wt[p][row] * sp[p];
        S[q] = x;
    }
    if (T_out) {
        if constexpr (DIAG) {
            for (int ch = tid; ch < DK; ch += 256) {
                float l = 0.f;
                for (int p = 0; p < np; ++p) l += Lg[p * DK + ch];
                if (t_layout == 3) reinterpret_cast<float*>(T_out)[pair * DK + ch] = __expf(l);
            }
            if (t_layout != 3) {   // dense diag(t), fp32 or bf16 hi/lo planes
                for (int it = tid; it < DK * DK; it += 256) {
                    const int r = it / DK, c = it % DK;
                    float l = 0.f;
                    if (r == c)
                        for (int p = 0; p < np; ++p) l += Lg[p * DK + r];
                    put_t(T_out, t_layout == 2, pair, DK, r, c, r == c ? __expf(l) : 0.f);
                }
            }
        } else {
            float l = 0.f;
            for (int p = 0; p < np; ++p) l += Lg[p];
            const float tval = __expf(l);
            if (t_layout == 1) {   // scalar
                if (tid == 0) reinterpret_cast<float*>(T_out)[pair] = tval;
            } else {               // dense t I, fp32 or bf16 hi/lo planes
                for (int it = tid; it < DK * DK; it += 256)
                    put_t(T_out, t_layout == 2, pair, DK, it / DK, it % DK, (it / DK == it % DK) ? tval : 0.f);
            }
        }
    }
}

template <int DK, int DV, bool BF16, int GATE>
static hipError_t launch_decay(int n_seg, int H, const int64_t* sb, const int64_t* se, int64_t n_tok,
                               const void* k, const void* v, const void* g, void* T_out, int t_layout,
                               float* S_out, float* ws, hipStream_t st)
{
    if (ws == nullptr) {
        hipLaunchKernelGGL((build_decay_kernel<DK, DV, BF16, GATE, false>), dim3(n_seg * H), dim3(256), 0, st, n_seg,
                           H, sb, se, n_tok, k, v, g, T_out, t_layout, S_out, nullptr);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((build_decay_kernel<DK, DV, BF16, GATE, true>), dim3(n_seg * H * kMaxPieces), dim3(256), 0,
                       st, n_seg, H, sb, se, n_tok, k, v, g, T_out, t_layout, S_out, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decay_fold_kernel<DK, DV, GATE == 2>), dim3(n_seg * H), dim3(256), 0, st, n_seg, H, sb, se,
                       n_tok, ws, T_out, t_layout, S_out);
    return hipGetLastError();
}

size_t decay_workspace_bytes(int dk, int dv, int H, int n_seg, int64_t n_tokens, bool diag)
{
    // pieces pay where segments average at least 4 chunks (256 tokens)
    if (n_seg < 1 || H < 1 || n_tokens < (int64_t)n_seg * 4 * CH) return 0;
    return ((size_t)n_seg * H * kMaxPieces * ((size_t)dk * dv + (diag ? dk : 1)) * sizeof(float) + 255) / 256 * 256;
}

hipError_t build_decay(int dk, int dv, bool in_bf16, int gate, int n_seg, int H, const int64_t* sb,
                       const int64_t* se, int64_t n_tok, const void* k, const void* v, const void* g,
                       void* T_out, int t_layout, float* S_out, void* ws, hipStream_t st)
{
    float* w = static_cast<float*>(ws);
#define HYPIC_GATES(DK_, DV_, B_)                                                                             \
    if (gate == 0) return launch_decay<DK_, DV_, B_, 0>(n_seg, H, sb, se, n_tok, k, v, g, T_out, t_layout, S_out, w, st); \
    if (gate == 1) return launch_decay<DK_, DV_, B_, 1>(n_seg, H, sb, se, n_tok, k, v, g, T_out, t_layout, S_out, w, st); \
    return launch_decay<DK_, DV_, B_, 2>(n_seg, H, sb, se, n_tok, k, v, g, T_out, t_layout, S_out, w, st);
#define HYPIC_CASE(DK_, DV_)                        \
    if (dk == DK_ && dv == DV_) {                   \
        if (in_bf16) { HYPIC_GATES(DK_, DV_, true) } \
        HYPIC_GATES(DK_, DV_, false)                \
    }
#define HYPIC_ROW(DK_) HYPIC_CASE(DK_, 16) HYPIC_CASE(DK_, 32) HYPIC_CASE(DK_, 64) HYPIC_CASE(DK_, 128)
    HYPIC_ROW(16) HYPIC_ROW(32) HYPIC_ROW(64) HYPIC_ROW(128)
#undef HYPIC_ROW
#undef HYPIC_CASE
#undef HYPIC_GATES
    return hipErrorNotSupported;
}

}  // namespace hypic
