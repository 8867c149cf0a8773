// seam.hip -- state-independent preparation of the seam windows.
//
// [ZH] (the Chinese HYPIC page), section 2.2: the first w tokens of every
// internal segment are kept out of the cache; at reuse the linear layers work
// out the window's own transition and state, advance the running state with
// it and send each window token's output to the attention layer above.
//
// For a window of w <= 16 tokens (padded to 16 with no-op tokens: k = v = q = 0,
// beta = 0, g = 0), with b the in-window inclusive cumulative log-gate and
// At = (I + Lt)^-1, Lt[t][s] = beta_t k_t.k_s (s < t), everything that does not
// depend on the running state R is
//     Wt[t] = sum_s At[t][s] beta_s k_s                 (16 x d_k)
//     U[t]  = sum_s e^{b_t-b_s} At[t][s] beta_s v_s     (16 x d_v)
//     Mo[t][s] = scale e^{b_t-b_s} (q_t . k_s), s <= t  (16 x 16)
// and the chain kernel (seam_chain.hip) then needs only (chunk form of the gated
// delta rule with its in-chunk outputs):
//     U' = U - diag(e^b) (Wt R)
//     O  = scale diag(e^b) (Q R) + Mo U'                 (window outputs)
//     R <- e^{b_w} R + K^T diag(e^{b_w - b}) U'          (state after the window)
// One workgroup (4 waves) per (chain, step, head) window.  The two 16 x 16 Gram
// products K K^T and Q K^T and the products Wt = Cw K, U = Cu V run on MFMA (bf16
// operands: exact for bf16 inputs, a hi/lo split for fp32 inputs and for the
// coefficients), the small triangular solve in fp32 on the vector ALUs.  Wt, q, k
// and Mo are written as bf16 hi/lo planes in MFMA fragment order (frag_off), so
// the chain kernel fetches each operand fragment as one contiguous 1 KiB.
#include "hypic_device.h"
#include "hypic_kernels.h"
#include "seam_layout.h"

namespace hypic {

namespace {

// hi/lo bf16 planes of 8 consecutive floats, written as two 16-byte stores (lo == NULL:
// the hi plane only, for values that bf16 holds exactly)
__device__ __forceinline__ void put_split8(uint16_t* hi, uint16_t* lo, const float* x)
{
    unsigned h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        __bf16 a0, b0, a1, b1;
        split_bf16(x[2 * i], a0, b0);
        split_bf16(x[2 * i + 1], a1, b1);
        h[i] = pack2(bf16_bits(a0), bf16_bits(a1));
        l[i] = pack2(bf16_bits(b0), bf16_bits(b1));
    }
    *reinterpret_cast<u32x4*>(hi) = u32x4{h[0], h[1], h[2], h[3]};
    if (lo) *reinterpret_cast<u32x4*>(lo) = u32x4{l[0], l[1], l[2], l[3]};
}

}  // namespace

template <int D>
__global__ __launch_bounds__(256) void seam_prep_kernel(
    int n_cj, int H, const int64_t* __restrict__ seam_start, int64_t n_tokens, int w,
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const void* __restrict__ gl, const void* __restrict__ beta, int in_bf16, float scale,
    unsigned char* __restrict__ ws, int v_ld)
{
    // v_ld: row length of v ([n_tokens][H][v_ld]); v points at this call's D value columns
    // (with v_ld < D, the channels past v_ld read as zeros: U has zero columns there)
    const int v_cols = v_ld < D ? v_ld : D;
    constexpr int W = kSeamMaxW;
    constexpr int LD = D + 4;                 // padded rows (float4 aligned)
    constexpr int KP = D < 32 ? 32 : D;       // contraction length padded to the MFMA K
    using R = SeamRec<D>;
    __shared__ __attribute__((aligned(16))) float Ks[W][LD];
    __shared__ __attribute__((aligned(16))) float Vs[W][LD];
    __shared__ __attribute__((aligned(16))) float Qs[W][LD];
    __shared__ float bs[W], bt[W], Gk[W][W + 1], Gq[W][W + 1], Cw[W][W + 1], Cu[W][W + 1];

    const int rec = blockIdx.x;             // (cj, h)
    const int cj = rec / H, h = rec % H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t s0 = seam_start[cj];
    if (s0 < 0 || s0 + w > n_tokens) return;  // uniform: no seam at this step
    unsigned char* rp = ws + (size_t)rec * R::kBytes;

    // ---- window tokens into LDS (fp32), padded tokens zero
    {
        constexpr int CG = D / 8;              // 8-channel groups per token
        for (int it = tid; it < W * CG; it += 256) {
            const int t = it / CG, c0 = (it % CG) * 8;
            float kx[8], vx[8], qx[8];
            if (t < w) {
                const size_t e = (size_t)(s0 + t) * H * D + (size_t)h * D + c0;
                const bool vok = c0 < v_cols;
                const size_t ev = ((size_t)(s0 + t) * H + h) * v_ld + (vok ? c0 : 0);
                if (in_bf16) {
                    const u32x4 a = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(k) + e);
                    const u32x4 b = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(v) + ev);
                    const u32x4 c = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(q) + e);
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        kx[2 * x] = __uint_as_float(a[x] << 16); kx[2 * x + 1] = __uint_as_float(a[x] & 0xFFFF0000u);
                        vx[2 * x] = __uint_as_float(b[x] << 16); vx[2 * x + 1] = __uint_as_float(b[x] & 0xFFFF0000u);
                        qx[2 * x] = __uint_as_float(c[x] << 16); qx[2 * x + 1] = __uint_as_float(c[x] & 0xFFFF0000u);
                    }
                } else {
                    const f32x4* a = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(k) + e);
                    const f32x4* b = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(v) + ev);
                    const f32x4* c = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(q) + e);
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        kx[x] = a[0][x]; kx[4 + x] = a[1][x];
                        vx[x] = b[0][x]; vx[4 + x] = b[1][x];
                        qx[x] = c[0][x]; qx[4 + x] = c[1][x];
                    }
                }
            } else {
#pragma unroll
                for (int x = 0; x < 8; ++x) kx[x] = vx[x] = qx[x] = 0.f;
            }
            if (c0 >= v_cols) {
#pragma unroll
                for (int x = 0; x < 8; ++x) vx[x] = 0.f;
            }
#pragma unroll
            for (int x = 0; x < 8; x += 4) {
                *reinterpret_cast<f32x4*>(&Ks[t][c0 + x]) = f32x4{kx[x], kx[x + 1], kx[x + 2], kx[x + 3]};
                *reinterpret_cast<f32x4*>(&Vs[t][c0 + x]) = f32x4{vx[x], vx[x + 1], vx[x + 2], vx[x + 3]};
                *reinterpret_cast<f32x4*>(&Qs[t][c0 + x]) = f32x4{qx[x], qx[x + 1], qx[x + 2], qx[x + 3]};
            }
        }
        if (tid < W) {
            const bool ok = tid < w;
            const size_t e = (size_t)(s0 + tid) * H + h;
            auto ld1 = [&](const void* base) -> float {
                return in_bf16 ? bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[e])
                               : reinterpret_cast<const float*>(base)[e];
            };
            bt[tid] = ok ? ld1(beta) : 0.f;
            Gk[tid][W] = ok ? ld1(gl) : 0.f;     // log-gates parked in the pad column
        }
    }
    __syncthreads();

    // ---- Gram products on MFMA: wave 0 K K^T, wave 1 Q K^T.  Wave 2: cumulative gates.
    const int g4 = lane >> 4, n16 = lane & 15;
    if (wave < 2) {
        const float (*X)[LD] = wave == 0 ? Ks : Qs;
        f32x4 acc = zero4();
#pragma unroll
        for (int ks = 0; ks < KP / 32; ++ks) {
            const int c0 = ks * 32 + 8 * g4;
            float xa[8], kb[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                xa[j] = c0 < D ? X[n16][c0 + j] : 0.f;   // A: row n16 of X
                kb[j] = c0 < D ? Ks[n16][c0 + j] : 0.f;  // B: column n16 of K^T = row n16 of K
            }
            bf16x8 ah, al, bh, bl;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                __bf16 x, y;
                split_bf16(xa[j], x, y); ah[j] = x; al[j] = y;
                split_bf16(kb[j], x, y); bh[j] = x; bl[j] = y;
            }
            acc = mma_bf16(ah, bh, acc);
            if (!in_bf16) {   // bf16 inputs are exact in one term
                acc = mma_bf16(ah, bl, acc);
                acc = mma_bf16(al, bh, acc);
            }
        }
        float (*G)[W + 1] = wave == 0 ? Gk : Gq;
#pragma unroll
        for (int i = 0; i < 4; ++i) G[4 * g4 + i][n16] = acc[i];
    } else if (wave == 2 && lane < W) {
        float acc = 0.f;
        for (int t = 0; t <= lane; ++t) acc += Gk[t][W];
        bs[lane] = acc;
    }
    __syncthreads();

    // ---- Lt in Cw (scratch), Mo planes, gate vectors
    {
        const int t = tid / W, s = tid % W;
        const float gk = Gk[t][s], gq = Gq[t][s];
        const float dts = bs[t] - bs[s];
        Cw[t][s] = s < t ? bt[t] * gk : 0.f;
        const float mo = s <= t ? scale * expf(dts) * gq : 0.f;
        __bf16 x, y;
        split_bf16(mo, x, y);
        if (t < w) {   // (rows past the window are never read: the chain zeroes them itself)
            reinterpret_cast<uint16_t*>(rp + R::kM)[frag_off(t, s, W)] = bf16_bits(x);
            reinterpret_cast<uint16_t*>(rp + R::kM + R::kPlaneM)[frag_off(t, s, W)] = bf16_bits(y);
        }
        {   // lane-ordered copies: thread (l, e) -> lane l, row t = 4 (l / 16) + e
            const int l = tid >> 2, e = tid & 3, tl = 4 * (l >> 4) + e;
            reinterpret_cast<float*>(rp + R::kEbL)[tid] = expf(bs[tl]);
            reinterpret_cast<float*>(rp + R::kEbwL)[tid] = expf(bs[W - 1] - bs[tl]);
        }
        if (tid == 0) reinterpret_cast<float*>(rp + R::kEbW)[0] = expf(bs[W - 1]);
    }
    __syncthreads();

    // ---- At = (I + Lt)^-1 by forward substitution, one column per thread; then the
    // coefficient matrices Cw = At diag(beta) and Cu = (e^{b_t - b_s}) o Cw
    if (tid < W) {
        float x[W];
#pragma unroll
        for (int r = 0; r < W; ++r) {
            float s = (r == tid) ? 1.f : 0.f;
#pragma unroll
            for (int c = 0; c < r; ++c) s -= Cw[r][c] * x[c];
            x[r] = s;
        }
#pragma unroll
        for (int r = 0; r < W; ++r) Gk[r][tid] = x[r];   // At (Gk is free now)
    }
    __syncthreads();
    {
        const int t = tid / W, s = tid % W;
        const float a = Gk[t][s] * bt[s];
        Cw[t][s] = a;
        Cu[t][s] = s <= t ? a * expf(bs[t] - bs[s]) : 0.f;
    }
    __syncthreads();

    // ---- Wt = Cw K and U = Cu V on MFMA: 16 x 16 times 16 x 16 tiles on v_mfma_f32_16x16x32_bf16
    // with the k-rows 16..31 zero (lanes g >= 2 carry zeros), Cw / Cu split into bf16 hi + lo,
    // K / V exact in bf16 for bf16 inputs (split too for fp32).  One tile (matrix, 16-column
    // block) per wave at a time.  U's accumulator tile is its record's lane order (one 16-byte
    // store per lane); Wt goes to its bf16 hi/lo planes.
    for (int tile = wave; tile < 2 * (D / 16); tile += 4) {
        const bool isu = tile >= D / 16;
        const int cb = isu ? tile - D / 16 : tile;
        const float (*C)[W + 1] = isu ? Cu : Cw;
        const float (*X)[LD] = isu ? Vs : Ks;
        bf16x8 ah, al, bh, bl;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const bool on = g4 < 2;
            const float a = on ? C[n16][8 * g4 + j] : 0.f;
            const float x = on ? X[8 * g4 + j][cb * 16 + n16] : 0.f;
            __bf16 h, l;
            split_bf16(a, h, l);
            ah[j] = h;
            al[j] = l;
            split_bf16(x, h, l);
            bh[j] = h;
            bl[j] = l;
        }
        f32x4 acc = mma_bf16(ah, bh, zero4());
        acc = mma_bf16(al, bh, acc);
        if (!in_bf16) acc = mma_bf16(ah, bl, acc);
        if (isu) {   // block cb, lane (g, n): rows 4g .. 4g+3 of column 16 cb + n
            if (4 * g4 < w) reinterpret_cast<f32x4*>(rp + R::kU)[cb * 64 + lane] = acc;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (4 * g4 + e >= w) continue;
                const int off = frag_off(4 * g4 + e, cb * 16 + n16, D);
                __bf16 h, l;
                split_bf16(acc[e], h, l);
                reinterpret_cast<uint16_t*>(rp + R::kW)[off] = bf16_bits(h);
                reinterpret_cast<uint16_t*>(rp + R::kW + R::kPlaneWD)[off] = bf16_bits(l);
            }
        }
    }
    // ---- q and k planes ([16][D], 8 channels per thread; bf16 q and k are exact in the hi
    // plane, their lo planes are neither written nor read)
    {
        constexpr int CG = D / 8;
        for (int it = tid; it < w * CG; it += 256) {   // (rows past the window are never read)
            const int t = it / CG, c0 = (it % CG) * 8;
            const int off = frag_off(t, c0, D) * 2;
            put_split8(reinterpret_cast<uint16_t*>(rp + R::kQ + off),
                       in_bf16 ? nullptr : reinterpret_cast<uint16_t*>(rp + R::kQ + R::kPlaneWD + off), &Qs[t][c0]);
            put_split8(reinterpret_cast<uint16_t*>(rp + R::kK + off),
                       in_bf16 ? nullptr : reinterpret_cast<uint16_t*>(rp + R::kK + R::kPlaneWD + off), &Ks[t][c0]);
        }
    }
}

hipError_t seam_prep(int d, int n_chain, int n_step, int H, const int64_t* seam_start, int64_t n_tokens,
                     int w, const void* q, const void* k, const void* v, const void* g, const void* beta,
                     bool in_bf16, float scale, void* ws, hipStream_t st, int v_ld)
{
    if (v_ld == 0) v_ld = d;
    const long long n_rec = (long long)n_chain * n_step * H;
    if (n_rec == 0) return hipSuccess;
#define HYPIC_CASE(D_)                                                                                       \
    if (d == D_) {                                                                                           \
        hipLaunchKernelGGL(seam_prep_kernel<D_>, dim3((unsigned)n_rec), dim3(256), 0, st, n_chain * n_step, \
                           H, seam_start, n_tokens, w, q, k, v, g, beta, (int)in_bf16, scale,                \
                           static_cast<unsigned char*>(ws), v_ld);                                           \
        return hipGetLastError();                                                                            \
    }
    HYPIC_CASE(16) HYPIC_CASE(32) HYPIC_CASE(64) HYPIC_CASE(128)
#undef HYPIC_CASE
    return hipErrorNotSupported;
}

size_t seam_record_bytes(int d)
{
    switch (d) {
    case 16: return SeamRec<16>::kBytes;
    case 32: return SeamRec<32>::kBytes;
    case 64: return SeamRec<64>::kBytes;
    case 128: return SeamRec<128>::kBytes;
    default: return 0;
    }
}

}  // namespace hypic
