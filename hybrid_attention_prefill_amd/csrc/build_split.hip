// build_split.hip -- segment parallelism inside one GPU for the gated-delta-rule build.
//
// A segment's pair is a fold of its pieces' pairs: for consecutive pieces C1, C2 of a
// segment, T(C1 C2) = T(C2) T(C1) and S(C1 C2) = T(C2) S(C1) + S(C2) -- the composition
// law of HYPIC ([ZH] = the Chinese HYPIC page, section 2.1), which its section 2.3 uses to
// build segments in parallel across workers.  Here the workers are the CUs: a long
// segment is one serial chain of 64-token chunks in one workgroup, so the longest
// segment of a prompt sets the build time while other CUs run out of work.  Segments
// longer than kPieceChunks chunks are cut into near-equal pieces on chunk boundaries,
// all pieces are built in one launch, longest first (LPT order), and a fold kernel
// composes each cut segment's pieces.
//
//   plan  (one workgroup): pieces per segment, workspace slots, LPT-ordered items
//   build (build_gdn.hip, items mode): one workgroup per (item, head)
//   fold  : X = [T | S] of the first piece, X <- T_k X + [0 | S_k] for the others
//
// How a segment is cut depends on its own length only, so its pair does not depend on
// the other segments of the call (the build of a range is deterministic).  The
// workspace holds the pairs of every piece after the first (the first is built into the
// caller's slot of the segment); for segments that do not overlap, floor(n_tokens /
// (64 kPieceChunks)) slots always suffice, and a segment whose pieces do not fit is
// built uncut.
#include "hypic_device.h"
#include "hypic_kernels.h"

namespace hypic {

namespace {

constexpr int kChunk = 64;         // tokens per chunk of the GDN build
constexpr int kPieceChunks = 16;   // longest piece, in chunks (segments up to this long are not cut)
constexpr int kBuckets = 64;       // LPT buckets by piece length (the last collects the rest)

struct SplitPlan {
    int64_t* ib;          // [n_items_max] item token range
    int64_t* ie;
    int32_t* out;         // [n_items_max] >= 0: caller's slot; < 0: workspace slot -1 - out
    int32_t* counts;      // [0] items, [1] cut segments
    int4* cut;            // [max_cut] cut segment, pieces, workspace slot of its second piece;
                          // pieces = 0 past the cut segments
    int32_t* npieces;     // [n_seg]
    int32_t* wsbase;      // [n_seg] workspace slot of the segment's second piece
    uint16_t* T_ws;       // [p_ws][H][2][d*d] bf16 hi / lo planes, fragment order
    float* S_ws;          // [p_ws][H][d][d]
};

struct SplitLayout {
    int p_ws = 0, n_items_max = 0, max_cut = 0;
    size_t off_ib = 0, off_ie = 0, off_out = 0, off_cnt = 0, off_cut = 0, off_np = 0, off_wb = 0,
           off_T = 0, off_S = 0, total = 0;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

SplitLayout split_layout(int d, int H, int n_seg, int64_t n_tokens)
{
    SplitLayout L;
    if ((d != 64 && d != 128) || n_seg <= 0 || H <= 0) return L;
    const int64_t p = n_tokens / (int64_t)(kChunk * kPieceChunks);
    if (p <= 0) return L;
    L.p_ws = p > (1 << 24) ? (1 << 24) : (int)p;
    L.n_items_max = n_seg + L.p_ws;
    L.max_cut = n_seg < L.p_ws ? n_seg : L.p_ws;   // a cut segment takes at least one slot
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = align256(o + bytes);
        return at;
    };
    L.off_ib = take(sizeof(int64_t) * L.n_items_max);
    L.off_ie = take(sizeof(int64_t) * L.n_items_max);
    L.off_out = take(sizeof(int32_t) * L.n_items_max);
    L.off_cnt = take(sizeof(int32_t) * 4);
    L.off_cut = take(sizeof(int4) * L.max_cut);
    L.off_np = take(sizeof(int32_t) * n_seg);
    L.off_wb = take(sizeof(int32_t) * n_seg);
    L.off_T = take(sizeof(uint16_t) * 2 * (size_t)L.p_ws * H * d * d);
    L.off_S = take(sizeof(float) * (size_t)L.p_ws * H * d * d);
    L.total = o;
    return L;
}

SplitPlan carve(void* ws, const SplitLayout& L)
{
    char* b = static_cast<char*>(ws);
    SplitPlan p;
    p.ib = reinterpret_cast<int64_t*>(b + L.off_ib);
    p.ie = reinterpret_cast<int64_t*>(b + L.off_ie);
    p.out = reinterpret_cast<int32_t*>(b + L.off_out);
    p.counts = reinterpret_cast<int32_t*>(b + L.off_cnt);
    p.cut = reinterpret_cast<int4*>(b + L.off_cut);
    p.npieces = reinterpret_cast<int32_t*>(b + L.off_np);
    p.wsbase = reinterpret_cast<int32_t*>(b + L.off_wb);
    p.T_ws = reinterpret_cast<uint16_t*>(b + L.off_T);
    p.S_ws = reinterpret_cast<float*>(b + L.off_S);
    return p;
}

__device__ __forceinline__ void clamp_range(int64_t& beg, int64_t& end, int64_t n_tokens) {
    beg = beg < 0 ? 0 : (beg > n_tokens ? n_tokens : beg);
    end = end < beg ? beg : (end > n_tokens ? n_tokens : end);
}

// Exclusive prefix sum over the 1024 threads of the workgroup; returns this thread's
// exclusive value and writes the total to *total (every thread).
__device__ int block_exclusive_scan(int x, int* wsum, int* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int v = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(v, o, 64);
        if (lane >= o) v += y;
    }
    if (lane == 63) wsum[wave] = v;
    __syncthreads();
    if (wave == 0) {   // exclusive scan of the 16 wave totals
        const int t = lane < 16 ? wsum[lane] : 0;
        int u = t;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
            const int y = __shfl_up(u, o, 64);
            if (lane >= o) u += y;
        }
        if (lane < 16) wsum[lane] = u - t;
        if (lane == 15) wsum[16] = u;
    }
    __syncthreads();
    const int r = wsum[wave] + v - x;
    *total = wsum[16];
    __syncthreads();   // wsum is reused by the next call
    return r;
}

__global__ __launch_bounds__(1024) void plan_pieces_kernel(int n_seg, const int64_t* __restrict__ sb,
                                                           const int64_t* __restrict__ se, int64_t n_tokens,
                                                           int p_ws, int max_cut, SplitPlan pl)
{
    __shared__ int hist[kBuckets], off[kBuckets], fill[kBuckets];
    __shared__ int wsum[17];
    __shared__ int ncut;
    const int tid = threadIdx.x;
    if (tid < kBuckets) {
        hist[tid] = 0;
        fill[tid] = 0;
    }
    if (tid == 0) ncut = 0;
    __syncthreads();

    // pieces per segment and the workspace slots of the pieces after the first
    int carry = 0;
    for (int base = 0; base < n_seg; base += 1024) {
        const int i = base + tid;
        int c = 0, n = 1;
        if (i < n_seg) {
            int64_t beg = sb[i], end = se[i];
            clamp_range(beg, end, n_tokens);
            c = (int)((end - beg + kChunk - 1) / kChunk);
            n = c > kPieceChunks ? (c + kPieceChunks - 1) / kPieceChunks : 1;
        }
        int total;
        const int wb = carry + block_exclusive_scan(n - 1, wsum, &total);
        carry += total;
        if (i < n_seg) {
            if (wb + (n - 1) > p_ws) n = 1;   // does not fit: built uncut
            pl.npieces[i] = n;
            pl.wsbase[i] = wb;
            const int bs = c / n, rem = c % n;
            if (rem) atomicAdd(&hist[min(bs + 1, kBuckets - 1)], rem);
            atomicAdd(&hist[min(bs, kBuckets - 1)], n - rem);
        }
    }
    __syncthreads();
    if (tid < 64) {   // longest pieces first: exclusive scan of the buckets from the last
        static_assert(kBuckets == 64, "one lane per bucket");
        const int b = kBuckets - 1 - tid;
        const int t = hist[b];
        int u = t;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(u, o, 64);
            if (tid >= o) u += y;
        }
        off[b] = u - t;
        if (tid == 63) pl.counts[0] = u;
    }
    __syncthreads();

    // items: piece p of a cut segment spans chunks [p bs + min(p, rem), +bs + (p < rem))
    for (int i = tid; i < n_seg; i += 1024) {
        int64_t beg = sb[i], end = se[i];
        clamp_range(beg, end, n_tokens);
        const int c = (int)((end - beg + kChunk - 1) / kChunk);
        const int n = pl.npieces[i], wb = pl.wsbase[i];
        const int bs = c / n, rem = c % n;
        for (int p = 0; p < n; ++p) {
            const int cnt = bs + (p < rem ? 1 : 0);
            const int b = min(cnt, kBuckets - 1);
            const int pos = off[b] + atomicAdd(&fill[b], 1);
            const int64_t t0 = beg + (int64_t)kChunk * (p * bs + min(p, rem));
            const int64_t t1 = min(end, t0 + (int64_t)kChunk * cnt);
            pl.ib[pos] = t0;
            pl.ie[pos] = t1;
            pl.out[pos] = p == 0 ? i : -1 - (wb + p - 1);
        }
        if (n > 1) pl.cut[atomicAdd(&ncut, 1)] = int4{i, n, wb, 0};
    }
    __syncthreads();
    if (tid == 0) pl.counts[1] = ncut;
    for (int j = ncut + tid; j < max_cut; j += 1024) pl.cut[j] = int4{0, 0, 0, 0};
}

// Fold of a cut segment's pieces, one workgroup (8 waves) per (segment, head, 64-column
// block of X = [T | S]): the block starts as the first piece's (in the caller's slot)
// and takes X <- T_k X + [0 | S_k] for the other pieces in order -- the composition law
// of [ZH] 2.1 -- then is written back.  X is re-split into bf16 hi/lo planes in LDS each
// step and T_k is used as cached (bf16 hi/lo planes): hi*hi + hi*lo + lo*hi on
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  Wave w owns row tile w % (d/16) and
// a group of the block's 16-column tiles.  The first step's operands are loaded together
// with the block's initial values.
template <int D>
struct FoldShape {
    static constexpr int NB = 64;               // columns per block
    static constexpr int NBLK = 2 * D / NB;     // blocks of X (T's, then S's)
    static constexpr int RTN = D / 16;          // row tiles
    static constexpr int WPT = 8 / RTN;         // waves per row tile
    static constexpr int CTF = NB / 16 / WPT;   // column tiles per wave
    static constexpr int KS = D / 32, LDB = D + 8;
};

template <int D>
__device__ __forceinline__ void fold_unit(int H, const SplitPlan& pl, void* __restrict__ T_out, int t_split,
                                          float* __restrict__ S_out, UnitSlot us, uint16_t* Rh, uint16_t* Rl)
{
    using F = FoldShape<D>;
    constexpr int NB = F::NB, NBLK = F::NBLK, RTN = F::RTN, CTF = F::CTF, KS = F::KS, LDB = F::LDB;
    const bool is_s = us.sub >= NBLK / 2;
    if (!is_s && T_out == nullptr) return;
    const int4 rec = pl.cut[us.unit / H];
    const int seg = rec.x, n = rec.y, wb = rec.z, h = us.unit % H;
    if (n < 2) return;
    const int col0 = (is_s ? us.sub - NBLK / 2 : us.sub) * NB;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rt = wave % RTN, cg = wave / RTN;
    const int g4 = lane >> 4, n16 = lane & 15;
    const size_t pair = (size_t)seg * H + h;
    auto col_of = [&](int ct) { return col0 + (cg * CTF + ct) * 16 + n16; };

    u32x4 th[KS], tl[KS];
    f32x4 sk[CTF];
    auto load_step = [&](int k) {   // T_k rows of this wave (A fragments); S_k block (S half)
        const size_t wp = (size_t)(wb + k - 1) * H + h;
        const uint16_t* T = pl.T_ws + wp * 2 * D * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int o = frag_off(rt * 16 + n16, ks * 32 + 8 * g4, D);
            th[ks] = *reinterpret_cast<const u32x4*>(T + o);
            tl[ks] = *reinterpret_cast<const u32x4*>(T + D * D + o);
        }
#pragma unroll
        for (int ct = 0; ct < CTF; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sk[ct][e] = is_s ? pl.S_ws[wp * D * D + (size_t)(rt * 16 + 4 * g4 + e) * D + col_of(ct)] : 0.f;
    };
    load_step(1);
    f32x4 acc[CTF];
#pragma unroll
    for (int ct = 0; ct < CTF; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = rt * 16 + 4 * g4 + e;
            acc[ct][e] = is_s ? S_out[pair * D * D + (size_t)row * D + col_of(ct)]
                              : get_t(T_out, t_split, pair, D, row, col_of(ct));
        }
    for (int k = 1; k < n; ++k) {
        if (k > 1) {
            load_step(k);
            __syncthreads();   // the planes' previous readers are done
        }
#pragma unroll
        for (int ct = 0; ct < CTF; ++ct) {
            unsigned h0, h1, l0, l1;
            pack_bf16_split(acc[ct], h0, h1, l0, l1);
            const int o = ((cg * CTF + ct) * 16 + n16) * LDB + rt * 16 + 4 * g4;
            *reinterpret_cast<u32x2*>(Rh + o) = u32x2{h0, h1};
            *reinterpret_cast<u32x2*>(Rl + o) = u32x2{l0, l1};
        }
        __syncthreads();
#pragma unroll
        for (int ct = 0; ct < CTF; ++ct) acc[ct] = sk[ct];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 ah = as_frag<bf16x8>(th[ks]), al = as_frag<bf16x8>(tl[ks]);
#pragma unroll
            for (int ct = 0; ct < CTF; ++ct) {
                const int o = ((cg * CTF + ct) * 16 + n16) * LDB + ks * 32 + 8 * g4;
                const bf16x8 bh = *reinterpret_cast<const bf16x8*>(Rh + o);
                const bf16x8 bl = *reinterpret_cast<const bf16x8*>(Rl + o);
                acc[ct] = mma_bf16(ah, bh, acc[ct]);
                acc[ct] = mma_bf16(ah, bl, acc[ct]);
                acc[ct] = mma_bf16(al, bh, acc[ct]);
            }
        }
    }
#pragma unroll
    for (int ct = 0; ct < CTF; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = rt * 16 + 4 * g4 + e;
            if (is_s) S_out[pair * D * D + (size_t)row * D + col_of(ct)] = acc[ct][e];
            else put_t(T_out, t_split, pair, D, row, col_of(ct), acc[ct][e]);
        }
}


// The grid strides over the (cut segment, head, block) units of this call (the plan's
// count of cut segments): a block's units stay on one XCD, and the blocks of one unit,
// which read the same T_k, are neighbours there.
template <int D>
__global__ __launch_bounds__(512) void fold_pieces_kernel(int H, SplitPlan pl, void* __restrict__ T_out, int t_split,
                                                          float* __restrict__ S_out)
{
    using F = FoldShape<D>;
    __shared__ __attribute__((aligned(16))) uint16_t Rh[F::NB * F::LDB];   // [column][row], bf16 hi
    __shared__ __attribute__((aligned(16))) uint16_t Rl[F::NB * F::LDB];   //                bf16 lo
    const int n_units = pl.counts[1] * H;
    for (int x = blockIdx.x;; x += gridDim.x) {
        const UnitSlot us = xcd_unit_slot(x, F::NBLK);
        if (us.unit >= n_units) return;
        if (x != (int)blockIdx.x) __syncthreads();   // the previous unit's LDS readers are done
        fold_unit<D>(H, pl, T_out, t_split, S_out, us, Rh, Rl);
    }
}

}  // namespace

size_t split_workspace_bytes(int d, int H, int n_seg, int64_t n_tokens)
{
    return split_layout(d, H, n_seg, n_tokens).total;
}

hipError_t build_gdn_split(int d, bool in_bf16, int n_seg, int H, const int64_t* sb, const int64_t* se,
                           int64_t n_tok, const void* k, const void* v, const void* g, const void* beta,
                           void* T_out, bool t_split, float* S_out, void* ws, hipStream_t st)
{
    const SplitLayout L = split_layout(d, H, n_seg, n_tok);
    if (L.total == 0 || ws == nullptr || (long long)L.n_items_max * H > 0x7fffffffLL)
        return build_gdn(d, in_bf16, n_seg, H, sb, se, n_tok, k, v, g, beta, T_out, t_split, S_out, BuildItems{}, BuildOut{}, st);
    const SplitPlan pl = carve(ws, L);
    hipLaunchKernelGGL(plan_pieces_kernel, dim3(1), dim3(1024), 0, st, n_seg, sb, se, n_tok, L.p_ws, L.max_cut, pl);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    BuildItems it;
    it.n_items = pl.counts;
    it.out = pl.out;
    it.T_ws = pl.T_ws;
    it.S_ws = pl.S_ws;
    e = build_gdn(d, in_bf16, L.n_items_max, H, pl.ib, pl.ie, n_tok, k, v, g, beta, T_out, t_split, S_out, it,
                  BuildOut{}, st);
    if (e != hipSuccess) return e;
    // one block per unit up to 1024 blocks (the units of this call are counted on the GPU)
    int grid = xcd_grid_size(L.max_cut * H, 2 * d / 64);
    grid = grid < 1024 ? grid : 1024;
    if (d == 128)
        hipLaunchKernelGGL(fold_pieces_kernel<128>, dim3(grid), dim3(512), 0, st, H, pl, T_out, (int)t_split, S_out);
    else
        hipLaunchKernelGGL(fold_pieces_kernel<64>, dim3(grid), dim3(512), 0, st, H, pl, T_out, (int)t_split, S_out);
    return hipGetLastError();
}

}  // namespace hypic
