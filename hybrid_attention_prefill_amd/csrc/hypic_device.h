// hypic_device.h -- device helpers shared by the gfx950 kernels of libhypic.
//
// MFMA shapes used (CDNA4, wave64):
//   v_mfma_f32_16x16x32_f16 / _bf16 : D(16x16,f32) += A(16x32) B(32x16)
//     A: lane l holds A[l%16][8*(l/16) + j], j = 0..7
//     B: lane l holds B[8*(l/16) + j][l%16], j = 0..7
//     D: lane l holds D[4*(l/16) + i][l%16], i = 0..3
//   v_mfma_f32_16x16x16_f16 : D(16x16,f32) += A(16x16) B(16x16)
//     A: lane l holds A[l%16][4*(l/16) + j], j = 0..3
//     B: lane l holds B[4*(l/16) + j][l%16]  (the D layout: a D tile packed to fp16 is a B operand)
//   v_mfma_f32_16x16x4_f32 : D(16x16) += A(16x4) B(4x16)
//     A: lane l holds A[l%16][l/16];  B: lane l holds B[l/16][l%16]
// These lane layouts are checked on the device by the test-suite.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hypic {

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

__device__ __forceinline__ f32x4 mma_f16(const f16x8& a, const f16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_f32(float a, float b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ---- scalar conversions -------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(((unsigned)b) << 16);
}
__device__ __forceinline__ uint16_t f16_bits(_Float16 h) { return __builtin_bit_cast(uint16_t, h); }
__device__ __forceinline__ uint16_t bf16_bits(__bf16 h) { return __builtin_bit_cast(uint16_t, h); }

// Round x to the operand type; `lo` receives the rounded remainder (3-term split).
__device__ __forceinline__ void split_f16(float x, _Float16& hi, _Float16& lo) {
    hi = (_Float16)x;
    lo = (_Float16)(x - (float)hi);
}
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
    hi = (__bf16)x;
    lo = (__bf16)(x - (float)hi);
}

// Pack two 16-bit values (low = a) into a dword.
__device__ __forceinline__ unsigned pack2(uint16_t a, uint16_t b) {
    return (unsigned)a | ((unsigned)b << 16);
}

// ---- accumulator tiles -> B operand (k = accumulator rows) -----------------------
// Two D tiles d0 (rows 0..15) and d1 (rows 16..31) of the same 16 columns, each
// already packed to 16-bit pairs per lane (p0 = rows 4g,4g+1; p1 = rows 4g+2,4g+3
// of tile 0; q0, q1 the same for tile 1), become the B fragment of the 32-row
// k-block: lane (g, n) receives rows 8g .. 8g+7 of column n.  Two cross-lane
// swaps: lanes 32..63 of the tile-0 words trade with lanes 0..31 of the tile-1
// words, then odd 16-lane rows of the first word trade with even rows of the
// second.
__device__ __forceinline__ u32x4 dtiles_to_bfrag(unsigned p0, unsigned p1, unsigned q0, unsigned q1) {
    auto s0 = __builtin_amdgcn_permlane32_swap(p0, q0, false, false);
    auto s1 = __builtin_amdgcn_permlane32_swap(p1, q1, false, false);
    // s0[0] = new p0 (tile0 rows 0-7 in lanes 0-31, tile1 rows 0-7 in lanes 32-63)
    // s0[1] = new q0 (tile0 rows 8-15 in lanes 0-31, tile1 rows 8-15 in lanes 32-63)
    auto t0 = __builtin_amdgcn_permlane16_swap(s0[0], s0[1], false, false);
    auto t1 = __builtin_amdgcn_permlane16_swap(s1[0], s1[1], false, false);
    return u32x4{t0[0], t1[0], t0[1], t1[1]};
}

template <typename T8>
__device__ __forceinline__ T8 as_frag(const u32x4& u) { return __builtin_bit_cast(T8, u); }

// Pack the 4 floats of a D tile lane into two 16-bit pairs of the operand type.  The
// pairs are converted together (round to nearest even, one v_cvt_pk_f16_f32 or
// v_cvt_pk_bf16_f32 per pair on gfx950); _split also returns the rounded remainders
// lo = x - hi (exact in fp32), rounded the same way.
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
__device__ __forceinline__ unsigned cvt2_f16(float a, float b) {
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{a, b}, f16x2));
}
__device__ __forceinline__ unsigned cvt2_bf16(float a, float b) {
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ f32x2 f16x2_to_f32(unsigned w) {
    return __builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2);
}
__device__ __forceinline__ f32x2 bf16x2_to_f32(unsigned w) {
    return f32x2{__uint_as_float(w << 16), __uint_as_float(w & 0xFFFF0000u)};
}
__device__ __forceinline__ void pack_f16(const f32x4& d, unsigned& w0, unsigned& w1) {
    w0 = cvt2_f16(d[0], d[1]);
    w1 = cvt2_f16(d[2], d[3]);
}
// x - (low / high fp16 half of w), exact (x - hi of x's fp16 rounding is representable in
// fp32), in one v_fma_mix_f32 that reads the fp16 operand in place
__device__ __forceinline__ float sub_f16_lo(unsigned w, float x) {
    float r;
    asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(w), "v"(x));
    return r;
}
__device__ __forceinline__ float sub_f16_hi(unsigned w, float x) {
    float r;
    asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(w), "v"(x));
    return r;
}
__device__ __forceinline__ void pack_f16_split(const f32x4& d, unsigned& h0, unsigned& h1,
                                               unsigned& l0, unsigned& l1) {
    h0 = cvt2_f16(d[0], d[1]);
    h1 = cvt2_f16(d[2], d[3]);
    l0 = cvt2_f16(sub_f16_lo(h0, d[0]), sub_f16_hi(h0, d[1]));
    l1 = cvt2_f16(sub_f16_lo(h1, d[2]), sub_f16_hi(h1, d[3]));
}
__device__ __forceinline__ void pack_bf16_split(const f32x4& d, unsigned& h0, unsigned& h1,
                                                unsigned& l0, unsigned& l1) {
    h0 = cvt2_bf16(d[0], d[1]);
    h1 = cvt2_bf16(d[2], d[3]);
    const f32x2 b0 = bf16x2_to_f32(h0), b1 = bf16x2_to_f32(h1);
    l0 = cvt2_bf16(d[0] - b0.x, d[1] - b0.y);
    l1 = cvt2_bf16(d[2] - b1.x, d[3] - b1.y);
}

// ---- fragment-ordered bf16 planes ---------------------------------------------
// A d_r x d_c matrix stored as [d_r/16][d_c/8][16][8] (16 x 8 blocks, row-major in a
// block, blocks row-major): the A operand of v_mfma_f32_16x16x32_bf16 for row tile rt
// and k-block ks -- lane l holding row rt*16 + l%16, columns ks*32 + 8(l/16) .. +7 --
// is then the 1 KiB at element (rt*(d_c/8) + ks*4)*128 + 8 l, one contiguous load.
__device__ __forceinline__ int frag_off(int row, int col, int dc) {
    return ((row >> 4) * (dc >> 3) + (col >> 3)) * 128 + (row & 15) * 8 + (col & 7);
}

// ---- one entry of a dense T in the cache: fp32 [pair][d][d] row-major, or (split)
// two bf16 planes [pair][2][d*d], hi = bf16(x) and lo = bf16(x - hi), fragment-ordered.
__device__ __forceinline__ void put_t(void* T, bool split, size_t pair, int d, int row, int col, float x) {
    const int dd = d * d;
    if (split) {
        __bf16 hi, lo;
        split_bf16(x, hi, lo);
        uint16_t* P = reinterpret_cast<uint16_t*>(T) + pair * 2 * dd;
        const int off = frag_off(row, col, d);
        P[off] = bf16_bits(hi);
        P[dd + off] = bf16_bits(lo);
    } else {
        reinterpret_cast<float*>(T)[pair * dd + (size_t)row * d + col] = x;
    }
}

// the inverse of put_t: one entry of a dense T (split: hi + lo)
__device__ __forceinline__ float get_t(const void* T, bool split, size_t pair, int d, int row, int col) {
    const int dd = d * d;
    if (split) {
        const uint16_t* P = reinterpret_cast<const uint16_t*>(T) + pair * 2 * dd;
        const int off = frag_off(row, col, d);
        return bf16_bits_to_f32(P[off]) + bf16_bits_to_f32(P[dd + off]);
    }
    return reinterpret_cast<const float*>(T)[pair * dd + (size_t)row * d + col];
}

// ---- workgroup barrier for LDS traffic only ------------------------------------
// Waits for this wave's LDS operations (lgkmcnt = 0), then s_barrier.  Unlike
// __syncthreads() it does not wait for outstanding vector-memory loads, so loads
// issued ahead of time (into registers, or global->LDS direct loads that only the
// issuing wave reads back) stay in flight across it.  The empty asm statements
// keep the compiler from moving memory accesses across the barrier.
// s_waitcnt immediate: vmcnt = 63 (unconstrained), expcnt = 7, lgkmcnt = 0.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// ---- grid -> XCD-aware unit mapping --------------------------------------------
// Workgroups are dispatched round-robin over the 8 XCDs (workgroup x runs on XCD
// x % 8).  Units are dealt to XCDs round-robin and the `nsub` workgroups of one
// unit are kept on the same XCD, so they share that XCD's L2.
struct UnitSlot { int unit, sub; };
__device__ __forceinline__ UnitSlot xcd_unit_slot(int x, int nsub) {
    const int xcd = x & 7, li = x >> 3;
    return UnitSlot{(li / nsub) * 8 + xcd, li % nsub};
}
static inline int xcd_grid_size(int n_units, int nsub) { return ((n_units + 7) / 8) * 8 * nsub; }

}  // namespace hypic
