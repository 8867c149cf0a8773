// build_common.h -- device helpers shared by the chunked build kernels.
#pragma once
#include "hypic_device.h"

namespace hypic {
namespace bld {

// fp32 16x16 block product on MFMA: returns A(16x16) B(16x16), D layout.
// An empty asm that "modifies" x: values derived from it inside a loop body are
// recomputed each iteration instead of being hoisted (and then spilled) by the compiler.
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

// A 16 x 16 block in the accumulator layout of v_mfma_f32_16x16x16_f16 (lane (g4, n16): rows
// 4 g4 .. 4 g4 + 3 of column n16) as fp16 hi / lo operand bits: the B operand of that product,
// or the A operand of the transposed block.
struct Hl16 {
    u32x2 h, l;
};
__device__ __forceinline__ Hl16 hl16(const f32x4& x) {
    unsigned a, b, c, d;
    pack_f16_split(x, a, b, c, d);
    return Hl16{u32x2{a, b}, u32x2{c, d}};
}
// 16 x 16 x 16 product with fp16 hi / lo operands (three products; lo x lo dropped)
__device__ __forceinline__ f32x4 mma16(const u32x2& ah, const u32x2& al, const u32x2& bh, const u32x2& bl, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, ah), __builtin_bit_cast(f16x4, bh), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, ah), __builtin_bit_cast(f16x4, bl), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, al), __builtin_bit_cast(f16x4, bh), c, 0, 0, 0);
    return c;
}
__device__ __forceinline__ f32x4 mm16(const Hl16& a, const Hl16& b) { return mma16(a.h, a.l, b.h, b.l, zero4()); }

// (I - N)^-1 for a strictly lower 16 x 16 block N (N^16 = 0), given N and N^T in the
// accumulator layout; returns the inverse transposed, in the accumulator layout:
//   (I - N)^-1 = P1 (I + N^4)(I + N^8),   P1 = (I + N)(I + N^2) = I + N + N^2 + N^3,
// formed transposed, Y^T = (I + N^8)^T (I + N^4)^T P1^T, as 16 x 16 products on MFMA (fp16
// hi / lo operands) with each identity term as a product's fp32 accumulator input.  A
// product's A operand is the accumulator layout of the transposed factor, so N and N^T are
// carried along.
__device__ __forceinline__ f32x4 inv16_t(const f32x4& nd, const f32x4& nt, int g4, int n16) {
    const Hl16 n1 = hl16(nd), n1t = hl16(nt);
    const f32x4 n2 = mm16(n1t, n1), n2t = mm16(n1, n1t);                    // N^2, (N^2)^T
    const Hl16 q2 = hl16(n2), q2t = hl16(n2t);
    f32x4 c1;   // I + N^T + (N^2)^T
#pragma unroll
    for (int e = 0; e < 4; ++e) c1[e] = nt[e] + n2t[e] + ((4 * g4 + e == opaque(n16)) ? 1.f : 0.f);   // (formed here, not kept)
    const f32x4 n4 = mm16(q2t, q2), n4t = mm16(q2, q2t);                    // N^4, (N^4)^T
    const f32x4 p1t = mma16(q2.h, q2.l, n1t.h, n1t.l, c1);                  // P1^T = c1 + (N^2)^T N^T
    const Hl16 q4 = hl16(n4), q4t = hl16(n4t), r1t = hl16(p1t);
    const f32x4 n8 = mm16(q4t, q4);                                         // N^8
    const f32x4 p2t = mma16(q4.h, q4.l, r1t.h, r1t.l, p1t);                 // (P1 (I + N^4))^T
    const Hl16 q8 = hl16(n8), r2t = hl16(p2t);
    return mma16(q8.h, q8.l, r2t.h, r2t.l, p2t);
}

__device__ __forceinline__ f32x4 mm16_f32(const float* A, int lda, const float* B, int ldb, int lane) {
    const int g4 = lane >> 4, n16 = lane & 15;
    f32x4 acc = zero4();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
        acc = mma_f32(A[n16 * lda + kb * 4 + g4], B[(kb * 4 + g4) * ldb + n16], acc);
    return acc;
}
__device__ __forceinline__ void st16_f32(float* dst, int ld, const f32x4& v, int lane, float sgn) {
    const int g4 = lane >> 4, n16 = lane & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[(4 * g4 + i) * ld + n16] = sgn * v[i];
}

template <int NSPLIT>
struct Frag;
template <>
struct Frag<1> {
    f16x8 h;
};
template <>
struct Frag<2> {
    f16x8 h, l;
};

// Load an operand fragment: 8 consecutive 16-bit values at row `row`, column `col`
// of each plane of a [NSPLIT][rows][LD] LDS array.
template <int NSPLIT, typename Arr>
__device__ __forceinline__ Frag<NSPLIT> frag_at(const Arr& a, int row, int col) {
    Frag<NSPLIT> f;
    f.h = *reinterpret_cast<const f16x8*>(&a[0][row][col]);
    if constexpr (NSPLIT == 2) f.l = *reinterpret_cast<const f16x8*>(&a[1][row][col]);
    return f;
}

template <int NSPLIT>
__device__ __forceinline__ f32x4 mma(const Frag<NSPLIT>& a, const Frag<NSPLIT>& b, f32x4 c) {
    c = mma_f16(a.h, b.h, c);
    if constexpr (NSPLIT == 2) {
        c = mma_f16(a.h, b.l, c);
        c = mma_f16(a.l, b.h, c);
    }
    return c;
}

// Two accumulator tiles (rows 0..15, 16..31 of a 32-row k-block) -> B fragment.
template <int NSPLIT>
__device__ __forceinline__ Frag<NSPLIT> dpair_to_frag(const f32x4& d0, const f32x4& d1) {
    Frag<NSPLIT> f;
    if constexpr (NSPLIT == 1) {
        unsigned p0, p1, q0, q1;
        pack_f16(d0, p0, p1);
        pack_f16(d1, q0, q1);
        f.h = as_frag<f16x8>(dtiles_to_bfrag(p0, p1, q0, q1));
    } else {
        unsigned p0, p1, pl0, pl1, q0, q1, ql0, ql1;
        pack_f16_split(d0, p0, p1, pl0, pl1);
        pack_f16_split(d1, q0, q1, ql0, ql1);
        f.h = as_frag<f16x8>(dtiles_to_bfrag(p0, p1, q0, q1));
        f.l = as_frag<f16x8>(dtiles_to_bfrag(pl0, pl1, ql0, ql1));
    }
    return f;
}

// bf16 hi + lo operand fragment (three-product split on v_mfma_f32_16x16x32_bf16).
struct FragB {
    bf16x8 h, l;
};
__device__ __forceinline__ FragB fragb_at(const uint16_t* hi, const uint16_t* lo, int ld, int row, int col) {
    FragB f;
    f.h = *reinterpret_cast<const bf16x8*>(hi + row * ld + col);
    f.l = *reinterpret_cast<const bf16x8*>(lo + row * ld + col);
    return f;
}
__device__ __forceinline__ f32x4 mma3(const FragB& a, const FragB& b, f32x4 c) {
    c = mma_bf16(a.h, b.h, c);
    c = mma_bf16(a.h, b.l, c);
    c = mma_bf16(a.l, b.h, c);
    return c;
}
__device__ __forceinline__ FragB dpair_to_fragb(const f32x4& d0, const f32x4& d1) {
    unsigned p0, p1, pl0, pl1, q0, q1, ql0, ql1;
    pack_bf16_split(d0, p0, p1, pl0, pl1);
    pack_bf16_split(d1, q0, q1, ql0, ql1);
    FragB f;
    f.h = as_frag<bf16x8>(dtiles_to_bfrag(p0, p1, q0, q1));
    f.l = as_frag<bf16x8>(dtiles_to_bfrag(pl0, pl1, ql0, ql1));
    return f;
}
__device__ __forceinline__ void put_bf16_split(uint16_t* hi, uint16_t* lo, float x) {
    __bf16 a, b;
    split_bf16(x, a, b);
    *hi = bf16_bits(a);
    *lo = bf16_bits(b);
}

template <int NSPLIT>
__device__ __forceinline__ void put16(uint16_t* hi, uint16_t* lo, float x) {
    if constexpr (NSPLIT == 1) {
        *hi = f16_bits((_Float16)x);
    } else {
        _Float16 a, b;
        split_f16(x, a, b);
        *hi = f16_bits(a);
        *lo = f16_bits(b);
    }
}

template <bool BF16>
__device__ __forceinline__ void load8(const void* base, size_t elem, float out[8]) {
    if constexpr (BF16) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(base) + elem);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            out[2 * e] = __uint_as_float(w[e] << 16);
            out[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
        }
    } else {
        const f32x4* p = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(base) + elem);
        const f32x4 a = p[0], b = p[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) { out[e] = a[e]; out[4 + e] = b[e]; }
    }
}
template <bool BF16>
__device__ __forceinline__ float load1(const void* base, size_t elem) {
    if constexpr (BF16) return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[elem]);
    else return reinterpret_cast<const float*>(base)[elem];
}

}  // namespace bld
}  // namespace hypic
