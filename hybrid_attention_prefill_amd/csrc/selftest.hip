// selftest.hip -- device check of the lane layouts the kernels rely on: the
// operand / result layouts of the three MFMA shapes and the accumulator-to-
// operand cross-lane shuffle.  Every access is inside the 64-lane wave and the
// fixed-size output buffer.
#include "hypic_device.h"
#include "hypic_kernels.h"

namespace hypic {

// out layout (floats), 2112 entries:
//   [0,256)    D (16x16, row-major) of mfma_f32_16x16x32_f16
//   [256,512)  D of mfma_f32_16x16x32_bf16
//   [512,768)  D of mfma_f32_16x16x4f32
//   [768,1280) B fragments made by dtiles_to_bfrag (64 lanes x 8 values)
//   [1280,1536) 16-byte global->LDS loads: lane l fetches in[4 g .. 4 g + 3] with
//              g = (7 l) % 64 and reads back LDS bytes [16 l, 16 l + 16)
//   [1536,1600) 4-byte global->LDS loads: lane l fetches in[(5 l) % 256], reads back [4 l, 4 l + 4)
//   [1600,1856) D of mfma_f32_16x16x16_f16 (A and B the first 16 columns / rows of the above)
//   [1856,2112) D of mfma_f32_16x16x16_f16 with the shuffle's tile0 packed as is as the B
//               operand (the accumulator layout is that operand's layout)
// Operands are filled assuming the documented lane layouts with small integer
// matrices (exact in every type); the host recomputes D = A B and the expected
// shuffle result and compares.
__global__ void selftest_layout_kernel(const float* in, float* out)
{
    __shared__ __attribute__((aligned(16))) float lds16[64 * 4];
    __shared__ __attribute__((aligned(16))) float lds4[64];
    const int l = threadIdx.x;
    const int g4 = l >> 4, n16 = l & 15;
    // A[i][k] = (3i + k) % 7 - 3,  B[k][j] = (5k + 2j) % 5 - 2
    f16x8 ah, bh;
    bf16x8 ab, bb;
    for (int j = 0; j < 8; ++j) {
        const int k = 8 * g4 + j;
        const float a = (float)((n16 * 3 + k) % 7 - 3);
        const float b = (float)((k * 5 + n16 * 2) % 5 - 2);
        ah[j] = (_Float16)a; bh[j] = (_Float16)b;
        ab[j] = (__bf16)a; bb[j] = (__bf16)b;
    }
    f32x4 d = mma_f16(ah, bh, zero4());
    for (int i = 0; i < 4; ++i) out[(4 * g4 + i) * 16 + n16] = d[i];
    d = mma_bf16(ab, bb, zero4());
    for (int i = 0; i < 4; ++i) out[256 + (4 * g4 + i) * 16 + n16] = d[i];
    // f32 16x16x4: A[i][k] with k = l/16 ; B[k][j] with k = l/16
    {
        const float a = (float)((n16 * 3 + g4) % 7 - 3);
        const float b = (float)((g4 * 5 + n16 * 2) % 5 - 2);
        d = mma_f32(a, b, zero4());
        for (int i = 0; i < 4; ++i) out[512 + (4 * g4 + i) * 16 + n16] = d[i];
    }
    // shuffle input: tile0[r][c] = 16 r + c, tile1[r][c] = 256 + 16 r + c (exact in fp16)
    f32x4 t0, t1;
    for (int i = 0; i < 4; ++i) {
        t0[i] = (float)((4 * g4 + i) * 16 + n16);
        t1[i] = (float)(256 + (4 * g4 + i) * 16 + n16);
    }
    unsigned p0, p1, q0, q1;
    pack_f16(t0, p0, p1);
    pack_f16(t1, q0, q1);
    const f16x8 f = as_frag<f16x8>(dtiles_to_bfrag(p0, p1, q0, q1));
    for (int j = 0; j < 8; ++j) out[768 + l * 8 + j] = (float)f[j];
    // global -> LDS direct loads (each lane's destination is implied by its lane id)
    __builtin_amdgcn_global_load_lds(in + ((7 * l) % 64) * 4, (__attribute__((address_space(3))) void*)lds16, 16, 0, 0);
    __builtin_amdgcn_global_load_lds(in + (5 * l) % 256, (__attribute__((address_space(3))) void*)lds4, 4, 0, 0);
    // 16x16x16 f16: A lane l holds A[l%16][4(l/16) + j], B lane l holds B[4(l/16) + j][l%16]
    {
        f16x4 a4, b4;
        for (int j = 0; j < 4; ++j) {
            const int k = 4 * g4 + j;
            a4[j] = (_Float16)(float)((n16 * 3 + k) % 7 - 3);
            b4[j] = (_Float16)(float)((k * 5 + n16 * 2) % 5 - 2);
        }
        d = __builtin_amdgcn_mfma_f32_16x16x16f16(a4, b4, zero4(), 0, 0, 0);
        for (int i = 0; i < 4; ++i) out[1600 + (4 * g4 + i) * 16 + n16] = d[i];
        d = __builtin_amdgcn_mfma_f32_16x16x16f16(a4, __builtin_bit_cast(f16x4, u32x2{p0, p1}), zero4(), 0, 0, 0);
        for (int i = 0; i < 4; ++i) out[1856 + (4 * g4 + i) * 16 + n16] = d[i];
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    for (int j = 0; j < 4; ++j) out[1280 + l * 4 + j] = lds16[l * 4 + j];
    out[1536 + l] = lds4[l];
}

hipError_t selftest_layouts(const float* in, float* out, hipStream_t st)
{
    hipLaunchKernelGGL(selftest_layout_kernel, dim3(1), dim3(64), 0, st, in, out);
    return hipGetLastError();
}

}  // namespace hypic
