// seam_layout.h -- per-(chain, step, head) record of the seam workspace.
//
// Every matrix the chain kernel feeds to the MFMA units is stored as two bf16
// planes, hi = bf16(x) and lo = bf16(x - hi), in fragment order (frag_off in
// hypic_device.h): one contiguous 16-byte load per lane is one operand fragment,
// and the chain kernel (seam_chain.hip) does no conversions.
#pragma once

namespace hypic {

constexpr int kSeamMaxW = 16;  // windows are padded to 16 tokens; the rows of tokens w .. 15 of
                                // the W, q, k, Mo and U parts are neither written nor read (the
                                // chain kernel keeps zeros in their place)

template <int D>
struct SeamRec {
    static constexpr int kPlaneWD = kSeamMaxW * D * 2;          // bytes of one [16][D] bf16 plane
    static constexpr int kW = 0;                                // [2][16][D] bf16  Wt = At diag(beta) K
    static constexpr int kQ = kW + 2 * kPlaneWD;                // [2][16][D] bf16  q (unscaled)
    static constexpr int kK = kQ + 2 * kPlaneWD;                // [2][16][D] bf16  k (token-major)
    static constexpr int kM = kK + 2 * kPlaneWD;                // [2][16][16] bf16 output mixing matrix Mo
    static constexpr int kPlaneM = kSeamMaxW * kSeamMaxW * 2;
    // Dword data in the D-fragment lane order of a 16 x 16 tile (lane l = 16 g + n holds
    // rows 4g .. 4g+3 of column n), so each wave fetches it with one 16-byte load per lane:
    static constexpr int kU = kM + 2 * kPlaneM;                 // [D/16][64][4] f32  U = A diag(beta) V,
                                                                //   block cb, lane (g, n): U[4g+e][16 cb + n]
    static constexpr int kEbL = kU + kSeamMaxW * D * 4;         // [64][4] f32  lane (g, n): e^{b_t}, t = 4g+e
    static constexpr int kEbwL = kEbL + 64 * 16;                // [64][4] f32  lane (g, n): e^{b_w - b_t}
    static constexpr int kEbW = kEbwL + 64 * 16;                // [1]  f32  e^{b_w}
    static constexpr int kBytes = (kEbW + 16 + 255) / 256 * 256;  // 256-byte records
};

}  // namespace hypic
