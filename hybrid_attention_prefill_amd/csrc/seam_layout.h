// seam_layout.h -- per-(chain, step, head) record of the seam workspace.
#pragma once

namespace hypic {

constexpr int kSeamMaxW = 16;  // windows are padded to 16 tokens

template <int D>
struct SeamRec {
    static constexpr int kWt = 0;                       // [16][D]  At diag(beta) K
    static constexpr int kU = kWt + kSeamMaxW * D;      // [16][D]  A diag(beta) V
    static constexpr int kMo = kU + kSeamMaxW * D;      // [16][16] output mixing matrix
    static constexpr int kEb = kMo + kSeamMaxW * kSeamMaxW;  // [16] e^{b_t}
    static constexpr int kEbw = kEb + kSeamMaxW;        // [16] e^{b_w - b_t}
    static constexpr int kEbW = kEbw + kSeamMaxW;       // [1]  e^{b_w}
    static constexpr int kKt = kEbW + 4;                // [D][16] window keys, channel-major (K^T)
    static constexpr int kFloats = (kKt + D * kSeamMaxW + 63) / 64 * 64;  // 256-byte records
};

}  // namespace hypic
