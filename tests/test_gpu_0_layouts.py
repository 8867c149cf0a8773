"""Device check of the MFMA lane layouts and the accumulator->operand lane
shuffle that every kernel relies on (expected values recomputed on the host)."""
import numpy as np
import pytest

from hybrid_attention_prefill_amd import binding as hb


@pytest.mark.gpu
def test_mfma_layouts_and_shuffle():
    print("selftest_layouts", flush=True)
    out = hb.selftest_layouts()
    i = np.arange(16)[:, None]
    k32 = np.arange(32)[None, :]
    A = ((3 * i + k32) % 7 - 3).astype(np.float64)                       # 16 x 32
    B = ((5 * np.arange(32)[:, None] + 2 * np.arange(16)[None, :]) % 5 - 2).astype(np.float64)
    D = A @ B
    np.testing.assert_array_equal(out[0:256].reshape(16, 16), D)          # f16
    np.testing.assert_array_equal(out[256:512].reshape(16, 16), D)        # bf16
    A4 = ((3 * i + np.arange(4)[None, :]) % 7 - 3).astype(np.float64)
    B4 = ((5 * np.arange(4)[:, None] + 2 * np.arange(16)[None, :]) % 5 - 2).astype(np.float64)
    np.testing.assert_array_equal(out[512:768].reshape(16, 16), A4 @ B4)  # f32
    frag = out[768:1280].reshape(64, 8)
    exp = np.empty((64, 8))
    for lane in range(64):
        g, n = lane // 16, lane % 16
        for j in range(8):
            row = 8 * g + j
            exp[lane, j] = row * 16 + n if row < 16 else 256 + (row - 16) * 16 + n
    np.testing.assert_array_equal(frag, exp)
    # global -> LDS direct loads: lane l's bytes land at LDS offset (size * l)
    lane = np.arange(64)
    g = (7 * lane) % 64
    np.testing.assert_array_equal(out[1280:1536].reshape(64, 4), (4 * g)[:, None] + np.arange(4)[None, :])
    np.testing.assert_array_equal(out[1536:1600], (5 * lane) % 256)
    # v_mfma_f32_16x16x16_f16, and a packed accumulator tile used directly as its B operand
    np.testing.assert_array_equal(out[1600:1856].reshape(16, 16), A[:, :16] @ B[:16, :])
    tile0 = np.arange(16)[:, None] * 16 + np.arange(16)[None, :]
    np.testing.assert_array_equal(out[1856:2112].reshape(16, 16), A[:, :16] @ tile0)
