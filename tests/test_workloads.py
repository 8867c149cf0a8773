"""Input-recipe checks: determinism, shapes, the 100k-token length mix, bf16 rounding."""
import numpy as np
import pytest
import torch

from hybrid_attention_prefill_amd import workloads as wl


def test_round_bf16_matches_torch_rne():
    x = np.random.default_rng(0).standard_normal(100_000).astype(np.float32) * 3
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0]   # ties
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(wl.round_bf16(x), ref)


def test_deterministic():
    a = wl.make("gdn-16h-d128-32k", n_heads=2, n_seg=2, seg_len=64)
    b = wl.make("gdn-16h-d128-32k", n_heads=2, n_seg=2, seg_len=64)
    for f in ("k", "v", "g", "beta", "q"):
        assert np.array_equal(getattr(a, f), getattr(b, f))


def test_100k_prompt_lengths_and_plan():
    W = wl.make("gdn-16h-d128-100k-seam", n_heads=1, d=16)
    L = W.seg_len
    assert L.sum() == 100_000 and L.min() >= 512 and len(L) == 128
    assert 600 < np.median(L) < 800
    assert W.cold.sum() == 26
    assert W.seam_start[0, 0] == -1
    assert np.array_equal(W.seam_start[0, 1:], W.seg_start[1:-1])
    assert np.array_equal(W.cache_begin[1:], W.seg_start[1:-1] + 8)
    assert W.cache_begin[0] == 0 and np.array_equal(W.cache_end, W.seg_start[1:])


def test_bf16_inputs_are_representable_and_keys_unit():
    W = wl.make("gdn-16h-d128-32k", n_heads=2, n_seg=1, seg_len=256)
    for f in ("k", "v", "g", "beta", "q"):
        x = getattr(W, f)
        assert np.array_equal(wl.round_bf16(x), x)
    nk = np.linalg.norm(W.k.astype(np.float64), axis=-1)
    assert np.all(np.abs(nk - 1) < 2 ** -7)
    assert np.all(W.g <= 0) and np.all((W.beta > 0) & (W.beta < 1))


def test_retnet_decay_stays_fp32():
    W = wl.make("retnet-8h-d64", n_heads=8, n_seg=1, seg_len=16)
    gam = np.exp(W.g.astype(np.float64))
    assert np.all(gam < 1.0)
    assert abs(gam[7] - (1 - 2.0 ** -12)) < 1e-7


@pytest.mark.parametrize("name", ["gdn-tiny-f32", "gdn-16h-d128-32k", "kda-32h-d128-131k"])
def test_stress_gates_mean_total(name):
    kw = dict(n_heads=2, n_seg=4)
    if name != "gdn-tiny-f32":
        kw["seg_len"] = 256
    W = wl.make(name, stress=True, **kw)
    L = int(W.seg_len[0])
    g = W.g.astype(np.float64).reshape(W.n_tokens, -1)
    tot = g.mean() * L      # expected log-decay over one segment
    assert abs(tot + 1.0) < 0.15
    assert W.beta.mean() < 0.05


def test_kda_reuse_plan():
    W = wl.make("kda-32h-d128-131k", n_heads=2, n_seg=4, seg_len=64, n_req=3, n_step=5, n_layers=2)
    assert W.pair_id.shape == (6, 5)
    assert np.all(W.pair_id[:3] < 4) and np.all(W.pair_id[3:] >= 4) and np.all(W.pair_id[3:] < 8)
    assert W.g.shape == (W.n_tokens, 2, 128)
