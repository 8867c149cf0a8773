"""hypic_compose parity with the fp64 oracle (bf16 hi/lo split MFMA)."""
import numpy as np
import pytest
import torch

import oracle
from hybrid_attention_prefill_amd import binding as hb
from _util import dev, rel_f, t_split, t_value

pytestmark = pytest.mark.gpu


def _pairs(seed, n_pair, H, d, t_norm=0.9):
    rng = np.random.default_rng(seed)
    T = rng.standard_normal((n_pair, H, d, d)) / np.sqrt(d)
    T *= t_norm / np.linalg.norm(T, ord=2, axis=(-2, -1))[..., None, None]   # contraction
    S = rng.standard_normal((n_pair, H, d, d))
    return T.astype(np.float32), S.astype(np.float32)


def _t_cache(T, layout):
    """The T cache in `layout` and the T values the oracle composes with."""
    if layout == hb.T_SPLIT:
        Tc = t_split(T)
        return Tc, t_value(Tc)
    return dev(T, torch.float32), T


@pytest.mark.parametrize("layout", [hb.T_DENSE, hb.T_SPLIT])
@pytest.mark.parametrize("d,H,n_chain,n_step", [(16, 1, 1, 2), (16, 3, 2, 9), (64, 8, 1, 16),
                                                (128, 16, 1, 32), (128, 4, 3, 7), (32, 2, 2, 5)])
def test_compose_matches_oracle(d, H, n_chain, n_step, layout):
    print(f"compose d={d} H={H} chains={n_chain} steps={n_step} layout={layout}", flush=True)
    n_pair = 11
    T, S = _pairs(d * 7 + H, n_pair, H, d)
    Tc, Tv = _t_cache(T, layout)
    rng = np.random.default_rng(5)
    ids = rng.integers(-1, n_pair, size=(n_chain, n_step)).astype(np.int32)
    ids[0, 0] = n_pair + 3          # out of range: skipped
    R0 = rng.standard_normal((n_chain, H, d, d)).astype(np.float32)
    ref = oracle.compose(Tv, S, np.where(ids >= n_pair, -1, ids), R0)   # the ABI skips such ids
    Rg = dev(R0, torch.float32)
    hb.compose(Tc, dev(S, torch.float32), dev(ids, torch.int32), Rg)
    torch.cuda.synchronize()
    err = rel_f(Rg.cpu().numpy(), ref)
    assert err.max() < 1e-4, err.max()


@pytest.mark.parametrize("layout", [hb.T_DENSE, hb.T_SPLIT])
@pytest.mark.parametrize("dk,dv", [(16, 128), (32, 64), (64, 16), (128, 32), (128, 64), (64, 128)])
def test_compose_rectangular_state(dk, dv, layout):
    """d_k != d_v: T is d_k x d_k, S and the running state d_k x d_v."""
    print(f"compose dk={dk} dv={dv} layout={layout}", flush=True)
    H, n_chain, n_step, n_pair = 3, 2, 12, 7
    rng = np.random.default_rng(dk * 131 + dv)
    T = rng.standard_normal((n_pair, H, dk, dk)) / np.sqrt(dk)
    T *= 0.9 / np.linalg.norm(T, ord=2, axis=(-2, -1))[..., None, None]
    T = T.astype(np.float32)
    S = rng.standard_normal((n_pair, H, dk, dv)).astype(np.float32)
    Tc, Tv = _t_cache(T, layout)
    ids = rng.integers(-1, n_pair, size=(n_chain, n_step)).astype(np.int32)
    R0 = rng.standard_normal((n_chain, H, dk, dv)).astype(np.float32)
    ref = oracle.compose(Tv, S, ids, R0)
    Rg = dev(R0, torch.float32)
    hb.compose(Tc, dev(S, torch.float32), dev(ids, torch.int32), Rg)
    torch.cuda.synchronize()
    err = rel_f(Rg.cpu().numpy(), ref)
    assert err.max() < 1e-4, err.max()


@pytest.mark.parametrize("layout", [hb.T_DENSE, hb.T_SPLIT])
def test_compose_many_chains_full_width(layout):
    """Enough (chain, head) units for the full-width column block (the batched path)."""
    d, H, n_chain, n_step, n_pair = 128, 16, 64, 3, 5
    print("compose many chains", layout, flush=True)
    T, S = _pairs(3, n_pair, H, d)
    Tc, Tv = _t_cache(T, layout)
    rng = np.random.default_rng(6)
    ids = rng.integers(0, n_pair, size=(n_chain, n_step)).astype(np.int32)
    R0 = np.zeros((n_chain, H, d, d), dtype=np.float32)
    Rg = dev(R0, torch.float32)
    hb.compose(Tc, dev(S, torch.float32), dev(ids, torch.int32), Rg)
    torch.cuda.synchronize()
    got = Rg.cpu().numpy()
    sample = [0, 17, 63]
    ref = oracle.compose(Tv, S, ids[sample], R0[sample])
    assert rel_f(got[sample], ref).max() < 1e-4


@pytest.mark.parametrize("layout", [hb.T_DENSE, hb.T_SPLIT])
def test_compose_identity_T_is_plain_sum(layout):
    d, H = 64, 2
    rng = np.random.default_rng(8)
    T = np.broadcast_to(np.eye(d, dtype=np.float32), (3, H, d, d)).copy()
    S = rng.standard_normal((3, H, d, d)).astype(np.float32)
    R0 = rng.standard_normal((1, H, d, d)).astype(np.float32)
    Rg = dev(R0, torch.float32)
    hb.compose(_t_cache(T, layout)[0], dev(S, torch.float32), dev(np.array([[0, 1, 2]], np.int32), torch.int32), Rg)
    torch.cuda.synchronize()
    ref = R0[0].astype(np.float64) + S.astype(np.float64).sum(axis=0)
    assert rel_f(Rg.cpu().numpy()[0], ref).max() < 1e-5


@pytest.mark.parametrize("n_step", [5, 21])
def test_compose_scalar_T(n_step):
    """Scalar T (steps taken in groups of 8 by the kernel: 5 and 21 cover a partial group
    and several), a skipped step and a repeated pair."""
    d, H = 64, 8
    rng = np.random.default_rng(9 + n_step)
    t = rng.uniform(0.5, 1.0, size=(6, H)).astype(np.float32)
    S = rng.standard_normal((6, H, d, d)).astype(np.float32)
    ids = np.array([[0, 1, -1, 5, 2]], np.int32) if n_step == 5 else rng.integers(-1, 6, size=(1, n_step)).astype(np.int32)
    ref = oracle.compose(t, S, ids, t_scalar=True)
    Rg = torch.zeros((1, H, d, d), device="cuda")
    hb.compose(dev(t, torch.float32), dev(S, torch.float32), dev(ids, torch.int32), Rg, t_layout=hb.T_SCALAR)
    torch.cuda.synchronize()
    assert rel_f(Rg.cpu().numpy(), ref).max() < 1e-6


@pytest.mark.parametrize("layout", [hb.T_DENSE, hb.T_SPLIT])
@pytest.mark.parametrize("n_chain,H", [(3, 2), (64, 16)])
def test_compose_long_chain_ring_refill(layout, n_chain, H):
    """Chains of 800 steps: the kernel's LDS ring of pair ids is refilled at steps 256, 512
    and 768, and runs of skipped ids end right before those points (the waves then meet at
    no step for a while).  Few chains run the narrow column blocks, 64 x 16 (chain, head)
    units the full-width ones; the latter are checked on sampled chains."""
    d, n_step, n_pair = 128, 800, 9
    print(f"compose long chain chains={n_chain} H={H} layout={layout}", flush=True)
    T, S = _pairs(41 + H, n_pair, H, d)
    Tc, Tv = _t_cache(T, layout)
    rng = np.random.default_rng(42)
    ids = rng.integers(0, n_pair, size=(n_chain, n_step)).astype(np.int32)
    for r in (256, 512, 768):
        ids[:, r - 7:r] = -1
        ids[::2, r - 1] = -1
        ids[1::2, r - 1] = 3
    ids[-1, 250:520] = -1
    R0 = rng.standard_normal((n_chain, H, d, d)).astype(np.float32)
    Rg = dev(R0, torch.float32)
    hb.compose(Tc, dev(S, torch.float32), dev(ids, torch.int32), Rg)
    torch.cuda.synchronize()
    got = Rg.cpu().numpy()
    sample = list(range(n_chain)) if n_chain <= 4 else [0, 1, 30, n_chain - 1]
    ref = oracle.compose_gemm(Tv, S, ids[sample], R0[sample])
    err = rel_f(got[sample], ref)
    print(f"  max rel_F {err.max():.2e}", flush=True)
    assert err.max() < 1e-4, err.max()
