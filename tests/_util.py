"""Helpers shared by the GPU parity tests (no method arithmetic here)."""
import numpy as np
import torch

T_FLOOR = 1e-30   # below this ||T_ref||_F the T of a pair is not exercised


def dev(x, dtype):
    """numpy -> device tensor; bf16 inputs are exactly representable, so the cast is exact."""
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(device="cuda", dtype=dtype)


def _frag_order(T):
    """[..., d, d] -> [..., d*d] in the SPLIT layout's order: 16 x 8 blocks, row-major."""
    d = T.shape[-1]
    x = T.reshape(*T.shape[:-2], d // 16, 16, d // 8, 8)
    return x.transpose(-3, -2).reshape(*T.shape[:-2], d * d)


def _row_major(P, d):
    """Inverse of _frag_order for a [..., d*d] plane."""
    x = P.reshape(*P.shape[:-1], d // 16, d // 8, 16, 8)
    return x.transpose(-3, -2).reshape(*P.shape[:-1], d, d)


def t_split(T):
    """fp32 T [..., d, d] (numpy or tensor) -> device bf16 SPLIT planes [..., 2, d*d]: hi = bf16(T),
    lo = bf16(T - hi), both round-to-nearest-even (torch's conversion), in fragment order."""
    T = torch.as_tensor(np.ascontiguousarray(T) if isinstance(T, np.ndarray) else T).to("cuda", torch.float32)
    hi = T.to(torch.bfloat16)
    lo = (T - hi.float()).to(torch.bfloat16)
    return torch.stack([_frag_order(hi), _frag_order(lo)], dim=-2).contiguous()


def t_value(T, d=None):
    """A T cache tensor in a dense layout -> float64 numpy [..., d, d] (SPLIT: hi + lo)."""
    if T.dtype == torch.bfloat16:
        d = int(round(T.shape[-1] ** 0.5)) if d is None else d
        hi = _row_major(T[..., 0, :].double(), d)
        lo = _row_major(T[..., 1, :].double(), d)
        return (hi + lo).cpu().numpy()
    return T.double().cpu().numpy()


def in_torch_dtype(W):
    return torch.bfloat16 if W.in_dtype == "bf16" else torch.float32


def workload_tensors(W):
    dt = in_torch_dtype(W)
    out = dict(k=dev(W.k, dt), v=dev(W.v, dt))
    out["g"] = dev(W.g, torch.float32 if W.gate == 0 else dt)
    out["beta"] = dev(W.beta, dt) if W.beta is not None else None
    out["q"] = dev(W.q, dt) if W.q is not None else None
    return out


def rel_f(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.sqrt(np.sum((x - ref) ** 2, axis=(-2, -1)))
    den = np.sqrt(np.sum(ref ** 2, axis=(-2, -1)))
    return num / np.where(den == 0, 1.0, den)


def assert_pairs_close(T, S, T_ref, S_ref, tol, what=""):
    """Per (segment, head) relative Frobenius error <= tol; T below the floor must stay tiny."""
    eS = rel_f(S, S_ref)
    assert np.all(np.isfinite(S)), f"{what}: non-finite S"
    assert eS.max() <= tol, f"{what}: S rel_F max {eS.max():.3e} > {tol:.1e}"
    if T is not None:
        nT = np.sqrt(np.sum(np.asarray(T_ref, dtype=np.float64) ** 2, axis=(-2, -1)))
        nG = np.sqrt(np.sum(np.asarray(T, dtype=np.float64) ** 2, axis=(-2, -1)))
        live = nT >= T_FLOOR
        eT = rel_f(T, T_ref)
        assert np.all(np.isfinite(T)), f"{what}: non-finite T"
        if live.any():
            assert eT[live].max() <= tol, f"{what}: T rel_F max {eT[live].max():.3e} > {tol:.1e}"
        assert np.all(nG[~live] <= 2 * T_FLOOR), f"{what}: T under the floor is not tiny"
        return float(eS.max()), float(eT[live].max()) if live.any() else None
    return float(eS.max()), None
