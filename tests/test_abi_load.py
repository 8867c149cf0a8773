"""The C-ABI library loads, exports every symbol include/hypic.h declares, and
rejects bad arguments before any launch (no GPU needed for these paths)."""
import ctypes
import os
import re

import pytest

from hybrid_attention_prefill_amd import binding as hb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hypic.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(hypic_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(hb.LIB_PATH):
        pytest.fail("libhypic.so is not built (python -m hybrid_attention_prefill_amd.build_lib)")
    return hb.load_library()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert {"hypic_segment_build", "hypic_compose", "hypic_seam_advance"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(hb.EXPORTED) == set(names)


def test_abi_version(lib):
    src = open(HEADER).read()
    v = int(re.search(r"#define HYPIC_ABI_VERSION (\d+)", src).group(1))
    assert hb.abi_version() == v


def _dims(**kw):
    base = dict(H=2, dk=16, dv=16, gate=hb.GATE_TOKEN, delta=1, in_dtype=hb.F32, t_layout=hb.T_DENSE)
    base.update(kw)
    return hb.make_dims(base["H"], base["dk"], base["dv"], gate=base["gate"], delta=base["delta"],
                        in_dtype=base["in_dtype"], t_layout=base["t_layout"])


@pytest.mark.parametrize("bad", [dict(H=0), dict(dk=24), dict(dv=256), dict(gate=3), dict(in_dtype=7),
                                 dict(t_layout=1), dict(t_layout=1, delta=0, gate=hb.GATE_DIAG), dict(t_layout=3),
                                 dict(t_layout=3, gate=hb.GATE_DIAG), dict(t_layout=3, delta=0),
                                 dict(t_layout=4), dict(t_layout=-1), dict(delta=3), dict(delta=-1),
                                 dict(t_layout=3, gate=hb.GATE_DIAG, delta=2)])
def test_invalid_dims_rejected(lib, bad):
    d = _dims(**bad)
    st = lib.hypic_compose(ctypes.byref(d), 1, 1, None, 0, None, None, None, None)
    assert st == hb.HYPIC_E_INVALID
    assert lib.hypic_last_error().decode()


@pytest.mark.parametrize("ok", [dict(t_layout=hb.T_SCALAR, gate=hb.GATE_HEAD, delta=0),
                                dict(t_layout=hb.T_SCALAR, gate=hb.GATE_TOKEN, delta=0),
                                dict(t_layout=hb.T_DIAG, gate=hb.GATE_DIAG, delta=0),
                                dict(t_layout=hb.T_SPLIT, gate=hb.GATE_DIAG, delta=0),
                                dict(t_layout=hb.T_SPLIT, gate=hb.GATE_DIAG, delta=2),
                                dict(t_layout=hb.T_DENSE, gate=hb.GATE_TOKEN, delta=2)])
def test_valid_layout_gate_pairs_accepted(lib, ok):
    d = _dims(**ok)
    assert lib.hypic_compose(ctypes.byref(d), 0, 1, None, 0, None, None, None, None) == hb.HYPIC_OK


def test_null_pointers_rejected(lib):
    d = _dims()
    assert lib.hypic_compose(None, 1, 1, None, 0, None, None, None, None) == hb.HYPIC_E_INVALID
    assert lib.hypic_compose(ctypes.byref(d), 1, 1, None, 1, None, None, None, None) == hb.HYPIC_E_INVALID
    assert lib.hypic_segment_build(ctypes.byref(d), 2, None, None, 10, None, None, None, None, None, None,
                                   None, 0, None) == hb.HYPIC_E_INVALID
    assert lib.hypic_segment_build(ctypes.byref(d), -1, None, None, 10, None, None, None, None, None, None,
                                   None, 0, None) == hb.HYPIC_E_INVALID


def test_empty_work_is_ok(lib):
    d = _dims()
    assert lib.hypic_compose(ctypes.byref(d), 0, 5, None, 0, None, None, None, None) == hb.HYPIC_OK
    assert lib.hypic_segment_build(ctypes.byref(d), 0, None, None, 0, None, None, None, None, None, None,
                                   None, 0, None) == hb.HYPIC_OK


def test_unsupported_reported(lib):
    # the delta rule with a per-head scalar gate (the delta-rule builds take token or channel gates)
    d = _dims(gate=hb.GATE_HEAD)
    p = ctypes.c_void_p(16)  # never dereferenced: the shape is rejected first
    st = lib.hypic_segment_build(ctypes.byref(d), 1, p, p, 4, p, p, p, p, p, p, None, 0, None)
    assert st == hb.HYPIC_E_UNSUPPORTED


def test_build_workspace_size(lib):
    """Build workspace: for the bf16 gated delta rule at d in {64, 128}, zero below one
    1024-token piece, growing with the token count; without the delta rule, 8 pieces per
    (segment, head) where segments average at least 256 tokens."""
    assert hb.build_workspace_bytes(16, 128, 128, 128, 100_000) > 0
    assert hb.build_workspace_bytes(16, 128, 128, 128, 1023) == 0
    assert hb.build_workspace_bytes(16, 16, 16, 128, 100_000) == 0
    assert hb.build_workspace_bytes(16, 128, 128, 128, 100_000, in_dtype=hb.F32) == 0
    assert hb.build_workspace_bytes(16, 128, 128, 128, 100_000, gate=hb.GATE_DIAG) == 0
    piece = lambda diag: 128 * 16 * 8 * (128 * 128 + (128 if diag else 1)) * 4
    assert hb.build_workspace_bytes(16, 128, 128, 128, 100_000, delta=False) >= piece(False)
    assert hb.build_workspace_bytes(16, 128, 128, 128, 100_000, gate=hb.GATE_DIAG, delta=False) >= piece(True)
    assert hb.build_workspace_bytes(16, 128, 128, 128, 128 * 256 - 1, delta=False) == 0
    one = hb.build_workspace_bytes(16, 128, 128, 128, 1024)
    two = hb.build_workspace_bytes(16, 128, 128, 128, 2 * 1024)
    assert two - one == 16 * 2 * 128 * 128 * 4            # one more slot: T planes + S per head


def test_short_build_workspace_rejected(lib):
    d = _dims(H=16, dk=128, dv=128, in_dtype=hb.BF16)
    need = hb.build_workspace_bytes(16, 128, 128, 4, 10_000)
    p = ctypes.c_void_p(256)  # never dereferenced: the size is rejected first
    st = lib.hypic_segment_build(ctypes.byref(d), 4, p, p, 10_000, p, p, p, p, p, p, p, need - 1, None)
    assert st == hb.HYPIC_E_INVALID and "workspace" in lib.hypic_last_error().decode()


def test_seam_workspace_size(lib):
    """Window records: 256-byte aligned, scaling with chains x steps x heads; 0 for bad arguments."""
    one = hb.seam_workspace_bytes(2, 128, 128, 1, 1, 8)
    assert one > 0 and one % 256 == 0 and one % 2 == 0
    assert hb.seam_workspace_bytes(2, 128, 128, 3, 5, 8) == 15 * one
    assert hb.seam_workspace_bytes(2, 128, 128, 1, 1, 17) == 0
    # d_k != d_v: the state advances in column blocks of at most d_k through one workspace
    assert hb.seam_workspace_bytes(2, 128, 64, 1, 1, 8) == one
    assert hb.seam_workspace_bytes(2, 64, 128, 1, 1, 8) == hb.seam_workspace_bytes(2, 64, 64, 1, 1, 8)
    assert hb.seam_workspace_bytes(2, 24, 24, 1, 1, 8) == 0
