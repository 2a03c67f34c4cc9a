"""The SSM_DEBUG twin of the library on the CPU: its launch-plan checks pass on
a sweep of shapes, ragged sizes and split choices of the three entry points
that take a workspace (ssm_debug_check_* run validation, plan and checks
without launching; pointers are compared, never dereferenced), they count,
and the regular build reports that it has none."""
import ctypes
import itertools
import os

import pytest

from test_abi import _addr, _bwd, _chunk, _scan


@pytest.fixture(scope="module")
def D():
    """The debug build (SSM_MI355X_DEBUG_LIB names another, e.g. a host-sanitized one)."""
    from selective_state_space_03_amd import binding
    from selective_state_space_03_amd import build as b

    path = os.environ.get("SSM_MI355X_DEBUG_LIB") or b.DEBUG_LIB_PATH
    if not os.path.exists(path):
        b.build()
    return binding.load(path)


@pytest.fixture(scope="module")
def R():
    from selective_state_space_03_amd import binding
    from selective_state_space_03_amd import build as b

    if not os.path.exists(binding.LIB_PATH):
        b.build()
    return binding.lib()


def _ok(L, fn, p, what):
    st = fn(ctypes.byref(p))
    assert st == 0, (what, L.ssm_status_string(st), L.ssm_last_error())


def test_regular_build_has_no_checks(R):
    if os.environ.get("SSM_MI355X_LIB") and R.ssm_debug_checks() != -1:
        pytest.skip("the library under test (SSM_MI355X_LIB) is a debug build")
    assert R.ssm_debug_checks() == -1
    assert R.ssm_debug_check_scan(ctypes.byref(_scan())) == 2  # SSM_ERR_UNSUPPORTED


def test_scan_plans(D):
    before = D.ssm_debug_checks()
    assert before >= 0
    n = 0
    for batch, seqlen, dim, split in itertools.product(
            (0, 1, 3, 8), (1, 3, 4, 7, 8, 9, 31, 65, 257, 1000, 2048, 4096), (16, 70, 136, 200, 7680),
            (0, 1, 2, 3, 5, 16, 32)):
        p = _scan(batch=batch, seqlen=seqlen, dim=dim, time_split=split)
        p.workspace_bytes = max(D.ssm_scan_workspace_size(ctypes.byref(p)), 1)
        _ok(D, D.ssm_debug_check_scan, p, (batch, seqlen, dim, split))
        n += 1
    # both discretisations, no conv, E-wide bf16 dt, no upper clip (no rescaled rows)
    for kw in (dict(discretization=1), dict(conv_w=None, conv_k=0, dt_rank1=0, dt_dtype=1, dt_w=None),
               dict(dt_max=float("inf"))):
        p = _scan(**kw)
        p.workspace_bytes = D.ssm_scan_workspace_size(ctypes.byref(p))
        _ok(D, D.ssm_debug_check_scan, p, kw)
        n += 1
    # the blocked single-pass scan: ragged tails, one partial block, batches
    for batch, seqlen, dim in itertools.product((1, 3, 8), (1, 15, 16, 17, 4096, 4099), (64, 192, 7680)):
        p = _scan(batch=batch, seqlen=seqlen, dim=dim, time_split=-1, dt_rank1=0, dt_dtype=1, dt_w=None)
        p.workspace_bytes = D.ssm_scan_workspace_size(ctypes.byref(p))
        _ok(D, D.ssm_debug_check_scan, p, ("blocked", batch, seqlen, dim))
        n += 1
    assert D.ssm_debug_checks() - before == n


def test_scan_plan_needs_its_workspace(D):
    """A workspace one byte short is refused by validation before any plan."""
    p = _scan(batch=8, seqlen=4096, dim=7680)
    need = D.ssm_scan_workspace_size(ctypes.byref(p))
    p.workspace_bytes = need - 1
    assert D.ssm_debug_check_scan(ctypes.byref(p)) == 3  # SSM_ERR_WORKSPACE


def test_chunk_plans(D):
    before = D.ssm_debug_checks()
    n = 0
    # the tuned path (N 64, chunk 128, P % 16 == 0) with its segments and pieces
    for batch, seqlen, heads, hd, seg in itertools.product(
            (1, 2), (1, 127, 128, 129, 1000, 4096, 65536), (8, 12, 80), (32, 96, 128), (0, 1, 2, 3, 5, 16)):
        p = _chunk(batch=batch, seqlen=seqlen, nheads=heads, headdim=hd, segments=seg)
        p.workspace_bytes = D.ssm_chunk_scan_workspace_size(ctypes.byref(p))
        p.workspace = _addr(20) if p.workspace_bytes else None
        _ok(D, D.ssm_debug_check_chunk, p, (batch, seqlen, heads, hd, seg))
        n += 1
    # the vector-ALU path: other chunk sizes, states, head dims and fp32 inputs
    for seqlen, q, N, hd, x_dtype in itertools.product((1, 63, 64, 65, 700), (64, 256), (16, 128), (40, 128), (0, 1)):
        p = _chunk(seqlen=seqlen, chunk_size=q, d_state=N, headdim=hd, x_dtype=x_dtype, bc_dtype=x_dtype)
        p.workspace_bytes = D.ssm_chunk_scan_workspace_size(ctypes.byref(p))
        _ok(D, D.ssm_debug_check_chunk, p, (seqlen, q, N, hd, x_dtype))
        n += 1
    assert D.ssm_debug_checks() - before == n


def test_bwd_plans(D):
    before = D.ssm_debug_checks()
    n = 0
    for batch, seqlen, dim, conv in itertools.product((1, 3), (1, 15, 16, 17, 63, 64, 65, 300, 2048),
                                                      (16, 40, 200, 7680), (True, False)):
        kw = dict(batch=batch, seqlen=seqlen, dim=dim)
        if not conv:
            kw.update(conv_w=None, conv_k=0, dconv_w=None)
        p = _bwd(**kw)
        p.workspace_bytes = D.ssm_scan_bwd_workspace_size(ctypes.byref(p))
        p.workspace = _addr(30)
        _ok(D, D.ssm_debug_check_scan_bwd, p, (batch, seqlen, dim, conv))
        n += 1
    assert D.ssm_debug_checks() - before == n
