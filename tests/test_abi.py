"""The C-ABI library on the CPU: it loads, exports every function the header
declares, its struct layouts match the ctypes mirror, and argument validation
rejects bad calls before anything reaches the GPU (no compute calls here)."""
import ctypes
import math
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm_mi355x.h")


@pytest.fixture(scope="module")
def L():
    from selective_state_space_03_amd import binding

    if not os.path.exists(binding.LIB_PATH):
        from selective_state_space_03_amd import build as b

        b.build()
    return binding.lib()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ssm_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_function(L):
    from selective_state_space_03_amd import binding

    names = _declared()
    assert set(names) == set(binding.EXPORTED), names
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (ssm_\w+)", out))
    for n in names:
        assert n in exported, f"{n} not exported"
        assert hasattr(L, n)


def test_struct_layouts_and_version(L):
    from selective_state_space_03_amd import binding

    assert L.ssm_abi_version() == 2
    assert L.ssm_params_sizeof(0) == ctypes.sizeof(binding.ScanParams)
    assert L.ssm_params_sizeof(1) == ctypes.sizeof(binding.DecodeParams)
    assert L.ssm_params_sizeof(2) == ctypes.sizeof(binding.ChunkParams)
    assert L.ssm_params_sizeof(3) == ctypes.sizeof(binding.ChunkDecodeParams)
    assert L.ssm_params_sizeof(4) == ctypes.sizeof(binding.LinearParams)
    assert L.ssm_params_sizeof(5) == ctypes.sizeof(binding.LayerParams)
    assert L.ssm_params_sizeof(6) == ctypes.sizeof(binding.ScanBwdParams)
    assert L.ssm_params_sizeof(7) == 0
    assert L.ssm_status_string(3) == b"SSM_ERR_WORKSPACE"


# Fake, well-separated, 256-byte aligned "device" addresses: validation only
# compares and range-checks pointers, it never dereferences them.
def _addr(i):
    return 0x10000000000 + i * 0x100000000


def _scan(**kw):
    from selective_state_space_03_amd import binding as b

    p = b.ScanParams()
    p.struct_size = ctypes.sizeof(b.ScanParams)
    p.batch, p.seqlen, p.dim, p.d_state, p.conv_k = 2, 64, 128, 16, 4
    p.x, p.y, p.A, p.B, p.C, p.dt, p.dt_w = (_addr(i) for i in range(1, 8))
    p.x_dtype = p.y_dtype = p.bc_dtype = 1
    p.dt_rank1 = 1
    p.dt_softplus = 1
    p.dt_min, p.dt_max = 1e-3, 0.1
    p.workspace, p.workspace_bytes = _addr(20), 1 << 30
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def _st(L, fn, p):
    return fn(ctypes.byref(p))


def test_scan_validation(L):
    ok = _scan()
    assert L.ssm_scan_check(ctypes.byref(ok)) == 0, L.ssm_last_error()
    assert L.ssm_scan_workspace_size(ctypes.byref(ok)) >= 2 * 64 * 32 * 4
    assert L.ssm_scan_check(ctypes.byref(_scan(discretization=1))) == 0, L.ssm_last_error()
    cases = {
        "discretization": (_scan(discretization=2), 1),
        "d_state": (_scan(d_state=8), 2),
        "neg": (_scan(batch=-1), 1),
        "bounds": (_scan(dt_min=0.5, dt_max=0.1), 1),
        "nan": (_scan(dt_min=math.nan), 1),
        "conv_k": (_scan(conv_w=_addr(9), conv_k=3), 2),
        "cache_without_conv": (_scan(conv_cache_in=_addr(9)), 1),
        "rank1_bf16": (_scan(dt_dtype=1), 2),
        "rank1_no_w": (_scan(dt_w=None), 1),
        "null_x": (_scan(x=None), 1),
        "split": (_scan(time_split=33), 1),
        "dtype": (_scan(x_dtype=5), 1),
        "z_dtype": (_scan(z=_addr(9), z_dtype=0), 2),
        "y_over_x": (_scan(y=_addr(1) + 64), 1),
        "workspace": (_scan(workspace_bytes=16), 3),
        "no_workspace": (_scan(workspace=None, workspace_bytes=0), 3),
        "ws_align": (_scan(workspace=_addr(20) + 8), 1),
        "struct": (_scan(struct_size=8), 1),
        "state_partial_alias": (_scan(ssm_state_in=_addr(10), ssm_state_out=_addr(10) + 4), 1),
    }
    for name, (p, want) in cases.items():
        assert L.ssm_scan_check(ctypes.byref(p)) == want, (name, L.ssm_last_error())
        assert L.ssm_last_error() != b""
    # the launching entry point returns the same code without touching a device
    bad = _scan(d_state=8)
    assert L.ssm_scan_fwd(ctypes.byref(bad), None) == 2
    # exact in-place aliasing of the state is allowed
    alias = _scan(ssm_state_in=_addr(10), ssm_state_out=_addr(10))
    assert L.ssm_scan_check(ctypes.byref(alias)) == 0
    assert L.ssm_scan_check(None) == 1


def _bulk(**kw):
    """A call the blocked scan takes: bf16 x / z / E-wide dt, no conv, dim % 64 == 0."""
    base = dict(batch=8, seqlen=4096, dim=7680, dt_rank1=0, dt_dtype=1, dt_w=None, z=_addr(9), z_dtype=1)
    base.update(kw)
    return _scan(**base)


def test_scan_blocked_selection(L):
    """time_split = SCAN_BLOCKED asks for the blocked single-pass scan and is
    refused (SSM_ERR_UNSUPPORTED) for calls it does not take; time_split = 0
    takes it at 768 or more 64-channel groups (its workspace: one 5120-byte
    record per batch row and 16-step block, then 1280 bytes of per-call
    values) and keeps the time-split kernels below that."""
    from selective_state_space_03_amd import binding as b

    ws = lambda p: L.ssm_scan_workspace_size(ctypes.byref(p))  # noqa: E731
    blk = 8 * 256 * 5120 + 1280
    assert ws(_bulk()) == blk
    assert ws(_bulk(time_split=b.SCAN_BLOCKED)) == blk
    assert ws(_bulk(time_split=4)) != blk
    assert ws(_bulk(seqlen=4097, time_split=b.SCAN_BLOCKED)) == 8 * 257 * 5120 + 1280
    assert ws(_bulk(batch=6)) != 6 * 256 * 5120 + 1280  # 720 groups: below the automatic threshold
    assert ws(_bulk(batch=6, time_split=b.SCAN_BLOCKED)) == 6 * 256 * 5120 + 1280
    assert L.ssm_scan_check(ctypes.byref(_bulk(time_split=b.SCAN_BLOCKED))) == 0, L.ssm_last_error()
    assert L.ssm_scan_check(ctypes.byref(_bulk(time_split=b.SCAN_BLOCKED, z=None, D=_addr(10)))) == 0
    refused = {
        "rank1": _bulk(dt_rank1=1, dt_dtype=0, dt_w=_addr(7)),
        "conv": _bulk(conv_w=_addr(11)),
        "dim": _bulk(dim=7616 + 32),
        "x_f32": _bulk(x_dtype=0, z_dtype=0),
        "dt_f32": _bulk(dt_dtype=0),
        "zoh": _bulk(discretization=1),
        "x_align": _bulk(x=_addr(1) + 2),
        "y_f32_align": _bulk(y_dtype=0, y=_addr(2) + 8),
        "state_align": _bulk(ssm_state_out=_addr(12) + 8),
    }
    for name, p in refused.items():
        p.time_split = b.SCAN_BLOCKED
        assert L.ssm_scan_check(ctypes.byref(p)) == 2, (name, L.ssm_last_error())
        assert b"blocked" in L.ssm_last_error(), name
        p.time_split = 0  # the library's own choice falls back to the time-split kernels
        assert L.ssm_scan_check(ctypes.byref(p)) == 0, (name, L.ssm_last_error())
        assert ws(p) != blk, name
    assert L.ssm_scan_check(ctypes.byref(_bulk(time_split=-2))) == 1


def test_scan_noalloc_validation(L):
    """ssm_scan_fwd_noalloc refuses, before touching a device: a NULL or
    mismatched struct, a workspace of the caller's (it uses its own scratch),
    and a call whose workspace would exceed the 64 MiB scratch."""
    fn = L.ssm_scan_fwd_noalloc
    assert fn(None, None) == 1
    assert fn(ctypes.byref(_scan(workspace=None, workspace_bytes=0, struct_size=8)), None) == 1
    assert fn(ctypes.byref(_scan()), None) == 1
    assert b"scratch" in L.ssm_last_error()
    assert fn(ctypes.byref(_scan(workspace=None, workspace_bytes=16)), None) == 1
    big = _scan(workspace=None, workspace_bytes=0, batch=64, seqlen=4096, dim=128)
    assert L.ssm_scan_workspace_size(ctypes.byref(big)) > 64 << 20
    assert fn(ctypes.byref(big), None) == 3
    assert b"at most 67108864" in L.ssm_last_error()


def test_empty_batch_calls_return_ok_without_launching(L):
    """batch = 0 through the sizing, validation and launch paths of the scan,
    the decode step and the chunked scan: OK, a zero workspace, nothing
    launched (no GPU here), and no division by the empty work count."""
    p = _scan(batch=0, x=None, y=None, B=None, C=None, dt=None, workspace=None, workspace_bytes=0)
    for split in (0, 1, 7, 32):
        p.time_split = split
        assert L.ssm_scan_workspace_size(ctypes.byref(p)) == 0
        assert L.ssm_scan_check(ctypes.byref(p)) == 0, L.ssm_last_error()
        assert L.ssm_scan_fwd(ctypes.byref(p), None) == 0, L.ssm_last_error()
    c = _chunk(batch=0, x=None, dt=None, B=None, C=None, out=None, workspace=None, workspace_bytes=0)
    assert L.ssm_chunk_scan_workspace_size(ctypes.byref(c)) == 0
    assert L.ssm_chunk_scan_fwd(ctypes.byref(c), None) == 0, L.ssm_last_error()


def _decode(**kw):
    from selective_state_space_03_amd import binding as b

    p = b.DecodeParams()
    p.struct_size = ctypes.sizeof(b.DecodeParams)
    p.batch, p.dim, p.d_state, p.conv_k = 64, 7680, 16, 4
    p.x, p.y, p.A, p.B, p.C, p.dt, p.dt_w, p.ssm_state, p.conv_w, p.conv_cache = (_addr(i) for i in range(1, 11))
    p.dt_rank1 = 1
    p.dt_min, p.dt_max = 1e-3, 0.1
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def test_decode_validation(L):
    assert L.ssm_decode_check(ctypes.byref(_decode())) == 0, L.ssm_last_error()
    assert L.ssm_decode_check(ctypes.byref(_decode(discretization=1))) == 0, L.ssm_last_error()
    cases = {
        "discretization": (_decode(discretization=-1), 1),
        "no_cache": (_decode(conv_cache=None), 1),
        "state_align": (_decode(ssm_state=_addr(8) + 4), 1),
        "d_state": (_decode(d_state=32), 2),
        "no_state": (_decode(ssm_state=None), 1),
        "y_over_state": (_decode(y=_addr(8) + 128), 1),
        "bc_align": (_decode(B=_addr(4) + 4), 1),
        "bc_align_bf16": (_decode(C=_addr(5) + 4, bc_dtype=1), 1),
        "conv_w_align": (_decode(conv_w=_addr(9) + 4), 1),
        "too_many_channels": (_decode(batch=1 << 20, dim=1 << 12), 2),
    }
    for name, (p, want) in cases.items():
        assert L.ssm_decode_check(ctypes.byref(p)) == want, (name, L.ssm_last_error())
    assert L.ssm_decode_step(ctypes.byref(_decode(d_state=32)), None) == 2
    # bf16 B/C need only 8-byte alignment
    assert L.ssm_decode_check(ctypes.byref(_decode(B=_addr(4) + 8, C=_addr(5) + 8, bc_dtype=1))) == 0


def _chunk(**kw):
    from selective_state_space_03_amd import binding as b

    p = b.ChunkParams()
    p.struct_size = ctypes.sizeof(b.ChunkParams)
    p.batch, p.seqlen, p.nheads, p.headdim, p.ngroups, p.d_state, p.chunk_size = 1, 1024, 8, 96, 1, 64, 128
    p.x, p.dt, p.A, p.B, p.C, p.out = (_addr(i) for i in range(1, 7))
    p.x_dtype = p.bc_dtype = 1
    p.dt_softplus = 1
    p.dt_min, p.dt_max = 1e-3, 0.1
    p.workspace, p.workspace_bytes = _addr(20), 1 << 32
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def test_chunk_validation(L):
    assert L.ssm_chunk_scan_check(ctypes.byref(_chunk())) == 0, L.ssm_last_error()
    cases = {
        "z_dtype": (_chunk(z=_addr(8), z_dtype=4), 1),
        "z_align": (_chunk(z=_addr(8) + 2), 1),
        "out_over_z": (_chunk(z=_addr(6) + 64), 1),
        "groups": (_chunk(ngroups=3), 1),
        "d_state": (_chunk(d_state=129), 2),
        "chunk": (_chunk(chunk_size=257, seqlen=1024), 2),
        "headdim": (_chunk(headdim=136), 2),
        "general_x_align": (_chunk(d_state=32, x=_addr(1) + 1), 1),
        "general_ws_small": (_chunk(d_state=32, workspace_bytes=1024), 3),
        "row_over_4GiB": (_chunk(seqlen=1 << 22), 2),
        "null_A": (_chunk(A=None), 1),
        "out_over_x": (_chunk(out=_addr(1) + 2), 1),
        "out_align": (_chunk(out=_addr(6) + 8), 1),
        "x_align": (_chunk(x=_addr(1) + 2), 1),
        "segments_neg": (_chunk(segments=-1), 1),
        "segments_big": (_chunk(segments=17), 1),
        "ws_small": (_chunk(segments=4, workspace_bytes=1024), 3),
        "ws_align": (_chunk(segments=4, workspace=_addr(20) + 16), 1),
    }
    for name, (p, want) in cases.items():
        assert L.ssm_chunk_scan_check(ctypes.byref(p)) == want, (name, L.ssm_last_error())
    assert L.ssm_chunk_scan_fwd(ctypes.byref(_chunk(d_state=200)), None) == 2
    # a sequence that is not a whole number of chunks is accepted
    assert L.ssm_chunk_scan_check(ctypes.byref(_chunk(seqlen=1000))) == 0, L.ssm_last_error()
    # the shapes of the vector-ALU kernels: other chunk sizes, d_state, headdim
    # and fp32 inputs (aligned to their element size only)
    for kw in (dict(chunk_size=64), dict(chunk_size=256), dict(d_state=16), dict(d_state=32), dict(d_state=128),
               dict(headdim=100), dict(x_dtype=0, bc_dtype=0), dict(x_dtype=0, x=_addr(1) + 4),
               dict(chunk_size=48, d_state=24, headdim=40, seqlen=1000)):
        assert L.ssm_chunk_scan_check(ctypes.byref(_chunk(**kw))) == 0, (kw, L.ssm_last_error())


def test_chunk_workspace_size(L):
    """Forced segments: per (batch, head), the state entering each segment
    after the first, one (P x N) state and one decay per summary piece of up
    to 16 chunks of the segments before the last; none for one segment."""
    L.ssm_chunk_scan_workspace_size.restype = ctypes.c_size_t
    size = lambda **kw: L.ssm_chunk_scan_workspace_size(ctypes.byref(_chunk(**kw)))
    P, N, heads = 96, 64, 8
    assert size(segments=1) == 0
    assert size(segments=1, seqlen=100) == 0
    # 8 chunks in 4 segments of 2: 3 incoming states, 3 pieces
    assert size(segments=4) == 4 * heads * (3 * P * N + 3 * (P * N + 1))
    # 36 chunks (ragged) in 2 segments of 18: 1 incoming state, 2 pieces
    assert size(segments=2, seqlen=4500) == 4 * heads * (P * N + 2 * (P * N + 1))
    # more segments than chunks: one chunk per segment
    assert size(segments=16, seqlen=300) == 4 * heads * (2 * P * N + 2 * (P * N + 1))
    assert size(segments=4, seqlen=0) == 0
    # the vector-ALU kernels: one (P x N) state and one decay per (batch,
    # chunk, head), each part rounded up to 256 bytes; segments do not matter
    rnd = lambda v: (v + 255) // 256 * 256  # noqa: E731
    assert size(d_state=32) == rnd(4 * 8 * heads * P * 32) + rnd(4 * 8 * heads)
    assert size(d_state=32, segments=4) == size(d_state=32)
    assert size(chunk_size=64, seqlen=1000) == rnd(4 * 16 * heads * P * N) + rnd(4 * 16 * heads)


def _cdec(**kw):
    from selective_state_space_03_amd import binding as b

    p = b.ChunkDecodeParams()
    p.struct_size = ctypes.sizeof(b.ChunkDecodeParams)
    p.batch, p.nheads, p.headdim, p.ngroups, p.d_state = 64, 80, 96, 1, 64
    p.x, p.dt, p.A, p.B, p.C, p.state, p.out = (_addr(i) for i in range(1, 8))
    p.x_dtype = p.bc_dtype = p.out_dtype = 1
    p.dt_softplus = 1
    p.dt_min, p.dt_max = 1e-3, 0.1
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def test_chunk_decode_validation(L):
    assert L.ssm_chunk_decode_check(ctypes.byref(_cdec())) == 0, L.ssm_last_error()
    for n in (16, 32, 128):
        assert L.ssm_chunk_decode_check(ctypes.byref(_cdec(d_state=n))) == 0, (n, L.ssm_last_error())
    cases = {
        "struct_size": (_cdec(struct_size=8), 1),
        "groups": (_cdec(ngroups=3), 1),
        "d_state": (_cdec(d_state=48), 2),
        "d_state_256": (_cdec(d_state=256), 2),
        "dtype": (_cdec(x_dtype=5), 1),
        "z_dtype": (_cdec(z=_addr(8), z_dtype=3), 1),
        "null_A": (_cdec(A=None), 1),
        "null_state": (_cdec(state=None), 1),
        "state_align": (_cdec(state=_addr(6) + 4), 1),
        "bc_align_bf16": (_cdec(B=_addr(4) + 8), 1),
        "bc_align_f32": (_cdec(bc_dtype=0, C=_addr(5) + 16), 1),
        "out_over_state": (_cdec(out=_addr(6) + 256), 1),
        "out_over_z": (_cdec(z=_addr(8), out=_addr(8) + 2), 1),
        "dt_nan": (_cdec(dt_min=math.nan), 1),
        "dt_order": (_cdec(dt_min=1.0, dt_max=0.5), 1),
        "too_many_rows": (_cdec(batch=1 << 20, nheads=64, headdim=64), 2),
    }
    for name, (p, want) in cases.items():
        assert L.ssm_chunk_decode_check(ctypes.byref(p)) == want, (name, L.ssm_last_error())
    assert L.ssm_last_error() != b""
    # batch 0 is a no-op that needs no buffers
    assert L.ssm_chunk_decode_step(ctypes.byref(_cdec(batch=0, x=None, state=None, out=None)), None) == 0
    assert L.ssm_chunk_decode_step(ctypes.byref(_cdec(d_state=48)), None) == 2
    # aligned to 8 elements is enough for B/C
    assert L.ssm_chunk_decode_check(ctypes.byref(_cdec(B=_addr(4) + 16, C=_addr(5) + 16))) == 0
    assert L.ssm_chunk_decode_check(ctypes.byref(_cdec(bc_dtype=0, B=_addr(4) + 32))) == 0


def _lin(**kw):
    from selective_state_space_03_amd import binding as b

    p = b.LinearParams()
    p.struct_size = ctypes.sizeof(b.LinearParams)
    p.rows, p.in_features, p.out_features = 2048, 2560, 15360
    p.x, p.weight, p.out = _addr(1), _addr(2), _addr(3)
    p.x_dtype, p.out_dtype = 1, 0
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def test_linear_validation(L):
    assert L.ssm_linear_check(ctypes.byref(_lin())) == 0, L.ssm_last_error()
    cases = {
        "struct_size": (_lin(struct_size=4), 1),
        "rows": (_lin(rows=-1), 1),
        "in_zero": (_lin(in_features=0), 1),
        "in_mult8": (_lin(in_features=2564), 2),
        "out_mult4": (_lin(out_features=15362), 2),
        "dtype": (_lin(x_dtype=7), 1),
        "null_w": (_lin(weight=None), 1),
        "x_align": (_lin(x=_addr(1) + 8), 1),
        "out_align": (_lin(out=_addr(3) + 4), 1),
        "out_over_x": (_lin(out=_addr(1) + 1024), 1),
        "out_over_w": (_lin(out=_addr(2) + 4096), 1),
        "ws_align": (_lin(workspace=_addr(4) + 16, workspace_bytes=1 << 20), 1),
        "ws_over_out": (_lin(workspace=_addr(3) + 256, workspace_bytes=1 << 20), 1),
        "ws_missing_f32": (_lin(x_dtype=0), 3),
        "ws_short_f32": (_lin(x_dtype=0, workspace=_addr(4), workspace_bytes=1 << 20), 3),
    }
    for name, (p, want) in cases.items():
        assert L.ssm_linear_check(ctypes.byref(p)) == want, (name, L.ssm_last_error())
    assert L.ssm_linear_fwd(ctypes.byref(_lin(rows=0, x=None, out=None)), None) == 0
    assert L.ssm_linear_fwd(ctypes.byref(_lin(in_features=12)), None) == 2
    # a bf16 input needs no workspace; an fp32 input its bf16 value and
    # remainder (rows x in_features each) and an fp32 product
    L.ssm_linear_workspace_size.restype = ctypes.c_size_t
    assert L.ssm_linear_workspace_size(ctypes.byref(_lin())) == 0
    assert L.ssm_linear_workspace_size(ctypes.byref(_lin(in_features=7680, out_features=2560))) == 0
    f32 = L.ssm_linear_workspace_size(ctypes.byref(_lin(in_features=7680, out_features=2560, x_dtype=0)))
    assert f32 == 2 * 2048 * 7680 * 2 + 2048 * 2560 * 4


def _layer(**kw):
    from selective_state_space_03_amd import binding as b

    p = b.LayerParams()
    p.struct_size = ctypes.sizeof(b.LayerParams)
    p.batch, p.seqlen, p.d_model, p.dim, p.d_state, p.conv_k = 1, 2048, 2560, 7680, 16, 4
    p.hidden, p.w_in, p.conv_w, p.w_x, p.dt_w, p.A, p.w_out, p.out = (_addr(i) for i in range(1, 9))
    p.hidden_dtype, p.out_dtype = 1, 1
    p.dt_softplus = 1
    p.dt_min, p.dt_max = 1e-3, 0.1
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def test_layer_validation(L):
    need = L.ssm_layer_workspace_size(ctypes.byref(_layer()))
    # x_branch, z and y in fp32 at least
    assert need >= 3 * 2048 * 7680 * 4
    ok = _layer(workspace=_addr(20), workspace_bytes=need)
    assert L.ssm_layer_check(ctypes.byref(ok)) == 0, L.ssm_last_error()
    cases = {
        "no_workspace": (_layer(), 3),
        "small_workspace": (_layer(workspace=_addr(20), workspace_bytes=need - 256), 3),
        "ws_align": (_layer(workspace=_addr(20) + 64, workspace_bytes=need), 1),
        "struct_size": (_layer(struct_size=12, workspace=_addr(20), workspace_bytes=need), 1),
        "d_state": (_layer(d_state=32, workspace=_addr(20), workspace_bytes=need), 2),
        "conv_k": (_layer(conv_k=3, workspace=_addr(20), workspace_bytes=need), 2),
        "dim": (_layer(dim=7600, workspace=_addr(20), workspace_bytes=need), 2),
        "d_model": (_layer(d_model=2564, workspace=_addr(20), workspace_bytes=need), 2),
        "null_w_x": (_layer(w_x=None, workspace=_addr(20), workspace_bytes=need), 1),
        "dtype": (_layer(out_dtype=9, workspace=_addr(20), workspace_bytes=need), 1),
        "out_over_hidden": (_layer(out=_addr(1) + 4096, workspace=_addr(20), workspace_bytes=need), 1),
        "ws_over_w_in": (_layer(workspace=_addr(2), workspace_bytes=need), 1),
        "hidden_align": (_layer(hidden=_addr(1) + 8, workspace=_addr(20), workspace_bytes=need), 1),
        "dt_order": (_layer(dt_min=0.5, dt_max=0.1, workspace=_addr(20), workspace_bytes=need), 1),
    }
    for name, (p, want) in cases.items():
        assert L.ssm_layer_check(ctypes.byref(p)) == want, (name, L.ssm_last_error())
    assert L.ssm_layer_fwd(ctypes.byref(_layer(batch=0, hidden=None, out=None)), None) == 0
    assert L.ssm_layer_fwd(ctypes.byref(_layer(d_state=8)), None) == 2


def _bwd(**kw):
    from selective_state_space_03_amd import binding as b

    p = b.ScanBwdParams()
    p.struct_size = ctypes.sizeof(b.ScanBwdParams)
    p.batch, p.seqlen, p.dim, p.d_state, p.conv_k = 1, 2048, 7680, 16, 4
    p.x, p.A, p.B, p.C, p.dt, p.dt_w, p.dy, p.conv_w = (_addr(i) for i in range(1, 9))
    p.x_dtype, p.bc_dtype, p.dy_dtype = 1, 1, 0
    p.dt_rank1, p.dt_softplus = 1, 1
    p.dt_min, p.dt_max = 1e-3, 0.1
    p.dx, p.dA, p.dB, p.dC, p.ddt, p.ddt_w, p.dconv_w = (_addr(i) for i in range(10, 17))
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def test_scan_bwd_validation(L):
    need = L.ssm_scan_bwd_workspace_size(ctypes.byref(_bwd()))
    assert need > 0
    ok = _bwd(workspace=_addr(30), workspace_bytes=need)
    assert L.ssm_scan_bwd_check(ctypes.byref(ok)) == 0, L.ssm_last_error()
    W = dict(workspace=_addr(30), workspace_bytes=need)
    cases = {
        "no_workspace": (_bwd(), 3),
        "struct_size": (_bwd(struct_size=4, **W), 1),
        "d_state": (_bwd(d_state=8, **W), 2),
        "dz_without_z": (_bwd(dz=_addr(20), **W), 1),
        "ddt_w_without_rank1": (_bwd(dt_rank1=0, dt_w=None, **W), 1),
        "dconv_without_conv": (_bwd(conv_w=None, **W), 1),
        "grad_over_input": (_bwd(dx=_addr(1) + 256, **W), 1),
        "grads_overlap": (_bwd(dB=_addr(10) + 64, **W), 1),
        "ws_over_grad": (_bwd(workspace=_addr(11), workspace_bytes=need), 1),
        "dy_dtype": (_bwd(dy_dtype=5, **W), 1),
        "bc_align": (_bwd(B=_addr(3) + 2, **W), 1),
    }
    for name, (p, want) in cases.items():
        assert L.ssm_scan_bwd_check(ctypes.byref(p)) == want, (name, L.ssm_last_error())
    assert L.ssm_scan_bwd(ctypes.byref(_bwd(batch=0)), None) == 0


def test_binding_refuses_cpu_tensors(L):
    import torch

    import selective_state_space_03_amd as ssm

    x = torch.zeros(1, 4, 8)
    with pytest.raises(ValueError):
        ssm.scan_fwd(x, torch.zeros(8, 16), torch.zeros(1, 4, 16), torch.zeros(1, 4, 16), torch.zeros(1, 4, 8))
