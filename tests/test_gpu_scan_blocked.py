"""GPU parity of the blocked single-pass scan (time_split = SCAN_BLOCKED)
against the oracle, through the C ABI: bf16 u / z / E-wide dt, no conv.

Block structure: L = 1 and 15 (one partial block), 16 and 64 (whole blocks
only), 17 and 257 (a ragged tail); channel groups 1 and 3 per batch row.  The
three forms of A: exact diagonal and the fp32 initialisation a model stores
(the same row in every channel: saturated blocks on the matrix cores), and
random per channel (step-by-step with a per-channel factor every step).  dt
saturated (most blocks on the matrix cores) and shifted off the clip (softplus
and both clip edges, step-by-step blocks).  Both output dtypes, no gate, no
skip, a starting state, in-place state, fp32 B/C, no softplus, no upper clip.
Tolerance 2e-3 max|y| (bf16 inputs, fp32 state)."""
import numpy as np
import pytest
import torch

import selective_state_space_03_amd as ssm
import ssm_workloads as W
from gpu_util import DEV, check, dev_tensor, np64, scan_oracle

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _run(w, *, y_dtype=torch.float32, z=True, D=True, state_in=None, state_out=True, bc_f32=False,
         dt_softplus=None, dt_max=None, time_split=ssm.SCAN_BLOCKED):
    o, d = w.opts, w.dims
    B, C = dev_tensor(w, "B"), dev_tensor(w, "C")
    if bc_f32:
        B, C = B.float(), C.float()
    st = None
    if state_out is True:
        st = torch.empty((d["batch"], d["dim"], 16), dtype=torch.float32, device=DEV)
    elif state_out is not None:
        st = state_out
    y = ssm.scan_fwd(dev_tensor(w, "x"), dev_tensor(w, "A"), B, C, dev_tensor(w, "dt"),
                     D=dev_tensor(w, "D") if D else None, z=dev_tensor(w, "z") if z else None,
                     dt_bias=dev_tensor(w, "dt_bias"),
                     dt_softplus=o["dt_softplus"] if dt_softplus is None else dt_softplus,
                     dt_min=o["dt_min"], dt_max=o["dt_max"] if dt_max is None else dt_max,
                     ssm_state_in=state_in, ssm_state_out=st, y_dtype=y_dtype, time_split=time_split)
    torch.cuda.synchronize()
    return y, st


def _oracle(w, *, z=True, D=True, state_in=None, dt_softplus=None, dt_max=None):
    """The oracle on the workload with the same variations."""
    from oracle import ssm_oracle as O

    o, f = w.opts, w.f64
    return O.ssm_layer_scan(f("x"), f("A"), f("B"), f("C"), D=f("D") if D else None, z=f("z") if z else None,
                            conv_w=None, conv_cache=None, dt_bias=f("dt_bias"),
                            dt_softplus=o["dt_softplus"] if dt_softplus is None else dt_softplus,
                            dt_min=float(o["dt_min"]), dt_max=float(o["dt_max"] if dt_max is None else dt_max),
                            ssm_state=state_in, dt=f("dt"))


@pytest.mark.parametrize("a_init", ["diag", "log_init", "random"])
@pytest.mark.parametrize("unsat", [False, True])
@pytest.mark.parametrize("seqlen", [1, 15, 16, 17, 64, 257])
def test_blocked_parity(seqlen, unsat, a_init):
    w = W.scan_bulk(batch=3, seqlen=seqlen, dim=192, unsaturated=unsat, a_init=a_init)
    y, st = _run(w)
    yo, ho, _ = scan_oracle(w)
    check(np64(y), yo, TOL, f"blocked y L={seqlen} unsat={unsat} A={a_init}")
    check(np64(st), ho, TOL, f"blocked state L={seqlen} unsat={unsat} A={a_init}")


@pytest.mark.parametrize("seqlen", [33, 300])
def test_blocked_bf16_out_no_gate_no_skip(seqlen):
    w = W.scan_bulk(batch=2, seqlen=seqlen, dim=64)
    y, st = _run(w, y_dtype=torch.bfloat16, z=False, D=False)
    yo, ho, _ = _oracle(w, z=False, D=False)
    check(np64(y), yo, TOL, f"blocked bf16 y L={seqlen}", out_bf16=True)
    check(np64(st), ho, TOL, f"blocked bf16 state L={seqlen}")


@pytest.mark.parametrize("in_place", [False, True])
def test_blocked_state_in(in_place):
    """A random starting state, read and (in place) overwritten."""
    w = W.scan_bulk(batch=2, seqlen=100, dim=128, unsaturated=True)
    rng = np.random.Generator(np.random.PCG64(41))
    s0 = rng.standard_normal((2, 128, 16)).astype(np.float32)
    st_in = torch.from_numpy(s0).to(DEV)
    y, st = _run(w, state_in=st_in, state_out=st_in if in_place else True)
    yo, ho, _ = _oracle(w, state_in=s0.astype(np.float64))
    check(np64(y), yo, TOL, "blocked y from a state")
    check(np64(st), ho, TOL, "blocked state from a state")
    if in_place:
        assert st is st_in


def test_blocked_fp32_bc_and_no_softplus():
    """fp32 B / C (the packing kernel's other input type; values exact in bf16)
    and dt = clip(pre, lo, hi) without softplus."""
    w = W.scan_bulk(batch=2, seqlen=80, dim=64, unsaturated=True)
    y, st = _run(w, bc_f32=True, dt_softplus=False)
    yo, ho, _ = _oracle(w, dt_softplus=False)
    check(np64(y), yo, TOL, "blocked fp32 B/C, no softplus y")
    check(np64(st), ho, TOL, "blocked fp32 B/C, no softplus state")


def test_blocked_without_upper_clip():
    """dt_max = +inf: the scaled form is off, every step carries its own decay."""
    w = W.scan_bulk(batch=2, seqlen=70, dim=64, unsaturated=True)
    y, st = _run(w, dt_max=float("inf"))
    yo, ho, _ = _oracle(w, dt_max=float("inf"))
    check(np64(y), yo, TOL, "blocked no upper clip y")
    check(np64(st), ho, TOL, "blocked no upper clip state")


def test_blocked_placed_off_clip_steps():
    """A saturated call with dt pushed off the clip at chosen (batch, step,
    channel) entries, so that a 16 x 16 tile of a wave holds: one step off the
    clip (first, middle and last step of a block), two steps in one channel,
    two steps in two channels, and three steps (the step-by-step path)."""
    w = W.scan_bulk(batch=2, seqlen=48, dim=64)
    dt = w.arrays["dt"]
    if not dt.flags.writeable:
        dt = w.arrays["dt"] = dt.copy()
    low = np.uint16(0xC0A0)  # bf16 -5.0: softplus(-5 + bias) < dt_max for any bias here
    for b, t, e in [(0, 3, 1), (0, 0, 17), (0, 15, 33), (0, 5, 50), (0, 9, 50), (0, 18, 2), (0, 27, 13),
                    (0, 20, 20), (0, 22, 21), (0, 30, 22), (1, 40, 63), (1, 47, 48), (1, 16, 0)]:
        dt[b, t, e] = low
    y, st = _run(w)
    yo, ho, _ = scan_oracle(w)
    check(np64(y), yo, TOL, "blocked y, placed off-clip steps")
    check(np64(st), ho, TOL, "blocked state, placed off-clip steps")


def test_library_choice_on_a_small_call():
    """time_split = 0 on a call with few channel groups keeps the time-split
    kernels; the blocked kernel on the same call agrees with the oracle too."""
    w = W.scan_bulk(batch=4, seqlen=512, dim=256)
    yo, ho, _ = scan_oracle(w)
    for split in (0, ssm.SCAN_BLOCKED):
        y, st = _run(w, time_split=split)
        check(np64(y), yo, TOL, f"y split={split}")
        check(np64(st), ho, TOL, f"state split={split}")


@pytest.mark.parametrize("bias", ["recipe", "equal", "descending", "extremes"])
def test_blocked_workgroup_order_from_bias(bias):
    """The bulk grid (batch 8, E 7680: 960 channel groups, runs of three and
    four groups per CU slot) over two blocks, with dt_bias ordering the groups
    of each run differently: the recipe's draw, every bias equal (ties), biases
    falling with the channel (every run reversed) and biases of +-1e30 in some
    channels.  y starts as NaN and every output is compared with the oracle,
    so a group written twice or never fails."""
    w = W.scan_bulk(batch=8, seqlen=32, dim=7680)
    b = np.array(w.arrays["dt_bias"], dtype=np.float32, copy=True)
    if bias == "equal":
        b[:] = np.float32(0.25)
    elif bias == "descending":
        b = np.linspace(1.0, -2.0, b.size, dtype=np.float32)
    elif bias == "extremes":
        b[5::97] = np.float32(-1e30)
        b[11::89] = np.float32(1e30)
    w.arrays["dt_bias"] = b
    o = w.opts
    y = torch.full((8, 32, 7680), float("nan"), dtype=torch.float32, device=DEV)
    st = torch.full((8, 7680, 16), float("nan"), dtype=torch.float32, device=DEV)
    ssm.scan_fwd(dev_tensor(w, "x"), dev_tensor(w, "A"), dev_tensor(w, "B"), dev_tensor(w, "C"), dev_tensor(w, "dt"),
                 D=dev_tensor(w, "D"), z=dev_tensor(w, "z"), dt_bias=dev_tensor(w, "dt_bias"),
                 dt_softplus=o["dt_softplus"], dt_min=o["dt_min"], dt_max=o["dt_max"], ssm_state_out=st, y=y,
                 time_split=ssm.SCAN_BLOCKED)
    torch.cuda.synchronize()
    yo, ho, _ = scan_oracle(w)
    assert not torch.isnan(y).any() and not torch.isnan(st).any()
    check(np64(y), yo, TOL, f"blocked y, bias {bias}")
    check(np64(st), ho, TOL, f"blocked state, bias {bias}")


@pytest.mark.parametrize("with_state,softplus", [(False, True), (True, True), (False, False)])
def test_blocked_one_channel_off_clip(with_state, softplus):
    """Saturated calls in which, inside a 16 x 16 tile, every step off the clip
    belongs to one channel: 3, 5, 8 and all 16 steps of a block (the
    one-channel path) and 2 steps (the per-step corrections), in channels at
    the first, a middle and the last lane column of a wave, in different
    waves and batch rows; next to tiles with two channels off and with one
    step off.  Against the oracle, fp32 output.  Without softplus (dt =
    clip(pre)) every other step is put at the clip by a pre-activation of 2."""
    w = W.scan_bulk(batch=2, seqlen=80, dim=128)
    dt = w.arrays["dt"]
    if not dt.flags.writeable:
        dt = w.arrays["dt"] = dt.copy()
    if not softplus:
        dt[:] = np.uint16(0x4000)  # bf16 2.0
    low = np.uint16(0xC0A0)  # bf16 -5.0: off the clip for any bias here
    cells = []
    cells += [(0, t, 0) for t in (1, 9)]                       # block 0, channel 0: two steps
    cells += [(0, t, 23) for t in (16, 18, 21, 27, 31)]        # block 1, channel 23: five steps
    cells += [(0, t, 47) for t in range(32, 48, 2)]            # block 2, channel 47: eight steps
    cells += [(1, t, 64) for t in range(48, 64)]               # block 3, batch 1, channel 64: every step
    cells += [(0, t, 33) for t in (50, 55, 60)]                # block 3, channel 33: three steps
    cells += [(1, t, 127) for t in (64, 79)]                   # block 4, last channel: first and last step
    cells += [(1, 3, 100), (1, 3, 101), (1, 20, 7), (1, 40, 90)]  # two channels / single steps elsewhere
    for b, t, e in cells:
        dt[b, t, e] = low
    st_in = None
    if with_state:
        rng = np.random.Generator(np.random.PCG64(31))
        st_in = rng.standard_normal((2, 128, 16)).astype(np.float32)
    y, st = _run(w, state_in=torch.from_numpy(st_in).to(DEV) if with_state else None, dt_softplus=softplus)
    yo, ho, _ = _oracle(w, state_in=st_in.astype(np.float64) if with_state else None, dt_softplus=softplus)
    check(np64(y), yo, TOL, "blocked y, one channel off the clip")
    check(np64(st), ho, TOL, "blocked state, one channel off the clip")
