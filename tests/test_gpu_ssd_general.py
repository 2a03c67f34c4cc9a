"""GPU parity of ssm_chunk_scan_fwd on the shapes outside the tuned matrix-core
kernel (other chunk sizes, d_state, headdims, fp32 x/B/C/z), which run the
vector-ALU chunked kernels, against the float64 oracle's chunked form and its
sequential recurrence.  Tolerances: 2e-3 max|out| with bf16 inputs, 1e-5 with
fp32 inputs (fp32 output in both)."""
import numpy as np
import pytest
import torch

import ssm_workloads as W
from gpu_util import DEV, check, np64, ssd_gpu, ssd_oracle

pytestmark = pytest.mark.gpu
TOL_BF16 = 2e-3
TOL_F32 = 1e-5


def _w(**kw):
    base = dict(batch=2, seqlen=1000, nheads=4, headdim=48, ngroups=2, d_state=64, chunk_size=128, unsaturated=True)
    base.update(kw)
    return W.ssd_long(**base)


def _to_f32(w, keys=("x", "B", "C", "z")):
    for k in keys:
        if k in w.arrays and k in w.bf16:
            w.arrays[k] = W.bf16_to_f32(w.arrays[k])
            w.bf16.discard(k)
    return w


def _both(w, tol):
    """The GPU result against the oracle's chunked form and its recurrence."""
    out, st = ssd_gpu(w)
    for sequential in (False, True):
        oo, so = ssd_oracle(w, sequential=sequential)
        check(np64(out), oo, tol, f"{w.name} out (sequential={sequential})")
        check(np64(st), so, tol, f"{w.name} state (sequential={sequential})")
    return out, st


@pytest.mark.parametrize("chunk", [64, 256])
def test_chunk_sizes(chunk):
    """chunk_size 64 and 256 (bf16 x/B/C, N 64), a ragged last chunk, 2 groups."""
    _both(_w(chunk_size=chunk), TOL_BF16)


@pytest.mark.parametrize("n", [16, 32, 128])
def test_state_sizes(n):
    """d_state 16, 32 and 128 at chunk 128 (bf16)."""
    _both(_w(d_state=n), TOL_BF16)


@pytest.mark.parametrize("chunk,n", [(128, 64), (64, 32), (256, 128)])
def test_fp32_inputs(chunk, n):
    """fp32 x, B and C (the tuned kernel's own shape too: N 64, chunk 128),
    held to the fp32 bound."""
    _both(_to_f32(_w(chunk_size=chunk, d_state=n)), TOL_F32)


def test_odd_shapes_gate_state_and_per_channel_D():
    """chunk 48, d_state 24, headdim 40 (no multiple of 16), a gate in fp32, a
    starting state and a per-channel D, bf16 output; 3 groups of 2 heads."""
    w = _w(chunk_size=48, d_state=24, headdim=40, nheads=6, ngroups=3, seqlen=500, gated=True)
    _to_f32(w, keys=("z",))
    rng = np.random.Generator(np.random.PCG64(51))
    st_in = rng.standard_normal((2, 6, 40, 24)).astype(np.float32)
    Dpc = rng.standard_normal((6, 40)).astype(np.float32)
    out, st = ssd_gpu(w, state_in=torch.from_numpy(st_in).to(DEV), D_override=Dpc, out_dtype=torch.bfloat16)
    oo, so = ssd_oracle(w, state_in=st_in, D_override=Dpc)
    check(np64(out), oo, TOL_BF16, "odd shapes out", out_bf16=True)
    check(np64(st), so, TOL_BF16, "odd shapes state")


def test_segments_have_no_effect_and_results_repeat():
    w = _w(chunk_size=64)
    o1, s1 = ssd_gpu(w)
    o2, s2 = ssd_gpu(w, segments=3)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


@pytest.mark.parametrize("seqlen", [0, 1, 63, 64, 65])
def test_short_sequences_from_a_state(seqlen):
    """No token (the state passes through), and sequences around one chunk of 64."""
    w = _w(chunk_size=64, seqlen=seqlen, d_state=32)
    rng = np.random.Generator(np.random.PCG64(52))
    st_in = rng.standard_normal((2, 4, 48, 32)).astype(np.float32)
    out, st = ssd_gpu(w, state_in=torch.from_numpy(st_in).to(DEV))
    if seqlen == 0:
        assert torch.equal(st, torch.from_numpy(st_in).to(DEV))
        return
    oo, so = ssd_oracle(w, state_in=st_in, sequential=True)
    check(np64(out), oo, TOL_BF16, f"L={seqlen} out")
    check(np64(st), so, TOL_BF16, f"L={seqlen} state")


def test_long_sequence_sampled_heads():
    """A long sequence at the layer's width: L 16384, 80 heads x 96, N 128,
    chunk 256 (bf16); oracle on heads 0, 41 and 79."""
    w = W.ssd_long(seqlen=16384, d_state=128, chunk_size=256, unsaturated=True)
    heads = [0, 41, 79]
    out, st = ssd_gpu(w)
    oo, so = ssd_oracle(w, heads=heads)
    hidx = torch.tensor(heads, device=DEV)
    check(np64(out.index_select(2, hidx)), oo, TOL_BF16, "long out")
    check(np64(st.index_select(1, hidx)), so, TOL_BF16, "long state")
