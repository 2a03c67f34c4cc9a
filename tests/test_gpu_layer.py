"""GPU parity of ssm_layer_fwd (in_proj, conv + SiLU, x_proj, scan with the
gate, out_proj) against the float64 oracle's ssm_layer_forward, through the C
ABI.  bf16 inputs and weights, fp32 activations and state: max|err| <= 2e-3
max|out| (plus the 2^-8 |out| format bound for a bf16 output); state and
conv cache likewise (the cache holds fp32 copies of in_proj outputs)."""
import numpy as np
import pytest
import torch

import ssm_workloads as W
from gpu_util import DEV, check, layer_gpu, layer_oracle, np64

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _small(**kw):
    base = dict(batch=2, seqlen=100, d_model=64, dim=256, d_state=16, seed=12)
    base.update(kw)
    return W.layer_prefill(**base)


@pytest.mark.parametrize("seqlen", [1, 3, 100, 200])
def test_layer_small(seqlen):
    """Token counts that leave partial 64-token tiles and sequences shorter
    than the conv window."""
    w = _small(seqlen=seqlen)
    out, st, cc = layer_gpu(w)
    oo, so, co = layer_oracle(w)
    check(np64(out), oo, TOL, f"layer out L={seqlen}")
    check(np64(st), so, TOL, f"layer state L={seqlen}")
    check(np64(cc), co, TOL, f"layer cache L={seqlen}")


def test_layer_bf16_out_and_wider():
    w = _small(batch=1, seqlen=300, d_model=512, dim=768)
    out, st, _ = layer_gpu(w, out_dtype=torch.bfloat16)
    oo, so, _ = layer_oracle(w)
    check(np64(out), oo, TOL, "layer out bf16", out_bf16=True)
    check(np64(st), so, TOL, "layer state")


def test_layer_prefill_split_matches_one_pass():
    """Layer over 70 tokens, then over the next 60 from the returned conv cache
    and state, against the oracle over all 130 tokens."""
    w = _small(seqlen=130)
    o1, s1, c1 = layer_gpu(w, tokens=slice(0, 70))
    o2, s2, c2 = layer_gpu(w, tokens=slice(70, 130), cache_in=c1, state_in=s1)
    oo, so, co = layer_oracle(w)
    check(np64(torch.cat([o1, o2], 1)), oo, TOL, "layer split out")
    check(np64(s2), so, TOL, "layer split state")
    check(np64(c2), co, TOL, "layer split cache")


def test_layer_deterministic():
    w = _small()
    a, sa, _ = layer_gpu(w)
    b, sb, _ = layer_gpu(w)
    assert torch.equal(a, b) and torch.equal(sa, sb)


def test_layer_full_size():
    """The Axon-SSM layer at the page's sizes: batch 1, 2048 tokens, D 2560,
    E 7680, N 16, random weights; the whole output against the oracle."""
    w = W.layer_prefill()
    out, st, cc = layer_gpu(w, out_dtype=torch.bfloat16)
    oo, so, co = layer_oracle(w)
    check(np64(out), oo, TOL, "layer full out", out_bf16=True)
    check(np64(st), so, TOL, "layer full state")
    check(np64(cc), co, TOL, "layer full cache")
