"""GPU parity of ssm_linear_fwd (the layer's projections on the matrix cores)
against the float64 oracle's `linear`, through the C ABI.  Inputs are exact
bf16 (or fp32) values and the accumulation is fp32: max|err| <= 1e-5
max|out| (plus the 2^-8 |out| format bound for a bf16 output)."""
import numpy as np
import pytest
import torch

import selective_state_space_03_amd as ssm
import ssm_workloads as W
from gpu_util import DEV, check, np64
from oracle import ssm_oracle as O

pytestmark = pytest.mark.gpu
TOL = 1e-5


def _bf16(shape, seed, scale=1.0):
    rng = np.random.Generator(np.random.PCG64(seed))
    bits = W.bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    return t, W.bf16_to_f32(bits).astype(np.float64)


@pytest.mark.parametrize("M,K,N", [(1, 8, 4), (300, 520, 388), (128, 64, 128), (257, 1000, 132), (64, 2560, 640)])
@pytest.mark.parametrize("x_f32", [False, True])
@pytest.mark.parametrize("out_bf16", [False, True])
def test_linear_shapes(M, K, N, x_f32, out_bf16):
    """Ragged tiles in M, N and K (K not a multiple of the 64-wide K step)."""
    x, xr = _bf16((M, K), 1 + M + K)
    if x_f32:
        rng = np.random.Generator(np.random.PCG64(7 + K))
        xr = rng.standard_normal((M, K)).astype(np.float32)
        x = torch.from_numpy(xr).to(DEV)
        xr = xr.astype(np.float64)
    w, wr = _bf16((N, K), 2 + N, 1.0 / np.sqrt(K))
    out = ssm.linear_fwd(x, w, out_dtype=torch.bfloat16 if out_bf16 else torch.float32)
    torch.cuda.synchronize()
    check(np64(out), O.linear(xr, wr), TOL, f"linear {M}x{K}x{N}", out_bf16=out_bf16)


def test_linear_batched_leading_dims_and_zero_rows():
    x, xr = _bf16((2, 3, 96), 3)
    w, wr = _bf16((40, 96), 4)
    out = ssm.linear_fwd(x, w, out_dtype=torch.float32)
    torch.cuda.synchronize()
    check(np64(out), O.linear(xr, wr), TOL, "linear (2, 3, 96)")
    e = ssm.linear_fwd(torch.empty((0, 96), dtype=torch.bfloat16, device=DEV), w)
    torch.cuda.synchronize()
    assert e.shape == (0, 40)


@pytest.mark.parametrize("which", ["in_proj", "out_proj"])
def test_layer_projection_full_size(which):
    """The layer's projections at full size (2048 tokens; in_proj 2560 -> 15360
    from bf16, out_proj 7680 -> 2560 from fp32); oracle on 96 sampled rows."""
    if which == "in_proj":
        x, xr = _bf16((2048, 2560), 5)
        w, wr = _bf16((15360, 2560), 6, 1.0 / np.sqrt(2560))
    else:
        rng = np.random.Generator(np.random.PCG64(8))
        xn = rng.standard_normal((2048, 7680)).astype(np.float32)
        x, xr = torch.from_numpy(xn).to(DEV), xn.astype(np.float64)
        w, wr = _bf16((2560, 7680), 9, 1.0 / np.sqrt(7680))
    out = ssm.linear_fwd(x, w, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = np.random.Generator(np.random.PCG64(10)).choice(2048, 96, replace=False)
    got = np64(out[torch.from_numpy(rows).to(DEV)])
    check(got, O.linear(xr[rows], wr), TOL, f"{which} full size")


def test_linear_deterministic():
    x, _ = _bf16((300, 520), 11)
    w, _ = _bf16((388, 520), 12)
    a = ssm.linear_fwd(x, w, out_dtype=torch.float32)
    b = ssm.linear_fwd(x, w, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
