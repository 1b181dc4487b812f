"""zo_mlp_loss_pair_noalloc against zo_mlp_loss_pair, through the C ABI.

The allocation-free entry point keeps the partial logits and row losses in the library's
static per-GPU scratch instead of a caller workspace; it runs the same kernels, so its two
losses must equal the workspace call's bit for bit.  Two calls in a row on one context (the
scratch keeps the first call's contents), the second on a smaller problem, and a shape
whose workspace would exceed the scratch is refused before anything runs.
"""
import ctypes

import numpy as np
import pytest
import torch

import forward_only_amd as zo
from forward_only_amd import _lib

pytestmark = pytest.mark.gpu


def _problem(batch, d_in, d_hid, d_out, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    M = d_hid * d_in + d_hid + d_out * d_hid + d_out
    theta = torch.from_numpy((rng.standard_normal(M) * 0.02).astype(np.float32)).cuda()
    X = torch.from_numpy(rng.standard_normal((batch, d_in)).astype(np.float32)).cuda()
    y = torch.from_numpy(rng.integers(0, d_out, batch).astype(np.int64)).cuda()
    return theta, X, y


def _noalloc(ctx, theta, X, y, d_hid, d_out, step, probe, alpha, bits, out):
    batch, d_in = X.shape
    return _lib.lib().zo_mlp_loss_pair_noalloc(
        ctx.handle, theta.data_ptr(), 0, step, probe, ctypes.c_float(alpha),
        None if bits is None else bits.data_ptr(), X.data_ptr(), y.data_ptr(), batch, d_in,
        d_hid, d_out, out.data_ptr(), out.data_ptr() + 8,
        torch.cuda.current_stream().cuda_stream)


def _with_workspace(ctx, theta, X, y, d_hid, d_out, step, probe, alpha, bits, out):
    batch, d_in = X.shape
    ws = torch.empty(zo.zo_mlp_workspace_bytes(batch, d_in, d_hid, d_out), dtype=torch.uint8,
                     device="cuda")
    st = _lib.lib().zo_mlp_loss_pair(
        ctx.handle, theta.data_ptr(), 0, step, probe, ctypes.c_float(alpha),
        None if bits is None else bits.data_ptr(), X.data_ptr(), y.data_ptr(), batch, d_in,
        d_hid, d_out, ws.data_ptr(), ws.numel(), out.data_ptr(), out.data_ptr() + 8,
        torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return st


@pytest.mark.parametrize("mode", ["regen", "bits"])
def test_noalloc_pair_equals_workspace_pair_twice(mode):
    ctx = zo.zo_init(3)
    # the workload's shape, then smaller ones (32 x 32 tiles, then 16 x 16 tiles)
    shapes = [(128, 768, 3072, 2), (32, 48, 64, 3), (48, 32, 48, 5)]
    for i, (batch, d_in, d_hid, d_out) in enumerate(shapes):
        print(f"[noalloc] {mode} call {i}: {batch}x{d_in}->{d_hid}->{d_out}", flush=True)
        theta, X, y = _problem(batch, d_in, d_hid, d_out, seed=40 + i)
        bits = (zo.zo_gen_probes(ctx, 5, 7, 1, 0, theta.numel())[0] if mode == "bits"
                else None)
        a = torch.full((2,), np.nan, dtype=torch.float64, device="cuda")
        b = torch.full((2,), -1.0, dtype=torch.float64, device="cuda")
        assert _noalloc(ctx, theta, X, y, d_hid, d_out, 5, 7, 1e-3, bits, a) == zo.ZO_OK
        torch.cuda.synchronize()
        assert _with_workspace(ctx, theta, X, y, d_hid, d_out, 5, 7, 1e-3, bits, b) == zo.ZO_OK
        got, want = a.cpu().numpy(), b.cpu().numpy()
        assert np.all(np.isfinite(got)), got
        assert np.array_equal(got.view(np.uint64), want.view(np.uint64)), (got, want)
        assert got[0] != got[1]                       # the two signs give two losses
    ctx.close()


def test_noalloc_pair_binding_and_limits():
    ctx = zo.zo_init(3)
    theta, X, y = _problem(32, 48, 64, 3, seed=9)
    op = torch.empty(1, dtype=torch.float64, device="cuda")
    om = torch.empty(1, dtype=torch.float64, device="cuda")
    zo.zo_mlp_loss_pair_noalloc(ctx, theta, 0, 1, 2, 1e-3, X, y, 64, 3, op, om)
    lp, lm = zo.zo_mlp_loss_pair(ctx, theta, 0, 1, 2, 1e-3, X, y, 64, 3)
    assert (op.item(), om.item()) == (lp.item(), lm.item())
    # a problem whose pair workspace exceeds the 1 MiB scratch is refused up front
    big = (256, 16, 4096, 2)
    assert zo.zo_mlp_workspace_bytes(*big) > zo.ZO_NOALLOC_SCRATCH_BYTES
    L = _lib.lib()
    st = L.zo_mlp_loss_pair_noalloc(ctx.handle, theta.data_ptr(), 0, 0, 0, ctypes.c_float(1e-3),
                                    None, X.data_ptr(), y.data_ptr(), *big, op.data_ptr(),
                                    om.data_ptr(), None)
    assert st == zo.ZO_EUNSUPPORTED
    st = L.zo_mlp_loss_pair_noalloc(ctx.handle, theta.data_ptr(), 0, 0, 0, ctypes.c_float(1e-3),
                                    None, X.data_ptr(), y.data_ptr(), 32, 48, 64, 3,
                                    op.data_ptr(), None, None)
    assert st == zo.ZO_EINVAL                         # no -alpha output
    torch.cuda.synchronize()
    ctx.close()
