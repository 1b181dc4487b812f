"""forward_only_amd -- the 1.5-SPSA perturb / probe-weight / update path on MI355X.

A thin Python face over libzo.so (include/zo.h).  Each function below has the name of the
C entry point it calls and only marshals arguments: it checks that tensors live on the
current GPU with the expected dtype and are contiguous, then passes their device pointers
and torch's current HIP stream (the library itself rejects misaligned pointers and bad
sizes).  All arithmetic runs in the library's HIP kernels; there is no CPU path.

    ctx = zo_init(seed)
    zo_perturb(ctx, theta, offset, step, probe, +eps)      # theta + eps*z_probe, in place
    ...
    c = zo_probe_weights(ctx, Lp, Lm, L0, eps, delta)
    zo_update(ctx, theta, offset, step, c, eta)             # theta - eta * sum c_i z_i
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import (ZO_BF16, ZO_EHIP, ZO_EINVAL, ZO_ENOMEM, ZO_EUNSUPPORTED, ZO_FP32,  # noqa: F401
                   ZO_MAX_NPERT, ZO_NOALLOC_SCRATCH_BYTES, ZO_OK, ZO_WEIGHTS_POWER, ZO_WEIGHTS_PRECOND,
                   ZO_WEIGHTS_SPSA_MEAN, ZOError)

__all__ = [
    "Context", "ZOError", "zo_init", "zo_destroy", "zo_bits_stride", "zo_gen_probes",
    "zo_perturb", "zo_perturb2", "zo_probe_weights", "zo_probe_weights_ex", "zo_update",
    "zo_restore_update", "zo_nonfinite_count", "zo_reset_nonfinite", "zo_quad_loss",
    "zo_quad_loss_probes",
    "zo_lowrank_quad_loss", "zo_mlp_workspace_bytes", "zo_mlp_loss", "zo_mlp_loss_perturbed",
    "zo_mlp_loss_pair", "zo_mlp_probes_workspace_bytes", "zo_mlp_loss_probes",
    "zo_mlp_loss_pair_noalloc", "zo_stream_rmw", "zo_tune_placement", "zo_set_slice_bytes",
    "zo_get_slice_bytes", "library_path",
]


def library_path() -> str:
    return _lib.LIB_PATH


class Context:
    """Owns one zo_ctx (probe seed, device counter); closes it on close() / GC."""

    def __init__(self, handle: int, seed: int):
        self._h = handle
        self.seed = seed

    @property
    def handle(self) -> int:
        if not self._h:
            raise ValueError("context is closed")
        return self._h

    def close(self) -> None:
        if self._h:
            h, self._h = self._h, None
            _lib.check(_lib.lib().zo_destroy(h), "zo_destroy")

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return ZO_FP32
    if t.dtype == torch.bfloat16:
        return ZO_BF16
    raise TypeError(f"parameters must be float32 or bfloat16, got {t.dtype}")


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if t.device.index is not None and t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} is on {t.device}, not on the current device "
                         f"cuda:{torch.cuda.current_device()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _row(bits, n: int, name: str = "bits"):
    """Device pointer of one probe's packed row over n params: a 1-D uint8 tensor of exactly
    zo_bits_stride(n) bytes (the library reads that many from the pointer), or None."""
    if bits is None:
        return None
    p = _dev(bits, name, torch.uint8)
    if bits.dim() != 1 or bits.numel() != zo_bits_stride(n):
        raise ValueError(f"{name} must be one packed row of {zo_bits_stride(n)} bytes, got "
                         f"shape {tuple(bits.shape)}")
    return p


def _rows(bits, npert: int, n: int):
    """Device pointer of n_pert packed rows over n params: a (n_pert, zo_bits_stride(n))
    uint8 tensor (row i at i * stride), or None."""
    if bits is None:
        return None
    p = _dev(bits, "bits", torch.uint8)
    if tuple(bits.shape) != (npert, zo_bits_stride(n)):
        raise ValueError(f"bits must have shape ({npert}, {zo_bits_stride(n)}), got "
                         f"{tuple(bits.shape)}")
    return p


def zo_init(seed: int) -> Context:
    h = ctypes.c_void_p()
    _lib.check(_lib.lib().zo_init(int(seed) & (2 ** 64 - 1), ctypes.byref(h)), "zo_init")
    return Context(h.value, int(seed))


def zo_destroy(ctx: Context) -> None:
    ctx.close()


def zo_bits_stride(n: int) -> int:
    return int(_lib.lib().zo_bits_stride(int(n)))


def zo_gen_probes(ctx: Context, step: int, probe0: int, n_probes: int, offset: int, n: int,
                  out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Packed sign rows, uint8 tensor of shape (n_probes, zo_bits_stride(n))."""
    stride = zo_bits_stride(n)
    if out is None:
        out = torch.empty((n_probes, stride), dtype=torch.uint8, device="cuda")
    if out.numel() < n_probes * stride:
        raise ValueError("out is too small")
    _lib.check(_lib.lib().zo_gen_probes(ctx.handle, step, probe0, n_probes, offset, n,
                                        _dev(out, "out", torch.uint8), _stream(stream)),
               "zo_gen_probes")
    return out


def zo_perturb(ctx: Context, theta: torch.Tensor, offset: int, step: int, probe: int,
               alpha: float, bits: torch.Tensor | None = None, stream=None) -> None:
    """theta <- theta + alpha * z_probe in place (theta fp32 or bf16)."""
    bp = _row(bits, theta.numel())
    _lib.check(_lib.lib().zo_perturb(ctx.handle, _dev(theta, "theta"), _dtype_code(theta),
                                     offset, theta.numel(), step, probe, float(alpha), bp,
                                     _stream(stream)), "zo_perturb")


def zo_perturb2(ctx: Context, theta: torch.Tensor, offset: int, step: int, probe_a: int,
                alpha_a: float, probe_b: int, alpha_b: float,
                bits_a: torch.Tensor | None = None, bits_b: torch.Tensor | None = None,
                stream=None) -> None:
    """theta <- theta + (+/-alpha_a) + (+/-alpha_b) in one pass (probes a and b)."""
    if (bits_a is None) != (bits_b is None):
        raise ValueError("give both packed rows or neither")
    pa = _row(bits_a, theta.numel(), "bits_a")
    pb = _row(bits_b, theta.numel(), "bits_b")
    _lib.check(_lib.lib().zo_perturb2(ctx.handle, _dev(theta, "theta"), _dtype_code(theta),
                                      offset, theta.numel(), step, probe_a, float(alpha_a),
                                      probe_b, float(alpha_b), pa, pb, _stream(stream)),
               "zo_perturb2")


def zo_probe_weights(ctx: Context, Lp: torch.Tensor, Lm: torch.Tensor, L0: torch.Tensor,
                     eps: float, delta: float, out: torch.Tensor | None = None,
                     stream=None) -> torch.Tensor:
    """c_i = g_i / max(|h_i|, delta) from float64 GPU tensors Lp[n], Lm[n], L0[1]."""
    n = Lp.numel()
    if Lm.numel() != n or L0.numel() < 1:
        raise ValueError("Lp and Lm must have the same length, L0 one element")
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device="cuda")
    if out.numel() < n:
        raise ValueError("out is too small")
    _lib.check(_lib.lib().zo_probe_weights(
        ctx.handle, _dev(Lp, "Lp", torch.float64), _dev(Lm, "Lm", torch.float64),
        _dev(L0, "L0", torch.float64), n, float(eps), float(delta),
        _dev(out, "out", torch.float32), _stream(stream)), "zo_probe_weights")
    return out


def zo_probe_weights_ex(ctx: Context, Lp: torch.Tensor, Lm: torch.Tensor,
                        L0: torch.Tensor | None, eps: float, delta: float, mode: int,
                        power: float = 1.0, out: torch.Tensor | None = None,
                        stream=None) -> torch.Tensor:
    """Weights in one of the pages' forms (ZO_WEIGHTS_PRECOND / _POWER / _SPSA_MEAN)."""
    n = Lp.numel()
    if Lm.numel() != n:
        raise ValueError("Lp and Lm must have the same length")
    if L0 is not None and L0.numel() < 1:
        raise ValueError("L0 must hold one element")
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device="cuda")
    if out.numel() < n:
        raise ValueError("out is too small")
    p0 = None if L0 is None else _dev(L0, "L0", torch.float64)
    _lib.check(_lib.lib().zo_probe_weights_ex(
        ctx.handle, _dev(Lp, "Lp", torch.float64), _dev(Lm, "Lm", torch.float64), p0, n,
        float(eps), float(delta), int(mode), float(power), _dev(out, "out", torch.float32),
        _stream(stream)), "zo_probe_weights_ex")
    return out


def zo_update(ctx: Context, theta: torch.Tensor, offset: int, step: int, c: torch.Tensor,
              eta: float, bits: torch.Tensor | None = None, stream=None) -> None:
    """theta <- theta - eta * sum_i c_i z_i in place; bits: (n_pert, stride) rows or None."""
    npert = c.numel()
    bp = _rows(bits, npert, theta.numel())
    _lib.check(_lib.lib().zo_update(ctx.handle, _dev(theta, "theta"), _dtype_code(theta),
                                    offset, theta.numel(), step, _dev(c, "c", torch.float32),
                                    npert, float(eta), bp, _stream(stream)), "zo_update")


def zo_restore_update(ctx: Context, theta: torch.Tensor, offset: int, step: int,
                      restore_probe: int, restore_alpha: float, c: torch.Tensor, eta: float,
                      bits: torch.Tensor | None = None, stream=None) -> None:
    """zo_perturb(restore_probe, restore_alpha) then zo_update, in one pass (bit-identical
    to the two calls)."""
    npert = c.numel()
    bp = _rows(bits, npert, theta.numel())
    _lib.check(_lib.lib().zo_restore_update(
        ctx.handle, _dev(theta, "theta"), _dtype_code(theta), offset, theta.numel(), step,
        int(restore_probe), float(restore_alpha), _dev(c, "c", torch.float32), npert,
        float(eta), bp, _stream(stream)), "zo_restore_update")


def zo_nonfinite_count(ctx: Context, stream=None) -> int:
    v = ctypes.c_uint32()
    _lib.check(_lib.lib().zo_nonfinite_count(ctx.handle, _stream(stream), ctypes.byref(v)),
               "zo_nonfinite_count")
    return int(v.value)


def zo_reset_nonfinite(ctx: Context, stream=None) -> None:
    _lib.check(_lib.lib().zo_reset_nonfinite(ctx.handle, _stream(stream)), "zo_reset_nonfinite")


def zo_quad_loss(ctx: Context, theta: torch.Tensor, a: torch.Tensor,
                 out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """1/2 sum a_j theta_j^2 in fp64 into a one-element float64 GPU tensor."""
    if a.numel() != theta.numel():
        raise ValueError("a and theta must have the same length")
    if out is None:
        out = torch.empty(1, dtype=torch.float64, device="cuda")
    _lib.check(_lib.lib().zo_quad_loss(ctx.handle, _dev(theta, "theta"), _dtype_code(theta),
                                       _dev(a, "a", torch.float32), theta.numel(),
                                       _dev(out, "out", torch.float64), _stream(stream)),
               "zo_quad_loss")
    return out


def zo_quad_loss_probes(ctx: Context, theta: torch.Tensor, a: torch.Tensor, offset: int,
                        step: int, probe0: int, n_probes: int, alpha: float,
                        bits: torch.Tensor | None = None, out_plus: torch.Tensor | None = None,
                        out_minus: torch.Tensor | None = None,
                        out_clean: torch.Tensor | None = None, stream=None):
    """The quadratic loss at theta +/- alpha * z_i for probes probe0 .. probe0 + n_probes - 1,
    each probe applied while theta is read (theta is not written); returns (out_plus,
    out_minus), float64 tensors of n_probes.  bits: None or (n_probes, zo_bits_stride(theta))
    rows.  out_clean (one float64, optional) also receives the loss at theta itself, equal to
    zo_quad_loss, from the first pass over theta."""
    if a.numel() != theta.numel():
        raise ValueError("a and theta must have the same length")
    if out_clean is not None and out_clean.numel() < 1:
        raise ValueError("out_clean is too small")
    for name, o in (("out_plus", out_plus), ("out_minus", out_minus)):
        if o is not None and o.numel() < n_probes:
            raise ValueError(f"{name} is too small")
    if out_plus is None:
        out_plus = torch.empty(max(n_probes, 1), dtype=torch.float64, device="cuda")
    if out_minus is None:
        out_minus = torch.empty(max(n_probes, 1), dtype=torch.float64, device="cuda")
    _lib.check(_lib.lib().zo_quad_loss_probes(
        ctx.handle, _dev(theta, "theta"), _dtype_code(theta), _dev(a, "a", torch.float32),
        offset, theta.numel(), step, probe0, n_probes, float(alpha),
        _rows(bits, n_probes, theta.numel()), _dev(out_plus, "out_plus", torch.float64),
        _dev(out_minus, "out_minus", torch.float64),
        None if out_clean is None else _dev(out_clean, "out_clean", torch.float64),
        _stream(stream)), "zo_quad_loss_probes")
    return out_plus, out_minus


def zo_lowrank_quad_loss(ctx: Context, theta: torch.Tensor, a: torch.Tensor, U: torch.Tensor,
                         out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """1/2 sum a_j theta_j^2 + 1/2 ||U theta||^2 (U: [r, n] float32) into a float64 tensor."""
    n = theta.numel()
    if a.numel() != n or (U.numel() and U.shape[-1] != n):
        raise ValueError("a must have n entries and U shape (r, n)")
    r = U.numel() // n if n else 0
    if out is None:
        out = torch.empty(1, dtype=torch.float64, device="cuda")
    up = _dev(U, "U", torch.float32) if U.numel() else None
    _lib.check(_lib.lib().zo_lowrank_quad_loss(ctx.handle, _dev(theta, "theta"),
                                               _dtype_code(theta), _dev(a, "a", torch.float32),
                                               up, r, n, _dev(out, "out", torch.float64),
                                               _stream(stream)), "zo_lowrank_quad_loss")
    return out


def zo_mlp_workspace_bytes(batch: int, d_in: int, d_hid: int, d_out: int) -> int:
    return int(_lib.lib().zo_mlp_workspace_bytes(batch, d_in, d_hid, d_out))


def _mlp_args(params, X, labels, d_hid, d_out, workspace, out):
    batch, d_in = X.shape
    nparams = d_hid * d_in + d_hid + d_out * d_hid + d_out
    if params.numel() != nparams:
        raise ValueError(f"params must hold {nparams} values")
    if labels.numel() != batch:
        raise ValueError("one label per row")
    need = zo_mlp_workspace_bytes(batch, d_in, d_hid, d_out)
    if workspace is None:
        workspace = torch.empty(max(need, 8), dtype=torch.uint8, device="cuda")
    if out is None:
        out = torch.empty(1, dtype=torch.float64, device="cuda")
    return (batch, d_in, _dev(params, "params", torch.float32), _dev(X, "X", torch.float32),
            _dev(labels, "labels", torch.int64), workspace, _dev(workspace, "workspace"),
            workspace.numel() * workspace.element_size(), out)


def zo_mlp_loss(ctx: Context, params: torch.Tensor, X: torch.Tensor, labels: torch.Tensor,
                d_hid: int, d_out: int, workspace: torch.Tensor | None = None,
                out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Mean cross-entropy of the MLP at `params` into a one-element float64 GPU tensor."""
    batch, d_in, pp, px, pl, ws, pw, wbytes, out = _mlp_args(params, X, labels, d_hid, d_out,
                                                             workspace, out)
    _lib.check(_lib.lib().zo_mlp_loss(ctx.handle, pp, px, pl, batch, d_in, d_hid, d_out, pw,
                                      wbytes, _dev(out, "out", torch.float64), _stream(stream)),
               "zo_mlp_loss")
    return out


def zo_mlp_loss_perturbed(ctx: Context, params: torch.Tensor, offset: int, step: int,
                          probe: int, alpha: float, X: torch.Tensor, labels: torch.Tensor,
                          d_hid: int, d_out: int, bits: torch.Tensor | None = None,
                          workspace: torch.Tensor | None = None,
                          out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """The MLP loss at params + alpha * z_probe, without writing params."""
    batch, d_in, pp, px, pl, ws, pw, wbytes, out = _mlp_args(params, X, labels, d_hid, d_out,
                                                             workspace, out)
    bp = _row(bits, params.numel())
    _lib.check(_lib.lib().zo_mlp_loss_perturbed(
        ctx.handle, pp, offset, step, probe, float(alpha), bp, px, pl, batch, d_in, d_hid,
        d_out, pw, wbytes, _dev(out, "out", torch.float64), _stream(stream)),
        "zo_mlp_loss_perturbed")
    return out


def zo_mlp_loss_pair(ctx: Context, params: torch.Tensor, offset: int, step: int, probe: int,
                     alpha: float, X: torch.Tensor, labels: torch.Tensor, d_hid: int,
                     d_out: int, bits: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None, out_plus: torch.Tensor | None = None,
                     out_minus: torch.Tensor | None = None, stream=None):
    """The MLP losses at params + alpha * z_probe and params - alpha * z_probe, in one
    launch sequence, without writing params; returns (out_plus, out_minus)."""
    batch, d_in, pp, px, pl, ws, pw, wbytes, out_plus = _mlp_args(params, X, labels, d_hid,
                                                                  d_out, workspace, out_plus)
    if out_minus is None:
        out_minus = torch.empty(1, dtype=torch.float64, device="cuda")
    bp = _row(bits, params.numel())
    _lib.check(_lib.lib().zo_mlp_loss_pair(
        ctx.handle, pp, offset, step, probe, float(alpha), bp, px, pl, batch, d_in, d_hid,
        d_out, pw, wbytes, _dev(out_plus, "out_plus", torch.float64),
        _dev(out_minus, "out_minus", torch.float64), _stream(stream)), "zo_mlp_loss_pair")
    return out_plus, out_minus


def zo_mlp_probes_workspace_bytes(batch: int, d_in: int, d_hid: int, d_out: int,
                                  n_probes: int) -> int:
    return int(_lib.lib().zo_mlp_probes_workspace_bytes(batch, d_in, d_hid, d_out, n_probes))


def zo_mlp_loss_probes(ctx: Context, params: torch.Tensor, offset: int, step: int, probe0: int,
                       n_probes: int, alpha: float, X: torch.Tensor, labels: torch.Tensor,
                       d_hid: int, d_out: int, bits: torch.Tensor | None = None,
                       workspace: torch.Tensor | None = None,
                       out_plus: torch.Tensor | None = None,
                       out_minus: torch.Tensor | None = None,
                       out_clean: torch.Tensor | None = None, stream=None):
    """The MLP losses at params +/- alpha * z_i for probes probe0 .. probe0 + n_probes - 1
    (up to 64 per launch sequence), without writing params; returns (out_plus, out_minus),
    float64 tensors of n_probes.  bits: None or (n_probes, zo_bits_stride(params)) rows.
    out_clean (one float64, optional) also receives the loss at params itself, equal to
    zo_mlp_loss, from the first launch sequence."""
    if out_clean is not None and out_clean.numel() < 1:
        raise ValueError("out_clean is too small")
    batch, d_in = X.shape
    if params.numel() != d_hid * d_in + d_hid + d_out * d_hid + d_out:
        raise ValueError("params must hold the MLP's parameters")
    if labels.numel() != batch:
        raise ValueError("one label per row")
    need = zo_mlp_probes_workspace_bytes(batch, d_in, d_hid, d_out, n_probes)
    if workspace is None:
        workspace = torch.empty(max(need, 8), dtype=torch.uint8, device="cuda")
    for name, o in (("out_plus", out_plus), ("out_minus", out_minus)):
        if o is not None and o.numel() < n_probes:
            raise ValueError(f"{name} is too small")
    if out_plus is None:
        out_plus = torch.empty(n_probes, dtype=torch.float64, device="cuda")
    if out_minus is None:
        out_minus = torch.empty(n_probes, dtype=torch.float64, device="cuda")
    _lib.check(_lib.lib().zo_mlp_loss_probes(
        ctx.handle, _dev(params, "params", torch.float32), offset, step, probe0, n_probes,
        float(alpha), _rows(bits, n_probes, params.numel()), _dev(X, "X", torch.float32),
        _dev(labels, "labels", torch.int64), batch, d_in, d_hid, d_out,
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _dev(out_plus, "out_plus", torch.float64), _dev(out_minus, "out_minus", torch.float64),
        None if out_clean is None else _dev(out_clean, "out_clean", torch.float64),
        _stream(stream)), "zo_mlp_loss_probes")
    return out_plus, out_minus


def zo_mlp_loss_pair_noalloc(ctx: Context, params: torch.Tensor, offset: int, step: int,
                             probe: int, alpha: float, X: torch.Tensor, labels: torch.Tensor,
                             d_hid: int, d_out: int, out_plus: torch.Tensor,
                             out_minus: torch.Tensor, bits: torch.Tensor | None = None,
                             stream=None) -> None:
    """zo_mlp_loss_pair with the library's static per-GPU scratch instead of a workspace:
    the call allocates nothing (the caller passes both one-element float64 outputs)."""
    batch, d_in = X.shape
    if params.numel() != d_hid * d_in + d_hid + d_out * d_hid + d_out:
        raise ValueError("params must hold the MLP's parameters")
    if labels.numel() != batch:
        raise ValueError("one label per row")
    _lib.check(_lib.lib().zo_mlp_loss_pair_noalloc(
        ctx.handle, _dev(params, "params", torch.float32), offset, step, probe, float(alpha),
        _row(bits, params.numel()), _dev(X, "X", torch.float32),
        _dev(labels, "labels", torch.int64), batch, d_in, d_hid, d_out,
        _dev(out_plus, "out_plus", torch.float64), _dev(out_minus, "out_minus", torch.float64),
        _stream(stream)), "zo_mlp_loss_pair_noalloc")


def zo_stream_rmw(ctx: Context, buf: torch.Tensor, mask: int = 0, stream=None) -> None:
    """Diagnostic: every 32-bit word of `buf` <- word ^ mask in place, in the perturb
    kernel's streaming order (mask 0: unchanged; timed, the in-place bandwidth ceiling of
    the memory `buf` occupies)."""
    nbytes = buf.numel() * buf.element_size()
    _lib.check(_lib.lib().zo_stream_rmw(ctx.handle, _dev(buf, "buf"), nbytes, int(mask) & 0xFFFFFFFF,
                                        _stream(stream)), "zo_stream_rmw")


def zo_tune_placement(ctx: Context, buf: torch.Tensor, stream=None) -> dict:
    """Time a pass over `buf` as one launch and as 1 GiB slices (contents unchanged), keep
    the faster form in the context; returns {"slice_bytes", "gbps_whole", "gbps_sliced"}."""
    sl, gw, gs = ctypes.c_uint64(), ctypes.c_double(), ctypes.c_double()
    nbytes = buf.numel() * buf.element_size()
    _lib.check(_lib.lib().zo_tune_placement(ctx.handle, _dev(buf, "buf"), nbytes,
                                            _stream(stream), ctypes.byref(sl), ctypes.byref(gw),
                                            ctypes.byref(gs)), "zo_tune_placement")
    return {"slice_bytes": int(sl.value), "gbps_whole": gw.value, "gbps_sliced": gs.value}


def zo_set_slice_bytes(ctx: Context, slice_bytes: int) -> None:
    """Issue the context's perturb passes per slice of `slice_bytes` (0: one launch)."""
    _lib.check(_lib.lib().zo_set_slice_bytes(ctx.handle, int(slice_bytes)), "zo_set_slice_bytes")


def zo_get_slice_bytes(ctx: Context) -> int:
    return int(_lib.lib().zo_get_slice_bytes(ctx.handle))
