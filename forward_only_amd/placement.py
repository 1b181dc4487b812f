"""Placement of a large parameter buffer in HBM.

The streaming bandwidth of a large allocation depends on the physical memory the driver
gives it, which neither the kernels nor the caller choose: on MI355X a 60 GB buffer read
and written back in place as one launch runs at about 6.0-6.1 TB/s on some allocations and
6.45 TB/s on others, while 1 GiB launches reach about 5.9-6.0 TB/s on either; so one launch
beats the slices by 2-5% on slow memory and by 8-9% on fast memory.  Allocations made while earlier ones are still held land on other
memory, so trying a few is enough to find a fast one.

`relocate` keeps the caller's buffer, allocates up to `tries` more buffers of its size while
holding the earlier ones (free memory allows three more for a 60 GB buffer on a 288 GB
device, seven for the 25.7 GB of a 13B-parameter bf16 set), times each with
`zo_tune_placement`, copies the contents into the fastest (a device-to-device copy) and
releases the others.  It is a one-time set-up step before a run of in-place passes, not part
of them.
"""
from __future__ import annotations

import torch

# Below this size the placement spread is not seen (and 1 GiB slices do not apply).
MIN_BYTES = 2 << 30


def _rate(r: dict) -> float:
    return max(r["gbps_whole"], r["gbps_sliced"])


def relocate(ctx, buf: torch.Tensor, tries: int = 7, headroom_bytes: int = 8 << 30,
             fast_ratio: float = 1.06, min_gain: float = 1.02, copy: bool = True):
    """Return (buffer, report): `buf` itself, or a same-shaped tensor on faster memory holding
    a copy of its contents.

    A placement counts as fast once one launch per pass beats 1 GiB slices by
    `fast_ratio`; the search stops there, after `tries` extra allocations, or when the
    device has less than the buffer's size plus `headroom_bytes` free.  A candidate replaces
    the original only if it is `min_gain` times faster.  The context's pass form is left set
    for the returned buffer.  With `copy=False` the contents are not carried over (for a
    buffer that is filled afterwards)."""
    from . import zo_tune_placement

    nbytes = buf.numel() * buf.element_size()
    if nbytes < MIN_BYTES:
        return buf, {"skipped": True, "reason": f"{nbytes} bytes < {MIN_BYTES}"}
    first = zo_tune_placement(ctx, buf)
    tried = [dict(first)]
    best, best_rate, best_i = buf, _rate(first), 0
    held = []
    fast = first["gbps_whole"] >= fast_ratio * first["gbps_sliced"]
    for _ in range(tries):
        if fast:
            break
        free, _total = torch.cuda.mem_get_info(buf.device)
        if free < nbytes + headroom_bytes:
            break
        try:
            cand = torch.empty_like(buf)
        except torch.cuda.OutOfMemoryError:       # fragmentation: stop searching
            break
        r = zo_tune_placement(ctx, cand)
        tried.append(dict(r))
        held.append(cand)
        if _rate(r) > best_rate:
            best, best_rate, best_i = cand, _rate(r), len(tried) - 1
        fast = r["gbps_whole"] >= fast_ratio * r["gbps_sliced"]
    if best is not buf and best_rate < min_gain * _rate(first):
        best, best_rate, best_i = buf, _rate(first), 0
    if best is not buf and copy:
        best.copy_(buf)
    cand = None
    held = None          # drops every candidate but the one kept
    torch.cuda.synchronize(buf.device)
    torch.cuda.empty_cache()
    final = zo_tune_placement(ctx, best)      # the context's pass form for this buffer
    return best, {"skipped": False, "tried": tried, "kept": best_i, "copied": best is not buf
                  and copy, "final": dict(final)}
