"""Host logic of placement.relocate, with the device calls replaced by scripted ones: which
allocation it keeps, when it stops searching, what it copies.  (The GPU test of the same
function runs it on real allocations.)"""
import numpy as np
import pytest
import torch

import forward_only_amd as zo
from forward_only_amd import placement


class Script:
    """zo_tune_placement stand-in: the n-th buffer it sees gets the n-th scripted rate pair
    (one launch, 1 GiB slices); a buffer seen again gets its earlier answer."""

    def __init__(self, rates):
        self.rates = list(rates)
        self.seen = {}
        self.calls = []

    def __call__(self, ctx, buf, stream=None):
        key = id(buf)
        if key not in self.seen:
            w, s = self.rates[len(self.seen)]
            self.seen[key] = {"slice_bytes": 0 if w >= s else 1 << 30, "gbps_whole": float(w),
                              "gbps_sliced": float(s)}
        self.calls.append(key)
        return dict(self.seen[key])


@pytest.fixture
def fake_device(monkeypatch):
    state = {"free": 1 << 40}
    monkeypatch.setattr(placement, "MIN_BYTES", 64)
    monkeypatch.setattr(torch.cuda, "mem_get_info", lambda dev=None: (state["free"], 1 << 41))
    monkeypatch.setattr(torch.cuda, "synchronize", lambda dev=None: None)
    monkeypatch.setattr(torch.cuda, "empty_cache", lambda: None)
    return state


def _buf():
    return torch.from_numpy(np.arange(4096, dtype=np.float32))


def test_fast_first_allocation_is_kept_without_search(fake_device, monkeypatch):
    script = Script([(6200, 5800)])
    monkeypatch.setattr(zo, "zo_tune_placement", script)
    b = _buf()
    out, rep = placement.relocate(None, b)
    assert out is b and rep["kept"] == 0 and not rep["copied"]
    assert len(rep["tried"]) == 1


def test_search_stops_at_the_first_fast_candidate_and_copies(fake_device, monkeypatch):
    script = Script([(5200, 5800), (5750, 5800), (6240, 5800), (6300, 5800)])
    monkeypatch.setattr(zo, "zo_tune_placement", script)
    b = _buf()
    out, rep = placement.relocate(None, b, tries=3)
    assert rep["kept"] == 2 and rep["copied"] and out is not b
    assert len(rep["tried"]) == 3                      # stopped before the fourth
    assert torch.equal(out, b)
    assert script.calls[-1] == id(out)                 # the context is tuned for the kept one
    assert rep["final"]["gbps_whole"] == 6240


def test_no_candidate_good_enough_keeps_the_original(fake_device, monkeypatch):
    # all slow; slices are the best any offers, within 2% of the original's
    script = Script([(5200, 5800), (5210, 5850), (5190, 5790), (5220, 5830)])
    monkeypatch.setattr(zo, "zo_tune_placement", script)
    b = _buf()
    out, rep = placement.relocate(None, b, tries=3)
    assert out is b and rep["kept"] == 0 and not rep["copied"]
    assert len(rep["tried"]) == 4


def test_best_of_slow_candidates_is_kept_when_clearly_faster(fake_device, monkeypatch):
    script = Script([(5200, 5600), (5300, 5900), (5250, 5800), (5100, 5700)])
    monkeypatch.setattr(zo, "zo_tune_placement", script)
    b = _buf()
    out, rep = placement.relocate(None, b, tries=3)
    assert rep["kept"] == 1 and torch.equal(out, b) and out is not b


def test_free_memory_limits_the_search(fake_device, monkeypatch):
    script = Script([(5200, 5800), (6200, 5800)])
    monkeypatch.setattr(zo, "zo_tune_placement", script)
    fake_device["free"] = 1 << 20                      # less than size + headroom
    b = _buf()
    out, rep = placement.relocate(None, b, tries=3)
    assert out is b and len(rep["tried"]) == 1


def test_copy_false_keeps_the_new_buffer_uninitialised(fake_device, monkeypatch):
    script = Script([(5200, 5800), (6200, 5800)])
    monkeypatch.setattr(zo, "zo_tune_placement", script)
    b = _buf()
    out, rep = placement.relocate(None, b, copy=False)
    assert out is not b and rep["kept"] == 1 and not rep["copied"]


def test_small_buffers_are_skipped(monkeypatch):
    script = Script([])
    monkeypatch.setattr(zo, "zo_tune_placement", script)
    b = torch.zeros(10)
    out, rep = placement.relocate(None, b)
    assert out is b and rep["skipped"] and script.calls == []


def test_an_allocation_failure_ends_the_search(fake_device, monkeypatch):
    script = Script([(5200, 5800), (6200, 5800)])
    monkeypatch.setattr(zo, "zo_tune_placement", script)

    def no_memory(*a, **k):
        raise torch.cuda.OutOfMemoryError("no memory")
    monkeypatch.setattr(torch, "empty_like", no_memory)
    b = _buf()
    out, rep = placement.relocate(None, b, tries=3)
    assert out is b and len(rep["tried"]) == 1 and rep["kept"] == 0
