"""cco_moe_plan_noalloc (the plan for callers that cannot allocate: scratch
in a fixed device array) against cco_moe_plan through the C ABI: the same
positions, counts, offsets, slot totals and status word, bit for bit, on
two calls in a row with the second smaller, plus an overflowing and an
invalid routing.  Runs alone in a fresh process and after the other GPU
tests (the array keeps every earlier call's contents)."""
import ctypes

import numpy as np
import pytest
import torch

from synth import get_config
from synth.gen import routing
from tests.gpu_util import make_moe, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def capi():
    from combine_symmetric_memory_amd import _capi
    assert torch.cuda.is_available()
    return _capi


def _noalloc(capi, idx, E, S, cap):
    T, K = idx.shape
    dev = torch.device("cuda")
    pos = torch.full((max(T, 1), K), -7, dtype=torch.int32, device=dev)
    counts = torch.full((E,), -7, dtype=torch.int32, device=dev)
    off = torch.full((E,), -7, dtype=torch.int32, device=dev)
    tot = torch.full((S,), -7, dtype=torch.int32, device=dev)
    status = torch.full((1,), -7, dtype=torch.int32, device=dev)
    idx_d = torch.from_numpy(np.ascontiguousarray(idx, np.int32)).to(dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = capi.lib.cco_moe_plan_noalloc(idx_d.data_ptr() if T else None, T, K, E, S, cap,
                                      pos.data_ptr(), counts.data_ptr(), off.data_ptr(),
                                      tot.data_ptr(), status.data_ptr(), stream)
    assert rc == capi.CCO_OK, capi.status_string(rc)
    torch.cuda.synchronize()
    return (pos[:T].cpu().numpy(), counts.cpu().numpy(), off.cpu().numpy(), tot.cpu().numpy(),
            int(status.cpu()[0]))


def _object_plan(moe, idx):
    dev = torch.device("cuda")
    moe.plan(torch.from_numpy(np.ascontiguousarray(idx, np.int32)).to(dev))
    code, _, _ = moe.status()
    pos, counts, off, tot = moe.read_routing()
    return pos, counts, off, tot, code


def _same(a, b, what):
    for name, x, y in zip(("pos", "counts", "expert_off", "slot_total", "status"), a, b):
        np.testing.assert_array_equal(np.asarray(x), np.asarray(y), err_msg=what + ": " + name)


def test_noalloc_plan_matches_the_object_plan(capi):
    cfg = get_config("dsv3")
    heap, moe = make_moe(cfg.with_(I=0))  # routing state only: no weights needed
    cap = moe.cap
    # the full batch (32 chunks), then a smaller one (one chunk), then a
    # multi-chunk one again: every call leaves the array behind for the next
    for T in (cfg.T, 200, 3000):
        idx, _ = routing(cfg, T)
        say("case: noalloc plan dsv3 routing T=%d" % T)
        _same(_noalloc(capi, idx, cfg.E, cfg.S, cap), _object_plan(moe, idx), "T=%d" % T)
    heap.destroy()


def test_noalloc_plan_overflow_and_bad_ids(capi):
    cfg = get_config("tiny")
    heap, moe = make_moe(cfg.with_(I=0))
    rng = np.random.default_rng(5)
    idx = rng.integers(0, cfg.E, size=(cfg.T, cfg.K)).astype(np.int32)
    idx[3, 1] = cfg.E
    say("case: noalloc plan, bad id")
    got = _noalloc(capi, idx, cfg.E, cfg.S, moe.cap)
    assert got[4] == capi.CCO_ERR_BAD_EXPERT
    _same(got, _object_plan(moe, idx), "bad id")
    # overflow: a small capacity, several chunks
    big = rng.integers(0, 2, size=(3000, 2)).astype(np.int32)
    say("case: noalloc plan, overflow")
    got = _noalloc(capi, big, 8, 4, 1000)
    assert got[4] == capi.CCO_ERR_CAPACITY
    assert (got[0] == -1).sum() == 6000 - 1000
    from oracle import oracle as orc
    ref = orc.plan(big, 8, 4, 1000)
    assert ref.status == orc.CAPACITY
    _same(got[:4], (ref.pos, ref.counts, ref.expert_off, ref.slot_total), "overflow vs oracle")
    heap.destroy()


def test_noalloc_plan_rejects_batches_beyond_its_scratch(capi):
    dev = torch.device("cuda")
    buf = torch.zeros(1 << 20, dtype=torch.int32, device=dev)
    p = buf.data_ptr()
    assert capi.lib.cco_moe_plan_noalloc(p, 1 << 17, 8, 256, 8, 1 << 20, p, p, p, p, p,
                                         None) == capi.CCO_ERR_TOO_LARGE
    assert capi.lib.cco_moe_plan_noalloc(p, 1 << 16, 8, 256, 8, 1 << 20, p + 2, p, p, p, p,
                                         None) == capi.CCO_ERR_INVALID_ARG
    assert capi.lib.cco_moe_plan_noalloc(p, 16, 8, 257, 8, 1 << 20, p, p, p, p, p,
                                         None) == capi.CCO_ERR_INVALID_ARG
    torch.cuda.synchronize()
