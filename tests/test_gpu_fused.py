"""GPU parity of the single-launch path (cco_moe_fused): plan, dispatch,
both expert GEMMs and combine in one persistent kernel.  Every stage against
the oracle as for the separate launches (plan and dispatch bit-exact, expert
within tolerance on the GPU's own receive rows, combine bit-exact on the GPU's
own expert rows, the whole path within tolerance from x); bit-identity with
the five separate launches where no GEMM tile is summed in K-ranges;
repeated launches (the kernel clears its own counters); error routings; the
full-size shapes."""
import gc

import numpy as np
import pytest
import torch

from synth import get_config
from synth.gen import bf16_bits, forced_edge_routing
from tests.gpu_util import make_case, make_moe, read_guards, run_path, say
from tests.test_gpu_parity import _check_all_stages

pytestmark = [pytest.mark.gpu, pytest.mark.skip(
    reason="cco_moe_fused is switched off: its kernel faulted the GPU on its first run "
           "(the small config) and the cause is not yet shown")]


@pytest.fixture(scope="module")
def ccm():
    import combine_symmetric_memory_amd as ccm
    assert torch.cuda.is_available()
    return ccm


@pytest.fixture(autouse=True)
def _free_device_memory():
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _fused(moe, c):
    out = moe.fused(c.idx, c.x, c.w, c.w13, c.w2)
    torch.cuda.synchronize()
    return out


def _windows(moe, S):
    _, st, _ = moe.status()
    hb = [moe.read_rows("hbuf", s, 0, int(st[s])) for s in range(S)] if moe.I else []
    ot = [moe.read_rows("out_tok", s, 0, int(st[s])) for s in range(S)] if moe.I else []
    return hb, ot


SMALL = [
    ("tiny", {}),
    ("multitile", dict(T=512, E=4, S=2, K=2, I=512, H=256)),
    ("mixedtiles", dict(T=1024, E=8, S=4, K=2, I=512, H=512)),
    ("identity", dict(T=300, E=16, S=4, K=4, I=0, H=1024)),
    ("k8rows14", dict(T=200, E=32, S=8, K=8, I=256, H=7168)),  # the fixed-length K=8 instantiation
    ("k2rows8", dict(T=256, E=8, S=8, K=2, I=256, H=4096)),    # the fixed-length K=2 instantiation
    ("oddk", dict(T=100, E=16, S=4, K=3, I=256, H=768)),       # the general instantiation
]


@pytest.mark.parametrize("name,kw", SMALL)
def test_fused_all_stages(ccm, orc, name, kw):
    cfg = get_config("tiny").with_(name=name, **kw)
    say("case: fused", name, cfg)
    c = make_case(cfg)
    heap, moe = make_moe(cfg)
    out = _fused(moe, c)
    code, _, _ = moe.status()
    assert code == ccm.CCO_OK, ccm.status_string(code)
    _check_all_stages(orc, moe, c, out)
    assert all((g == 0xA5).all() for g in read_guards(moe)), "a window overran its guard bytes"
    heap.destroy()


@pytest.mark.parametrize("name,kw", [
    ("b4b-k2", dict(T=1024, E=8, S=4, K=2, I=256, H=256)),
    ("b4b-k3", dict(T=300, E=12, S=4, K=3, I=256, H=256)),
    ("b4b-k8", dict(T=600, E=32, S=8, K=8, I=256, H=256)),
])
def test_fused_matches_the_separate_launches_bit_for_bit(ccm, name, kw):
    # GEMMs of 8 K-steps, which the separate launches never cut into
    # K-ranges: the fused kernel computes the same tiles
    cfg = get_config("tiny").with_(name=name, **kw)
    say("case: fused vs separate", name, cfg)
    c = make_case(cfg)
    heap, moe = make_moe(cfg)
    ref_out, _ = run_path(moe, c)
    ref_out = bf16_bits(ref_out)
    ref_hb, ref_ot = _windows(moe, cfg.S)
    for rep in range(3):  # repeated launches reuse the counters the kernel clears
        out = bf16_bits(_fused(moe, c))
        hb, ot = _windows(moe, cfg.S)
        assert moe.status()[0] == ccm.CCO_OK
        np.testing.assert_array_equal(out, ref_out, err_msg="launch %d" % rep)
        for s in range(cfg.S):
            np.testing.assert_array_equal(hb[s], ref_hb[s])
            np.testing.assert_array_equal(ot[s], ref_ot[s])
    # and the separate launches after the fused one still agree
    again, _ = run_path(moe, c)
    np.testing.assert_array_equal(bf16_bits(again), ref_out)
    heap.destroy()


def test_fused_edge_routings_and_errors(ccm, orc):
    cfg = get_config("decode").with_(name="fused-edges", T=64, E=64, I=256, H=1024)
    idx, w = forced_edge_routing(cfg.T, cfg.K, cfg.E, cfg.S, n_empty=8, n_one=8, n_two=8)
    c = make_case(cfg, idx_w=(idx, w))
    heap, moe = make_moe(cfg)
    out = _fused(moe, c)
    assert moe.status()[0] == ccm.CCO_OK
    _check_all_stages(orc, moe, c, out)
    # an invalid id: reported, and the kernel still finishes
    bad = c.idx_np.copy()
    bad[3, 2] = cfg.E
    cb = make_case(cfg, idx_w=(bad, c.w_np))
    _fused(moe, cb)
    assert moe.status()[0] == ccm.CCO_ERR_BAD_EXPERT
    # the next clean launch clears it
    out = _fused(moe, c)
    assert moe.status()[0] == ccm.CCO_OK
    _check_all_stages(orc, moe, c, out)
    heap.destroy()
    # a slot overflow: the pairs past the capacity are dropped, as in the oracle
    small = get_config("tiny").with_(name="fused-overflow", K=2, E=4, S=4)
    heap1, moe1 = make_moe(small)
    dup = np.zeros((small.T, 2), np.int32)
    c3 = make_case(small, idx_w=(dup, np.full((small.T, 2), 0.5, np.float32)))
    out3 = _fused(moe1, c3)
    assert moe1.status()[0] == ccm.CCO_ERR_CAPACITY
    ref = orc.pipeline(c3.x_np, c3.w_np, c3.idx_np, small.E, small.S, moe1.cap,
                       bf16_bits(c3.w13), bf16_bits(c3.w2), allow_overflow=True)
    np.testing.assert_array_equal(moe1.read_routing()[0], ref.plan.pos)
    from tests.gpu_util import assert_close
    assert_close(bf16_bits(out3), ref.out, "fused combine after an overflow")
    assert all((g == 0xA5).all() for g in read_guards(moe1)), "overflow wrote past a window"
    heap1.destroy()


def test_fused_rejects_bad_arguments(ccm):
    from combine_symmetric_memory_amd import _capi
    cfg = get_config("tiny")
    c = make_case(cfg)
    heap, moe = make_moe(cfg)
    lib, h, INV = _capi.lib, moe.handle, ccm.CCO_ERR_INVALID_ARG
    out = torch.empty((cfg.T + 1, cfg.H), dtype=torch.bfloat16, device="cuda")
    args = [c.idx.data_ptr(), c.x.data_ptr(), c.w.data_ptr(), c.w13.data_ptr(), c.w2.data_ptr(),
            out.data_ptr()]
    assert lib.cco_moe_fused(h, *args, cfg.T + 1, None) == INV  # above max_tokens
    for i, off in ((0, 2), (1, 8), (2, 2), (3, 2), (4, 8), (5, 2)):
        bad = list(args)
        bad[i] += off
        assert lib.cco_moe_fused(h, *bad, cfg.T, None) == INV, i
    assert lib.cco_moe_fused(h, *args, cfg.T, None) == ccm.CCO_OK
    torch.cuda.synchronize()
    heap.destroy()
    big = get_config("tiny").with_(name="k12", K=12, E=16)
    heap2, moe2 = make_moe(big)
    assert lib.cco_moe_fused(moe2.handle, *args, 1, None) == INV  # top-k above 8
    heap2.destroy()
