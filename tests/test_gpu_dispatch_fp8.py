"""GPU parity of the 8-bit dispatch (tokens the caller quantized, with fp32
scales) against the oracle: receive rows and metadata bit-exact, bytes past
each row's token and scales untouched, guard bytes intact, host-side
rejections, and sampled rows at the DeepSeek-V3 shape."""
import ctypes

import numpy as np
import pytest
import torch

from synth import get_config
from synth.gen import quantized_activations, routing
from tests.gpu_util import make_moe, read_guards, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ccm():
    import combine_symmetric_memory_amd as ccm
    assert torch.cuda.is_available()
    return ccm


def _inputs(cfg, ns_block, T=None):
    """x8 uint8 [T, H], scales fp32 [T, ns] (None for ns_block == 0), idx, w."""
    if ns_block:
        x8, sc = quantized_activations(cfg, T, block=ns_block)
    else:
        rng = np.random.default_rng([cfg.seed, 7])
        x8 = rng.integers(0, 256, (cfg.T if T is None else T, cfg.H), dtype=np.uint8)
        sc = None
    idx, w = routing(cfg, x8.shape[0])
    return x8, sc, np.ascontiguousarray(idx, np.int32), np.ascontiguousarray(w, np.float32)


def _dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _read_rows8(moe, s, n):
    """Receive rows [0, n) of slot s as raw bytes [n, 2H]."""
    return moe.read_window(s, moe.layout.disp_x, n * 2 * moe.H).reshape(n, 2 * moe.H)


def _check_against_oracle(orc, moe, cfg, x8, sc, idx, w):
    ns = 0 if sc is None else sc.shape[1]
    H, E, S, cap = cfg.H, cfg.E, cfg.S, moe.cap
    ref = orc.plan(idx, E, S, cap)
    assert ref.status == orc.OK
    pos, counts, _, tot = moe.read_routing()
    np.testing.assert_array_equal(pos, ref.pos)
    np.testing.assert_array_equal(tot, ref.slot_total)
    d = orc.dispatch_fp8(x8, np.zeros((x8.shape[0], 0), np.float32) if sc is None else sc,
                         w, idx, ref.pos, E, S, cap)
    for s in range(S):
        n = int(ref.slot_total[s])
        rows = _read_rows8(moe, s, n)
        np.testing.assert_array_equal(rows[:, :H + 4 * ns], d.disp_x[s, :n, :H + 4 * ns])
        meta = moe.read_rows("meta", s, 0, n)
        np.testing.assert_array_equal(meta["src"], d.meta_src[s, :n])
        np.testing.assert_array_equal(meta["w"], d.meta_w[s, :n])
        np.testing.assert_array_equal(meta["e"], d.meta_e[s, :n])
    return ref


@pytest.mark.parametrize("name,over,block,T", [
    ("tiny", {}, 128, None),                                   # ns = 2
    ("dsv3", {"I": 0}, 128, 300),                              # ns = 56, top-8 fast path
    ("tiny", {"H": 1024, "E": 12, "S": 4, "K": 3, "I": 0}, 4, 77),   # ns = 256: scales past 64 lanes
    ("tiny", {"H": 8208, "I": 0, "K": 2}, 16, 33),             # rows past one chunk; ns = 513
    ("tiny", {"H": 48, "E": 4, "S": 2, "K": 1, "I": 0}, 0, 50),    # no scales, 3 vectors per row
    ("mixtral", {"I": 0}, 128, 200),                           # 4 vectors per lane, top-2
    ("tiny", {"H": 8192, "E": 16, "S": 4, "K": 6, "I": 0}, 128, 40),  # 8 vectors per lane, top-6
])
def test_dispatch_fp8_matches_oracle(ccm, orc, name, over, block, T):
    cfg = get_config(name, **over)
    if T is not None:
        cfg = cfg.with_(T=T)
    say("case: fp8 dispatch %s H=%d K=%d E=%d S=%d T=%d block=%d" %
        (name, cfg.H, cfg.K, cfg.E, cfg.S, cfg.T, block))
    x8, sc, idx, w = _inputs(cfg, block)
    heap, moe = make_moe(cfg)
    moe.plan(_dev(idx))
    moe.dispatch_fp8(_dev(x8), _dev(sc), _dev(w))
    torch.cuda.synchronize()
    assert moe.status()[0] == ccm.CCO_OK
    _check_against_oracle(orc, moe, cfg, x8, sc, idx, w)
    assert all((g == 0xA5).all() for g in read_guards(moe)), "a window overran its guard bytes"
    heap.destroy()


def test_dispatch_fp8_leaves_the_rest_of_each_row(ccm, orc):
    # a bf16 dispatch fills whole rows; the 8-bit dispatch of the same routing
    # then rewrites bytes [0, H + 4 ns) only
    cfg = get_config("tiny").with_(I=0, H=512, T=90)
    x8, sc, idx, w = _inputs(cfg, 32)      # ns = 16
    ns = sc.shape[1]
    heap, moe = make_moe(cfg)
    xb = torch.randn(cfg.T, cfg.H, dtype=torch.float32).to(torch.bfloat16).cuda()
    moe.plan(_dev(idx))
    moe.dispatch(xb, _dev(w))
    torch.cuda.synchronize()
    before = [_read_rows8(moe, s, moe.read_routing()[3][s]) for s in range(cfg.S)]
    moe.dispatch_fp8(_dev(x8), _dev(sc), _dev(w))
    torch.cuda.synchronize()
    _check_against_oracle(orc, moe, cfg, x8, sc, idx, w)
    for s in range(cfg.S):
        after = _read_rows8(moe, s, before[s].shape[0])
        np.testing.assert_array_equal(after[:, cfg.H + 4 * ns:], before[s][:, cfg.H + 4 * ns:])
    heap.destroy()


def test_dispatch_fp8_empty_batch_and_rejections(ccm):
    cfg = get_config("tiny")
    heap, moe = make_moe(cfg)
    L, h = ccm.lib, moe.handle
    x8, sc, idx, w = _inputs(cfg, 128)
    idx_d, w_d, sc_d = _dev(idx), _dev(w), _dev(sc)
    # T = 0 after a plan of 0 tokens: nothing launched, success
    moe.plan(idx_d[:0])
    assert L.cco_moe_dispatch_fp8(h, None, None, 0, None, 0, None) == ccm.CCO_OK
    moe.plan(idx_d)
    T, H = cfg.T, cfg.H
    flat = torch.zeros(T * H + 16, dtype=torch.uint8, device="cuda")
    x8_d = flat[:T * H].view(T, H)
    odd = flat[1:1 + T * H]                        # not 16-byte aligned
    p = ctypes.c_void_p
    # (x8, scales, ns, T): each is rejected before any launch
    bad = [
        (p(odd.data_ptr()), p(sc_d.data_ptr()), 2, T),      # misaligned tokens
        (p(x8_d.data_ptr()), p(sc_d.data_ptr() + 2), 2, T), # misaligned scales
        (p(x8_d.data_ptr()), p(sc_d.data_ptr()), H // 4 + 1, T),  # scales past the row
        (p(x8_d.data_ptr()), p(sc_d.data_ptr()), -1, T),
        (p(x8_d.data_ptr()), None, 2, T),                   # ns > 0 without scales
        (None, p(sc_d.data_ptr()), 2, T),
        (p(x8_d.data_ptr()), p(sc_d.data_ptr()), 2, T - 1), # T differs from the plan
    ]
    for a in bad:
        assert L.cco_moe_dispatch_fp8(h, a[0], a[1], a[2], p(w_d.data_ptr()), a[3], None) == \
            ccm.CCO_ERR_INVALID_ARG, a
    heap.destroy()
    # H % 16 != 0: the 8-bit rows would not be whole 16-byte vectors
    cfg8 = get_config("tiny").with_(H=40, I=0, T=16)
    heap8, moe8 = make_moe(cfg8)
    x8, sc, idx, w = _inputs(cfg8, 0)
    moe8.plan(_dev(idx))
    with pytest.raises(ccm.CcoError):
        moe8.dispatch_fp8(_dev(x8), None, _dev(w))
    heap8.destroy()


def test_identity_combine_refuses_8bit_rows(ccm):
    # identity experts: combine would read the 8-bit rows through the view
    # as bf16; the caller's own expert output (a foreign pointer) is fine,
    # and a bf16 dispatch makes the rows bf16 again.  (The SwiGLU expert
    # reads 8-bit rows as such: tests/test_gpu_expert_fp8.py.)
    cfg = get_config("tiny").with_(I=0)
    x8, sc, idx, w = _inputs(cfg, 128)
    heap, moe = make_moe(cfg)
    moe.plan(_dev(idx))
    moe.dispatch_fp8(_dev(x8), _dev(sc), _dev(w))
    with pytest.raises(ccm.CcoError):
        moe.combine(_dev(w))
    tot = moe.read_routing()[3]
    own = [torch.zeros((max(int(tot[s]), 1), cfg.H), dtype=torch.bfloat16, device="cuda")
           for s in range(cfg.S)]
    out, code = moe.combine(_dev(w), expert_out=own)
    assert code == ccm.CCO_INFO_COPIED
    torch.cuda.synchronize()
    assert not out.float().abs().sum().item()
    xb = torch.randn(cfg.T, cfg.H).to(torch.bfloat16).cuda()
    moe.dispatch(xb, _dev(w))
    out, code = moe.combine(_dev(w))
    torch.cuda.synchronize()
    assert code == ccm.CCO_OK
    heap.destroy()


def test_dispatch_fp8_dsv3_full_sampled(ccm, orc):
    # the full DeepSeek-V3 shape (T = 8192, H = 7168, top-8, 256 experts over
    # 8 slots, 1 x 128 block scales): positions bit-exact against the oracle's
    # plan, and the rows of 512 sampled tokens against x8 and scales
    cfg = get_config("dsv3").with_(I=0)
    say("case: fp8 dispatch dsv3 full size, sampled rows")
    x8, sc, idx, w = _inputs(cfg, 128)
    ns, H, K = sc.shape[1], cfg.H, cfg.K
    heap, moe = make_moe(cfg)
    moe.plan(_dev(idx))
    moe.dispatch_fp8(_dev(x8), _dev(sc), _dev(w))
    torch.cuda.synchronize()
    assert moe.status()[0] == ccm.CCO_OK
    ref = orc.plan(idx, cfg.E, cfg.S, moe.cap)
    pos = moe.read_routing()[0]
    np.testing.assert_array_equal(pos, ref.pos)
    rng = np.random.default_rng(11)
    toks = np.sort(rng.choice(cfg.T, 512, replace=False))
    toks[0], toks[-1] = 0, cfg.T - 1
    rb = 2 * H
    for t in toks:
        for j in range(K):
            e = int(idx[t, j])
            s, r = e // cfg.eps, int(ref.pos[t, j])
            row = moe.read_window(s, moe.layout.disp_x + r * rb, H + 4 * ns)
            assert bytes(row[:H]) == bytes(x8[t]), (t, j)
            assert bytes(row[H:]) == sc[t].tobytes(), (t, j)
            m = moe.read_rows("meta", s, r, 1)
            assert (int(m["src"][0]), int(m["e"][0])) == (t * K + j, e)
            assert m["w"][0] == w[t, j]
    heap.destroy()
