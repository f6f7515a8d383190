"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times.  Plan and dispatch are compared with the oracle in full
(bit-exact); the expert on every row of a stratified set of experts; combine
on sampled tokens (bit-exact on the GPU's own expert rows) and end to end on
sampled tokens from x (within tolerance)."""
import gc

import numpy as np
import pytest
import torch

from synth import get_config
from synth.gen import bf16_bits
from tests.gpu_util import assert_close, make_case, make_moe, run_path, say, weights_host

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _free_device_memory():
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _plan_and_dispatch_exact(orc, moe, c):
    cfg = c.cfg
    ref = orc.plan(c.idx_np, cfg.E, cfg.S, moe.cap)
    assert ref.status == orc.OK
    code, st, cnt = moe.status()
    assert code == 0
    pos, counts, off, tot = moe.read_routing()
    np.testing.assert_array_equal(counts, ref.counts)
    np.testing.assert_array_equal(off, ref.expert_off)
    np.testing.assert_array_equal(tot, ref.slot_total)
    np.testing.assert_array_equal(pos, ref.pos)
    # DISP_X[slot(e)][pos[t][j]] == x[t] for every pair (closed form of the
    # oracle's dispatch, checked slot by slot to bound host memory)
    eps = cfg.eps
    slot = c.idx_np // eps
    for s in range(cfg.S):
        n = int(ref.slot_total[s])
        rows = moe.read_rows("disp_x", s, 0, n)
        tt, jj = np.nonzero(slot == s)
        order = np.empty(n, np.int64)
        order[ref.pos[tt, jj]] = tt
        np.testing.assert_array_equal(rows, c.x_np[order])
        meta = moe.read_rows("meta", s, 0, n)
        src = np.empty(n, np.int64)
        src[ref.pos[tt, jj]] = tt * cfg.K + jj
        np.testing.assert_array_equal(meta["src"], src)
        np.testing.assert_array_equal(meta["e"], c.idx_np.ravel()[src])
        np.testing.assert_array_equal(meta["w"], c.w_np.ravel()[src])
    return ref


def _sample_experts(counts, k=4):
    nz = np.nonzero(counts)[0]
    order = nz[np.argsort(counts[nz], kind="stable")]
    picks = {int(order[0]), int(order[-1]), int(order[len(order) // 2]),
             int(order[len(order) // 4])}
    return sorted(picks)[:k]


def _expert_rows_parity(orc, moe, c, ref, experts):
    cfg = c.cfg
    for e in experts:
        n = int(ref.counts[e])
        s, o = e // cfg.eps, int(ref.expert_off[e])
        X = moe.read_rows("disp_x", s, o, n)
        Y = moe.read_rows("out_tok", s, o, n)
        w13e, w2e = weights_host(c, e)
        say("  expert %d: %d rows" % (e, n))
        assert_close(Y, orc.swiglu_rows(X, w13e, w2e), "expert %d" % e)


def _combine_tokens_parity(orc, moe, c, ref, out, tokens, identity):
    cfg = c.cfg
    got = bf16_bits(out)[tokens]
    rows = []
    for t in tokens:
        for j in range(cfg.K):
            e = int(c.idx_np[t, j])
            s, p = e // cfg.eps, int(ref.pos[t, j])
            rows.append(moe.read_rows("disp_x" if identity else "out_tok", s, p, 1)[0])
    np.testing.assert_array_equal(got, orc.combine_rows(rows, c.w_np[tokens]))
    return got


def _end_to_end_tokens(orc, c, tokens, got):
    """Oracle from x for the sampled tokens: each chosen expert's SwiGLU on
    x[t] (the expert rows of a token do not depend on other tokens)."""
    cfg = c.cfg
    rows = []
    cache = {}
    for t in tokens:
        for j in range(cfg.K):
            e = int(c.idx_np[t, j])
            if e not in cache:
                cache[e] = weights_host(c, e)
            rows.append(orc.swiglu_rows(c.x_np[t:t + 1], *cache[e])[0])
    assert_close(got, orc.combine_rows(rows, c.w_np[tokens]), "end to end, %d tokens" % len(tokens))


def test_dsv3_full(orc):
    cfg = get_config("dsv3")
    say("case: dsv3 full size", cfg)
    c = make_case(cfg)
    heap, moe = make_moe(cfg)
    out, code = run_path(moe, c)
    assert code == 0
    ref = _plan_and_dispatch_exact(orc, moe, c)
    _expert_rows_parity(orc, moe, c, ref, _sample_experts(ref.counts))
    tokens = np.random.default_rng(0).choice(cfg.T, size=24, replace=False)
    tokens = np.unique(np.concatenate([tokens, [0, cfg.T - 1]]))
    got = _combine_tokens_parity(orc, moe, c, ref, out, tokens, identity=False)
    _end_to_end_tokens(orc, c, tokens[:8], got[:8])
    heap.destroy()


def test_zipf_identity_full(orc):
    cfg = get_config("zipf")
    say("case: zipf identity full size", cfg)
    c = make_case(cfg)
    heap, moe = make_moe(cfg)
    out, code = run_path(moe, c)
    assert code == 0
    ref = _plan_and_dispatch_exact(orc, moe, c)
    # identity experts: the combine of every token from x, bit-exact
    got = bf16_bits(out)
    K = cfg.K
    rows = [c.x_np[t] for t in range(cfg.T) for _ in range(K)]
    np.testing.assert_array_equal(got, orc.combine_rows(rows, c.w_np))
    heap.destroy()


def test_decode_full(orc):
    cfg = get_config("decode")
    say("case: decode full size", cfg)
    c = make_case(cfg)
    heap, moe = make_moe(cfg)
    out, code = run_path(moe, c)
    assert code == 0
    ref = _plan_and_dispatch_exact(orc, moe, c)
    _expert_rows_parity(orc, moe, c, ref, _sample_experts(ref.counts, k=4))
    tokens = np.arange(0, cfg.T, 17)
    got = _combine_tokens_parity(orc, moe, c, ref, out, tokens, identity=False)
    _end_to_end_tokens(orc, c, tokens[:6], got[:6])
    heap.destroy()


def test_mixtral_full(orc):
    cfg = get_config("mixtral")
    say("case: mixtral full size", cfg)
    c = make_case(cfg)
    heap, moe = make_moe(cfg)
    out, code = run_path(moe, c)
    assert code == 0
    ref = _plan_and_dispatch_exact(orc, moe, c)
    # a row sample per expert (first, last and a middle block of rows)
    for e in range(cfg.E):
        n = int(ref.counts[e])
        s, o = e // cfg.eps, int(ref.expert_off[e])
        w13e, w2e = weights_host(c, e)
        for r0, r1 in ((0, 3), (n // 2, n // 2 + 2), (n - 3, n)):
            X = moe.read_rows("disp_x", s, o + r0, r1 - r0)
            Y = moe.read_rows("out_tok", s, o + r0, r1 - r0)
            assert_close(Y, orc.swiglu_rows(X, w13e, w2e), "expert %d rows %d:%d" % (e, r0, r1))
    tokens = np.array([0, 1, 2047, cfg.T - 1])
    got = _combine_tokens_parity(orc, moe, c, ref, out, tokens, identity=False)
    _end_to_end_tokens(orc, c, tokens, got)
    heap.destroy()
