"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times.  Plan and dispatch are compared with the oracle in full
(bit-exact); the expert on the first and last row of every expert that has
rows (every m-tile kind: full, partial, the 128-row remainder tiles), and on
one row of every 256-row m-tile where the GEMM splits its last tiles; combine
on every token (bit-exact on the GPU's own expert rows, read slot by slot) and
end to end on sampled tokens from x (within tolerance).  Repeated runs of the
full dsv3 batch, with a smaller batch in between, are bit-identical."""
import dataclasses
import gc
from concurrent.futures import ThreadPoolExecutor

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


def _combine_all_tokens_exact(orc, moe, c, ref, out):
    """Combine of every token, bit-exact against the oracle's combine of the
    GPU's own expert rows; the staging rows are read slot by slot into a
    [S][max slot total][H] array (the oracle addresses rows as slot * rows +
    pos, so any per-slot row count at least the slot totals serves)."""
    cfg = c.cfg
    n = int(ref.slot_total.max())
    src = np.zeros((cfg.S, n, cfg.H), np.uint16)
    for s in range(cfg.S):
        src[s, :ref.slot_total[s]] = moe.read_rows("out_tok", s, 0, int(ref.slot_total[s]))
    want = orc.combine_tokens(src, c.w_np, c.idx_np, ref.pos, cfg.E, cfg.S)
    got = bf16_bits(out)
    np.testing.assert_array_equal(got, want)
    say("  combine: all %d tokens bit-exact" % cfg.T)
    return got


def _rows_parity(orc, moe, c, ref, picks, label):
    """picks: {expert: [row offsets inside the expert]}; each expert's rows
    through the oracle's SwiGLU, experts in parallel (the oracle releases the
    interpreter lock)."""
    cfg = c.cfg

    def one(e):
        s, o = e // cfg.eps, int(ref.expert_off[e])
        rows = sorted(set(picks[e]))
        X = np.stack([moe.read_rows("disp_x", s, o + r, 1)[0] for r in rows])
        Y = np.stack([moe.read_rows("out_tok", s, o + r, 1)[0] for r in rows])
        w13e, w2e = weights_host(c, e)
        return e, Y, orc.swiglu_rows(X, w13e, w2e, nthreads=2)

    with ThreadPoolExecutor(max_workers=8) as ex:
        res = list(ex.map(one, sorted(picks)))
    Y = np.concatenate([r[1] for r in res])
    R = np.concatenate([r[2] for r in res])
    say("  %s: %d experts, %d rows" % (label, len(res), len(Y)))
    assert_close(Y, R, label)


def _first_last_rows(counts):
    return {int(e): [0, int(counts[e]) - 1] for e in np.nonzero(counts)[0]}


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
    _rows_parity(orc, moe, c, ref, _first_last_rows(ref.counts), "first and last row of every expert")
    got = _combine_all_tokens_exact(orc, moe, c, ref, out)
    tokens = np.random.default_rng(0).choice(cfg.T, size=24, replace=False)
    tokens = np.unique(np.concatenate([tokens, [0, cfg.T - 1]]))
    _end_to_end_tokens(orc, c, tokens[:8], got[tokens[:8]])
    heap.destroy()


def _window_digests(moe, S):
    import hashlib
    _, st, _ = moe.status()
    d = []
    for s in range(S):
        for which in ("hbuf", "out_tok"):
            rows = moe.read_rows(which, s, 0, int(st[s]))
            d.append(hashlib.blake2b(rows.tobytes(), digest_size=16).hexdigest())
    return d


def test_dsv3_full_repeated_runs_are_bit_identical():
    # the GEMMs' hand-out (per-XCD ranges, stealing, the next tile claimed
    # during the epilogue) decides only who computes a tile: repeated runs of
    # the full batch, with a smaller batch in between (which leaves the
    # counters at other values), give the same bits in every window and in out
    cfg = get_config("dsv3")
    say("case: dsv3 full size, repeated runs", cfg)
    c = make_case(cfg)
    heap, moe = make_moe(cfg)
    out0, code = run_path(moe, c)
    assert code == 0
    ref_out = bf16_bits(out0)
    ref_win = _window_digests(moe, cfg.S)
    small = dataclasses.replace(make_case(cfg, T=cfg.T // 2, weights=False), w13=c.w13, w2=c.w2)
    for rep in range(2):
        out_s, code = run_path(moe, small)
        assert code == 0
        out, code = run_path(moe, c)
        assert code == 0 and moe.status()[0] == 0
        np.testing.assert_array_equal(bf16_bits(out), ref_out, err_msg="run %d" % rep)
        assert _window_digests(moe, cfg.S) == ref_win, "windows differ on run %d" % rep
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
    # every row of every expert (2048 rows in all)
    picks = {int(e): list(range(int(ref.counts[e]))) for e in np.nonzero(ref.counts)[0]}
    _rows_parity(orc, moe, c, ref, picks, "every row of every expert")
    got = _combine_all_tokens_exact(orc, moe, c, ref, out)
    tokens = np.arange(0, cfg.T, 17)
    _end_to_end_tokens(orc, c, tokens[:6], got[tokens[:6]])
    heap.destroy()


def test_mixtral_full(orc):
    cfg = get_config("mixtral")
    say("case: mixtral full size", cfg)
    c = make_case(cfg)
    heap, moe = make_moe(cfg)
    out, code = run_path(moe, c)
    assert code == 0
    ref = _plan_and_dispatch_exact(orc, moe, c)
    # the down projection splits its last tiles into K-ranges here: one row
    # of every 256-row m-tile of every expert (a different offset in each),
    # plus each expert's first, middle and last rows
    picks = {}
    for e in range(cfg.E):
        n = int(ref.counts[e])
        rows = [0, 1, 2, n // 2, n // 2 + 1, n - 3, n - 2, n - 1]
        rows += [min(n - 1, m * 256 + (37 * m + 5) % 256) for m in range((n + 255) // 256)]
        picks[e] = rows
    _rows_parity(orc, moe, c, ref, picks, "rows of every m-tile")
    got = _combine_all_tokens_exact(orc, moe, c, ref, out)
    tokens = np.array([0, 1, 2047, cfg.T - 1])
    _end_to_end_tokens(orc, c, tokens, got[tokens])
    heap.destroy()


@pytest.mark.skip(reason="cco_moe_fused is switched off: its kernel faulted the GPU on its "
                         "first run (the small config) and the cause is not yet shown")
@pytest.mark.parametrize("name", ["dsv3", "decode", "mixtral"])
def test_fused_full(orc, name):
    """The single-launch path at full size: plan and dispatch bit-exact,
    the first and last row of every expert within tolerance, combine of every
    token bit-exact on the GPU's own expert rows; against the separate
    launches, identical where they sum no tile in K-ranges (dsv3, decode) and
    within tolerance where they do (mixtral's down projection)."""
    import combine_symmetric_memory_amd as ccm
    cfg = get_config(name)
    say("case: fused full size", cfg)
    c = make_case(cfg)
    heap, moe = make_moe(cfg)
    sep, code = run_path(moe, c)
    assert code == 0
    sep = bf16_bits(sep)
    out = moe.fused(c.idx, c.x, c.w, c.w13, c.w2)
    torch.cuda.synchronize()
    code, _, _ = moe.status()
    assert code == ccm.CCO_OK, ccm.status_string(code)
    ref = _plan_and_dispatch_exact(orc, moe, c)
    _rows_parity(orc, moe, c, ref, _first_last_rows(ref.counts), "fused: first and last rows")
    got = _combine_all_tokens_exact(orc, moe, c, ref, out)
    if name == "mixtral":
        assert_close(got, sep, "fused vs separate launches")
    else:
        np.testing.assert_array_equal(got, sep)
    heap.destroy()
