"""GPU parity of the expert on 8-bit receive rows (cco_moe_expert after
cco_moe_dispatch_fp8): the gate/up GEMM reads each row's e4m3 values and
fp32 block scales in place and multiplies bf16(binary32(e4m3 * scale)).

Against the oracle: the expert rows within tolerance of the oracle's SwiGLU
on oracle.dequant_e4m3_rows of the GPU's own receive rows, combine bit-exact
on the GPU's own expert rows.  Against the bf16 path: a bf16 dispatch of the
oracle's dequantized tokens gives bit-identical HBUF, expert rows and
combine output (same tiles, same K order, same bf16 operands).  Scale blocks
of 1, 2, 4, 8 and 16 K-steps, no scales, half tiles and split K-ranges, ragged
and empty batches, eleven seeded random shapes, the full DeepSeek-V3 and
Mixtral shapes, and the host-side rejections."""
import gc
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from synth import get_config
from synth.gen import bf16_bits, expert_weights, quantized_activations, routing
from tests.gpu_util import assert_close, make_moe, say

pytestmark = pytest.mark.gpu


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


def _dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _inputs(cfg, block, T=None, scaled=True):
    """x8 [T, H] e4m3 bytes, scales [T, H / block] (None when not scaled:
    the codes alone are the values), idx, w."""
    x8, sc = quantized_activations(cfg, T, block=block)
    idx, w = routing(cfg, x8.shape[0])
    return (x8, sc if scaled else None, np.ascontiguousarray(idx, np.int32),
            np.ascontiguousarray(w, np.float32))


def _token_rows(x8, sc):
    """Tokens laid out as receive rows [T, 2H]: values, scale bytes, zeros."""
    T, H = x8.shape
    rows = np.zeros((T, 2 * H), np.uint8)
    rows[:, :H] = x8
    if sc is not None:
        rows[:, H:H + 4 * sc.shape[1]] = np.ascontiguousarray(sc, np.float32).view(np.uint8)
    return rows


def _read_rows8(moe, s, r0, n):
    H = moe.H
    return moe.read_window(s, moe.layout.disp_x + r0 * 2 * H, n * 2 * H).reshape(n, 2 * H)


def _run_fp8(moe, x8, sc, idx, w, w13, w2):
    moe.plan(_dev(idx))
    moe.dispatch_fp8(_dev(x8), _dev(sc), _dev(w))
    moe.expert(w13, w2)
    out, code = moe.combine(_dev(w))
    torch.cuda.synchronize()
    return out, code


def _run_bf16(moe, xb, idx, w, w13, w2):
    moe.plan(_dev(idx))
    moe.dispatch(xb, _dev(w))
    moe.expert(w13, w2)
    out, code = moe.combine(_dev(w))
    torch.cuda.synchronize()
    return out, code


def _windows(moe, tot):
    hb = [moe.read_rows("hbuf", s, 0, int(tot[s])) for s in range(moe.S)]
    ot = [moe.read_rows("out_tok", s, 0, int(tot[s])) for s in range(moe.S)]
    return hb, ot


CASES = [
    # name, config overrides, scale block (values), T, scaled
    ("tiny-b64", {}, 64, None, True),                                        # 1 K-step per scale
    ("split-b128", dict(T=512, E=8, S=4, K=2, I=512, H=1024), 128, None, True),  # half tiles,
                                                                             # K-ranges
    ("row-b512", dict(T=300, E=12, S=4, K=3, I=256, H=512), 512, None, True),    # 1 scale per row
    ("k8-b256", dict(T=200, E=32, S=8, K=8, I=256, H=2048), 256, None, True),    # 4 K-steps each
    ("ragged-b128", dict(E=16, S=4, K=4, I=512, H=768), 128, 77, True),          # 6 blocks of 2
    ("noscale", dict(T=300, E=8, S=4, K=2, I=256, H=1024), 128, None, False),    # the codes alone
]


def _check_against_oracle(ccm, orc, cfg, moe, x8, sc, idx, w, w13, w2, out):
    """Receive rows and positions bit-exact; every expert's rows within
    tolerance of the oracle's SwiGLU on the dequantized GPU receive rows;
    combine bit-exact on the GPU's own expert rows."""
    ns = 0 if sc is None else sc.shape[1]
    E, S, cap = cfg.E, cfg.S, moe.cap
    ref = orc.plan(idx, E, S, cap)
    pos, counts, off, tot = moe.read_routing()
    np.testing.assert_array_equal(pos, ref.pos)
    d = orc.dispatch_fp8(x8, np.zeros((x8.shape[0], 0), np.float32) if sc is None else sc,
                         w, idx, ref.pos, E, S, cap)
    full = np.zeros((S, cap, cfg.H), np.uint16)
    w13h, w2h = bf16_bits(w13), bf16_bits(w2)
    for s in range(S):
        n = int(ref.slot_total[s])
        rows = _read_rows8(moe, s, 0, n)
        np.testing.assert_array_equal(rows[:, :cfg.H + 4 * ns], d.disp_x[s, :n, :cfg.H + 4 * ns])
        X = orc.dequant_e4m3_rows(rows, ns)
        Y = moe.read_rows("out_tok", s, 0, n)
        full[s, :n] = Y
        for e in range(s * cfg.eps, (s + 1) * cfg.eps):
            c, o = int(ref.counts[e]), int(ref.expert_off[e])
            if c == 0:
                continue
            assert_close(Y[o:o + c], orc.swiglu_rows(X[o:o + c], w13h[e], w2h[e]),
                         "expert %d (%d rows)" % (e, c))
    np.testing.assert_array_equal(bf16_bits(out),
                                  orc.combine_tokens(full, w, idx, ref.pos, E, S))


@pytest.mark.parametrize("name,over,block,T,scaled", CASES)
def test_expert_8bit_matches_oracle(ccm, orc, name, over, block, T, scaled):
    cfg = get_config("tiny").with_(name=name, **over)
    say("case: 8-bit expert vs oracle", name, cfg, "block", block, "T", T, "scaled", scaled)
    x8, sc, idx, w = _inputs(cfg, block, T, scaled)
    heap, moe = make_moe(cfg)
    w13, w2 = expert_weights(cfg, "cuda")
    out, code = _run_fp8(moe, x8, sc, idx, w, w13, w2)
    assert code == ccm.CCO_OK and moe.status()[0] == ccm.CCO_OK
    _check_against_oracle(ccm, orc, cfg, moe, x8, sc, idx, w, w13, w2, out)
    heap.destroy()


@pytest.mark.parametrize("name,over,block,T,scaled", [
    ("tiny-b64", {}, 64, None, True),
    ("split-b128", dict(T=512, E=8, S=4, K=2, I=512, H=1024), 128, None, True),
    ("k8-b256", dict(T=200, E=32, S=8, K=8, I=256, H=2048), 256, None, True),
    ("noscale", dict(T=300, E=8, S=4, K=2, I=256, H=1024), 128, None, False),
    ("one-token", dict(E=16, S=4, K=4, I=512, H=1024), 1024, 1, True),
])
def test_expert_8bit_is_the_bf16_path_on_dequantized_tokens(ccm, orc, name, over, block, T,
                                                            scaled):
    cfg = get_config("tiny").with_(name=name, **over)
    say("case: 8-bit expert vs bf16 path", name, cfg, "block", block, "scaled", scaled)
    x8, sc, idx, w = _inputs(cfg, block, T, scaled)
    ns = 0 if sc is None else sc.shape[1]
    xb = torch.from_numpy(orc.dequant_e4m3_rows(_token_rows(x8, sc), ns).view(np.int16)) \
        .view(torch.bfloat16).cuda()
    heap, moe = make_moe(cfg)
    w13, w2 = expert_weights(cfg, "cuda")
    out8, code = _run_fp8(moe, x8, sc, idx, w, w13, w2)
    assert code == ccm.CCO_OK and moe.status()[0] == ccm.CCO_OK
    tot = moe.read_routing()[3]
    hb8, ot8 = _windows(moe, tot)
    outb, code = _run_bf16(moe, xb, idx, w, w13, w2)
    assert code == ccm.CCO_OK and moe.status()[0] == ccm.CCO_OK
    hbb, otb = _windows(moe, tot)
    for s in range(cfg.S):
        np.testing.assert_array_equal(hb8[s], hbb[s], err_msg="HBUF slot %d" % s)
        np.testing.assert_array_equal(ot8[s], otb[s], err_msg="expert rows slot %d" % s)
    assert torch.equal(out8.view(torch.int16), outb.view(torch.int16))
    # and the 8-bit path again after the bf16 one: the rows are read as 8-bit
    # only after an 8-bit dispatch
    again, _ = _run_fp8(moe, x8, sc, idx, w, w13, w2)
    assert torch.equal(again.view(torch.int16), out8.view(torch.int16))
    heap.destroy()


def _random_8bit_shapes(n=10, seed=77):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        S = int(rng.choice([1, 2, 4, 8]))
        E = S * int(rng.integers(1, 9))
        K = int(rng.choice([1, 2, 3, 4, 6, 8]))
        H = 256 * int(rng.integers(1, 9))
        I = 128 * int(rng.integers(1, 5))
        T = int(rng.choice([1, 7, 64, 257, 600]))
        blocks = [b for b in (64, 128, 256, 512, 1024, 2048) if H % b == 0]
        block = int(rng.choice(blocks))
        scaled = rng.random() < 0.85
        if K > E or T * K > 5000:
            continue
        out.append((H, I, E, S, K, T, block, scaled))
    return out


@pytest.mark.parametrize("H,I,E,S,K,T,block,scaled",
                         _random_8bit_shapes() + [(512, 256, 8, 2, 2, 300, 128, False)])
def test_expert_8bit_random_shape(ccm, orc, H, I, E, S, K, T, block, scaled):
    cfg = get_config("tiny").with_(name="random8", H=H, I=I, E=E, S=S, K=K, T=T)
    say("case: 8-bit random H=%d I=%d E=%d S=%d K=%d T=%d block=%d scaled=%s" %
        (H, I, E, S, K, T, block, scaled))
    x8, sc, idx, w = _inputs(cfg, block, T, scaled)
    ns = 0 if sc is None else sc.shape[1]
    heap, moe = make_moe(cfg)
    w13, w2 = expert_weights(cfg, "cuda")
    out8, code = _run_fp8(moe, x8, sc, idx, w, w13, w2)
    assert code == ccm.CCO_OK and moe.status()[0] == ccm.CCO_OK
    _check_against_oracle(ccm, orc, cfg, moe, x8, sc, idx, w, w13, w2, out8)
    tot = moe.read_routing()[3]
    hb8, ot8 = _windows(moe, tot)
    xb = torch.from_numpy(orc.dequant_e4m3_rows(_token_rows(x8, sc), ns).view(np.int16)) \
        .view(torch.bfloat16).cuda()
    outb, code = _run_bf16(moe, xb, idx, w, w13, w2)
    assert code == ccm.CCO_OK
    hbb, otb = _windows(moe, tot)
    for s in range(S):
        np.testing.assert_array_equal(hb8[s], hbb[s], err_msg="HBUF slot %d" % s)
        np.testing.assert_array_equal(ot8[s], otb[s], err_msg="expert rows slot %d" % s)
    assert torch.equal(out8.view(torch.int16), outb.view(torch.int16))
    heap.destroy()


def test_expert_8bit_rejections_and_empty_batch(ccm):
    # scale blocks that are not whole runs of a power of two of 64-value
    # K-steps are refused before any launch; a bf16 dispatch clears the state
    cases = [(dict(H=256), 32), (dict(H=768), 192), (dict(H=1280), 640)]
    for over, block in cases:
        cfg = get_config("tiny").with_(name="rej", **over)
        say("case: 8-bit expert rejects", over, "block", block)
        x8, sc, idx, w = _inputs(cfg, block)
        heap, moe = make_moe(cfg)
        w13, w2 = expert_weights(cfg, "cuda")
        moe.plan(_dev(idx))
        moe.dispatch_fp8(_dev(x8), _dev(sc), _dev(w))
        with pytest.raises(ccm.CcoError):
            moe.expert(w13, w2)
        xb = torch.randn(cfg.T, cfg.H).to(torch.bfloat16).cuda()
        moe.dispatch(xb, _dev(w))
        moe.expert(w13, w2)
        torch.cuda.synchronize()
        assert moe.status()[0] == ccm.CCO_OK
        heap.destroy()
    # an empty batch: every call is a no-op
    cfg = get_config("tiny")
    heap, moe = make_moe(cfg)
    w13, w2 = expert_weights(cfg, "cuda")
    moe.plan(torch.zeros((0, cfg.K), dtype=torch.int32, device="cuda"))
    moe.dispatch_fp8(torch.zeros((0, cfg.H), dtype=torch.uint8, device="cuda"),
                     torch.zeros((0, 2), dtype=torch.float32, device="cuda"),
                     torch.zeros((0, cfg.K), dtype=torch.float32, device="cuda"))
    moe.expert(w13, w2)
    out, code = moe.combine(torch.zeros((0, cfg.K), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    assert code == ccm.CCO_OK and out.shape[0] == 0
    heap.destroy()


def test_expert_8bit_dsv3_full_size(ccm, orc):
    # the full DeepSeek-V3 shape (T = 8192, H = 7168, I = 2048, top-8 of 256
    # experts over 8 slots, 1 x 128 block scales): the first and last row of
    # every expert with rows against the oracle, and the whole path
    # bit-identical to the bf16 path on the oracle's dequantized tokens
    cfg = get_config("dsv3")
    say("case: 8-bit expert dsv3 full size")
    x8, sc, idx, w = _inputs(cfg, 128)
    ns = sc.shape[1]
    heap, moe = make_moe(cfg)
    w13, w2 = expert_weights(cfg, "cuda")
    out8, code = _run_fp8(moe, x8, sc, idx, w, w13, w2)
    assert code == ccm.CCO_OK and moe.status()[0] == ccm.CCO_OK
    ref = orc.plan(idx, cfg.E, cfg.S, moe.cap)
    pos, counts, off, tot = moe.read_routing()
    np.testing.assert_array_equal(pos, ref.pos)
    w13h, w2h = bf16_bits(w13), bf16_bits(w2)

    def one(e):
        # the expert's first and last row, through the oracle's SwiGLU
        s, o, c = int(e) // cfg.eps, int(ref.expert_off[e]), int(ref.counts[e])
        rows = sorted({0, c - 1})
        X = np.concatenate([orc.dequant_e4m3_rows(_read_rows8(moe, s, o + r, 1), ns)
                            for r in rows])
        Y = np.stack([moe.read_rows("out_tok", s, o + r, 1)[0] for r in rows])
        return Y, orc.swiglu_rows(X, w13h[e], w2h[e], nthreads=2)

    with ThreadPoolExecutor(max_workers=8) as ex:
        res = list(ex.map(one, [int(e) for e in np.nonzero(ref.counts)[0]]))
    Y = np.concatenate([r[0] for r in res])
    say("  %d experts, %d sampled rows" % (len(res), len(Y)))
    assert_close(Y, np.concatenate([r[1] for r in res]), "expert rows (sampled)")
    ot8 = [moe.read_rows("out_tok", s, 0, int(tot[s])) for s in range(cfg.S)]
    xb = torch.from_numpy(orc.dequant_e4m3_rows(_token_rows(x8, sc), ns).view(np.int16)) \
        .view(torch.bfloat16).cuda()
    outb, code = _run_bf16(moe, xb, idx, w, w13, w2)
    assert code == ccm.CCO_OK
    for s in range(cfg.S):
        np.testing.assert_array_equal(ot8[s], moe.read_rows("out_tok", s, 0, int(tot[s])),
                                      err_msg="expert rows slot %d" % s)
    assert torch.equal(out8.view(torch.int16), outb.view(torch.int16))
    say("  whole path bit-identical to the bf16 path")
    heap.destroy()


def test_expert_8bit_mixtral_full_size(ccm, orc):
    # the full Mixtral shape (T = 4096, H = 4096, top-2 of 8 experts, one per
    # slot, I = 14336; gate/up bound by the matrix cores, down split into
    # K-ranges in its last round): one row of every 256-row m-tile of every
    # expert against the oracle, and the whole path bit-identical to the bf16
    # path on the oracle's dequantized tokens
    cfg = get_config("mixtral")
    say("case: 8-bit expert mixtral full size")
    x8, sc, idx, w = _inputs(cfg, 128)
    ns = sc.shape[1]
    heap, moe = make_moe(cfg)
    w13, w2 = expert_weights(cfg, "cuda")
    out8, code = _run_fp8(moe, x8, sc, idx, w, w13, w2)
    assert code == ccm.CCO_OK and moe.status()[0] == ccm.CCO_OK
    ref = orc.plan(idx, cfg.E, cfg.S, moe.cap)
    tot = moe.read_routing()[3]
    w13h, w2h = bf16_bits(w13), bf16_bits(w2)

    def one(e):
        s, o, c = e // cfg.eps, int(ref.expert_off[e]), int(ref.counts[e])
        rows = sorted({min(c - 1, m + (7 * m // 256) % 256) for m in range(0, c, 256)} | {c - 1})
        X = np.concatenate([orc.dequant_e4m3_rows(_read_rows8(moe, s, o + r, 1), ns)
                            for r in rows])
        Y = np.stack([moe.read_rows("out_tok", s, o + r, 1)[0] for r in rows])
        return Y, orc.swiglu_rows(X, w13h[e], w2h[e], nthreads=2)

    with ThreadPoolExecutor(max_workers=8) as ex:
        res = list(ex.map(one, [int(e) for e in np.nonzero(ref.counts)[0]]))
    Y = np.concatenate([r[0] for r in res])
    say("  %d experts, %d sampled rows" % (len(res), len(Y)))
    assert_close(Y, np.concatenate([r[1] for r in res]), "expert rows (sampled)")
    ot8 = [moe.read_rows("out_tok", s, 0, int(tot[s])) for s in range(cfg.S)]
    xb = torch.from_numpy(orc.dequant_e4m3_rows(_token_rows(x8, sc), ns).view(np.int16)) \
        .view(torch.bfloat16).cuda()
    outb, code = _run_bf16(moe, xb, idx, w, w13, w2)
    assert code == ccm.CCO_OK
    for s in range(cfg.S):
        np.testing.assert_array_equal(ot8[s], moe.read_rows("out_tok", s, 0, int(tot[s])),
                                      err_msg="expert rows slot %d" % s)
    assert torch.equal(out8.view(torch.int16), outb.view(torch.int16))
    say("  whole path bit-identical to the bf16 path")
    heap.destroy()


def test_expert_8bit_decode_full_size(ccm, orc):
    # the decode shape (T = 256, H = 7168, top-8 of 256 experts over 8
    # slots, I = 2048): every expert holds a few rows, all of them in
    # 128 x 512 remainder tiles, and both GEMMs cut their one short round
    # into K-ranges.  The first and last row of every expert against the
    # oracle, and the whole path bit-identical to the bf16 path on the
    # oracle's dequantized tokens
    cfg = get_config("decode")
    say("case: 8-bit expert decode full size")
    x8, sc, idx, w = _inputs(cfg, 128)
    ns = sc.shape[1]
    heap, moe = make_moe(cfg)
    w13, w2 = expert_weights(cfg, "cuda")
    out8, code = _run_fp8(moe, x8, sc, idx, w, w13, w2)
    assert code == ccm.CCO_OK and moe.status()[0] == ccm.CCO_OK
    ref = orc.plan(idx, cfg.E, cfg.S, moe.cap)
    tot = moe.read_routing()[3]
    w13h, w2h = bf16_bits(w13), bf16_bits(w2)

    def one(e):
        s, o, c = e // cfg.eps, int(ref.expert_off[e]), int(ref.counts[e])
        rows = sorted({0, c - 1})
        X = np.concatenate([orc.dequant_e4m3_rows(_read_rows8(moe, s, o + r, 1), ns)
                            for r in rows])
        Y = np.stack([moe.read_rows("out_tok", s, o + r, 1)[0] for r in rows])
        return Y, orc.swiglu_rows(X, w13h[e], w2h[e], nthreads=2)

    with ThreadPoolExecutor(max_workers=8) as ex:
        res = list(ex.map(one, [int(e) for e in np.nonzero(ref.counts)[0]]))
    Y = np.concatenate([r[0] for r in res])
    say("  %d experts, %d sampled rows" % (len(res), len(Y)))
    assert_close(Y, np.concatenate([r[1] for r in res]), "expert rows (sampled)")
    ot8 = [moe.read_rows("out_tok", s, 0, int(tot[s])) for s in range(cfg.S)]
    xb = torch.from_numpy(orc.dequant_e4m3_rows(_token_rows(x8, sc), ns).view(np.int16)) \
        .view(torch.bfloat16).cuda()
    outb, code = _run_bf16(moe, xb, idx, w, w13, w2)
    assert code == ccm.CCO_OK
    for s in range(cfg.S):
        np.testing.assert_array_equal(ot8[s], moe.read_rows("out_tok", s, 0, int(tot[s])),
                                      err_msg="expert rows slot %d" % s)
    assert torch.equal(out8.view(torch.int16), outb.view(torch.int16))
    say("  whole path bit-identical to the bf16 path")
    heap.destroy()
