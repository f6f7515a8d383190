"""Pins for the CPU oracle: each function is checked against something other
than itself -- brute force on tiny inputs, library routines (numpy stable
argsort and bincount, float64 matmul, torch's bf16 conversion), exact
rational rounding, and closed forms -- so that a dropped term, a wrong index
or a transposed operand anywhere in the oracle fails a test here."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from synth import get_config
from synth.gen import activations, bf16_bits, bits_to_bf16, expert_weights, routing
from tests.combine_cases import (_adversarial_combine_case, _bf16_of, _chain,
                                 _round_rational)

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


# ------------------------------------------------------------------ bf16 ---

def _torch_bf16_bits(v: np.ndarray) -> np.ndarray:
    return bf16_bits(torch.from_numpy(np.asarray(v, np.float32)).to(torch.bfloat16))


def _exact_bf16(d: float) -> int:
    """Nearest bf16 to d by exact rational comparison, ties to even mantissa."""
    # enumerate the two bf16 neighbours bracketing d: scan bit patterns near
    # the truncation of d's binary32 encoding
    f32 = np.float32(d)
    u = int(np.array([f32], np.float32).view(np.uint32)[0]) >> 16
    cands = []
    for b in (u - 1, u, u + 1):
        b &= 0xFFFF
        val = np.array([b << 16], np.uint32).view(np.float32)[0]
        if np.isfinite(val):
            cands.append((abs(Fraction(float(val)) - Fraction(d)), b))
    best = min(c[0] for c in cands)
    ties = [b for dist, b in cands if dist == best]
    if len(ties) == 1:
        return ties[0]
    return [b for b in ties if b % 2 == 0][0]


def test_bf16_f32_rounding_matches_torch(orc):
    rng = np.random.default_rng(123)
    vals = np.concatenate([
        rng.standard_normal(4000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-38).astype(np.float32),  # denormals
        (rng.standard_normal(2000) * 1e30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.4e38, -3.4e38, np.inf, -np.inf], np.float32),
    ])
    # exact ties: bf16 value + half an ulp, both parities of the kept bit
    base = rng.integers(0x3000, 0x4f00, size=2000).astype(np.uint32)
    ties = ((base << 16) | 0x8000).view(np.float32)
    vals = np.concatenate([vals, ties])
    ours = np.array([orc.f32_to_bf16(float(v)) for v in vals], np.uint16)
    np.testing.assert_array_equal(ours, _torch_bf16_bits(vals))


def test_bf16_f64_rounding_is_exact(orc):
    rng = np.random.default_rng(7)
    vals = list(rng.standard_normal(1500) * 10.0 ** rng.integers(-6, 6, 1500))
    # doubles just above / below / on a bf16 midpoint: the binary32 of these
    # is exactly the midpoint, which is where double rounding would go wrong
    for b in rng.integers(0x3800, 0x4800, size=300):
        mid = float(np.array([(int(b) << 16) | 0x8000], np.uint32).view(np.float32)[0])
        vals += [mid, mid * (1 + 2.0 ** -40), mid * (1 - 2.0 ** -40), -mid * (1 + 2.0 ** -40)]
    for d in vals:
        assert orc.f64_to_bf16(float(d)) == _exact_bf16(float(d)), d


# ------------------------------------------------------------------ plan ---

def _brute_plan(idx, E, S):
    """Definition by brute force: count earlier pairs with the same expert."""
    T, K = idx.shape
    eps = E // S
    flat = [int(v) for v in idx.ravel()]
    counts = [flat.count(e) for e in range(E)]
    off = []
    for e in range(E):
        s = e // eps
        off.append(sum(counts[s * eps:e]))
    pos = np.zeros((T, K), np.int64)
    for f, e in enumerate(flat):
        pos.flat[f] = off[e] + sum(1 for g in range(f) if flat[g] == e)
    tot = [sum(counts[s * eps:(s + 1) * eps]) for s in range(S)]
    return np.array(counts), np.array(off), np.array(tot), pos


@pytest.mark.parametrize("T,K,E,S", [(1, 1, 1, 1), (5, 2, 4, 2), (17, 3, 8, 4),
                                     (33, 4, 16, 16), (9, 8, 8, 1)])
def test_plan_brute_force(orc, T, K, E, S):
    rng = np.random.default_rng(T * 100 + K)
    idx = rng.integers(0, E, size=(T, K)).astype(np.int32)  # duplicates allowed
    cap = T * K
    p = orc.plan(idx, E, S, cap)
    assert p.status == orc.OK
    c, o, tot, pos = _brute_plan(idx, E, S)
    np.testing.assert_array_equal(p.counts, c)
    np.testing.assert_array_equal(p.expert_off, o)
    np.testing.assert_array_equal(p.slot_total, tot)
    np.testing.assert_array_equal(p.pos, pos)


def _numpy_plan_check(orc, idx, E, S):
    T, K = idx.shape
    eps = E // S
    cap = max(1, T * K)
    p = orc.plan(idx, E, S, cap)
    assert p.status == orc.OK
    flat = idx.ravel().astype(np.int64)
    counts = np.bincount(flat, minlength=E)
    np.testing.assert_array_equal(p.counts, counts)
    assert p.counts.sum() == T * K
    # slot order = stable sort of the flat pairs by expert id, restarted at
    # every slot boundary
    order = np.argsort(flat, kind="stable")
    sorted_e = flat[order]
    for s in range(S):
        sel = (sorted_e // eps) == s
        pairs = order[sel]                      # flat ids in slot order
        assert p.slot_total[s] == pairs.size
        np.testing.assert_array_equal(p.pos.ravel()[pairs], np.arange(pairs.size))
    # offsets: first row of each expert inside its slot
    for e in range(E):
        s = e // eps
        assert p.expert_off[e] == counts[s * eps:e].sum()


def test_plan_library_routine_random_shapes(orc):
    rng = np.random.default_rng(2024)
    for trial in range(60):
        E = int(rng.choice([1, 2, 8, 64, 256]))
        S = int(rng.choice([s for s in (1, 2, 4, 8) if E % s == 0]))
        K = int(rng.integers(1, 9))
        T = int(rng.integers(0, 301))
        idx = rng.integers(0, E, size=(T, K)).astype(np.int32)
        _numpy_plan_check(orc, idx, E, S)


@pytest.mark.parametrize("name", ["tiny", "mixtral", "dsv3", "decode", "zipf"])
def test_plan_invariants_on_configs(orc, name):
    cfg = get_config(name)
    idx, _ = routing(cfg)
    p = orc.plan(idx, cfg.E, cfg.S, cfg.cap)
    assert p.status == orc.OK
    _numpy_plan_check(orc, idx, cfg.E, cfg.S)
    # every (token, k) appears exactly once: pos restricted to a slot is a
    # bijection onto [0, slot_total)
    eps = cfg.eps
    slot = idx // eps
    for s in range(cfg.S):
        ps = np.sort(p.pos[slot == s])
        np.testing.assert_array_equal(ps, np.arange(p.slot_total[s]))


def test_plan_errors(orc):
    idx = np.array([[0, 1], [2, 8]], np.int32)
    assert orc.plan(idx, 8, 4, 100).status == orc.BAD_EXPERT
    idx = np.array([[0, -1]], np.int32)
    assert orc.plan(idx, 8, 4, 100).status == orc.BAD_EXPERT
    # every token to expert 0 of slot 0, over capacity
    idx = np.zeros((10, 1), np.int32)
    assert orc.plan(idx, 8, 4, 9).status == orc.CAPACITY
    assert orc.plan(idx, 8, 4, 10).status == orc.OK


@pytest.mark.parametrize("seed,T,K,E,S,cap", [(1, 40, 3, 8, 2, 30), (2, 25, 2, 4, 4, 9),
                                              (3, 64, 4, 8, 1, 200), (4, 7, 5, 2, 1, 20)])
def test_plan_overflow_drops_the_rows_past_capacity(orc, seed, T, K, E, S, cap):
    # brute force: a pair keeps the row the uncapped plan gives it when that
    # row is inside the slot, and is dropped (-1) otherwise
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, E, size=(T, K)).astype(np.int32)
    c, o, tot, pos = _brute_plan(idx, E, S)
    p = orc.plan(idx, E, S, cap)
    assert p.status == (orc.CAPACITY if tot.max() > cap else orc.OK)
    assert tot.max() > cap  # the shapes above do overflow
    np.testing.assert_array_equal(p.counts, c)
    np.testing.assert_array_equal(p.slot_total, tot)
    np.testing.assert_array_equal(p.pos, np.where(pos < cap, pos, -1))
    # dispatch and combine skip the dropped pairs
    H = 16
    x = _torch_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    w = rng.random((T, K)).astype(np.float32)
    d = orc.dispatch(x, w, idx, p.pos, E, S, cap)
    eps = E // S
    filled = np.zeros((S, cap), bool)
    for t in range(T):
        for j in range(K):
            if p.pos[t, j] >= 0:
                filled[idx[t, j] // eps, p.pos[t, j]] = True
                np.testing.assert_array_equal(d.disp_x[idx[t, j] // eps, p.pos[t, j]], x[t])
    assert (d.meta_src[~filled] == -1).all()
    out = orc.combine_tokens(d.disp_x, w, idx, p.pos, E, S)
    keep = np.where(p.pos >= 0, w, np.float32(0))
    np.testing.assert_array_equal(out, orc.combine_tokens(d.disp_x, keep, idx,
                                                          np.where(p.pos >= 0, p.pos, 0), E, S))


# -------------------------------------------------------------- dispatch ---

def test_dispatch_closed_form(orc):
    cfg = get_config("tiny")
    x = bf16_bits(activations(cfg))
    idx, w = routing(cfg)
    p = orc.plan(idx, cfg.E, cfg.S, cfg.cap)
    d = orc.dispatch(x, w, idx, p.pos, cfg.E, cfg.S, cfg.cap)
    eps = cfg.eps
    seen = np.zeros((cfg.S, cfg.cap), bool)
    for t in range(cfg.T):
        for j in range(cfg.K):
            e = idx[t, j]
            s, r = e // eps, p.pos[t, j]
            np.testing.assert_array_equal(d.disp_x[s, r], x[t])
            assert d.meta_src[s, r] == t * cfg.K + j
            assert d.meta_w[s, r] == w[t, j]
            assert d.meta_e[s, r] == e
            seen[s, r] = True
    # rows past each slot's total are untouched
    for s in range(cfg.S):
        assert seen[s, :p.slot_total[s]].all() and not seen[s, p.slot_total[s]:].any()
        assert not d.disp_x[s, p.slot_total[s]:].any()
    # inside an expert's segment the source pairs strictly increase (stable)
    for e in range(cfg.E):
        s, o, n = e // eps, p.expert_off[e], p.counts[e]
        assert np.all(np.diff(d.meta_src[s, o:o + n]) > 0)
        assert np.all(d.meta_e[s, o:o + n] == e)


def _fp8_case(seed, T, H, K, E, S, ns):
    rng = np.random.default_rng(seed)
    x8 = rng.integers(0, 256, (T, H), dtype=np.uint8)
    sc = rng.standard_normal((T, ns)).astype(np.float32)
    idx = rng.integers(0, E, (T, K)).astype(np.int32)
    w = rng.random((T, K)).astype(np.float32)
    return x8, sc, idx, w


def test_dispatch_fp8_with_no_scales_is_the_bf16_dispatch_of_the_same_bytes(orc):
    # H bytes per token read as H/2 bf16 values: the bf16 dispatch (pinned
    # above) must place the same bytes in the same rows, with the same metadata
    T, H, K, E, S = 50, 64, 3, 8, 4
    x8, sc, idx, w = _fp8_case(1, T, H, K, E, S, 0)
    cap = T * min(K, E // S)
    p = orc.plan(idx, E, S, cap)
    d8 = orc.dispatch_fp8(x8, sc, w, idx, p.pos, E, S, cap)
    d16 = orc.dispatch(x8.view(np.uint16), w, idx, p.pos, E, S, cap)
    np.testing.assert_array_equal(d8.disp_x[:, :, :H], d16.disp_x.view(np.uint8))
    assert not d8.disp_x[:, :, H:].any()
    for a, b in ((d8.meta_src, d16.meta_src), (d8.meta_w, d16.meta_w), (d8.meta_e, d16.meta_e)):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("T,H,K,E,S,ns", [(1, 16, 1, 1, 1, 4), (9, 32, 2, 4, 2, 1),
                                          (23, 64, 3, 8, 4, 16), (40, 128, 4, 16, 8, 7)])
def test_dispatch_fp8_brute_force(orc, T, H, K, E, S, ns):
    x8, sc, idx, w = _fp8_case(T * 31 + ns, T, H, K, E, S, ns)
    cap = T * min(K, E // S)
    p = orc.plan(idx, E, S, cap)
    d = orc.dispatch_fp8(x8, sc, w, idx, p.pos, E, S, cap)
    eps = E // S
    hits = np.zeros((S, cap), np.int32)
    for t in range(T):
        for j in range(K):
            s, r = idx[t, j] // eps, p.pos[t, j]
            row = d.disp_x[s, r]
            assert bytes(row[:H]) == bytes(x8[t])
            assert bytes(row[H:H + 4 * ns]) == sc[t].tobytes()
            assert not row[H + 4 * ns:].any()
            assert (d.meta_src[s, r], d.meta_e[s, r]) == (t * K + j, idx[t, j])
            assert d.meta_w[s, r] == w[t, j]
            hits[s, r] += 1
    # every pair lands exactly once, in a row below its slot's total;
    # nothing else is written
    for s in range(S):
        n = p.slot_total[s]
        assert (hits[s, :n] == 1).all() and not hits[s, n:].any()
        assert not d.disp_x[s, n:].any()


# ---------------------------------------------------------------- expert ---

def _f32(bits):
    return bits_to_bf16(bits).to(torch.float64).numpy()


def _numpy_swiglu(X, w13_e, w2_e):
    """float64 matmuls (library routine) with h and y rounded to bf16 by
    torch's conversion."""
    I = w13_e.shape[0] // 2
    x = _f32(X)
    g = x @ _f32(w13_e[:I]).T
    u = x @ _f32(w13_e[I:]).T
    h = (g / (1.0 + np.exp(-g))) * u
    hb = torch.from_numpy(h).to(torch.bfloat16).to(torch.float64).numpy()
    y = hb @ _f32(w2_e).T
    return bf16_bits(torch.from_numpy(y).to(torch.bfloat16)), hb


def _ulp_diff(a, b):
    ai = a.astype(np.int32)
    bi = b.astype(np.int32)
    # bf16 sign-magnitude -> ordered integers
    ai = np.where(ai & 0x8000, 0x8000 - ai, ai)
    bi = np.where(bi & 0x8000, 0x8000 - bi, bi)
    return np.abs(ai - bi)


@pytest.mark.parametrize("n,H,I", [(1, 16, 8), (7, 64, 32), (40, 256, 96), (3, 96, 200)])
def test_swiglu_matches_float64_matmul(orc, n, H, I):
    g = torch.Generator().manual_seed(n * 1000 + H + I)
    X = bf16_bits(torch.randn(n, H, generator=g).to(torch.bfloat16))
    w13 = bf16_bits((torch.randn(2 * I, H, generator=g) * 0.1).to(torch.bfloat16))
    w2 = bf16_bits((torch.randn(H, I, generator=g) * 0.1).to(torch.bfloat16))
    Y = orc.swiglu_rows(X, w13, w2, nthreads=3)
    ref, _ = _numpy_swiglu(X, w13, w2)
    ud = _ulp_diff(Y, ref)
    # same definition, different summation order in double: only a value
    # sitting on a bf16 rounding boundary may land one ulp away
    assert ud.max() <= 1
    assert (ud > 0).mean() < 0.02
    # a transposed or swapped operand would be far off
    yf, rf = _f32(Y), _f32(ref)
    assert np.abs(yf - rf).max() <= 1e-2 * np.abs(rf).max() + 1e-30


def test_swiglu_gate_up_not_swapped(orc):
    # gate and up play different roles: silu(g)*u != silu(u)*g
    H, I = 4, 2
    X = bf16_bits(torch.tensor([[1.0, 0, 0, 0]]).to(torch.bfloat16))
    w13 = np.zeros((2 * I, H), np.float32)
    w13[0, 0], w13[1, 0] = 30.0, -30.0     # gate: g = (30, -30)
    w13[2, 0], w13[3, 0] = 1.0, 1.0        # up:   u = (1, 1)
    wd = np.zeros((H, I), np.float32)
    wd[0, 0] = 1.0
    wd[1, 1] = 1.0
    Y = orc.swiglu_rows(X, bf16_bits(torch.from_numpy(w13).to(torch.bfloat16)),
                        bf16_bits(torch.from_numpy(wd).to(torch.bfloat16)))
    y = _f32(Y)[0]
    # silu(30) = 30 to far below bf16 resolution; silu(-30) ~ -2.8e-12
    assert y[0] == 30.0
    assert -1e-11 < y[1] < 0.0
    assert y[2] == 0.0 and y[3] == 0.0


def test_swiglu_zero_projections_give_zero(orc):
    g = torch.Generator().manual_seed(5)
    H, I, n = 64, 48, 9
    X = bf16_bits(torch.randn(n, H, generator=g).to(torch.bfloat16))
    w13 = bf16_bits(torch.randn(2 * I, H, generator=g).to(torch.bfloat16))
    w2 = bf16_bits(torch.randn(H, I, generator=g).to(torch.bfloat16))
    for zero_rows in (slice(0, I), slice(I, 2 * I)):  # gate = 0, then up = 0
        wz = w13.copy()
        wz[zero_rows] = 0
        Y = orc.swiglu_rows(X, wz, w2)
        assert not (Y & 0x7FFF).any()  # +0 or -0 everywhere


# --------------------------------------------------------------- combine ---

def test_combine_identity_expert(orc):
    cfg = get_config("tiny")
    x = bf16_bits(activations(cfg))
    idx, w = routing(cfg)
    p = orc.plan(idx, cfg.E, cfg.S, cfg.cap)
    d = orc.dispatch(x, w, idx, p.pos, cfg.E, cfg.S, cfg.cap)
    out = orc.combine_tokens(d.disp_x, w, idx, p.pos, cfg.E, cfg.S)
    # identity experts: out[t] = (sum_j w[t,j]) * x[t], to one bf16 ulp
    ref = w.astype(np.float64).sum(1, keepdims=True) * _f32(x)
    refb = bf16_bits(torch.from_numpy(ref).to(torch.bfloat16))
    assert _ulp_diff(out, refb).max() <= 1


def test_combine_k1_unit_weight_is_copy_and_zero_weight_is_zero(orc):
    rng = np.random.default_rng(3)
    T, H, E, S = 50, 32, 4, 2
    x = bf16_bits(torch.from_numpy(rng.standard_normal((T, H), dtype=np.float32)).to(torch.bfloat16))
    idx = rng.integers(0, E, size=(T, 1)).astype(np.int32)
    cap = T
    p = orc.plan(idx, E, S, cap)
    d = orc.dispatch(x, np.ones((T, 1), np.float32), idx, p.pos, E, S, cap)
    out = orc.combine_tokens(d.disp_x, np.ones((T, 1), np.float32), idx, p.pos, E, S)
    np.testing.assert_array_equal(out, x)
    out0 = orc.combine_tokens(d.disp_x, np.zeros((T, 1), np.float32), idx, p.pos, E, S)
    assert not (out0 & 0x7FFF).any()


def test_combine_weights_follow_columns(orc):
    # distinct rows and weights per column: a misaligned weight index shows
    rng = np.random.default_rng(11)
    T, K, H, E, S = 20, 3, 16, 6, 3
    src = bf16_bits(torch.from_numpy(rng.standard_normal((S, T * K, H), dtype=np.float32)).to(torch.bfloat16))
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, K)).astype(np.float32)
    p = orc.plan(idx, E, S, T * K)
    out = orc.combine_tokens(src, w, idx, p.pos, E, S)
    eps = E // S
    ref = np.zeros((T, H))
    for t in range(T):
        for j in range(K):
            ref[t] += float(w[t, j]) * _f32(src[idx[t, j] // eps, p.pos[t, j]])
    refb = bf16_bits(torch.from_numpy(ref).to(torch.bfloat16))
    assert _ulp_diff(out, refb).max() <= 1
    # combine_rows is the same arithmetic on explicit row pointers
    rows = [src[idx[t, j] // eps, p.pos[t, j]] for t in range(T) for j in range(K)]
    np.testing.assert_array_equal(orc.combine_rows(rows, w), out)



# ------------------------------------------- combine, exact fp32 fma chain ---
#
# The combine reading fixes fp32 accumulation with one fused multiply-add per
# routed row, in column order j = 0..K-1, and one final rounding to bf16.  The
# pins above only bound the result to a bf16 ulp of a float64 sum, which an
# unfused product-then-add or a reversed column loop would also meet.  The
# model below rebuilds the chain from its mathematical definition -- exact
# rationals, each fma rounded once to the nearest binary32 (ties to even) --
# and the oracle must match it bit for bit, on inputs built so that the
# unfused and the reversed chains give different bf16 results.

def _random_combine_case(seed: int, nt: int, K: int, H: int):
    rng = np.random.default_rng(seed)
    y = _torch_bf16_bits(rng.standard_normal((nt, K, H)).astype(np.float32))
    w = rng.random((nt, K)).astype(np.float32)
    return y, w


@pytest.mark.parametrize("kind,seed,nt,K,H", [("adversarial", 1, 96, 2, 4),
                                              ("adversarial", 2, 96, 4, 4),
                                              ("adversarial", 3, 96, 8, 4),
                                              ("random", 4, 16, 8, 32),
                                              ("random", 5, 12, 3, 40)])
def test_combine_is_the_exact_fp32_fma_chain_in_column_order(orc, kind, seed, nt, K, H):
    make = _adversarial_combine_case if kind == "adversarial" else _random_combine_case
    y, w = make(seed, nt, K, H)
    rows = [y[q, j] for q in range(nt) for j in range(K)]
    got = orc.combine_rows(rows, w)
    want = np.array([[_chain(w[q], y[q], h) for h in range(H)] for q in range(nt)], np.uint16)
    np.testing.assert_array_equal(got, want)
    # the same rows through the slot layout and the plan's positions
    E, S = K, 1
    idx = np.tile(np.arange(K, dtype=np.int32), (nt, 1))
    p = orc.plan(idx, E, S, nt * K)
    src = np.zeros((S, nt * K, H), np.uint16)
    for q in range(nt):
        for j in range(K):
            src[0, p.pos[q, j]] = y[q, j]
    np.testing.assert_array_equal(orc.combine_tokens(src, w, idx, p.pos, E, S), want)
    if kind == "adversarial":
        # the inputs tell the reading from its near neighbours: the unfused
        # chain, and the fused chain in reverse column order (K > 1)
        unfused = np.array([[_chain(w[q], y[q], h, fused=False) for h in range(H)]
                            for q in range(nt)], np.uint16)
        rev = np.array([[_chain(w[q], y[q], h, reverse=True) for h in range(H)]
                        for q in range(nt)], np.uint16)
        assert (unfused != want).sum() >= 10, "inputs do not separate fused from unfused"
        assert (rev != want).sum() >= 10, "inputs do not separate the column orders"


def test_round_rational_matches_binary32_and_bf16(orc):
    # the model's rounding against numpy's binary32 and the oracle's bf16 on
    # random doubles (a double -> binary32 conversion is itself one rounding)
    rng = np.random.default_rng(9)
    vals = rng.standard_normal(400) * 10.0 ** rng.integers(-30, 30, 400)
    for d in vals:
        q = Fraction(float(d))
        assert _round_rational(q, 24) == Fraction(float(np.float32(d)))
        assert _bf16_of(_round_rational(q, 8)) == orc.f64_to_bf16(float(d))


# -------------------------------------------------------------- pipeline ---

def test_tiny_pipeline_brute_force(orc):
    """End to end on the small config against an independent formulation:
    per token, per chosen expert, SwiGLU by float64 matmul, weighted sum."""
    cfg = get_config("tiny")
    xt = activations(cfg)
    x = bf16_bits(xt)
    idx, w = routing(cfg)
    w13t, w2t = expert_weights(cfg, "cpu")
    w13, w2 = bf16_bits(w13t), bf16_bits(w2t)
    r = orc.pipeline(x, w, idx, cfg.E, cfg.S, cfg.cap, w13, w2, nthreads=4)
    ref = np.zeros((cfg.T, cfg.H))
    for t in range(cfg.T):
        for j in range(cfg.K):
            e = idx[t, j]
            y, _ = _numpy_swiglu(x[t:t + 1], w13[e], w2[e])
            ref[t] += float(w[t, j]) * _f32(y)[0]
    refb = bf16_bits(torch.from_numpy(ref).to(torch.bfloat16))
    o, rb = _f32(r.out), _f32(refb)
    assert np.abs(o - rb).max() <= 2e-2 * np.abs(rb).max()
    assert _ulp_diff(r.out, refb).max() <= 2


# ---- the expert's input from 8-bit receive rows (oracle.dequant_e4m3_rows)

def _e4m3_codes_f32():
    """Every e4m3 code decoded by torch's float8_e4m3fn (a library routine)."""
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()


def _rows_8bit(q: np.ndarray, scales: np.ndarray | None) -> np.ndarray:
    """Receive rows [n, 2H]: the H code bytes, then the fp32 scales' bytes."""
    n, H = q.shape
    rows = np.zeros((n, 2 * H), np.uint8)
    rows[:, :H] = q
    if scales is not None:
        rows[:, H:H + 4 * scales.shape[1]] = np.ascontiguousarray(scales, np.float32).view(np.uint8)
    return rows


def test_e4m3_decode_on_every_code():
    """With no scales the expert input is the decoded value itself: every
    finite code against torch's e4m3fn decode (exact in bf16), the two NaN
    codes to a NaN."""
    from oracle import oracle as orc
    q = np.arange(256, dtype=np.uint8).reshape(1, 256)
    got = orc.dequant_e4m3_rows(_rows_8bit(q, None), 0)[0]
    ref = _e4m3_codes_f32()
    for c in range(256):
        if c in (0x7F, 0xFF):
            assert (got[c] & 0x7F80) == 0x7F80 and (got[c] & 0x7F) != 0, c
            continue
        bits = int(np.array([ref[c]], np.float32).view(np.uint32)[0])
        assert bits & 0xFFFF == 0, c  # e4m3 values are bf16 values
        assert got[c] == bits >> 16, (c, got[c], bits >> 16)


def _exact_two_step(code_val: float, s: float) -> int:
    """bf16 of round_binary32(code * s), from exact rationals (a zero
    product keeps the IEEE sign of the factors)."""
    p = Fraction(float(code_val)) * Fraction(float(s))
    if p == 0:
        return 0x8000 if np.copysign(1.0, code_val) * np.copysign(1.0, s) < 0 else 0
    return _bf16_of(_round_rational(_round_rational(p, 24), 8))


def _exact_one_step(code_val: float, s: float) -> int:
    p = Fraction(float(code_val)) * Fraction(float(s))
    return _bf16_of(_round_rational(p, 8))


def _is_tie(p: Fraction, prec: int) -> bool:
    """p lies exactly half-way between two numbers of `prec` significant bits."""
    if p == 0:
        return False
    a = abs(p)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    n = a / Fraction(2) ** (max(e, -126) - (prec - 1))
    return n - n.numerator // n.denominator == Fraction(1, 2)


def _dequant_witnesses(seed: int = 7):
    """(code, scale) pairs: exact products that are binary32 ties; binary32
    products that are bf16 ties; and products that the binary32 rounding
    moves onto a bf16 tie, so that rounding twice gives another bf16 than
    rounding the exact product once."""
    rng = np.random.default_rng(seed)
    vals = _e4m3_codes_f32()
    code_of = {float(vals[c]): c for c in range(128) if np.isfinite(vals[c])}
    # binary32 ties: a 4-bit significand times a random 24-bit one
    f32_ties = []
    multi = [code_of[v] for v in (1.125, 1.375, 1.625, 1.875, 1.25, 1.75)]
    while len(f32_ties) < 8:
        c = int(rng.choice(multi))
        s = float(np.float32(rng.uniform(1.0, 2.0) * 2.0 ** int(rng.integers(-20, 20))))
        if _is_tie(Fraction(float(vals[c])) * Fraction(s), 24):
            f32_ties.append((c, s))
    # bf16 ties: 1.0 times a binary32 whose low 16 bits are 0x8000
    one = code_of[1.0]
    bf16_ties = []
    for k in range(8):
        upper = (0x3F00 + (k << 7) + 2 * int(rng.integers(0, 64))) & 0x7FFF
        bf16_ties.append((one, float(np.array([(upper << 16) | 0x8000], np.uint32).view(np.float32)[0])))
    # double rounding: binary32 F a bf16 tie with an even upper half; a scale
    # near F / q whose exact product rounds to F in binary32 but lies above it
    double = []
    for k in range(64):
        if len(double) >= 8:
            break
        upper = 0x3F00 + 2 * int(rng.integers(0, 1 << 10))
        F = float(np.array([(upper << 16) | 0x8000], np.uint32).view(np.float32)[0])
        c = multi[k % len(multi)]
        qv = float(vals[c])
        s0 = np.float32(F / qv)
        for step in range(-40, 41):
            s = float(np.nextafter(s0, np.float32(np.inf if step > 0 else -np.inf)) if step else s0)
            for _ in range(abs(step) - 1):
                s = float(np.nextafter(np.float32(s), np.float32(np.inf if step > 0 else -np.inf)))
            p = Fraction(qv) * Fraction(s)
            if p > Fraction(F) and _round_rational(p, 24) == Fraction(F):
                double.append((c, s))
                break
    return f32_ties, bf16_ties, double


def test_dequant_rounds_the_scaled_value_twice_to_nearest_even():
    """Decoded value times its block's scale, rounded to binary32 and then to
    bf16 (both to nearest even): against exact rationals on random codes and
    scales (each value with its block's scale, ns = 1, 2, 4), and on
    constructed codes and scales whose product is an exact binary32 tie, an
    exact bf16 tie, or a value one rounding of which would give another
    bf16."""
    from oracle import oracle as orc
    vals = _e4m3_codes_f32()
    f32_ties, bf16_ties, double = _dequant_witnesses()
    assert len(double) >= 4 and len(bf16_ties) == 8
    rng = np.random.default_rng(3)
    finite = np.array([c for c in range(256) if np.isfinite(vals[c])], np.uint8)
    for ns in (1, 2, 4):
        H = 256
        q = rng.choice(finite, size=(3, H)).astype(np.uint8)
        sc = (rng.uniform(0.5, 2.0, (3, ns)) * 2.0 ** rng.integers(-12, 12, (3, ns))).astype(np.float32)
        got = orc.dequant_e4m3_rows(_rows_8bit(q, sc), ns)
        blk = H // ns
        for r in range(3):
            for k in range(H):
                want = _exact_two_step(vals[q[r, k]], sc[r, k // blk])
                assert got[r, k] == want, (ns, r, k, got[r, k], want)
    # the witnesses themselves, one scale each (ns = number of them, blocks of 1)
    for c, s in f32_ties + bf16_ties + double:
        q = np.full((1, 64), c, np.uint8)
        sc = np.full((1, 1), s, np.float32)
        got = orc.dequant_e4m3_rows(_rows_8bit(q, sc), 1)[0, 0]
        assert got == _exact_two_step(vals[c], s), (c, s)
    assert any(_exact_two_step(vals[c], s) != _exact_one_step(vals[c], s) for c, s in double)
