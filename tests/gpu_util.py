"""Helpers for the GPU parity tests: build the inputs, run the path through
the C ABI, read results back.  Oracle comparisons live in the tests."""
from __future__ import annotations

import sys
from dataclasses import dataclass

import numpy as np
import torch

from synth import MoEConfig
from synth.gen import activations, bf16_bits, expert_weights, routing

TOL = 2e-2  # max|err| <= TOL * max|ref| for the bf16 expert and combine outputs


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@dataclass
class Case:
    cfg: MoEConfig
    T: int
    x: torch.Tensor          # bf16 [T, H] device
    idx: torch.Tensor        # int32 [T, K] device
    w: torch.Tensor          # fp32 [T, K] device
    w13: torch.Tensor | None
    w2: torch.Tensor | None
    x_np: np.ndarray         # uint16 [T, H]
    idx_np: np.ndarray
    w_np: np.ndarray


def make_case(cfg: MoEConfig, T: int | None = None, idx_w=None, weights=True) -> Case:
    T = cfg.T if T is None else T
    xt = activations(cfg, T)
    if idx_w is None:
        idx_np, w_np = routing(cfg, T)
    else:
        idx_np, w_np = idx_w
    dev = torch.device("cuda")
    w13 = w2 = None
    if weights and cfg.I > 0:
        w13, w2 = expert_weights(cfg, dev)
    return Case(cfg, T, xt.to(dev), torch.from_numpy(np.ascontiguousarray(idx_np)).to(dev),
                torch.from_numpy(np.ascontiguousarray(w_np)).to(dev), w13, w2,
                bf16_bits(xt), np.ascontiguousarray(idx_np, np.int32),
                np.ascontiguousarray(w_np, np.float32))


def make_moe(cfg: MoEConfig, max_tokens: int | None = None):
    from combine_symmetric_memory_amd import MoE, SymHeap, required_slot_bytes
    mt = cfg.T if max_tokens is None else max_tokens
    need = required_slot_bytes(mt, cfg.H, cfg.K, cfg.E, cfg.I, cfg.S)
    assert need > 0
    heap = SymHeap(cfg.S, need)
    moe = MoE(heap, mt, cfg.H, cfg.K, cfg.E, cfg.I)
    return heap, moe


def run_path(moe, c: Case, expert_out=None):
    moe.plan(c.idx)
    moe.dispatch(c.x, c.w)
    moe.expert(c.w13, c.w2)
    out, code = moe.combine(c.w, expert_out=expert_out)
    torch.cuda.synchronize()
    return out, code


def f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def assert_close(got_bits: np.ndarray, ref_bits: np.ndarray, what: str, tol: float = TOL):
    g, r = f32(got_bits).astype(np.float64), f32(ref_bits).astype(np.float64)
    assert np.isfinite(g).all(), what + ": non-finite values"
    err = np.abs(g - r).max() if g.size else 0.0
    bound = tol * (np.abs(r).max() if r.size else 0.0)
    say("  %s: max|err| = %.3e, bound %.3e (max|ref| %.3e)" % (what, err, bound,
                                                            np.abs(r).max() if r.size else 0))
    assert err <= bound, "%s: max|err| %.4e > %.4e" % (what, err, bound)


def weights_host(c: Case, e: int):
    return bf16_bits(c.w13[e]), bf16_bits(c.w2[e])


def read_guards(moe) -> list[np.ndarray]:
    lay = moe.layout
    out = []
    for s in range(moe.S):
        for off, n in ((lay.disp_x, lay.disp_x_bytes), (lay.disp_meta, lay.disp_meta_bytes),
                       (lay.hbuf, lay.hbuf_bytes), (lay.out_tok, lay.out_tok_bytes)):
            if n:
                out.append(moe.read_window(s, off + n, 256))
    return out
