"""Seeded generators: activations, routing, expert weights.

Independent streams keep each draw reproducible on its own:
  x        numpy default_rng([seed, 0]), N(0, 1) fp32 -> bf16
  routing  numpy default_rng([seed, 2]) (router logits, Gumbel noise, biases)
  weights  torch.Generator per expert e, seeded (seed + 1) * 1_000_003 + e,
           N(0, std) fp32 -> bf16, drawn on the device that will hold them
"""
from __future__ import annotations

import numpy as np
import torch

from .configs import MoEConfig


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def bits_to_bf16(a: np.ndarray) -> torch.Tensor:
    """numpy uint16 bit patterns -> bf16 tensor on the host."""
    return torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).view(torch.bfloat16)


def activations(cfg: MoEConfig, T: int | None = None) -> torch.Tensor:
    """x [T, H] bf16 on the host, N(0, 1)."""
    T = cfg.T if T is None else T
    rng = np.random.default_rng([cfg.seed, 0])
    x = rng.standard_normal((T, cfg.H), dtype=np.float32)
    return torch.from_numpy(x).to(torch.bfloat16)


def _topk_desc(score: np.ndarray, k: int) -> np.ndarray:
    """Column order: descending score, ties to the lower expert id."""
    order = np.argsort(-score, axis=1, kind="stable")
    return order[:, :k]


def routing(cfg: MoEConfig, T: int | None = None) -> tuple[np.ndarray, np.ndarray]:
    """(idx int32 [T, K], w float32 [T, K]); columns in descending score."""
    T = cfg.T if T is None else T
    E, K = cfg.E, cfg.K
    rng = np.random.default_rng([cfg.seed, 2])
    kind = cfg.routing
    if kind == "softmax_topk":
        # p = softmax(logits) over all experts; weights are p at the chosen ids
        logits = rng.standard_normal((T, E))
        p = np.exp(logits - logits.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        idx = _topk_desc(p, K)
        w = np.take_along_axis(p, idx, axis=1)
    elif kind == "softmax_selected":
        # top-k of N(0,1) logits, softmax over the selected logits only
        logits = rng.standard_normal((T, E))
        idx = _topk_desc(logits, K)
        sel = np.take_along_axis(logits, idx, axis=1)
        w = np.exp(sel - sel.max(axis=1, keepdims=True))
        w /= w.sum(axis=1, keepdims=True)
    elif kind == "biased_sigmoid":
        # select on logits + per-expert bias; weight sigmoid(score) renormalised
        bias = rng.normal(0.0, 0.5, size=E)
        logits = rng.standard_normal((T, E))
        s = logits + bias[None, :]
        idx = _topk_desc(s, K)
        sig = 1.0 / (1.0 + np.exp(-np.take_along_axis(s, idx, axis=1)))
        w = sig / sig.sum(axis=1, keepdims=True)
    elif kind == "zipf":
        # expert popularity p_e ~ (e+1)^-1.2; K distinct experts per token by
        # Gumbel-top-k on log p; weights p renormalised over the chosen ones
        p = (np.arange(E, dtype=np.float64) + 1.0) ** -1.2
        p /= p.sum()
        g = rng.gumbel(size=(T, E))
        idx = _topk_desc(np.log(p)[None, :] + g, K)
        pw = p[idx]
        w = pw / pw.sum(axis=1, keepdims=True)
    else:
        raise ValueError("unknown routing kind %r" % kind)
    return np.ascontiguousarray(idx, np.int32), np.ascontiguousarray(w, np.float32)


def forced_edge_routing(T: int, K: int, E: int, S: int, seed: int = 0,
                        n_empty: int = 4, n_one: int = 4, n_two: int = 4
                        ) -> tuple[np.ndarray, np.ndarray]:
    """Routing with experts forced empty, and experts with exactly one and
    exactly two rows; the remaining experts take random distinct picks.
    Expert ids of each kind are spread over the slots."""
    rng = np.random.default_rng([seed, 3])
    perm = rng.permutation(E)
    empty = perm[:n_empty]
    one = perm[n_empty:n_empty + n_one]
    two = perm[n_empty + n_one:n_empty + n_one + n_two]
    rest = np.sort(perm[n_empty + n_one + n_two:])
    assert len(rest) >= K
    idx = np.empty((T, K), np.int64)
    for t in range(T):
        idx[t] = rng.choice(rest, size=K, replace=False)
    # overwrite column K-1 of distinct tokens with the 1-row and 2-row experts
    special = list(one) + [e for e in two for _ in range(2)]
    assert len(special) <= T
    toks = rng.choice(T, size=len(special), replace=False)
    for t, e in zip(toks, special):
        idx[t, K - 1] = e
    w = rng.random((T, K))
    w /= w.sum(axis=1, keepdims=True)
    return np.ascontiguousarray(idx, np.int32), np.ascontiguousarray(w, np.float32)


def expert_weights(cfg: MoEConfig, device: str | torch.device = "cpu",
                   experts: list[int] | None = None):
    """(w13 [E, 2I, H], w2 [E, H, I]) bf16 on `device`, N(0, std).

    w13 rows 0..I-1 are the gate projection, rows I..2I-1 the up projection;
    both matrices are K-contiguous like nn.Linear.weight.  With `experts`
    given, only those experts are drawn (stacked in that order); the values
    of expert e do not depend on which others are drawn.
    """
    if cfg.I == 0:
        return None, None
    device = torch.device(device)
    ids = list(range(cfg.E)) if experts is None else list(experts)
    H, I = cfg.H, cfg.I
    w13 = torch.empty((len(ids), 2 * I, H), dtype=torch.bfloat16, device=device)
    w2 = torch.empty((len(ids), H, I), dtype=torch.bfloat16, device=device)
    for n, e in enumerate(ids):
        g = torch.Generator(device=device)
        g.manual_seed((cfg.seed + 1) * 1_000_003 + int(e))
        a = torch.randn((2 * I, H), generator=g, device=device, dtype=torch.float32)
        w13[n] = (a * cfg.weight_std).to(torch.bfloat16)
        del a
        b = torch.randn((H, I), generator=g, device=device, dtype=torch.float32)
        w2[n] = (b * cfg.weight_std).to(torch.bfloat16)
        del b
    return w13, w2


def quantized_activations(cfg: MoEConfig, T: int | None = None, block: int = 128
                          ) -> tuple[np.ndarray, np.ndarray]:
    """Tokens as a caller would quantize them before an 8-bit dispatch:
    x (as drawn by `activations`) in blocks of `block` values along H, each
    block scaled by its absolute maximum / 448 and cast to OCP e4m3 by torch.
    Returns (x8 uint8 [T, H] raw bytes, scales fp32 [T, H // block]).  The
    dispatch moves these bytes without reading them, so only their shape
    and realism matter here."""
    x = activations(cfg, T).float()
    T, H = x.shape
    assert H % block == 0
    xb = x.view(T, H // block, block)
    sc = xb.abs().amax(dim=2).clamp_min(1e-12) / 448.0
    q = (xb / sc.unsqueeze(2)).to(torch.float8_e4m3fn).view(T, H)
    return q.view(torch.uint8).numpy().copy(), sc.numpy().astype(np.float32)
