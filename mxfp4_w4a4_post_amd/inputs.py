"""Seeded synthetic inputs for the MACaQ W4A4 linear layer.

This module is the only code that the HIP path and the CPU oracle share: it
draws activations, calibration rows, weights and MoE routing, and holds none
of the method's arithmetic (no scale, no Hadamard, no quantization). Every
draw is fp32 from numpy ``default_rng([config, shape, stream])`` and is
rounded once to bf16 (round-to-nearest-even) by torch.

Streams: 0 outlier channels, 1 calibration rows, 2 evaluation rows,
3 weights, 4 routing.

The pages measure trained models (Qwen3 in vLLM, Llama-3-8B) on text; these
seeded tensors stand in for those layers' activations and weights at the
same layer shapes. The distributions are:

* tiny / decode: N(0, 1) activations with 4 seeded channels x50;
* prefill 8B-shaped: Student-t(3) with round(1% of K) channels x30;
* large prefill: Student-t(3) with round(0.5% of K) channels x100;
* weights N(0, 0.02^2) (N(0, 0.015^2) for the large prefill);
* MoE: 4096 tokens, top-8 of 128 experts with Zipf(1.1) popularity (Gumbel
  top-k over log-popularity of a seeded permutation), rows in expert-major
  order.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

CALIB_ROWS = 64

# Shapes of the five workloads. Each linear shape is (K, N).
TINY = dict(name="tiny", M=16, shapes=[(256, 256)], blocks=[32])
PREFILL_8B = dict(name="prefill-8b", M=2048, shapes=[(4096, 4096), (4096, 14336), (14336, 4096)], blocks=[32])
DECODE_32B = dict(name="decode-32b", Ms=[1, 8, 32, 64], shapes=[(5120, 25600), (25600, 5120)], blocks=[32])
MOE = dict(name="moe-128e", tokens=4096, experts=128, top_k=8, hidden=2048, ffn=768, zipf=1.1, blocks=[32])
PREFILL_LARGE = dict(name="prefill-large", M=8192, shapes=[(8192, 28672), (28672, 8192)], blocks=[32, 64, 128])

WORKLOAD_SPECS = {1: TINY, 2: PREFILL_8B, 3: DECODE_32B, 4: MOE, 5: PREFILL_LARGE}


def _rng(cfg: int, shape_idx: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([cfg, shape_idx, stream])


def to_bf16(a: np.ndarray) -> torch.Tensor:
    """fp32 numpy -> bf16 torch (CPU), round-to-nearest-even."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 torch tensor -> numpy uint16 array of its bits (CPU copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _act_recipe(cfg: int):
    """(distribution, outlier fraction or count, outlier factor)."""
    if cfg in (1, 3, 4):
        return "normal", 4, 50.0
    if cfg == 2:
        return "student3", 0.01, 30.0
    if cfg == 5:
        return "student3", 0.005, 100.0
    raise ValueError("unknown workload %r" % cfg)


def outlier_channels(cfg: int, shape_idx: int, K: int) -> np.ndarray:
    _, amount, _ = _act_recipe(cfg)
    n = amount if isinstance(amount, int) else int(round(amount * K))
    n = max(0, min(n, K))
    return np.sort(_rng(cfg, shape_idx, 0).choice(K, size=n, replace=False))


def _draw_acts(rng: np.random.Generator, cfg: int, rows: int, K: int, chans: np.ndarray) -> np.ndarray:
    dist, _, factor = _act_recipe(cfg)
    if dist == "normal":
        x = rng.standard_normal((rows, K), dtype=np.float32)
    else:
        x = rng.standard_t(3.0, size=(rows, K)).astype(np.float32)
    if chans.size:
        x[:, chans] *= np.float32(factor)
    return x


def activations(cfg: int, shape_idx: int, M: int, K: int, stream: int = 2) -> torch.Tensor:
    """[M, K] bf16 activation rows of workload `cfg` (stream 2: evaluation)."""
    chans = outlier_channels(cfg, shape_idx, K)
    return to_bf16(_draw_acts(_rng(cfg, shape_idx, stream), cfg, M, K, chans))


def calibration(cfg: int, shape_idx: int, K: int, rows: int = CALIB_ROWS) -> torch.Tensor:
    """[rows, K] bf16 calibration rows: same distribution and outlier channels."""
    return activations(cfg, shape_idx, rows, K, stream=1)


def weights(cfg: int, shape_idx: int, N: int, K: int) -> torch.Tensor:
    sigma = 0.015 if cfg == 5 else 0.02
    w = _rng(cfg, shape_idx, 3).standard_normal((N, K), dtype=np.float32)
    w *= np.float32(sigma)
    return to_bf16(w)


@dataclass
class LinearCase:
    """One linear layer of a workload: bf16 x [M, K], calibration [64, K], W [N, K]."""
    cfg: int
    shape_idx: int
    M: int
    K: int
    N: int
    b: int
    x: torch.Tensor
    xcal: torch.Tensor
    w: torch.Tensor

    @property
    def name(self) -> str:
        return "%s M=%d K=%d N=%d b=%d" % (WORKLOAD_SPECS[self.cfg]["name"], self.M, self.K, self.N, self.b)


def linear_case(cfg: int, shape_idx: int = 0, M: int | None = None, b: int | None = None,
                K: int | None = None, N: int | None = None, with_weights: bool = True) -> LinearCase:
    """Build one linear layer of workload `cfg` (1, 2, 3 or 5).

    ``M``/``K``/``N`` override the workload's sizes (smaller parity cases keep
    the same distributions); ``b`` picks the Hadamard block.
    """
    spec = WORKLOAD_SPECS[cfg]
    if cfg == 4:
        raise ValueError("the MoE workload is built by moe_case")
    k0, n0 = spec["shapes"][shape_idx]
    K = k0 if K is None else K
    N = n0 if N is None else N
    if M is None:
        M = spec["M"] if "M" in spec else spec["Ms"][-1]
    b = spec["blocks"][0] if b is None else b
    x = activations(cfg, shape_idx, M, K)
    xcal = calibration(cfg, shape_idx, K)
    w = weights(cfg, shape_idx, N, K) if with_weights else torch.empty(0, K, dtype=torch.bfloat16)
    return LinearCase(cfg, shape_idx, M, K, N, b, x, xcal, w)


@dataclass
class MoECase:
    """Grouped layer: expert-major rows, offsets [E+1], per-expert calibration and weights."""
    T: int
    E: int
    K: int
    N: int
    b: int
    x: torch.Tensor          # [T, K] bf16, expert-major
    offsets: np.ndarray      # int32 [E+1]
    token_of_row: np.ndarray  # int64 [T] source token of each row
    xcal: torch.Tensor       # [E, 64, K] bf16
    w: torch.Tensor          # [E, N, K] bf16
    counts: np.ndarray = field(default=None)


def moe_topk(tokens: int, experts: int, top_k: int, zipf: float, seed_cfg: int = 4):
    """Top-k expert choice per token with Zipf(`zipf`) expert popularity.

    Logits are ln p(pi(e)) + Gumbel(0, 1) with p(r) proportional to r^-zipf
    and pi a seeded permutation of the experts; each token takes its k
    largest logits. Returns (ids int32 [T, k], routing weights fp32 [T, k]:
    the softmax of the token's k chosen logits).
    """
    rng = _rng(seed_cfg, 0, 4)
    ranks = np.arange(1, experts + 1, dtype=np.float64)
    p = ranks ** (-zipf)
    p /= p.sum()
    perm = rng.permutation(experts)
    logp = np.log(p[perm])
    g = rng.gumbel(size=(tokens, experts))
    logits = logp[None, :] + g
    topk = np.argsort(-logits, axis=1, kind="stable")[:, :top_k]
    chosen = np.take_along_axis(logits, topk, axis=1)
    wexp = np.exp(chosen - chosen.max(axis=1, keepdims=True))
    weights = (wexp / wexp.sum(axis=1, keepdims=True)).astype(np.float32)
    return topk.astype(np.int32), weights


def moe_routing(tokens: int, experts: int, top_k: int, zipf: float, seed_cfg: int = 4):
    """The grouped layer's row order for the routing of `moe_topk`: rows sorted
    by expert, then token. Returns (row -> token index, offsets[E+1])."""
    topk, _ = moe_topk(tokens, experts, top_k, zipf, seed_cfg)
    tok = np.repeat(np.arange(tokens), top_k)
    exp_ = topk.reshape(-1)
    order = np.lexsort((tok, exp_))  # by expert, then token
    counts = np.bincount(exp_, minlength=experts)
    offsets = np.zeros(experts + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    return tok[order], offsets


def moe_case(proj: str = "gate_up", tokens: int | None = None, experts: int | None = None,
             with_weights: bool = True) -> MoECase:
    """The MoE workload: `gate_up` (K=2048 -> N=1536, gate and up side by side)
    or `down` (K=768 -> N=2048). Down-projection inputs are drawn with the
    same recipe at K=768. ``tokens``/``experts`` shrink it for parity runs."""
    spec = MOE
    tokens = spec["tokens"] if tokens is None else tokens
    E = spec["experts"] if experts is None else experts
    top_k = min(spec["top_k"], E)
    if proj == "gate_up":
        K, N, sidx = spec["hidden"], 2 * spec["ffn"], 0
    elif proj == "down":
        K, N, sidx = spec["ffn"], spec["hidden"], 1
    else:
        raise ValueError(proj)
    tok_of_row, offsets = moe_routing(tokens, E, top_k, spec["zipf"])
    x_tok = _draw_acts(_rng(4, sidx, 2), 4, tokens, K, outlier_channels(4, sidx, K))
    x = to_bf16(x_tok[tok_of_row])
    chans = outlier_channels(4, sidx, K)
    cal = _draw_acts(_rng(4, sidx, 1), 4, E * CALIB_ROWS, K, chans).reshape(E, CALIB_ROWS, K)
    xcal = to_bf16(cal)
    if with_weights:
        w = _rng(4, sidx, 3).standard_normal((E, N, K), dtype=np.float32)
        w *= np.float32(0.02)
        wt = to_bf16(w)
    else:
        wt = torch.empty(E, 0, K, dtype=torch.bfloat16)
    counts = np.diff(offsets)
    return MoECase(int(offsets[-1]), E, K, N, spec["blocks"][0], x, offsets, tok_of_row, xcal, wt, counts)


@dataclass
class MoEBlockCase:
    """The MoE block: T bf16 tokens [T, H], top-k ids and routing weights
    [T, k], per-expert calibration rows for the gate/up input [E, 64, H] and
    for the down input [E, 64, F], and bf16 weights gate, up [E, F, H] and
    down [E, H, F]."""
    T: int
    E: int
    k: int
    H: int
    F: int
    b: int
    x: torch.Tensor
    ids: np.ndarray
    w: np.ndarray
    xcal_gu: torch.Tensor
    xcal_dn: torch.Tensor
    w_gate: torch.Tensor
    w_up: torch.Tensor
    w_dn: torch.Tensor


def moe_block_case(tokens: int | None = None, experts: int | None = None, top_k: int | None = None,
                   hidden: int | None = None, ffn: int | None = None, b: int | None = None,
                   with_weights: bool = True) -> MoEBlockCase:
    """The MoE workload as a whole block (defaults: 4096 tokens, 128 experts,
    top-8, hidden 2048, expert FFN 768, b = 32). Token activations follow the
    MoE recipe at K = hidden; the down projection's calibration rows are
    drawn with the same recipe at K = ffn (a stand-in for the gated
    activations of calibration text). Smaller sizes keep the distributions."""
    spec = MOE
    T = spec["tokens"] if tokens is None else tokens
    E = spec["experts"] if experts is None else experts
    k = min(spec["top_k"] if top_k is None else top_k, E)
    H = spec["hidden"] if hidden is None else hidden
    F = spec["ffn"] if ffn is None else ffn
    b = spec["blocks"][0] if b is None else b
    ids, w = moe_topk(T, E, k, spec["zipf"])
    chans_h = outlier_channels(4, 0, H)
    chans_f = outlier_channels(4, 1, F)
    x = to_bf16(_draw_acts(_rng(4, 0, 2), 4, T, H, chans_h))
    xcal_gu = to_bf16(_draw_acts(_rng(4, 0, 1), 4, E * CALIB_ROWS, H, chans_h).reshape(E, CALIB_ROWS, H))
    xcal_dn = to_bf16(_draw_acts(_rng(4, 1, 1), 4, E * CALIB_ROWS, F, chans_f).reshape(E, CALIB_ROWS, F))
    if with_weights:
        rng = _rng(4, 2, 3)
        wg = rng.standard_normal((E, F, H), dtype=np.float32) * np.float32(0.02)
        wu = rng.standard_normal((E, F, H), dtype=np.float32) * np.float32(0.02)
        wd = rng.standard_normal((E, H, F), dtype=np.float32) * np.float32(0.02)
        w_gate, w_up, w_dn = to_bf16(wg), to_bf16(wu), to_bf16(wd)
    else:
        w_gate = w_up = torch.empty(E, 0, H, dtype=torch.bfloat16)
        w_dn = torch.empty(E, 0, F, dtype=torch.bfloat16)
    return MoEBlockCase(T, E, k, H, F, b, x, ids, w, xcal_gu, xcal_dn, w_gate, w_up, w_dn)
