"""Seeded synthetic inputs for the block-diffusion MoE denoise step.

This module is the only code shared by the CPU oracle (``oracle/``) and the
HIP path (``block_diffusion_moe_amd``).  It draws random tensors and lays them
out; it contains none of the method's arithmetic (no routing, no expert math,
no softmax, no unmask rule).

Sources of the shapes (page titles, then section):

* "Clover-35B-A3B: how a diffusion model gets to 680 tokens a second, read from
  its files" (below: the files page), section "What Clover is": hidden 2,048,
  256 routed experts, 8 routed per token, one shared expert, vocabulary
  248,320, block_size 32, mask_token_id 151669, threshold 0.95; gate and up are
  2,048 by 512 and down is 512 by 2,048; the output head is untied.
* The files page, section "How it writes", step 1: a fresh block is 32 slots
  all holding the mask token.

Layouts (all row-major, the reduction dimension contiguous):

* x, residual            [T][H]     bf16
* w_router               [E][H]     fp32      router_bias [E] fp32 or None
* w_gate, w_up           [E][I][H]  bf16      (output-major: row i of expert e)
* w_down                 [E][H][I]  bf16
* ws_gate, ws_up         [I][H]     bf16      ws_down [H][I] bf16 (shared expert)
* h                      [T][H]     bf16      w_head [V][H] bf16
* tokens                 [T]        int32

Workload recipes (seeded; weights from ``seed``, token blocks from
``block_seed``) are described next to each generator.  Generation runs on the
device that is asked for (torch's generator for that device), so a block made
on ``cuda`` differs from one made on ``cpu`` with the same seeds; the parity
tests always feed the *same* tensors to both sides.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

MASK_ID_CLOVER = 151669
THRESHOLD = 0.95


@dataclass(frozen=True)
class MoEShape:
    T: int          # tokens in the block (block size x number of blocks)
    H: int          # hidden size
    E: int          # routed experts
    I: int          # expert intermediate size
    k: int          # routed experts per token
    shared: bool = True


@dataclass(frozen=True)
class HeadShape:
    T: int
    H: int
    V: int
    mask_id: int


# The five workloads.  "tiny" is the small case the oracle finishes instantly;
# "layer" is one Clover-shaped MoE layer over one 32-slot block; "head" is the
# untied output head over one block; "stack" is 40 layers shaped like "layer";
# "skew" is 8 concurrent blocks through one layer with a log-Zipf router bias.
TINY = MoEShape(T=8, H=64, E=16, I=32, k=2)
TINY_HEAD = HeadShape(T=8, H=64, V=512, mask_id=0)
LAYER = MoEShape(T=32, H=2048, E=256, I=512, k=8)
HEAD = HeadShape(T=32, H=2048, V=248320, mask_id=MASK_ID_CLOVER)
SKEW = MoEShape(T=256, H=2048, E=256, I=512, k=8)
STACK_LAYERS = 40


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal(g, shape, std, device, chunk_rows: int = 0) -> torch.Tensor:
    """N(0, std^2) in fp32, drawn in row chunks so that big tensors do not need
    a second full-size temporary on the host."""
    shape = tuple(shape)
    if not chunk_rows or shape[0] <= chunk_rows:
        return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std
    out = torch.empty(shape, device=device, dtype=torch.float32)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        out[r0:r1] = torch.randn((r1 - r0,) + shape[1:], generator=g, device=device,
                                 dtype=torch.float32) * std
    return out


def _normal_bf16(g, shape, std, device, chunk_rows: int = 8) -> torch.Tensor:
    """N(0, std^2) drawn in fp32 and stored as bf16 (torch's round-to-nearest-even)."""
    shape = tuple(shape)
    out = torch.empty(shape, device=device, dtype=torch.bfloat16)
    step = max(1, chunk_rows)
    for r0 in range(0, shape[0], step):
        r1 = min(shape[0], r0 + step)
        out[r0:r1] = (torch.randn((r1 - r0,) + shape[1:], generator=g, device=device,
                                  dtype=torch.float32) * std).to(torch.bfloat16)
    return out


@dataclass
class MoEInputs:
    shape: MoEShape
    x: torch.Tensor
    w_router: torch.Tensor
    router_bias: Optional[torch.Tensor]
    w_gate: torch.Tensor
    w_up: torch.Tensor
    w_down: torch.Tensor
    ws_gate: Optional[torch.Tensor]
    ws_up: Optional[torch.Tensor]
    ws_down: Optional[torch.Tensor]
    residual: Optional[torch.Tensor] = None
    # fp32 originals before the single bf16 rounding (tiny workload only)
    fp32: dict = field(default_factory=dict)


def moe_weights(shape: MoEShape, seed: int, device="cpu", std: float = 0.02,
                router_std: float = 0.02, keep_fp32: bool = False):
    """Expert, shared-expert and router weights of one layer.

    Draw order from one generator seeded with ``seed``: router [E][H] fp32,
    then per expert gate, up, down, then the shared expert's gate, up, down.
    All N(0, std^2); the router stays fp32, the rest is rounded once to bf16.
    """
    s = shape
    g = _gen(device, seed)
    w_router = _normal(g, (s.E, s.H), router_std, device)
    w_gate = torch.empty((s.E, s.I, s.H), device=device, dtype=torch.bfloat16)
    w_up = torch.empty((s.E, s.I, s.H), device=device, dtype=torch.bfloat16)
    w_down = torch.empty((s.E, s.H, s.I), device=device, dtype=torch.bfloat16)
    orig = {}
    if keep_fp32:
        orig = {"w_gate": torch.empty((s.E, s.I, s.H), dtype=torch.float32, device=device),
                "w_up": torch.empty((s.E, s.I, s.H), dtype=torch.float32, device=device),
                "w_down": torch.empty((s.E, s.H, s.I), dtype=torch.float32, device=device)}
    for e in range(s.E):
        for name, dst, shp in (("w_gate", w_gate, (s.I, s.H)), ("w_up", w_up, (s.I, s.H)),
                               ("w_down", w_down, (s.H, s.I))):
            f = torch.randn(shp, generator=g, device=device, dtype=torch.float32) * std
            dst[e] = f.to(torch.bfloat16)
            if keep_fp32:
                orig[name][e] = f
    ws = [None, None, None]
    if s.shared:
        for j, shp in enumerate(((s.I, s.H), (s.I, s.H), (s.H, s.I))):
            f = torch.randn(shp, generator=g, device=device, dtype=torch.float32) * std
            ws[j] = f.to(torch.bfloat16)
            if keep_fp32:
                orig[("ws_gate", "ws_up", "ws_down")[j]] = f
    return w_router, w_gate, w_up, w_down, ws[0], ws[1], ws[2], orig


def moe_router(shape: MoEShape, seed: int, device="cpu", router_std: float = 0.02):
    """Only the router of ``moe_weights(shape, seed)`` (it is that generator's
    first draw), for statistics that need no expert weights."""
    g = _gen(device, seed)
    return _normal(g, (shape.E, shape.H), router_std, device)


def moe_tokens(shape: MoEShape, block_seed: int, device="cpu", with_residual: bool = False,
               keep_fp32: bool = False):
    """Token block x ~ N(0,1) [T][H] rounded to bf16 (and an independent
    residual stream of the same law when asked for)."""
    g = _gen(device, 1_000_003 + block_seed)
    xf = torch.randn((shape.T, shape.H), generator=g, device=device, dtype=torch.float32)
    res = None
    rf = None
    if with_residual:
        rf = torch.randn((shape.T, shape.H), generator=g, device=device, dtype=torch.float32)
        res = rf.to(torch.bfloat16)
    orig = {"x": xf, "residual": rf} if keep_fp32 else {}
    return xf.to(torch.bfloat16), res, orig


def zipf_router_bias(E: int, seed: int, s: float = 1.1, device="cpu") -> torch.Tensor:
    """Per-expert router offset for the load-skew workload: a seeded random
    permutation assigns ranks 1..E to the experts and expert e gets
    -s * ln(rank_e) added to its fp32 logit, i.e. a Zipf(s) prior on the
    routing probabilities (a few experts take most tokens)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(7_000_001 + seed)
    rank = torch.randperm(E, generator=g).to(torch.float64) + 1.0
    return (-s * torch.log(rank)).to(torch.float32).to(device)


def moe_inputs(shape: MoEShape, seed: int = 0, block_seed: int = 1, device="cpu",
               with_residual: bool = False, zipf_s: Optional[float] = None,
               keep_fp32: bool = False) -> MoEInputs:
    wr, wg, wu, wd, sg, su, sd, orig = moe_weights(shape, seed, device, keep_fp32=keep_fp32)
    x, res, orig_t = moe_tokens(shape, block_seed, device, with_residual, keep_fp32)
    bias = zipf_router_bias(shape.E, seed, zipf_s, device) if zipf_s else None
    orig.update(orig_t)
    return MoEInputs(shape, x, wr, bias, wg, wu, wd, sg, su, sd, res, orig)


def tiny_inputs(seed: int = 0, block_seed: int = 1, with_residual: bool = False) -> MoEInputs:
    """The tiny workload: fp32 N(0,0.02) weights and N(0,1) activations, each
    rounded once to bf16 (the kernels take bf16); the fp32 originals are kept."""
    return moe_inputs(TINY, seed, block_seed, "cpu", with_residual, keep_fp32=True)


def skew_inputs(seed: int = 0, block_seed: int = 1, device="cpu") -> MoEInputs:
    return moe_inputs(SKEW, seed, block_seed, device, zipf_s=1.1)


# ----------------------------------------------------------------------------
# Output head
# ----------------------------------------------------------------------------

@dataclass
class HeadInputs:
    shape: HeadShape
    h: torch.Tensor
    w_head: torch.Tensor
    tokens: torch.Tensor
    boosted_rows: list
    boosted_tokens: list
    mask_boost_rows: list = field(default_factory=list)


def head_weights(shape: HeadShape, seed: int, device="cpu", std: float = 0.02) -> torch.Tensor:
    g = _gen(device, 2_000_003 + seed)
    rows = max(1, (1 << 22) // shape.H)
    return _normal_bf16(g, (shape.V, shape.H), std, device, chunk_rows=rows)


def head_block(shape: HeadShape, w_head: torch.Tensor, block_seed: int, n_boost: int = 10,
               boost: Optional[float] = None, boost_all: bool = False,
               committed_rows: int = 0, mask_boost_rows: int = 0,
               mask_boost: float = 30.0) -> HeadInputs:
    """Hidden states for one block whose logit rows are mostly flat.

    g_t ~ N(0,1) [H]; a seeded set of ``n_boost`` rows (all rows when
    ``boost_all``) gets one seeded non-mask token v_t whose logit is raised by
    ``boost``: h_t = g_t + boost * w_{v_t} / |w_{v_t}|^2, so h_t . w_{v_t}
    grows by exactly ``boost`` before the bf16 rounding of h.  The default
    boost is +12 at small vocabularies and +20 at the full one (a +12 boost
    does not reach 0.95 over 248,319 flat competitors).  ``mask_boost_rows``
    rows (never boosted ones) raise the mask token's own logit by
    ``mask_boost`` (it must never be chosen).  ``committed_rows`` rows start already committed
    (a seeded non-mask token id); all other rows hold the mask id.
    """
    s = shape
    dev = w_head.device
    g = torch.Generator(device="cpu")
    g.manual_seed(3_000_017 + block_seed)
    if boost is None:
        boost = 12.0 if s.V <= 4096 else 20.0
    perm = torch.randperm(s.T, generator=g).tolist()
    rows = list(range(s.T)) if boost_all else sorted(perm[:n_boost])
    toks = []
    for _ in rows:
        while True:
            v = int(torch.randint(0, s.V, (1,), generator=g))
            if v != s.mask_id:
                break
        toks.append(v)
    gd = _gen(dev, 4_000_037 + block_seed)
    hf = torch.randn((s.T, s.H), generator=gd, device=dev, dtype=torch.float32)
    for r, v in zip(rows, toks):
        w = w_head[v].to(torch.float32)
        hf[r] += boost * w / torch.dot(w, w)
    free = [r for r in torch.randperm(s.T, generator=g).tolist() if r not in rows]
    mrows = sorted(free[:mask_boost_rows])
    if mask_boost_rows:
        w = w_head[s.mask_id].to(torch.float32)
        for r in mrows:
            hf[r] += mask_boost * w / torch.dot(w, w)
    tokens = torch.full((s.T,), s.mask_id, dtype=torch.int32)
    crow = torch.randperm(s.T, generator=g)[:committed_rows].tolist()
    for r in crow:
        while True:
            v = int(torch.randint(0, s.V, (1,), generator=g))
            if v != s.mask_id:
                break
        tokens[r] = v
    return HeadInputs(s, hf.to(torch.bfloat16), w_head, tokens.to(dev), rows, toks, mrows)


# ----------------------------------------------------------------------------
# Host copies for the oracle (plumbing: bit patterns, no arithmetic)
# ----------------------------------------------------------------------------

def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor (any device) -> numpy uint16 bit patterns on the host."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f32_host(t: Optional[torch.Tensor]) -> Optional[np.ndarray]:
    if t is None:
        return None
    return t.detach().to("cpu", torch.float32).contiguous().numpy()


class LazyPool:
    """Bounds the host copies of several lazy layers: views created with the
    same pool and different keys (one key per layer) share it, and indexing a
    view whose key differs from the last one used drops the cached experts of
    every other key.  A stack walked layer by layer then holds one layer's
    touched experts on the host at a time."""

    def __init__(self):
        self.current = None
        self.views = []

    def use(self, key):
        if key != self.current:
            for v in self.views:
                if v.key != key:
                    v._cache.clear()
            self.current = key


class LazyExperts:
    """Indexable view of a [E][...] bf16 weight tensor that copies one expert
    to the host (as uint16 bits) only when it is indexed: the oracle touches
    only the experts it routes to, so a 1.6 GB layer on the device costs only
    the touched experts' bytes on the host."""

    def __init__(self, t: torch.Tensor, pool: Optional[LazyPool] = None, key=None):
        self.t = t
        self.shape = tuple(t.shape)
        self._cache = {}
        self.pool, self.key = pool, key
        if pool is not None:
            pool.views.append(self)

    def __len__(self):
        return self.shape[0]

    def __getitem__(self, e):
        e = int(e)
        if self.pool is not None:
            self.pool.use(self.key)
        if e not in self._cache:
            self._cache[e] = bf16_bits(self.t[e])
        return self._cache[e]


def moe_host(inp: MoEInputs, lazy: bool = False, pool: Optional[LazyPool] = None,
             key=None) -> dict:
    """Host views of a MoE input set for the oracle (``pool``/``key``: see
    LazyPool)."""
    conv = (lambda t: LazyExperts(t, pool, key)) if lazy else bf16_bits
    d = {
        "x": bf16_bits(inp.x),
        "w_router": f32_host(inp.w_router),
        "router_bias": f32_host(inp.router_bias),
        "w_gate": conv(inp.w_gate),
        "w_up": conv(inp.w_up),
        "w_down": conv(inp.w_down),
        "ws_gate": None if inp.ws_gate is None else bf16_bits(inp.ws_gate),
        "ws_up": None if inp.ws_up is None else bf16_bits(inp.ws_up),
        "ws_down": None if inp.ws_down is None else bf16_bits(inp.ws_down),
        "residual": None if inp.residual is None else bf16_bits(inp.residual),
        "k": inp.shape.k,
    }
    return d


__all__ = [n for n in dir() if not n.startswith("_")]
