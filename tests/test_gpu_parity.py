"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every case feeds the same seeded tensors to both sides.  Bar: top-k expert
indices and unmask decisions bit-exact (tokens whose k-th/(k+1)-th router
logit gap, or rows whose top-2 logit gap or distance to the threshold, is
below 1e-4 are excluded from the integer comparison); bf16 outputs within
1e-2 absolute + 2e-2 relative of the oracle; fp32 weights and confidences
within 2e-5 relative.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import head as ohead, norm as onorm
from tests.conftest import gpu_available
from tests.gpu_common import (assert_bf16_close, compare_head, compare_moe, oracle_head,
                              oracle_moe, run_head, run_moe, say)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def bdm():
    if not gpu_available():
        pytest.skip("no GPU")
    import block_diffusion_moe_amd as b
    b.load()
    return b


# --------------------------------------------------------------------------
# MoE layer
# --------------------------------------------------------------------------

def _to_dev(inp: synth.MoEInputs) -> synth.MoEInputs:
    f = lambda t: None if t is None else t.to(DEV)  # noqa: E731
    return synth.MoEInputs(inp.shape, f(inp.x), f(inp.w_router), f(inp.router_bias),
                           f(inp.w_gate), f(inp.w_up), f(inp.w_down), f(inp.ws_gate),
                           f(inp.ws_up), f(inp.ws_down), f(inp.residual))


LAYOUTS = pytest.mark.parametrize("layout", [0, 1], ids=["rowmajor", "packed"])


@pytest.mark.parametrize("rows,cols", [(16, 32), (17, 64), (1000, 96), (48, 2048)])
def test_pack_weights_bit_exact(bdm, rows, cols):
    """The packed copy is exactly the documented permutation (checked with an
    independent numpy index computation), with zero padding rows."""
    say(f"case pack rows={rows} cols={cols}")
    g = torch.Generator(device=DEV).manual_seed(rows * cols)
    w = torch.randn(rows, cols, generator=g, device=DEV).to(torch.bfloat16)
    p = bdm.bdm_pack_weights(w)
    torch.cuda.synchronize()
    got = synth.bf16_bits(p.data)
    src = synth.bf16_bits(w)
    rp = (rows + 15) // 16 * 16
    full = np.zeros((rp, cols), dtype=np.uint16)
    full[:rows] = src
    # element (r, k) goes to tile (r//16, k//32), lane (k%32)//8*16 + r%16, item k%8
    r = np.arange(rp)[:, None]
    k = np.arange(cols)[None, :]
    dst = (((r // 16) * (cols // 32) + k // 32) * 64 + ((k % 32) // 8) * 16 + r % 16) * 8 + k % 8
    want = np.empty(rp * cols, dtype=np.uint16)
    want[dst.reshape(-1)] = full.reshape(-1)
    assert got.shape[0] == rp * cols
    assert np.array_equal(got, want)


@LAYOUTS
@pytest.mark.parametrize("seed", [0, 1, 2, 3])
@pytest.mark.parametrize("variant", ["plain", "residual", "noshared", "norenorm", "bias"])
def test_moe_tiny(bdm, seed, variant, layout):
    say(f"case moe tiny seed={seed} variant={variant} layout={layout}")
    inp = _to_dev(synth.moe_inputs(synth.TINY, seed=seed, block_seed=seed + 1,
                                   with_residual=variant == "residual",
                                   zipf_s=1.1 if variant == "bias" else None))
    kw = dict(renorm=variant != "norenorm", shared=variant != "noshared")
    y, idx, w = run_moe(bdm, inp, layout=layout, **kw)
    o = oracle_moe(inp, **kw)
    compare_moe(y, idx, w, o)


# (T, H, E, I, k): ragged token counts, several tiles, k = 1 and k = 16,
# hidden sizes that leave some of the four K-slice waves empty
SHAPES = [
    (1, 64, 16, 32, 2),
    (5, 128, 8, 64, 8),
    (17, 256, 64, 96, 4),
    (33, 192, 32, 32, 1),
    (40, 512, 128, 128, 16),
    (64, 2048, 256, 512, 8),
    (100, 1024, 64, 1024, 2),
    (7, 2048, 1024, 64, 3),
]


@LAYOUTS
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "T%d_H%d_E%d_I%d_k%d" % s)
def test_moe_shapes(bdm, shape, layout):
    T, H, E, I, k = shape
    say(f"case moe shape T={T} H={H} E={E} I={I} k={k} layout={layout}")
    s = synth.MoEShape(T=T, H=H, E=E, I=I, k=k)
    inp = synth.moe_inputs(s, seed=T + E, block_seed=k, device=DEV, with_residual=True)
    y, idx, w = run_moe(bdm, inp, layout=layout)
    o = oracle_moe(inp, lazy=True)
    compare_moe(y, idx, w, o)


ALL_LAYOUTS = pytest.mark.parametrize("layout", [0, 1, 2], ids=["rowmajor", "packed", "gu_pairs"])


@pytest.fixture(scope="module")
def clover_layer():
    """One Clover-shaped layer and its oracle result (computed once)."""
    inp = synth.moe_inputs(synth.LAYER, seed=0, block_seed=1, device=DEV, with_residual=True)
    return inp, oracle_moe(inp, lazy=True)


@ALL_LAYOUTS
def test_moe_clover_layer_full(bdm, clover_layer, layout):
    """One Clover-shaped layer (H 2048, 256 experts, I 512, top-8, shared),
    32-token block, every output element against the oracle, in each weight
    layout (gu_pairs: gate/up packed as pairs, the benchmark's layout)."""
    say(f"case moe clover layer T=32 full layout={layout}")
    inp, o = clover_layer
    y, idx, w = run_moe(bdm, inp, layout=layout)
    say(f"  touched experts: {o['touched']}")
    compare_moe(y, idx, w, o)


def test_moe_clover_layer_inplace_residual(bdm):
    """residual == y (the stack's in-place residual add) gives the same bits
    as a separate output buffer."""
    say("case moe clover layer in-place residual")
    inp = synth.moe_inputs(synth.LAYER, seed=0, block_seed=2, device=DEV, with_residual=True)
    y_sep, _, _ = run_moe(bdm, inp)
    buf = inp.residual.clone()
    bdm.bdm_moe_block_forward(inp.x, inp.w_router, inp.w_gate, inp.w_up, inp.w_down, 8,
                              ws_gate=inp.ws_gate, ws_up=inp.ws_up, ws_down=inp.ws_down,
                              residual=buf, y=buf)
    torch.cuda.synchronize()
    assert torch.equal(buf.view(torch.int16), y_sep.view(torch.int16))


@pytest.fixture(scope="module")
def skew_layer():
    """The load-skew workload (eight 32-token blocks, T = 256, log-Zipf router
    offset) and its oracle result over every token (computed once)."""
    inp = synth.skew_inputs(seed=0, block_seed=1, device=DEV)
    return inp, oracle_moe(inp, residual=False, lazy=True)


@ALL_LAYOUTS
def test_moe_skew_all_tokens(bdm, skew_layer, layout):
    """The load-skew workload: the routing and every output element of all
    256 tokens against the oracle, in each weight layout."""
    say(f"case moe skew T=256 all tokens layout={layout}")
    inp, o = skew_layer
    y, idx, w = run_moe(bdm, inp, residual=False, layout=layout)
    counts = np.bincount(idx.cpu().numpy().reshape(-1), minlength=256)
    say(f"  touched {int((counts > 0).sum())} experts, busiest {int(counts.max())} tokens")
    assert int(counts.max()) > 64          # the hottest expert spans several 64-token items
    compare_moe(y, idx, w, o)


@pytest.mark.parametrize("T,coreset", [(8, False), (32, False), (32, True), (256, False),
                                       (512, False)])
def test_moe_prenorm_equals_rmsnorm_then_layer(bdm, T, coreset):
    """x_norm given: the layer normalises its raw input itself (inside the
    router below 512 tokens, a separate RMSNorm launch from 512); the
    normalised rows, routing and output equal bdm_rmsnorm followed by the
    layer bit for bit, also in place (x is the residual and the output)."""
    say(f"case moe pre-norm T={T} coreset={coreset}")
    s = synth.MoEShape(T=T, H=2048, E=256, I=512, k=8)
    inp = synth.moe_inputs(s, seed=31, block_seed=T, device=DEV)
    x = (inp.x.float() * 2.5).to(torch.bfloat16)          # a residual stream, not unit RMS
    kw = dict(ws_gate=inp.ws_gate, ws_up=inp.ws_up, ws_down=inp.ws_down)
    if coreset:
        kw.update(coreset_top_p=0.9, coreset_block=32,
                  n_kept=torch.zeros(1, dtype=torch.int32, device=DEV))
    xn = torch.empty_like(x)
    bdm.bdm_rmsnorm(x, xn, eps=1e-6)
    ref, idx0 = torch.empty_like(x), torch.empty((T, s.k), dtype=torch.int32, device=DEV)
    bdm.bdm_moe_block_forward(xn, inp.w_router, inp.w_gate, inp.w_up, inp.w_down, s.k,
                              residual=x, y=ref, topk_idx=idx0, **kw)
    xn2, y2 = torch.empty_like(x), torch.empty_like(x)
    idx2 = torch.empty_like(idx0)
    bdm.bdm_moe_block_forward(x, inp.w_router, inp.w_gate, inp.w_up, inp.w_down, s.k,
                              residual=x, y=y2, topk_idx=idx2, x_norm=xn2, **kw)
    buf, xn3 = x.clone(), torch.empty_like(x)
    bdm.bdm_moe_block_forward(buf, inp.w_router, inp.w_gate, inp.w_up, inp.w_down, s.k,
                              residual=buf, y=buf, x_norm=xn3, **kw)
    torch.cuda.synchronize()
    assert torch.equal(xn2.view(torch.int16), xn.view(torch.int16))
    assert torch.equal(xn3.view(torch.int16), xn.view(torch.int16))
    assert torch.equal(idx2, idx0)
    assert torch.equal(y2.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(buf.view(torch.int16), ref.view(torch.int16))


def test_moe_repeatable_bitwise(bdm):
    say("case moe repeatability (and row-major == packed bits)")
    inp = synth.moe_inputs(synth.LAYER, seed=0, block_seed=3, device=DEV, with_residual=True)
    outs = [run_moe(bdm, inp) for _ in range(2)] + [run_moe(bdm, inp, layout=1)]
    for y, idx, w in outs[1:]:
        assert torch.equal(y.view(torch.int16), outs[0][0].view(torch.int16))
        assert torch.equal(idx, outs[0][1])
        assert torch.equal(w.view(torch.int32), outs[0][2].view(torch.int32))


def test_moe_workspace_poison_independent(bdm):
    """Results do not depend on what the workspace held before the call."""
    say("case moe workspace poison")
    inp = synth.moe_inputs(synth.MoEShape(48, 512, 64, 128, 4), seed=5, device=DEV)
    s = inp.shape
    n = bdm.bdm_moe_workspace_bytes(s.T, s.H, s.I, s.E, s.k, True)
    outs = []
    for fill in (0x00, 0xFF, 0x7F):
        ws = torch.full((n,), fill, dtype=torch.uint8, device=DEV)
        y = torch.empty((s.T, s.H), dtype=torch.bfloat16, device=DEV)
        bdm.bdm_moe_block_forward(inp.x, inp.w_router, inp.w_gate, inp.w_up, inp.w_down, s.k,
                                  ws_gate=inp.ws_gate, ws_up=inp.ws_up, ws_down=inp.ws_down,
                                  y=y, ws=ws)
        torch.cuda.synchronize()
        outs.append(y)
    assert all(torch.equal(o.view(torch.int16), outs[0].view(torch.int16)) for o in outs)


def test_uniform_router_ties_on_gpu(bdm):
    """All-zero router: every logit ties, the picks are experts 0..k-1 with
    weight 1/k (the tie rule, bit-exact)."""
    say("case moe uniform router")
    inp = synth.moe_inputs(synth.MoEShape(16, 256, 32, 64, 4), seed=9, device=DEV)
    inp.w_router.zero_()
    y, idx, w = run_moe(bdm, inp, residual=False)
    assert torch.equal(idx.cpu(), torch.arange(4, dtype=torch.int32).repeat(16, 1))
    assert torch.all(w == 0.25)
    o = oracle_moe(inp, residual=False)
    assert_bf16_close(y, o["y"])


# --------------------------------------------------------------------------
# Head + unmask
# --------------------------------------------------------------------------

def test_pack_gate_up_layout(bdm):
    """The pair buffer holds the plain packed groups of gate and up,
    alternating (16-row groups: 2g = gate g, 2g + 1 = up g)."""
    say("case pack gate/up pair buffer")
    s = synth.MoEShape(T=8, H=256, E=4, I=96, k=2)
    inp = synth.moe_inputs(s, seed=7, block_seed=1, device=DEV)
    g, u = bdm.bdm_pack_gate_up(inp.w_gate, inp.w_up)
    pg, pu = bdm.bdm_pack_weights(inp.w_gate), bdm.bdm_pack_weights(inp.w_up)
    S = 16 * s.H
    pair = g.data.view(-1, 2, S)
    torch.cuda.synchronize()
    assert torch.equal(pair[:, 0].reshape(-1).view(torch.int16), pg.data.view(torch.int16))
    assert torch.equal(pair[:, 1].reshape(-1).view(torch.int16), pu.data.view(torch.int16))
    assert u.data_ptr() == g.data_ptr() + 2 * S


@pytest.mark.parametrize("case", ["tiny", "T5_H128", "T17_I96", "H192", "noshared", "clover32",
                                  "clover512", "skew256", "I96_T400"])
def test_moe_gate_up_pair_layout_equals_tiles(bdm, case):
    """Gate/up packed as pairs give the bits of the plain tile layout, on the
    few-token and the many-token kernels (routing, weights, outputs)."""
    say(f"case gate/up pair layout {case}")
    shapes = {"tiny": (8, 64, 16, 32, 2), "T5_H128": (5, 128, 8, 64, 8),
              "T17_I96": (17, 256, 64, 96, 4), "H192": (33, 192, 32, 32, 1),
              "noshared": (24, 512, 32, 64, 4), "clover32": (32, 2048, 256, 512, 8),
              "clover512": (512, 2048, 256, 512, 8), "skew256": (256, 2048, 256, 512, 8),
              "I96_T400": (400, 512, 8, 96, 3)}
    T, H, E, I, k = shapes[case]
    shp = synth.MoEShape(T=T, H=H, E=E, I=I, k=k)
    inp = synth.moe_inputs(shp, seed=T + E, block_seed=3, device=DEV, with_residual=True,
                           zipf_s=1.1 if case == "skew256" else None)
    shared = case != "noshared"
    a = run_moe(bdm, inp, layout=1, shared=shared)
    b = run_moe(bdm, inp, layout=2, shared=shared)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1], b[1]) and torch.equal(a[2].view(torch.int32), b[2].view(torch.int32))
    if case == "tiny":
        compare_moe(*b, oracle_moe(inp))


@LAYOUTS
@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("variant", ["plain", "committed", "maskboost", "all_boosted"])
def test_head_tiny(bdm, seed, variant, layout):
    say(f"case head tiny seed={seed} variant={variant} layout={layout}")
    s = synth.TINY_HEAD
    W = synth.head_weights(s, seed).to(DEV)
    blk = synth.head_block(s, W, block_seed=seed + 1, n_boost=3,
                           committed_rows=3 if variant == "committed" else 0,
                           mask_boost_rows=2 if variant == "maskboost" else 0,
                           boost_all=variant == "all_boosted")
    out = run_head(bdm, blk, layout=layout)
    o = oracle_head(blk)
    compare_head(out, o, blk.tokens.cpu().numpy())


@LAYOUTS
@pytest.mark.parametrize("V,T", [(2, 3), (17, 5), (1000, 33), (4097, 40), (70001, 64)])
def test_head_ragged(bdm, V, T, layout):
    say(f"case head ragged V={V} T={T} layout={layout}")
    s = synth.HeadShape(T=T, H=256, V=V, mask_id=V // 3)
    W = synth.head_weights(s, V).to(DEV)
    blk = synth.head_block(s, W, block_seed=T, n_boost=min(T, 4), committed_rows=1)
    out = run_head(bdm, blk, layout=layout)
    o = oracle_head(blk)
    compare_head(out, o, blk.tokens.cpu().numpy())


@LAYOUTS
def test_head_clover_full(bdm, layout):
    """Untied 248,320 x 2048 head, 32 positions, 10 boosted rows (+20) among
    flat ones: every row's argmax/conf and the commit decisions."""
    say(f"case head clover full layout={layout}")
    s = synth.HEAD
    W = synth.head_weights(s, 0, device=DEV)
    blk = synth.head_block(s, W, block_seed=1, n_boost=10)
    out = run_head(bdm, blk, layout=layout)
    o = oracle_head(blk)
    assert o["n_committed"] == 10
    compare_head(out, o, blk.tokens.cpu().numpy())
    # a second block: rows already committed, the mask token boosted in two rows
    blk2 = synth.head_block(s, W, block_seed=2, n_boost=10, committed_rows=5, mask_boost_rows=2)
    out2 = run_head(bdm, blk2, layout=layout)
    compare_head(out2, oracle_head(blk2), blk2.tokens.cpu().numpy())


@LAYOUTS
def test_head_clover_fallback(bdm, layout):
    """Every row boosted by only +12 over 248,319 flat competitors: no row
    reaches 0.95, so exactly one row (the most confident) commits."""
    say("case head clover fallback")
    s = synth.HEAD
    W = synth.head_weights(s, 0, device=DEV)
    blk = synth.head_block(s, W, block_seed=4, boost=12.0, boost_all=True)
    out = run_head(bdm, blk, layout=layout)
    o = oracle_head(blk)
    assert o["n_committed"] == 1
    compare_head(out, o, blk.tokens.cpu().numpy())
    out_nf = run_head(bdm, blk, fallback=False, layout=layout)
    assert int(out_nf[3].item()) == 0
    assert torch.equal(out_nf[0].cpu(), blk.tokens.cpu())


@LAYOUTS
@pytest.mark.parametrize("T", [32, 100])
def test_head_two_phase_and_vocab_shards(bdm, layout, T):
    """Phase 1 + phase 2 equals the fused call bit for bit, and the head
    computed as three vocabulary shards (each with its vocab_offset, the
    mask row in the middle shard) and merged once gives the same argmax and
    decisions, with confidences within the fp32 merge-order tolerance (100
    rows: two passes in each shard's launch)."""
    say(f"case head two-phase + shards T={T} layout={layout}")
    s = synth.HeadShape(T=T, H=2048, V=100000, mask_id=51234)
    W = synth.head_weights(s, 3, device=DEV)
    blk = synth.head_block(s, W, block_seed=5, n_boost=10, committed_rows=3, mask_boost_rows=2)
    fused = run_head(bdm, blk, layout=layout)
    P = bdm.bdm_head_stat_parts()
    T = s.T
    cuts = [0, 33000, 67000, s.V]
    sm = torch.empty((T, P * 3), dtype=torch.float32, device=DEV)
    ss = torch.empty_like(sm)
    sa = torch.empty((T, P * 3), dtype=torch.int32, device=DEV)
    for i in range(3):
        Wi = W[cuts[i]:cuts[i + 1]]
        if layout:
            Wi = bdm.bdm_pack_weights(Wi.contiguous())
        cols = slice(i * P, (i + 1) * P)
        bdm.bdm_lm_head_stats(blk.h, Wi, s.mask_id, sm[:, cols], ss[:, cols], sa[:, cols],
                              vocab_offset=cuts[i])
    tok = blk.tokens.clone()
    am = torch.empty(T, dtype=torch.int32, device=DEV)
    cf = torch.empty(T, dtype=torch.float32, device=DEV)
    nc = torch.empty(1, dtype=torch.int32, device=DEV)
    bdm.bdm_unmask_from_stats(sm, ss, sa, s.mask_id, 0.95, True, tok, argmax=am, conf=cf,
                              n_committed=nc)
    # one shard over the whole vocabulary through the two phases = the fused call
    sm1 = torch.empty((T, P), dtype=torch.float32, device=DEV)
    ss1, sa1 = torch.empty_like(sm1), torch.empty((T, P), dtype=torch.int32, device=DEV)
    Wf = bdm.bdm_pack_weights(W) if layout else W
    bdm.bdm_lm_head_stats(blk.h, Wf, s.mask_id, sm1, ss1, sa1)
    tok1 = blk.tokens.clone()
    am1, cf1, nc1 = torch.empty_like(am), torch.empty_like(cf), torch.empty_like(nc)
    bdm.bdm_unmask_from_stats(sm1, ss1, sa1, s.mask_id, 0.95, True, tok1, argmax=am1, conf=cf1,
                              n_committed=nc1)
    torch.cuda.synchronize()
    for x, z in zip(fused, (tok1, am1, cf1, nc1)):
        assert torch.equal(x.view(torch.int32), z.view(torch.int32))
    o = oracle_head(blk)
    compare_head((tok, am, cf, nc), o, blk.tokens.cpu().numpy())


@pytest.mark.parametrize("T,V", [(33, 70001), (64, 70001), (100, 70001), (130, 70001),
                                 (255, 70001), (97, 1000)])
def test_head_wide_pass_equals_32_row_calls(bdm, T, V):
    """Up to 64 rows share one pass over the head weights, and up to 255 rows
    run as several passes in one launch (2 .. 4 of them, workgroups of one
    vocabulary range side by side); every row's partial statistics equal
    those of the same row computed in a call of at most 32 rows, bit for bit
    (the per-row arithmetic and the vocabulary ranges do not change).  V =
    1000 leaves most ranges empty.  (From 256 rows the head runs as a tiled
    GEMM whose sums run in another order: test_head_gemm_rows.)"""
    say(f"case head wide pass T={T} V={V}")
    s = synth.HeadShape(T=T, H=2048, V=V, mask_id=5)
    W = synth.head_weights(s, 6, device=DEV)
    blk = synth.head_block(s, W, block_seed=T, n_boost=8)
    P = bdm.bdm_head_stat_parts()
    for Wl in (W, bdm.bdm_pack_weights(W)):
        wide = [torch.empty((T, P), dtype=dt, device=DEV)
                for dt in (torch.float32, torch.float32, torch.int32)]
        bdm.bdm_lm_head_stats(blk.h, Wl, s.mask_id, *wide)
        narrow = [torch.empty_like(x) for x in wide]
        for t0 in range(0, T, 32):
            t1 = min(T, t0 + 32)
            bdm.bdm_lm_head_stats(blk.h[t0:t1].contiguous(), Wl, s.mask_id,
                                  *[x[t0:t1] for x in narrow])
        torch.cuda.synchronize()
        for x, z in zip(wide, narrow):
            assert torch.equal(x.view(torch.int32), z.view(torch.int32))


@LAYOUTS
@pytest.mark.parametrize("T,V,H", [(256, 70001, 2048), (300, 70001, 2048), (512, 248320, 2048),
                                   (2048, 70001, 2048), (300, 1000, 2048), (700, 4099, 256),
                                   (260, 5000, 64)])
def test_head_gemm_rows(bdm, T, V, H, layout):
    """From 256 rows (several blocks in one call) the head is a tiled GEMM
    (256 rows x 256 vocabulary rows per tile, the whole K per tile, the
    online softmax folded per tile): every row's argmax and conf against the
    oracle and the commit rule per 32-row block.  Ragged row counts (a
    partial last row block), V = 1,000 (most ranges empty), small H."""
    say(f"case head GEMM rows T={T} V={V} H={H} layout={layout}")
    s = synth.HeadShape(T=T, H=H, V=V, mask_id=V // 7)
    W = synth.head_weights(s, T + 3, device=DEV)
    blk = synth.head_block(s, W, block_seed=T + 4, n_boost=T // 3, committed_rows=7)
    w_head = bdm.bdm_pack_weights(W) if layout else W
    tokens = blk.tokens.clone()
    am = torch.full((T,), -1, dtype=torch.int32, device=DEV)
    cf = torch.full((T,), float("nan"), dtype=torch.float32, device=DEV)
    nc = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    bdm.bdm_lm_head_unmask(blk.h, w_head, s.mask_id, 0.95, True, tokens, argmax=am, conf=cf,
                           n_committed=nc, block_tokens=32)
    torch.cuda.synchronize()
    o = ohead.head_unmask(synth.bf16_bits(blk.h), synth.bf16_bits(W), blk.tokens.cpu().numpy(),
                          s.mask_id, 0.95, True, block=32)
    o["mask_id"] = s.mask_id
    compare_head((tokens, am, cf, nc), o, blk.tokens.cpu().numpy())


@LAYOUTS
@pytest.mark.parametrize("T", [65, 130, 255])
def test_head_many_rows(bdm, T, layout):
    """Several 64-row passes in one launch against the oracle: every row's
    argmax/conf and the commit decisions."""
    say(f"case head many rows T={T} layout={layout}")
    s = synth.HeadShape(T=T, H=2048, V=70001, mask_id=777)
    W = synth.head_weights(s, T + 1, device=DEV)
    blk = synth.head_block(s, W, block_seed=T + 2, n_boost=T // 3, committed_rows=5)
    out = run_head(bdm, blk, layout=layout)
    o = oracle_head(blk)
    compare_head(out, o, blk.tokens.cpu().numpy())


@pytest.mark.parametrize("layout", [0, 1])
def test_head_rule_per_block(bdm, layout):
    """Two blocks of 32 in one call, the rule per block: block 0 has rows
    above the threshold, block 1 none (its most confident masked row is
    committed by the fallback, as it would be alone)."""
    say(f"case head rule per block layout={layout}")
    s = synth.HeadShape(T=32, H=2048, V=70001, mask_id=321)
    W = synth.head_weights(s, 8, device=DEV)
    b0 = synth.head_block(s, W, block_seed=11, n_boost=10)
    b1 = synth.head_block(s, W, block_seed=12, boost=12.0, boost_all=True)
    h = torch.cat([b0.h, b1.h]).contiguous()
    tok = torch.cat([b0.tokens, b1.tokens]).contiguous()
    Wl = bdm.bdm_pack_weights(W) if layout else W
    am = torch.empty(64, dtype=torch.int32, device=DEV)
    cf = torch.empty(64, dtype=torch.float32, device=DEV)
    nc = torch.empty(1, dtype=torch.int32, device=DEV)
    out = tok.clone()
    bdm.bdm_lm_head_unmask(h, Wl, s.mask_id, 0.95, True, out, argmax=am, conf=cf,
                           n_committed=nc, block_tokens=32)
    torch.cuda.synchronize()
    o = ohead.head_unmask(synth.bf16_bits(h), synth.bf16_bits(W), tok.cpu().numpy(), s.mask_id,
                          0.95, True, block=32)
    assert o["committed"][32:].sum() == 1 and o["committed"][:32].sum() >= 1
    o["mask_id"] = s.mask_id
    compare_head((out, am, cf, nc), o, tok.cpu().numpy())
    # each block alone gives the same rows
    for b, blk in enumerate((b0, b1)):
        one = blk.tokens.clone()
        bdm.bdm_lm_head_unmask(blk.h, Wl, s.mask_id, 0.95, True, one)
        torch.cuda.synchronize()
        assert torch.equal(one, out[32 * b:32 * (b + 1)])


def test_head_repeatable_bitwise(bdm):
    say("case head repeatability")
    s = synth.HeadShape(T=32, H=2048, V=65536, mask_id=3)
    W = synth.head_weights(s, 1, device=DEV)
    blk = synth.head_block(s, W, block_seed=7, n_boost=10)
    a = run_head(bdm, blk)
    b = run_head(bdm, blk)
    c = run_head(bdm, blk, layout=1)
    for x, z in list(zip(a, b)) + list(zip(a, c)):
        assert torch.equal(x.view(torch.int32), z.view(torch.int32))


# --------------------------------------------------------------------------
# RMSNorm
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T,H", [(1, 64), (32, 2048), (37, 704)])
def test_rmsnorm(bdm, T, H):
    say(f"case rmsnorm T={T} H={H}")
    g = torch.Generator(device=DEV).manual_seed(T * H)
    x = (torch.randn(T, H, generator=g, device=DEV) * 3).to(torch.bfloat16)
    out = torch.empty_like(x)
    bdm.bdm_rmsnorm(x, out, eps=1e-6)
    torch.cuda.synchronize()
    ref = onorm.rmsnorm(synth.bf16_bits(x), 1e-6)
    exact = assert_bf16_close(out, ref, what="rmsnorm")
    assert exact > 0.98
    bdm.bdm_rmsnorm(x, x, eps=1e-6)            # in place
    torch.cuda.synchronize()
    assert torch.equal(x.view(torch.int16), out.view(torch.int16))
