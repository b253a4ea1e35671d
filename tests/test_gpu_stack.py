"""GPU parity on the 40-layer stack at full size.

Forty independent Clover-shaped layers (seeds 100..139) run one denoise step
over a 32-slot block,

    x_{l+1} = x_l + MoE_l(RMSNorm(x_l))      (in-place residual, y == residual)

on the weights the benchmark times: gate/up packed as pairs, down packed as
MFMA tiles.  The oracle reads the row-major copies of the same weights, one
layer's touched experts at a time.

1. Teacher-forced: every layer, every one of the 32 tokens, against the oracle
   layer fed the GPU's own input to that layer (top-k ids exact away from a
   near tie, weights to 2e-5, outputs to the contract tolerance).
2. End to end: the oracle chained over the 40 layers from the same block.
   Single-ulp rounding differences upstream change a layer's input a little,
   so a token may route differently at a later layer; every such flip must be
   explained by that input difference (the oracle's k-th/(k+1)-th logit gap
   at most 2 |dxn| max_e |w_e| + 1e-4, a bound on how far the difference can
   move two logits apart), the flips per layer are reported, and tokens that
   never flipped end within a tolerance grown from the per-layer one.
3. One step of the loop driver (bdm_denoise_block, max_steps 1: embedding,
   the 40 layers, final RMSNorm, head + unmask) equals the single calls
   composed, bit for bit, and against oracle.denoise.denoise_step on the same
   block: argmax of every row away from a near tie or a routing flip, conf
   within the end-to-end tolerance, and the commit decisions.

Page "Clover-35B-A3B: how a diffusion model gets to 680 tokens a second, read
from its files", sections "What Clover is" (40 layers) and "How it writes",
steps 1-4.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import bf16, denoise as oden, head as ohead, moe as omoe, norm as onorm
from tests.conftest import gpu_available
from tests.gpu_common import ATOL, RTOL, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
N_LAYERS = synth.STACK_LAYERS
S = synth.LAYER
# tolerance of the chained comparison: each layer may leave its output up to
# one per-layer tolerance away from the oracle's (different fp32 summation
# order before the bf16 rounding), the residual stream carries that
# difference on, and differences of independent layers add like a random
# walk: sqrt(40) ~ 6.3 per-layer tolerances after the 40 layers
E2E_GROW = float(np.sqrt(N_LAYERS))


@pytest.fixture(scope="module")
def bdm():
    if not gpu_available():
        pytest.skip("no GPU")
    import block_diffusion_moe_amd as b
    b.load()
    return b


@pytest.fixture(scope="module")
def stack(bdm):
    """The 40 layers (row-major for the oracle, gate/up pairs for the GPU),
    and the GPU's per-layer records over one block."""
    say(f"fixture stack {N_LAYERS} layers T={S.T} gate/up pairs")
    inputs, packed = [], []
    pk = bdm.bdm_pack_weights
    for l in range(N_LAYERS):
        inp = synth.moe_inputs(S, seed=100 + l, block_seed=1, device=DEV)
        g, u = bdm.bdm_pack_gate_up(inp.w_gate, inp.w_up)
        sg, su = bdm.bdm_pack_gate_up(inp.ws_gate, inp.ws_up)
        packed.append({"w_router": inp.w_router, "w_gate": g, "w_up": u,
                       "w_down": pk(inp.w_down), "ws_gate": sg, "ws_up": su,
                       "ws_down": pk(inp.ws_down)})
        inputs.append(inp)
    torch.cuda.synchronize()
    say("  weights generated and packed")
    x = inputs[0].x.clone()                    # the block's hidden state
    xn = torch.empty_like(x)
    idx = torch.empty((S.T, S.k), dtype=torch.int32, device=DEV)
    wts = torch.empty((S.T, S.k), dtype=torch.float32, device=DEV)
    ws = bdm.workspace(bdm.bdm_moe_workspace_bytes(S.T, S.H, S.I, S.E, S.k, True), DEV)
    fused = torch.empty_like(x)
    rec = []
    bdm.bdm_rmsnorm(x, xn, eps=1e-6)
    x0 = x.clone()
    for l, W in enumerate(packed):
        x_in, xn_in = x.clone(), xn.clone()
        # the layer also writes RMSNorm of its output (the next layer's input)
        bdm.bdm_moe_block_forward(xn, W["w_router"], W["w_gate"], W["w_up"], W["w_down"], S.k,
                                  ws_gate=W["ws_gate"], ws_up=W["ws_up"],
                                  ws_down=W["ws_down"], residual=x, y=x, topk_idx=idx,
                                  topk_w=wts, ws=ws, y_norm=fused)
        bdm.bdm_rmsnorm(x, xn, eps=1e-6)
        torch.cuda.synchronize()
        assert torch.equal(fused.view(torch.int16), xn.view(torch.int16)), f"layer {l} y_norm"
        rec.append({"x_in": synth.bf16_bits(x_in), "xn_in": synth.bf16_bits(xn_in),
                    "x_out": synth.bf16_bits(x), "idx": idx.cpu().numpy().copy(),
                    "w": wts.cpu().numpy().copy()})
    say("  stack ran on the GPU (fused RMSNorm == bdm_rmsnorm bit for bit at every layer)")
    yield {"inputs": inputs, "packed": packed, "x0": x0, "rec": rec, "ws": ws}
    del inputs, packed, rec
    torch.cuda.empty_cache()


def _err_tol(g_bits, o_bits, grow=1.0):
    g, o = bf16.to_f64(g_bits), bf16.to_f64(o_bits)
    return np.abs(g - o), grow * (ATOL + RTOL * np.abs(o))


def test_stack_40_layers_teacher_forced_all_tokens(stack):
    """Every layer, all 32 tokens, on the GPU's own input to the layer."""
    say("case stack teacher-forced, 40 layers x 32 tokens")
    worst, excluded = 0.0, 0
    for l, (inp, r) in enumerate(zip(stack["inputs"], stack["rec"])):
        err, tol = _err_tol(r["xn_in"], onorm.rmsnorm(r["x_in"], 1e-6))
        assert np.all(err <= tol), f"layer {l} rmsnorm"
        h = synth.moe_host(inp, lazy=True)
        o = omoe.moe_block(r["xn_in"], h["w_router"], h["w_gate"], h["w_up"], h["w_down"], S.k,
                           h["ws_gate"], h["ws_up"], h["ws_down"], residual=r["x_in"])
        keep = ~o["near_tie"]
        excluded += int((~keep).sum())
        assert np.array_equal(r["idx"][keep], o["idx"][keep]), f"layer {l}: top-k ids differ"
        np.testing.assert_allclose(r["w"][keep], o["w"][keep], rtol=2e-5, atol=1e-6)
        err, tol = _err_tol(r["x_out"][keep], o["y"][keep])
        assert np.all(err <= tol), f"layer {l}: {int(np.sum(err > tol))} outputs off"
        worst = max(worst, float(np.max(err / tol)))
    say(f"  40 layers x 32 tokens: worst err/tol {worst:.3f}, near-tie token-layers "
        f"excluded {excluded} of {N_LAYERS * S.T}")


def test_stack_40_layers_oracle_chain(stack):
    """The oracle chained over all 40 layers from the same block (config 4
    end to end): routing flips per layer, each certified by the input
    difference, and the final outputs of the tokens that never flipped."""
    say("case stack end to end: the oracle chained over 40 layers")
    xo = stack["rec"][0]["x_in"]                    # the same block on both sides
    flipped = np.zeros(S.T, dtype=bool)
    flips, worst_in = [], 0.0
    for l, (inp, r) in enumerate(zip(stack["inputs"], stack["rec"])):
        xno = onorm.rmsnorm(xo, 1e-6)
        h = synth.moe_host(inp, lazy=True)
        o = omoe.moe_block(xno, h["w_router"], h["w_gate"], h["w_up"], h["w_down"], S.k,
                           h["ws_gate"], h["ws_up"], h["ws_down"], residual=xo)
        same = np.array([set(a) == set(b) for a, b in zip(r["idx"], o["idx"])])
        n_flip = int((~same).sum())
        flips.append(n_flip)
        if n_flip:
            # certificate: a set change needs two logits to cross, which the
            # input difference bounds (Cauchy-Schwarz per expert row)
            dxn = bf16.to_f64(r["xn_in"]) - bf16.to_f64(xno)
            wmax = float(np.max(np.linalg.norm(h["w_router"].astype(np.float64), axis=1)))
            l32 = o["logits"].astype(np.float64)
            srt = -np.sort(-l32, axis=1)
            gap = srt[:, S.k - 1] - srt[:, S.k]
            bound = 2.0 * np.linalg.norm(dxn, axis=1) * wmax + 1e-4
            for t in np.flatnonzero(~same):
                say(f"  layer {l} token {t}: oracle gap {gap[t]:.3e}, bound {bound[t]:.3e}")
                assert gap[t] <= bound[t], f"layer {l} token {t}: unexplained routing flip"
        flipped |= ~same
        worst_in = max(worst_in, float(np.max(np.abs(bf16.to_f64(r["xn_in"])
                                                     - bf16.to_f64(xno)))))
        xo = o["y"]
    say(f"  routing flips per layer: {flips}; tokens ever flipped: {int(flipped.sum())}; "
        f"largest layer-input difference {worst_in:.3e}")
    keep = ~flipped
    assert keep.sum() >= S.T // 2, "most tokens must route identically through the stack"
    err, tol = _err_tol(stack["rec"][-1]["x_out"][keep], xo[keep], E2E_GROW)
    say(f"  final outputs of {int(keep.sum())} unflipped tokens: max err {err.max():.3e}, "
        f"worst err/tol {float(np.max(err / tol)):.3f} (tolerance x{E2E_GROW:g}), bit-exact "
        f"{float(np.mean(err == 0)):.4f}")
    assert np.all(err <= tol)


def test_denoise_step_40_layers_against_oracle(stack, bdm):
    """One loop step over the full stack and head: equal to the single calls
    composed, and against oracle.denoise.denoise_step."""
    HS = synth.HEAD
    say("case denoise step 40 layers + head against the oracle")
    g = torch.Generator(device=DEV)
    g.manual_seed(917)
    emb = torch.randn((HS.V, S.H), generator=g, device=DEV).to(torch.bfloat16)
    w_head = synth.head_weights(HS, 2, device=DEV)
    w_head_p = bdm.bdm_pack_weights(w_head)
    gt = torch.Generator(device="cpu")
    gt.manual_seed(918)
    ids = torch.randperm(HS.V - 1, generator=gt)[:S.T]
    ids = ids + (ids >= HS.mask_id).long()
    tok0 = ids.to(torch.int32)
    tok0[torch.randperm(S.T, generator=gt)[:16]] = HS.mask_id     # 16 masked, 16 committed
    tok0 = tok0.to(DEV)
    # the loop's step
    one = tok0.clone()
    steps, commits = bdm.bdm_denoise_block(one, emb, bdm.MoeStack(stack["packed"]), w_head_p,
                                           S.k, HS.mask_id, 0.95, max_steps=1)
    # the same step from the single calls, with argmax and conf
    x = emb[tok0.long()].contiguous()
    xn, xn2 = torch.empty_like(x), torch.empty_like(x)
    bdm.bdm_rmsnorm(x, xn, eps=1e-6)
    for W in stack["packed"]:
        # each layer writes the next layer's normalised input (a second buffer:
        # y_norm may not alias the layer's input)
        bdm.bdm_moe_block_forward(xn, W["w_router"], W["w_gate"], W["w_up"], W["w_down"], S.k,
                                  ws_gate=W["ws_gate"], ws_up=W["ws_up"],
                                  ws_down=W["ws_down"], residual=x, y=x, ws=stack["ws"],
                                  y_norm=xn2)
        xn, xn2 = xn2, xn
    ref = tok0.clone()
    am = torch.empty(S.T, dtype=torch.int32, device=DEV)
    cf = torch.empty(S.T, dtype=torch.float32, device=DEV)
    nc = torch.zeros(1, dtype=torch.int32, device=DEV)
    bdm.bdm_lm_head_unmask(xn, w_head_p, HS.mask_id, 0.95, True, ref, argmax=am, conf=cf,
                           n_committed=nc)
    torch.cuda.synchronize()
    assert steps == 1 and commits == [int(nc.item())]
    assert torch.equal(one, ref), "the loop's step differs from the single calls composed"
    say(f"  loop step == single calls; GPU commits {commits[0]}")
    # the oracle's step on the same block and weights
    pool = synth.LazyPool()
    layers = [synth.moe_host(inp, lazy=True, pool=pool, key=l)
              for l, inp in enumerate(stack["inputs"])]
    o = oden.denoise_step(tok0.cpu().numpy(), synth.bf16_bits(emb), layers,
                          synth.bf16_bits(w_head), S.k, HS.mask_id, 0.95)
    gam, gcf, gtok = am.cpu().numpy(), cf.cpu().numpy(), one.cpu().numpy()
    # rows whose routing differs anywhere in the stack (or sits at a near
    # tie) can take other experts: only the others are compared
    flip = o["near_route"].copy()
    # the GPU's final hidden state against the oracle's
    err, tol = _err_tol(synth.bf16_bits(xn), o["h"], E2E_GROW)
    rows_off = np.any(err > tol, axis=1)
    say(f"  final hidden rows beyond the end-to-end tolerance: {int(rows_off.sum())}, "
        f"routing near ties/flips in {int(flip.sum())} rows")
    keep = ~(flip | rows_off | o["near_tie"])
    assert keep.sum() >= S.T // 2
    assert np.array_equal(gam[keep], o["argmax"][keep]), "argmax differs"
    rel = np.abs(gcf[keep] - o["conf"][keep]) / o["conf"][keep]
    say(f"  {int(keep.sum())} rows compared: argmax equal, conf max rel diff {rel.max():.3e}")
    assert np.all(rel <= 2e-2)
    # commit decisions: rows already committed never change; the oracle's
    # threshold commits hold on the GPU; with no row at the threshold the
    # fallback commits the lowest position among the most confident masked
    # rows (the 16 masked rows embed the same token, so their hidden rows
    # are identical and their confidences equal on both sides)
    masked = tok0.cpu().numpy() == HS.mask_id
    done = ~masked
    assert np.array_equal(gtok[done], tok0.cpu().numpy()[done])
    assert int(nc.item()) == o["n_committed"]
    thr = o["committed"] & (o["conf"].astype(np.float32) >= np.float32(0.95))
    assert np.array_equal(gtok[thr & keep], o["tokens"][thr & keep])
    if not thr.any():
        gpu_row = int(np.flatnonzero(gtok != tok0.cpu().numpy())[0])
        orc_row = int(np.flatnonzero(o["committed"])[0])
        say(f"  fallback: GPU commits row {gpu_row}, oracle row {orc_row}")
        assert gpu_row == orc_row
        if keep[gpu_row]:
            assert gtok[gpu_row] == o["tokens"][orc_row]
    del emb, w_head, w_head_p, layers
    torch.cuda.empty_cache()
