"""GPU parity of the verify epilogue (bdm_lm_head_verify) against oracle.verify.

Causal hidden rows come from synth.head_block: every row raises one seeded
token's logit by a fixed boost over flat competitors, and the candidates are
those tokens except at the chosen rejection rows, where a random other token
stands.  Bar: per-row accept decisions and argmax exact away from a near
call (a candidate probability within 1e-4 relative of its bound, an argmax
gap below 1e-4); p_cand within 2e-5 relative and entropy within 1e-4
absolute + 1e-5 relative of the oracle; the GPU's own outputs obey the
prefix rule exactly; tokens_out and n_accepted equal the oracle's whenever
no near call falls on a row that decides them.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import verify as over
from tests.conftest import gpu_available
from tests.gpu_common import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
LAYOUTS = pytest.mark.parametrize("layout", [0, 1], ids=["rowmajor", "packed"])


@pytest.fixture(scope="module")
def bdm():
    if not gpu_available():
        pytest.skip("no GPU")
    import block_diffusion_moe_amd as b
    b.load()
    return b


def _inputs(shape, w_seed, blk_seed, boost, reject_rows, device=DEV):
    """h [T1][H], W, candidates [T1-1] (boosted tokens; random at reject_rows)."""
    W = synth.head_weights(shape, w_seed, device=device)
    blk = synth.head_block(shape, W, block_seed=blk_seed, boost=boost, boost_all=True)
    T = shape.T - 1
    cand = torch.tensor(blk.boosted_tokens[:T], dtype=torch.int32)
    g = torch.Generator().manual_seed(77 + blk_seed)
    for r in reject_rows:
        while True:
            v = int(torch.randint(0, shape.V, (1,), generator=g))
            if v != int(cand[r]):
                break
        cand[r] = v
    return blk.h, W, cand.to(device)


def _run(bdm, h, W, cand, rule, layout, ratio=0.9, delta=0.6):
    T1 = h.shape[0]
    Wl = bdm.bdm_pack_weights(W) if layout else W
    acc = torch.full((T1 - 1,), -7, dtype=torch.int32, device=DEV)
    am = torch.full((T1,), -7, dtype=torch.int32, device=DEV)
    pc = torch.full((T1 - 1,), -7.0, dtype=torch.float32, device=DEV)
    ent = torch.full((T1,), -7.0, dtype=torch.float32, device=DEV)
    tok, na = bdm.bdm_lm_head_verify(h, Wl, cand, rule, ratio, delta, accept=acc, argmax=am,
                                     p_cand=pc, entropy=ent)
    torch.cuda.synchronize()
    return {"tokens": tok.cpu().numpy().astype(np.int64), "n": int(na.item()),
            "accept": acc.cpu().numpy().astype(bool), "argmax": am.cpu().numpy().astype(np.int64),
            "p_cand": pc.cpu().numpy().astype(np.float64),
            "entropy": ent.cpu().numpy().astype(np.float64)}


def _oracle(h, W, cand, rule, ratio=0.9, delta=0.6):
    return over.verify(synth.bf16_bits(h), synth.bf16_bits(W), cand.cpu().numpy(), rule, ratio,
                       delta)


def _compare(g, o, cand, rule):
    cand = cand.cpu().numpy().astype(np.int64)
    T = len(cand)
    # the GPU's own outputs follow the prefix rule exactly
    assert set(np.unique(g["accept"].astype(int))) <= {0, 1}
    r = over.accept_prefix(g["accept"])
    assert g["n"] == r
    assert np.array_equal(g["tokens"][:r], cand[:r])
    assert g["tokens"][r] == g["argmax"][r]
    assert (g["tokens"][r + 1:] == -1).all()
    # per row, against the oracle
    tie = o["gap"] < 1e-4
    assert np.array_equal(g["argmax"][~tie], o["argmax"][~tie])
    near = o["near"]
    assert np.array_equal(g["accept"][~near], o["accept"][~near]), (g["accept"], o["accept"])
    np.testing.assert_allclose(g["p_cand"], o["p_cand"], rtol=2e-5, atol=1e-30)
    np.testing.assert_allclose(g["entropy"], o["entropy"], rtol=1e-5, atol=1e-4)
    ro = o["n_accepted"]
    unsure = near[:min(ro + 1, T)].any() or tie[ro]     # rows that decide the outputs
    if not unsure:
        assert g["n"] == ro
        assert np.array_equal(g["tokens"], o["tokens"])
    return ro


@LAYOUTS
@pytest.mark.parametrize("rule", ["threshold", "exact"])
@pytest.mark.parametrize("reject", [(), (0,), (4,), (2, 6)], ids=["none", "r0", "r4", "r2r6"])
def test_verify_tiny(bdm, rule, reject, layout):
    """T1 = 9 rows, H = 256, V = 1000 (a ragged last row group)."""
    say(f"case verify tiny rule={rule} reject={reject} layout={layout}")
    s = synth.HeadShape(T=9, H=256, V=1000, mask_id=0)
    h, W, cand = _inputs(s, 11, 3, 12.0, reject)
    g = _run(bdm, h, W, cand, rule, layout)
    o = _oracle(h, W, cand, rule)
    _compare(g, o, cand, rule)
    if rule == "exact":
        # boosted candidates are the argmax; a random one almost never is
        assert o["n_accepted"] == (reject[0] if reject else 8)


@pytest.mark.parametrize("boost", [3.0, 6.0])
def test_verify_tiny_mixed_decisions(bdm, boost):
    """Weak boosts over a near-flat row: probabilities near the entropy bound,
    so the threshold rule both accepts and rejects (the near calls skipped)."""
    say(f"case verify mixed boost={boost}")
    s = synth.HeadShape(T=33, H=512, V=4097, mask_id=0)
    h, W, cand = _inputs(s, 5, 9, boost, tuple(range(1, 32, 3)))
    for rule in ("threshold", "exact"):
        g = _run(bdm, h, W, cand, rule, 0)
        o = _oracle(h, W, cand, rule)
        _compare(g, o, cand, rule)


def test_verify_ratio_binds(bdm):
    """A small ratio caps the bound: min(ratio, delta e^-H) = ratio on sharp rows."""
    say("case verify ratio binds")
    s = synth.HeadShape(T=9, H=256, V=1000, mask_id=0)
    h, W, cand = _inputs(s, 2, 4, 5.0, (3,))
    for ratio, delta in ((0.05, 0.6), (0.9, 5.0), (1.0, 1.0)):
        g = _run(bdm, h, W, cand, "threshold", 1, ratio, delta)
        o = _oracle(h, W, cand, "threshold", ratio, delta)
        _compare(g, o, cand, "threshold")


@pytest.mark.parametrize("T1,H,V", [(1, 256, 1000), (2, 512, 17), (70, 1024, 4097),
                                    (33, 2048, 70001)])
def test_verify_shapes(bdm, T1, H, V):
    """No candidates (only the new token), one, several 32-row chunks with a
    ragged one, every supported hidden size."""
    say(f"case verify shape T1={T1} H={H} V={V}")
    s = synth.HeadShape(T=T1, H=H, V=V, mask_id=0)
    h, W, cand = _inputs(s, T1, H, 12.0 if V > 100 else 4.0, (T1 // 2,) if T1 > 3 else ())
    for layout in (0, 1):
        for rule in ("threshold", "exact"):
            g = _run(bdm, h, W, cand, rule, layout)
            o = _oracle(h, W, cand, rule)
            _compare(g, o, cand, rule)
    if T1 == 1:
        assert g["n"] == 0 and g["tokens"][0] == g["argmax"][0]


def test_verify_out_of_range_candidates(bdm):
    """Ids outside [0, V) are never accepted and get probability 0."""
    say("case verify out-of-range candidates")
    s = synth.HeadShape(T=9, H=256, V=1000, mask_id=0)
    h, W, cand = _inputs(s, 1, 1, 12.0, ())
    cand[2] = -1
    cand[5] = s.V
    g = _run(bdm, h, W, cand, "threshold", 0, ratio=0.9, delta=0.0)  # bound 0 accepts the rest
    assert g["p_cand"][2] == 0.0 and g["p_cand"][5] == 0.0
    assert not g["accept"][2] and not g["accept"][5]
    assert g["accept"][[0, 1, 3, 4, 6, 7]].all()
    assert g["n"] == 2 and g["tokens"][2] == g["argmax"][2]


@LAYOUTS
@pytest.mark.parametrize("rule,reject", [("threshold", (20,)), ("exact", (20,)),
                                         ("threshold", ())])
def test_verify_clover_full(bdm, rule, reject, layout):
    """The untied 248,320 x 2048 head over 32 candidates + 1 bonus row: every
    row checked; boost +20 makes each boosted candidate the argmax with
    probability near 1."""
    say(f"case verify clover rule={rule} reject={reject} layout={layout}")
    s = synth.HeadShape(T=33, H=2048, V=248320, mask_id=synth.HEAD.mask_id)
    h, W, cand = _inputs(s, 0, 21, 20.0, reject)
    g = _run(bdm, h, W, cand, rule, layout)
    o = _oracle(h, W, cand, rule)
    ro = _compare(g, o, cand, rule)
    assert ro == (reject[0] if reject else 32)
    assert g["n"] == ro
    del W
    torch.cuda.empty_cache()


def test_verify_repeatable_bitwise(bdm):
    say("case verify repeatability")
    s = synth.HeadShape(T=33, H=2048, V=65536, mask_id=0)
    h, W, cand = _inputs(s, 4, 8, 8.0, (7, 19))
    a = _run(bdm, h, W, cand, "threshold", 0)
    b = _run(bdm, h, W, cand, "threshold", 0)
    c = _run(bdm, h, W, cand, "threshold", 1)
    for key in a:
        x, y, z = (np.asarray(d[key]) for d in (a, b, c))
        assert np.array_equal(x, y) and np.array_equal(x, z), key
