"""The C-ABI library loads and exports every symbol include/bdmoe.h declares;
host-side workspace arithmetic and argument validation (CPU only: no call
here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bdmoe.h")


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"BDM_API\s+[\w\s\*]+?\b(bdm_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from block_diffusion_moe_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libbdmoe.so not built (python -m block_diffusion_moe_amd.build)")
    return binding.load()


def test_header_declares_the_entry_points():
    syms = declared_symbols()
    assert syms == sorted(["bdm_version", "bdm_status_string", "bdm_moe_workspace_bytes",
                           "bdm_moe_block_forward", "bdm_head_workspace_bytes",
                           "bdm_lm_head_unmask", "bdm_rmsnorm", "bdm_packed_weight_elems",
                           "bdm_pack_weights", "bdm_pack_gate_up", "bdm_head_stat_parts",
                           "bdm_lm_head_stats",
                           "bdm_unmask_from_stats", "bdm_moe_block_forward_coreset",
                           "bdm_denoise_workspace_bytes", "bdm_denoise_block",
                           "bdm_head_verify_workspace_bytes", "bdm_lm_head_verify",
                           "bdm_moe_block_forward_noalloc", "bdm_debug_bounds"])


def test_library_exports_every_declared_symbol(lib):
    from block_diffusion_moe_amd import binding
    for name in declared_symbols():
        assert hasattr(lib, name), name
    assert sorted(binding.EXPORTS) == declared_symbols()
    assert lib.bdm_version() >= 100
    for st in (0, -1, -2, -3, -4, -5, 7):
        assert isinstance(lib.bdm_status_string(st), bytes)


def test_debug_bounds_library_and_release_answer(lib):
    """The bounds-checked build exports the same symbols (and holds gfx950
    code); the release library answers bdm_debug_bounds with
    BDM_ERR_NOT_DEBUG_BUILD before any device call."""
    from block_diffusion_moe_amd import binding
    assert os.path.exists(binding.DEBUG_LIB_PATH), "libbdmoe_debug.so not built"
    dbg = ctypes.CDLL(binding.DEBUG_LIB_PATH)
    for name in declared_symbols():
        assert hasattr(dbg, name), name
    dbg.bdm_version.restype = ctypes.c_int
    assert dbg.bdm_version() == lib.bdm_version()
    assert b"gfx950" in open(binding.DEBUG_LIB_PATH, "rb").read()
    dbg.bdm_debug_bounds.restype = ctypes.c_int
    assert dbg.bdm_debug_bounds(None) == -1
    v = ctypes.c_uint(123)
    assert lib.bdm_debug_bounds(ctypes.byref(v)) == binding.BDM_ERR_NOT_DEBUG_BUILD
    assert v.value == 0
    assert lib.bdm_debug_bounds(None) == -1
    assert b"debug" in lib.bdm_status_string(binding.BDM_ERR_NOT_DEBUG_BUILD)
    with pytest.raises(binding.BdmError):
        binding.bdm_debug_bounds()


def test_library_is_gfx950_code_object():
    from block_diffusion_moe_amd import binding
    blob = open(binding.LIB_PATH, "rb").read()
    assert b"gfx950" in blob


def test_moe_workspace_bytes(lib):
    from block_diffusion_moe_amd import binding as b
    n = b.bdm_moe_workspace_bytes(32, 2048, 512, 256, 8, True)
    P = 32 * 9
    # expert outputs [P][H] fp32 and activations [P][I] bf16 dominate
    assert n >= P * 2048 * 4 + P * 512 * 2 + 32 * 256 * 4
    assert n % 256 == 0
    assert b.bdm_moe_workspace_bytes(32, 2048, 512, 256, 8, False) <= n
    size = ctypes.c_size_t(0)
    assert lib.bdm_moe_workspace_bytes(0, 2048, 512, 256, 8, 1, ctypes.byref(size)) == -1
    assert lib.bdm_moe_workspace_bytes(32, 2048, 512, 256, 9999, 1, ctypes.byref(size)) == -1
    assert lib.bdm_moe_workspace_bytes(32, 2047, 512, 256, 8, 1, ctypes.byref(size)) == -2
    assert lib.bdm_moe_workspace_bytes(32, 4096, 512, 256, 8, 1, ctypes.byref(size)) == -2
    assert lib.bdm_moe_workspace_bytes(32, 2048, 500, 256, 8, 1, ctypes.byref(size)) == -2
    assert lib.bdm_moe_workspace_bytes(4096, 2048, 512, 256, 8, 1, ctypes.byref(size)) == -2
    assert lib.bdm_moe_workspace_bytes(2048, 2048, 512, 256, 8, 1, ctypes.byref(size)) == 0
    assert lib.bdm_moe_workspace_bytes(32, 2048, 512, 256, 17, 1, ctypes.byref(size)) == -2
    assert lib.bdm_moe_workspace_bytes(32, 2048, 512, 256, 8, 2, ctypes.byref(size)) == -1
    assert lib.bdm_moe_workspace_bytes(32, 2048, 512, 256, 8, 1, None) == -1


def test_head_workspace_bytes(lib):
    from block_diffusion_moe_amd import binding as b
    n = b.bdm_head_workspace_bytes(32, 2048, 248320)
    assert n >= 32 * 970 * 12
    size = ctypes.c_size_t(0)
    assert lib.bdm_head_workspace_bytes(32, 2048, 1, ctypes.byref(size)) == -1
    assert lib.bdm_head_workspace_bytes(32, 2000, 512, ctypes.byref(size)) == -2


def _fake(addr):
    return ctypes.c_void_p(addr)


def test_moe_validation_rejects_before_launch(lib):
    """Bad arguments return an error code without touching the device (the
    pointers below are never dereferenced)."""
    A = _fake(1 << 20)        # 16-byte aligned fake address
    size = 1 << 30
    good = dict(x=A, T=32, H=2048, wr=A, bias=None, E=256, k=8, renorm=1, wg=A, wu=A, wd=A,
                I=512, sg=A, su=A, sd=A, lay=0, res=None, y=_fake(2 << 20), idx=None, w=None,
                ws=_fake(1 << 24), wsb=size, stream=None)

    def call(**kw):
        a = dict(good, **kw)
        return lib.bdm_moe_block_forward(a["x"], a["T"], a["H"], a["wr"], a["bias"], a["E"],
                                         a["k"], a["renorm"], a["wg"], a["wu"], a["wd"], a["I"],
                                         a["sg"], a["su"], a["sd"], a["lay"], a["res"], a["y"],
                                         a.get("yn"), a.get("xn"), a["idx"], a["w"], a["ws"],
                                         a["wsb"], a["stream"])

    assert call(x=None) == -1
    assert call(y=None) == -1
    assert call(ws=None) == -1
    assert call(sd=None) == -1                    # shared trio must be all or none
    assert call(renorm=2) == -1
    assert call(lay=3) == -1
    # gate/up pair layout: up must follow gate by one 16-row group (16 H
    # elements), for the routed and the shared expert alike; with both pairs
    # right the call gets as far as the workspace check
    G, SG = 1 << 28, 1 << 29
    pair = dict(lay=2, wg=_fake(G), wu=_fake(G + 32 * 2048), sg=_fake(SG), su=_fake(SG + 32 * 2048))
    assert call(lay=2) == -1                      # w_up == w_gate
    assert call(**dict(pair, su=_fake(SG))) == -1
    assert call(**dict(pair, wu=_fake(G + 32 * 1024))) == -1
    assert call(**dict(pair, wsb=1)) == -3
    assert call(**dict(pair, lay=1, wsb=1)) == -3
    assert call(k=0) == -1
    assert call(k=300) == -1
    assert call(H=100) == -2
    assert call(I=48) == -2
    assert call(x=_fake((1 << 20) + 2)) == -1     # misaligned
    assert call(ws=_fake((1 << 24) + 16)) == -1   # workspace not 256-aligned
    assert call(y=A) == -1                        # y aliases x
    Y = _fake(1 << 22)
    assert call(y=Y, yn=Y) == -1                  # y_norm aliases y
    assert call(y=Y, yn=A) == -1                  # y_norm aliases x
    assert call(y=Y, yn=_fake((1 << 23) + 8)) == -1   # y_norm misaligned
    assert call(wsb=1024) == -3
    # x_norm: x is the raw input; it may then be y, but x_norm aliases nothing
    XN = _fake(1 << 25)
    assert call(y=A, xn=XN, wsb=1024) == -3       # x == y allowed: reaches the size check
    assert call(y=Y, xn=A) == -1                  # x_norm aliases x
    assert call(y=Y, xn=Y) == -1                  # x_norm aliases y
    assert call(y=Y, yn=XN, xn=XN) == -1          # x_norm aliases y_norm
    assert call(y=Y, xn=_fake((1 << 25) + 4)) == -1   # misaligned


def test_head_and_rmsnorm_validation(lib):
    A = _fake(1 << 20)
    T = ctypes.c_void_p(3 << 20)
    W = _fake(1 << 24)

    def head(**kw):
        a = dict(h=A, T=32, H=2048, w=A, V=248320, lay=0, mask=151669, thr=0.95, fb=1, blk=0,
                 tok=T, am=None, cf=None, nc=None, ws=W, wsb=1 << 30, st=None)
        a.update(kw)
        return lib.bdm_lm_head_unmask(a["h"], a["T"], a["H"], a["w"], a["V"], a["lay"],
                                      a["mask"], a["thr"], a["fb"], a["blk"], a["tok"], a["am"],
                                      a["cf"], a["nc"], a["ws"], a["wsb"], a["st"])

    assert head(h=None) == -1
    assert head(tok=None) == -1
    assert head(mask=248320) == -1
    assert head(mask=-1) == -1
    assert head(thr=float("nan")) == -1
    assert head(fb=3) == -1
    assert head(blk=-1) == -1
    assert head(lay=5) == -1
    assert head(T=0) == -1
    assert head(T=4096) == -2
    assert head(wsb=16) == -3
    assert lib.bdm_rmsnorm(None, None, 1e-6, 32, 2048, A, None) == -1
    assert lib.bdm_rmsnorm(A, None, -1.0, 32, 2048, A, None) == -1
    assert lib.bdm_rmsnorm(A, None, 1e-6, 32, 100, A, None) == -2


def test_packed_weight_size_and_pack_validation(lib):
    from block_diffusion_moe_amd import binding as b
    assert b.bdm_packed_weight_elems(248320, 2048) == 248320 * 2048
    assert b.bdm_packed_weight_elems(17, 64) == 32 * 64           # rows padded to 16
    assert b.bdm_packed_weight_elems(256 * 512, 2048) == 256 * 512 * 2048
    n = ctypes.c_size_t(0)
    assert lib.bdm_packed_weight_elems(16, 48, ctypes.byref(n)) == -1   # cols % 32
    assert lib.bdm_packed_weight_elems(0, 64, ctypes.byref(n)) == -1
    A, B = _fake(1 << 20), _fake(1 << 26)
    assert lib.bdm_pack_weights(None, 16, 64, B, None) == -1
    assert lib.bdm_pack_weights(A, 16, 64, _fake((1 << 20) + 64), None) == -1   # overlap
    assert lib.bdm_pack_weights(A, 16, 64, _fake((1 << 26) + 8), None) == -1    # misaligned
    p = lib.bdm_pack_gate_up
    C = _fake(1 << 27)
    assert p(None, A, 16, 64, B, None) == -1
    assert p(A, None, 16, 64, B, None) == -1
    assert p(A, C, 16, 64, None, None) == -1
    assert p(A, C, 24, 64, B, None) == -1                          # rows % 16
    assert p(A, C, 16, 48, B, None) == -1                          # cols % 32
    assert p(A, C, 0, 64, B, None) == -1
    assert p(A, C, 16, 64, _fake((1 << 20) + 1024), None) == -1    # dst overlaps gate
    assert p(A, C, 16, 64, _fake((1 << 27) - 2048), None) == -1    # dst overlaps up
    assert p(A, C, 16, 64, _fake((1 << 26) + 8), None) == -1       # misaligned


def test_two_phase_head_validation(lib):
    A = _fake(1 << 20)
    S = _fake(1 << 22)
    assert lib.bdm_lm_head_stats(None, 32, 2048, A, 1000, 0, 0, 5, S, S, S, 1024, None) == -1
    assert lib.bdm_lm_head_stats(A, 32, 2048, A, 1000, -1, 0, 5, S, S, S, 1024, None) == -1
    assert lib.bdm_lm_head_stats(A, 32, 2048, A, 1000, 0, 3, 5, S, S, S, 1024, None) == -1
    assert lib.bdm_lm_head_stats(A, 32, 2000, A, 1000, 0, 0, 5, S, S, S, 1024, None) == -2
    u = lib.bdm_unmask_from_stats
    assert u(S, S, S, 32, 0, 8, 5, 0.95, 1, 0, A, None, None, None, None) == -1
    assert u(S, S, S, 32, 16, 8, 5, 0.95, 1, 0, A, None, None, None, None) == -1
    assert u(S, S, S, 32, 8, 8, 5, 0.95, 1, 0, None, None, None, None, None) == -1
    assert lib.bdm_unmask_from_stats(S, S, S, 4000, 8, 8, 5, 0.95, 1, 0, A, None, None, None,
                                     None) == -2
    assert lib.bdm_unmask_from_stats(S, S, S, 32, 8, 8, 5, 0.95, 1, -2, A, None, None, None,
                                     None) == -1


def test_calibration_library_exports():
    """The calibration kernels (counter-calibration copy, read-bandwidth
    probe) live in their own library and reject arguments they cannot serve
    (checks only, no launch)."""
    import ctypes
    import os
    path = os.path.join(ROOT, "block_diffusion_moe_amd", "libbdmcal.so")
    if not os.path.exists(path):
        pytest.fail("libbdmcal.so not built (python -m block_diffusion_moe_amd.build)")
    cal = ctypes.CDLL(path)
    f = cal.bdmcal_stream_copy
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_long, ctypes.c_void_p]
    assert f(None, _fake(1 << 20), 16384, None) == -1
    assert f(_fake(1 << 20), _fake(1 << 21), 16000, None) == -1
    assert f(_fake(1 << 20), _fake(1 << 20), 16384, None) == -1
    r = cal.bdmcal_stream_read
    r.restype = ctypes.c_int
    r.argtypes = [ctypes.c_void_p, ctypes.c_long, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    assert r(None, 1 << 20, _fake(1 << 21), 4, None) == -1
    assert r(_fake(1 << 20), 1000, _fake(1 << 21), 4, None) == -1
    assert r(_fake(1 << 20), 1 << 20, None, 4, None) == -1
    assert r(_fake(1 << 20), 1 << 20, _fake(1 << 21), 0, None) == -1
    g = cal.bdmcal_stream_read_region
    g.restype = ctypes.c_int
    g.argtypes = [ctypes.c_void_p, ctypes.c_long, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    assert g(None, 1 << 20, _fake(1 << 21), 4, None) == -1
    assert g(_fake(1 << 20), 1000, _fake(1 << 21), 4, None) == -1
    assert g(_fake(1 << 20), 1 << 20, _fake(1 << 21), 0, None) == -1
    assert g(_fake(1 << 20), 1 << 14, _fake(1 << 21), 2, None) == -1   # under one batch each


def test_coreset_validation(lib):
    A = _fake(1 << 20)
    size = 1 << 30

    def call(top_p=0.9, block=32, T=32):
        return lib.bdm_moe_block_forward_coreset(
            A, T, 2048, A, None, 256, 8, 1, top_p, block, A, A, A, 512, A, A, A, 0, None, A,
            None, None, None, None, None, A, size, None)
    assert call(top_p=0.0) == -1
    assert call(top_p=-0.5) == -1
    assert call(top_p=1.5) == -1
    assert call(top_p=float("nan")) == -1
    assert call(block=0) == -1
    assert call(block=33) == -1
    assert call(T=4000) == -2


def test_denoise_validation(lib):
    from block_diffusion_moe_amd.binding import MoeLayerC
    A = _fake(1 << 20)
    lay = (MoeLayerC * 2)()
    for i in range(2):
        for f, _ in MoeLayerC._fields_:
            setattr(lay[i], f, 1 << 20)
        lay[i].router_bias = None
    steps = ctypes.c_int(-1)
    size = 1 << 30

    def call(**kw):
        a = dict(tokens=A, T=32, emb=A, V=248320, H=2048, layers=lay, L=2, E=256, k=8, I=512,
                 renorm=1, head=A, layout=0, mask=151669, thr=0.95, top_p=0.0, blk=0, steps=32)
        a.update(kw)
        return lib.bdm_denoise_block(a["tokens"], a["T"], a["emb"], a["V"], a["H"], a["layers"],
                                     a["L"], a["E"], a["k"], a["I"], a["renorm"], a["head"],
                                     a["layout"], a["mask"], a["thr"], a["top_p"], a["blk"],
                                     a["steps"],
                                     ctypes.byref(steps), None, A, size, None)
    assert call(tokens=None) == -1
    assert call(mask=248320) == -1
    assert call(steps=-1) == -1
    assert call(layout=3) == -1
    assert call(layout=2) == -1                 # gate/up pairs: w_up != w_gate + 16 H
    assert call(thr=float("inf")) == -1
    assert call(top_p=-0.1) == -1
    assert call(top_p=1.5) == -1
    assert call(top_p=float("nan")) == -1
    assert call(blk=-1) == -1
    assert call(T=4000) == -2
    assert call(H=2000) == -2
    lay[1].ws_gate = None                       # shared trio broken in one layer
    assert call() == -1
    lay[1].ws_up = None
    lay[1].ws_down = None                       # layers disagree on the shared expert
    assert call() == -1
    size_t = ctypes.c_size_t(0)
    assert lib.bdm_denoise_workspace_bytes(32, 2048, 512, 256, 8, 1, ctypes.byref(size_t)) == 0
    m = ctypes.c_size_t(0)
    assert lib.bdm_moe_workspace_bytes(32, 2048, 512, 256, 8, 1, ctypes.byref(m)) == 0
    assert size_t.value > m.value


def test_verify_validation(lib):
    A = _fake(1 << 20)

    def call(**kw):
        a = dict(h=A, T1=33, H=2048, w=A, V=248320, lay=0, cand=A, rule=1, ratio=0.9,
                 delta=0.6, tok=A, na=A, ws=A, wsb=1 << 30)
        a.update(kw)
        return lib.bdm_lm_head_verify(a["h"], a["T1"], a["H"], a["w"], a["V"], a["lay"],
                                      a["cand"], a["rule"], a["ratio"], a["delta"], a["tok"],
                                      a["na"], None, None, None, None, a["ws"], a["wsb"], None)
    assert call(h=None) == -1
    assert call(tok=None) == -1
    assert call(na=None) == -1
    assert call(cand=None) == -1
    assert call(rule=2) == -1
    assert call(ratio=float("nan")) == -1
    assert call(delta=float("inf")) == -1
    assert call(lay=3) == -1
    assert call(T1=0) == -1
    assert call(V=1) == -1
    assert call(T1=2049) == -2
    assert call(H=2112) == -2          # multiple of 64, not of 256
    assert call(H=768) == -2           # multiple of 256 outside {256, 512, 1024, 2048}
    assert call(wsb=16) == -3
    n = ctypes.c_size_t(0)
    assert lib.bdm_head_verify_workspace_bytes(33, 2048, 248320, ctypes.byref(n)) == 0
    h = ctypes.c_size_t(0)
    assert lib.bdm_head_workspace_bytes(33, 2048, 248320, ctypes.byref(h)) == 0
    assert n.value > h.value
    assert lib.bdm_head_verify_workspace_bytes(33, 768, 248320, ctypes.byref(n)) == -2


def test_binding_weight_layout_detection():
    """The binding's choice of weight_layout from the kinds of expert
    matrices it is given (host logic only: no library call)."""
    from block_diffusion_moe_amd import binding as bd
    I, H = 32, 64
    rm = torch.zeros((2, I, H), dtype=torch.bfloat16)
    down = bd.Packed(torch.zeros(2 * H * I, dtype=torch.bfloat16), (2, H, I))
    plain = bd.Packed(torch.zeros(2 * I * H, dtype=torch.bfloat16), (2, I, H))
    buf = torch.zeros(2 * 2 * I * H, dtype=torch.bfloat16)
    g = bd.Packed(buf, (2, I, H), 0, "gate")
    u = bd.Packed(buf, (2, I, H), 16 * H, "up")
    assert bd._expert_layout(rm, rm, rm, None, None, None) == bd.BDM_LAYOUT_ROW_MAJOR
    assert bd._expert_layout(plain, plain, down, None, None, None) == bd.BDM_LAYOUT_MFMA_TILES
    assert bd._expert_layout(g, u, down, None, None, None) == bd.BDM_LAYOUT_MFMA_TILES_GU
    with pytest.raises(ValueError):                     # row-major mixed with packed
        bd._expert_layout(rm, plain, down, None, None, None)
    with pytest.raises(ValueError):                     # gate and up swapped
        bd._expert_layout(u, g, down, None, None, None)
    with pytest.raises(ValueError):                     # halves of different buffers
        bd._expert_layout(g, bd.Packed(buf.clone(), (2, I, H), 16 * H, "up"), down,
                          None, None, None)
    with pytest.raises(ValueError):                     # shared expert not a pair
        bd._expert_layout(g, u, down, plain, plain, down)
    short = torch.zeros(2 * I * H + 16 * H, dtype=torch.bfloat16)
    with pytest.raises(ValueError):                     # buffer shorter than both matrices
        bd._expert_layout(bd.Packed(short, (2, I, H), 0, "gate"),
                          bd.Packed(short, (2, I, H), 16 * H, "up"), down, None, None, None)


def test_noalloc_validation(lib):
    """The allocation-free MoE entry point rejects, before any device call,
    null pointers, bad shapes and sizes whose workspace exceeds its static
    buffer (the pointers below are never dereferenced)."""
    from block_diffusion_moe_amd import binding
    A = _fake(1 << 20)

    def call(T=32, x=A, H=2048, E=256, k=8, I=512, y=_fake(2 << 20)):
        return lib.bdm_moe_block_forward_noalloc(x, T, H, A, None, E, k, 1, A, A, A, I, A, A, A,
                                                 0, None, y, None, None, None, None)

    assert call(x=None) == -1
    assert call(y=None) == -1
    assert call(k=0) == -1
    assert call(H=100) == -2
    assert call(T=4096) == -2
    for T in (512, 1024, 2048):                  # need more than the static buffer
        assert binding.bdm_moe_workspace_bytes(T, 2048, 512, 256, 8, True) > \
            binding.BDM_STATIC_SCRATCH_BYTES
        assert call(T=T) == -3
    assert binding.bdm_moe_workspace_bytes(256, 2048, 512, 256, 8, True) <= \
        binding.BDM_STATIC_SCRATCH_BYTES
