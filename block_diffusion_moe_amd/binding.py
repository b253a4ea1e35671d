"""ctypes binding of libbdmoe.so: the C entry points under the same names.

Argument marshalling only: torch tensors are checked for device, dtype,
shape and contiguity and passed as raw device pointers together with the
caller's current HIP stream; every step of the computation runs in the HIP
kernels of the library.  A missing library raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbdmoe.so")
# the same entry points with device-side bounds checks (bdm_debug_bounds)
DEBUG_LIB_PATH = os.path.join(_HERE, "libbdmoe_debug.so")

BDM_OK = 0
BDM_MASK_ID_CLOVER = 151669
BDM_THRESHOLD_DEFAULT = 0.95
BDM_LAYOUT_ROW_MAJOR = 0
BDM_LAYOUT_MFMA_TILES = 1
BDM_LAYOUT_MFMA_TILES_GU = 2

_c_int, _c_float, _c_size, _vp = ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p

_SIGS = {
    "bdm_version": (_c_int, []),
    "bdm_status_string": (ctypes.c_char_p, [_c_int]),
    "bdm_debug_bounds": (_c_int, [ctypes.POINTER(ctypes.c_uint)]),
    "bdm_moe_workspace_bytes": (_c_int, [_c_int] * 6 + [ctypes.POINTER(_c_size)]),
    "bdm_moe_block_forward": (_c_int, [_vp, _c_int, _c_int, _vp, _vp, _c_int, _c_int, _c_int,
                                       _vp, _vp, _vp, _c_int, _vp, _vp, _vp, _c_int, _vp, _vp,
                                       _vp, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "bdm_moe_block_forward_noalloc": (_c_int, [_vp, _c_int, _c_int, _vp, _vp, _c_int, _c_int,
                                               _c_int, _vp, _vp, _vp, _c_int, _vp, _vp, _vp,
                                               _c_int, _vp, _vp, _vp, _vp, _vp, _vp]),
    "bdm_moe_block_forward_coreset": (_c_int, [_vp, _c_int, _c_int, _vp, _vp, _c_int, _c_int,
                                               _c_int, _c_float, _c_int, _vp, _vp, _vp, _c_int,
                                               _vp, _vp, _vp, _c_int, _vp, _vp, _vp, _vp, _vp,
                                               _vp, _vp, _vp, _c_size, _vp]),
    "bdm_head_workspace_bytes": (_c_int, [_c_int, _c_int, _c_int, ctypes.POINTER(_c_size)]),
    "bdm_denoise_workspace_bytes": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                             ctypes.POINTER(_c_size)]),
    "bdm_denoise_block": (_c_int, [_vp, _c_int, _vp, _c_int, _c_int, _vp, _c_int, _c_int,
                                   _c_int, _c_int, _c_int, _vp, _c_int, ctypes.c_int32,
                                   _c_float, _c_float, _c_int, _c_int, ctypes.POINTER(_c_int),
                                   _vp, _vp, _c_size, _vp]),
    "bdm_lm_head_unmask": (_c_int, [_vp, _c_int, _c_int, _vp, _c_int, _c_int, ctypes.c_int32,
                                    _c_float, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _c_size,
                                    _vp]),
    "bdm_head_verify_workspace_bytes": (_c_int, [_c_int, _c_int, _c_int,
                                                 ctypes.POINTER(_c_size)]),
    "bdm_lm_head_verify": (_c_int, [_vp, _c_int, _c_int, _vp, _c_int, _c_int, _vp, _c_int,
                                    _c_float, _c_float, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                    _c_size, _vp]),
    "bdm_head_stat_parts": (_c_int, [ctypes.POINTER(_c_int)]),
    "bdm_lm_head_stats": (_c_int, [_vp, _c_int, _c_int, _vp, _c_int, _c_int, _c_int,
                                   ctypes.c_int32, _vp, _vp, _vp, _c_int, _vp]),
    "bdm_unmask_from_stats": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, ctypes.c_int32,
                                       _c_float, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp]),
    "bdm_packed_weight_elems": (_c_int, [ctypes.c_long, _c_int, ctypes.POINTER(_c_size)]),
    "bdm_pack_weights": (_c_int, [_vp, ctypes.c_long, _c_int, _vp, _vp]),
    "bdm_pack_gate_up": (_c_int, [_vp, _vp, ctypes.c_long, _c_int, _vp, _vp]),
    "bdm_rmsnorm": (_c_int, [_vp, _vp, _c_float, _c_int, _c_int, _vp, _vp]),
}

EXPORTS = tuple(_SIGS)

_lib = None


class BdmError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed with status {status}: {bdm_status_string(status)}")
        self.status = status


def load(path: str = None) -> ctypes.CDLL:
    """Load the library (once): `path`, else $BDM_LIBRARY, else libbdmoe.so
    (DEBUG_LIB_PATH is the bounds-checked build).  torch is imported first so
    the library binds to the HIP runtime torch uses."""
    global _lib
    if _lib is not None:
        return _lib
    if path is None:
        path = os.environ.get("BDM_LIBRARY") or LIB_PATH
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m block_diffusion_moe_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class Packed:
    """A bf16 weight tensor in the MFMA-tile layout (see bdm_pack_weights):
    `data` holds the packed elements, `shape` the logical row-major shape
    (the last dimension is the reduction dimension).  A gate or up matrix of
    a gate/up pair (bdm_pack_gate_up) shares `data` with its partner:
    `offset` elements in, `pair` the name of its role ("gate" or "up")."""

    def __init__(self, data: torch.Tensor, shape, offset: int = 0, pair=None):
        self.data = data
        self.shape = tuple(shape)
        self.device = data.device
        self.dtype = data.dtype
        self.offset = int(offset)
        self.pair = pair

    def data_ptr(self):
        return self.data.data_ptr() + 2 * self.offset


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(t, name: str, dtype, shape=None, device=None):
    if t is None:
        return
    if isinstance(t, Packed):
        if t.dtype != dtype or not t.data.is_cuda or not t.data.is_contiguous():
            raise ValueError(f"{name}: packed data must be a contiguous device {dtype} tensor")
        if device is not None and t.device != device:
            raise ValueError(f"{name}: on {t.device}, expected {device}")
        if shape is not None and t.shape != tuple(shape):
            raise ValueError(f"{name}: logical shape {t.shape}, expected {tuple(shape)}")
        rows = 1
        for d in t.shape[:-1]:
            rows *= d
        if t.data.numel() < bdm_packed_weight_elems(rows, t.shape[-1]):
            raise ValueError(f"{name}: packed buffer too small")
        return
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def _raise(fn: str, st: int):
    if st != BDM_OK:
        raise BdmError(fn, st)


def bdm_version() -> int:
    return load().bdm_version()


def bdm_status_string(status: int) -> str:
    return load().bdm_status_string(status).decode()


BDM_ERR_NOT_DEBUG_BUILD = -5


def bdm_debug_bounds() -> int:
    """The debug build's bounds-check violation bits since the last call
    (0: none), cleared; synchronises with the device.  Raises BdmError on
    the release library."""
    v = ctypes.c_uint(0)
    _raise("bdm_debug_bounds", load().bdm_debug_bounds(ctypes.byref(v)))
    return int(v.value)


def bdm_moe_workspace_bytes(T, H, I, E, k, has_shared) -> int:
    n = _c_size(0)
    _raise("bdm_moe_workspace_bytes", load().bdm_moe_workspace_bytes(T, H, I, E, k, int(has_shared),
                                                                     ctypes.byref(n)))
    return n.value


def bdm_head_workspace_bytes(T, H, V) -> int:
    n = _c_size(0)
    _raise("bdm_head_workspace_bytes", load().bdm_head_workspace_bytes(T, H, V, ctypes.byref(n)))
    return n.value


def bdm_packed_weight_elems(rows: int, cols: int) -> int:
    n = _c_size(0)
    _raise("bdm_packed_weight_elems", load().bdm_packed_weight_elems(int(rows), int(cols),
                                                                     ctypes.byref(n)))
    return n.value


def bdm_pack_weights(w: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> Packed:
    """Packed (MFMA-tile) copy of a row-major bf16 weight tensor; all leading
    dimensions are folded into rows (an expert stack [E][I][H] packs as one
    [E*I][H] matrix)."""
    _check(w, "w", torch.bfloat16)
    cols = w.shape[-1]
    rows = w.numel() // cols
    n = bdm_packed_weight_elems(rows, cols)
    if out is None:
        out = torch.empty(n, dtype=torch.bfloat16, device=w.device)
    _check(out, "out", torch.bfloat16, device=w.device)
    if out.numel() < n:
        raise ValueError("out: too small for the packed copy")
    _raise("bdm_pack_weights", load().bdm_pack_weights(_ptr(w), rows, cols, _ptr(out),
                                                       _stream(stream)))
    return Packed(out, w.shape)


def bdm_pack_gate_up(w_gate: torch.Tensor, w_up: torch.Tensor, out=None, stream=None):
    """The gate and up matrices of a layer (or of its shared expert) packed
    into one buffer whose 16-row groups alternate gate, up
    (BDM_LAYOUT_MFMA_TILES_GU); returns the (gate, up) `Packed` views, to be
    passed as w_gate / w_up (or ws_gate / ws_up) together."""
    _check(w_gate, "w_gate", torch.bfloat16)
    _check(w_up, "w_up", torch.bfloat16, tuple(w_gate.shape), w_gate.device)
    cols = w_gate.shape[-1]
    rows = w_gate.numel() // cols
    n = 2 * rows * cols
    if out is None:
        out = torch.empty(n, dtype=torch.bfloat16, device=w_gate.device)
    _check(out, "out", torch.bfloat16, device=w_gate.device)
    if out.numel() < n:
        raise ValueError("out: too small for the packed pair")
    _raise("bdm_pack_gate_up", load().bdm_pack_gate_up(_ptr(w_gate), _ptr(w_up), rows, cols,
                                                       _ptr(out), _stream(stream)))
    return (Packed(out, w_gate.shape, 0, "gate"), Packed(out, w_up.shape, 16 * cols, "up"))


def _expert_layout(gate, up, down, sgate, sup, sdown) -> int:
    """weight_layout of one layer's expert matrices: all row-major, all
    packed plainly, or gate/up (and the shared expert's) as packed pairs."""
    mats = [t for t in (gate, up, down, sgate, sup, sdown) if t is not None]
    packed = [isinstance(t, Packed) for t in mats]
    if any(packed) and not all(packed):
        raise ValueError("expert weights must be all row-major or all packed")
    if not all(packed):
        return BDM_LAYOUT_ROW_MAJOR
    pairs = [(gate, up)] + ([(sgate, sup)] if sgate is not None else [])
    roles = [t.pair for g, u in pairs for t in (g, u)]
    if all(r is None for r in roles) and down.pair is None and (sdown is None or
                                                                sdown.pair is None):
        return BDM_LAYOUT_MFMA_TILES
    for g, u in pairs:
        if g.pair != "gate" or u.pair != "up" or g.data is not u.data or \
                u.offset != g.offset + 16 * g.shape[-1]:
            raise ValueError("gate/up must both come from one bdm_pack_gate_up call "
                             "(routed and shared alike)")
        rows = 1
        for d in g.shape[:-1]:
            rows *= d
        if rows % 16 or g.data.numel() - g.offset < 2 * rows * g.shape[-1]:
            raise ValueError("gate/up pair: rows not a multiple of 16, or the buffer "
                             "holds less than both matrices")
    if down.pair is not None or (sdown is not None and sdown.pair is not None):
        raise ValueError("down matrices are packed with bdm_pack_weights")
    return BDM_LAYOUT_MFMA_TILES_GU


def workspace(nbytes: int, device) -> torch.Tensor:
    """Device scratch buffer (torch allocations are 256-byte aligned)."""
    return torch.empty(max(1, nbytes), dtype=torch.uint8, device=device)


def bdm_moe_block_forward(x, w_router, w_gate, w_up, w_down, k: int, *, router_bias=None,
                          ws_gate=None, ws_up=None, ws_down=None, residual=None, y=None,
                          topk_idx=None, topk_w=None, renorm: bool = True, ws=None, stream=None,
                          coreset_top_p=None, coreset_block: int = 32, n_kept=None,
                          y_norm=None, x_norm=None):
    """y = MoE layer over the block x (see include/bdmoe.h).  ``y`` may be
    ``residual`` (in-place residual add); a new tensor is made when None.
    Expert weights may be row-major tensors or all `Packed`.  ``y_norm``
    (optional) receives RMSNorm(y), the next layer's input.  ``x_norm``
    (optional): x is un-normalised; the layer takes RMSNorm(x) itself, writes
    it there and computes y = residual + MoE(RMSNorm(x)).  With
    ``coreset_top_p`` the block coreset selector runs first
    (bdm_moe_block_forward_coreset; ``n_kept`` receives |kept| per block)."""
    T, H = x.shape
    E, I, _ = w_gate.shape
    dev = x.device
    if y is None:
        y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _check(x, "x", torch.bfloat16, (T, H))
    _check(w_router, "w_router", torch.float32, (E, H), dev)
    _check(router_bias, "router_bias", torch.float32, (E,), dev)
    _check(w_gate, "w_gate", torch.bfloat16, (E, I, H), dev)
    _check(w_up, "w_up", torch.bfloat16, (E, I, H), dev)
    _check(w_down, "w_down", torch.bfloat16, (E, H, I), dev)
    _check(ws_gate, "ws_gate", torch.bfloat16, (I, H), dev)
    _check(ws_up, "ws_up", torch.bfloat16, (I, H), dev)
    _check(ws_down, "ws_down", torch.bfloat16, (H, I), dev)
    _check(residual, "residual", torch.bfloat16, (T, H), dev)
    _check(y, "y", torch.bfloat16, (T, H), dev)
    _check(y_norm, "y_norm", torch.bfloat16, (T, H), dev)
    _check(x_norm, "x_norm", torch.bfloat16, (T, H), dev)
    _check(topk_idx, "topk_idx", torch.int32, (T, k), dev)
    _check(topk_w, "topk_w", torch.float32, (T, k), dev)
    has_shared = ws_gate is not None
    layout = _expert_layout(w_gate, w_up, w_down, ws_gate, ws_up, ws_down)
    need = bdm_moe_workspace_bytes(T, H, I, E, k, has_shared)
    if ws is None:
        ws = workspace(need, dev)
    if coreset_top_p is None:
        st = load().bdm_moe_block_forward(
            _ptr(x), T, H, _ptr(w_router), _ptr(router_bias), E, int(k), int(renorm),
            _ptr(w_gate), _ptr(w_up), _ptr(w_down), I, _ptr(ws_gate), _ptr(ws_up),
            _ptr(ws_down), layout, _ptr(residual), _ptr(y), _ptr(y_norm), _ptr(x_norm),
            _ptr(topk_idx), _ptr(topk_w), _ptr(ws), ws.numel(), _stream(stream))
        _raise("bdm_moe_block_forward", st)
        return y
    nb = (T + coreset_block - 1) // max(1, coreset_block)
    _check(n_kept, "n_kept", torch.int32, (nb,), dev)
    st = load().bdm_moe_block_forward_coreset(
        _ptr(x), T, H, _ptr(w_router), _ptr(router_bias), E, int(k), int(renorm),
        float(coreset_top_p), int(coreset_block), _ptr(w_gate), _ptr(w_up), _ptr(w_down), I,
        _ptr(ws_gate), _ptr(ws_up), _ptr(ws_down), layout, _ptr(residual), _ptr(y),
        _ptr(y_norm), _ptr(x_norm), _ptr(topk_idx), _ptr(topk_w), _ptr(n_kept), _ptr(ws),
        ws.numel(), _stream(stream))
    _raise("bdm_moe_block_forward_coreset", st)
    return y


BDM_STATIC_SCRATCH_BYTES = 32 << 20


def bdm_moe_block_forward_noalloc(x, w_router, w_gate, w_up, w_down, k: int, *,
                                  router_bias=None, ws_gate=None, ws_up=None, ws_down=None,
                                  residual=None, y=None, topk_idx=None, topk_w=None,
                                  renorm: bool = True, stream=None, y_norm=None):
    """bdm_moe_block_forward with the library's static per-device scratch
    buffer instead of a workspace (nothing is allocated by the call when
    ``y`` is given).  Calls that overlap on one device race."""
    T, H = x.shape
    E, I, _ = w_gate.shape
    dev = x.device
    if y is None:
        y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _check(x, "x", torch.bfloat16, (T, H))
    _check(w_router, "w_router", torch.float32, (E, H), dev)
    _check(router_bias, "router_bias", torch.float32, (E,), dev)
    _check(w_gate, "w_gate", torch.bfloat16, (E, I, H), dev)
    _check(w_up, "w_up", torch.bfloat16, (E, I, H), dev)
    _check(w_down, "w_down", torch.bfloat16, (E, H, I), dev)
    _check(ws_gate, "ws_gate", torch.bfloat16, (I, H), dev)
    _check(ws_up, "ws_up", torch.bfloat16, (I, H), dev)
    _check(ws_down, "ws_down", torch.bfloat16, (H, I), dev)
    _check(residual, "residual", torch.bfloat16, (T, H), dev)
    _check(y, "y", torch.bfloat16, (T, H), dev)
    _check(y_norm, "y_norm", torch.bfloat16, (T, H), dev)
    _check(topk_idx, "topk_idx", torch.int32, (T, k), dev)
    _check(topk_w, "topk_w", torch.float32, (T, k), dev)
    layout = _expert_layout(w_gate, w_up, w_down, ws_gate, ws_up, ws_down)
    st = load().bdm_moe_block_forward_noalloc(
        _ptr(x), T, H, _ptr(w_router), _ptr(router_bias), E, int(k), int(renorm),
        _ptr(w_gate), _ptr(w_up), _ptr(w_down), I, _ptr(ws_gate), _ptr(ws_up), _ptr(ws_down),
        layout, _ptr(residual), _ptr(y), _ptr(y_norm), _ptr(topk_idx), _ptr(topk_w),
        _stream(stream))
    _raise("bdm_moe_block_forward_noalloc", st)
    return y


class MoeLayerC(ctypes.Structure):
    """bdm_moe_layer of include/bdmoe.h."""
    _fields_ = [(n, ctypes.c_void_p) for n in ("w_router", "router_bias", "w_gate", "w_up",
                                               "w_down", "ws_gate", "ws_up", "ws_down")]


def bdm_denoise_workspace_bytes(T, H, I, E, k, has_shared=True) -> int:
    n = _c_size(0)
    _raise("bdm_denoise_workspace_bytes", load().bdm_denoise_workspace_bytes(
        T, H, I, E, k, int(has_shared), ctypes.byref(n)))
    return n.value


class MoeStack:
    """The layers of a pre-norm expert stack checked and marshalled once into
    the host array of bdm_moe_layer structs bdm_denoise_block takes (the
    tensors stay referenced here).  `layers`: list of dicts with w_router,
    router_bias (optional), w_gate, w_up, w_down, ws_gate, ws_up, ws_down
    (tensors, or all expert matrices `Packed`, gate/up possibly as
    bdm_pack_gate_up pairs: the same kind in every layer)."""

    def __init__(self, layers):
        if not layers:
            raise ValueError("at least one layer")
        self.layers = list(layers)
        E, I, H = self.layers[0]["w_gate"].shape
        dev = self.layers[0]["w_router"].device
        self.E, self.I, self.H = E, I, H
        self.has_shared = self.layers[0].get("ws_gate") is not None
        self.arr = (MoeLayerC * len(self.layers))()
        for i, lw in enumerate(self.layers):
            _check(lw["w_router"], "w_router", torch.float32, (E, H), dev)
            _check(lw.get("router_bias"), "router_bias", torch.float32, (E,), dev)
            _check(lw["w_gate"], "w_gate", torch.bfloat16, (E, I, H), dev)
            _check(lw["w_up"], "w_up", torch.bfloat16, (E, I, H), dev)
            _check(lw["w_down"], "w_down", torch.bfloat16, (E, H, I), dev)
            for nm, shp in (("ws_gate", (I, H)), ("ws_up", (I, H)), ("ws_down", (H, I))):
                _check(lw.get(nm), nm, torch.bfloat16, shp, dev)
            for f, _ in MoeLayerC._fields_:
                ptr = _ptr(lw.get(f))
                setattr(self.arr[i], f, None if ptr is None else ptr.value)
            lay = _expert_layout(*[lw.get(n) for n in ("w_gate", "w_up", "w_down", "ws_gate",
                                                       "ws_up", "ws_down")])
            if i > 0 and lay != self.layout:
                raise ValueError("every layer's expert weights must be of one kind")
            self.layout = lay
        self.packed = self.layout != BDM_LAYOUT_ROW_MAJOR
        self.device = dev

    def __len__(self):
        return len(self.layers)


def bdm_denoise_block(tokens, w_embed, layers, w_head, k: int, mask_id: int,
                      threshold: float = 0.95, max_steps=None, renorm: bool = True, ws=None,
                      stream=None, coreset_top_p=None, block_tokens: int = 0):
    """The denoise loop over the block `tokens` (int32 device [T], updated in
    place).  `layers`: a MoeStack, or the list of layer dicts it takes
    (marshalled on every call then).  `coreset_top_p`: route every layer
    through the block coreset selector at that top_p (None: plain top-k).
    `block_tokens` > 0: the rows are several blocks of that many slots, each
    with its own commit rule.  Returns (steps, commits per step, summed over
    the blocks)."""
    T = tokens.shape[0]
    V, H = w_embed.shape
    dev = tokens.device
    stack = layers if isinstance(layers, MoeStack) else MoeStack(layers)
    _check(tokens, "tokens", torch.int32, (T,))
    _check(w_embed, "w_embed", torch.bfloat16, (V, H), dev)
    _check(w_head, "w_head", torch.bfloat16, (V, H), dev)
    if stack.H != H or stack.device != dev:
        raise ValueError("the stack's hidden size or device differs from w_embed's")
    if isinstance(w_head, Packed) != stack.packed:
        raise ValueError("expert and head weights must be all row-major or all packed")
    layout = stack.layout
    need = bdm_denoise_workspace_bytes(T, H, stack.I, stack.E, k, stack.has_shared)
    if ws is None:
        ws = workspace(need, dev)
    limit = (T if block_tokens <= 0 else min(T, int(block_tokens))) if max_steps is None \
        else int(max_steps)
    steps = _c_int(0)
    commits = (ctypes.c_int32 * max(1, limit))()
    _raise("bdm_denoise_block", load().bdm_denoise_block(
        _ptr(tokens), T, _ptr(w_embed), V, H, stack.arr, len(stack), stack.E, int(k), stack.I,
        int(renorm), _ptr(w_head), layout, int(mask_id), float(threshold),
        float(coreset_top_p or 0.0), int(block_tokens), limit, ctypes.byref(steps), commits,
        _ptr(ws), ws.numel(), _stream(stream)))
    return steps.value, [int(commits[i]) for i in range(steps.value)]


def bdm_lm_head_unmask(h, w_head, mask_id: int, threshold: float, fallback: bool, tokens,
                       argmax=None, conf=None, n_committed=None, ws=None, stream=None,
                       block_tokens: int = 0):
    """Head + commit rule; ``block_tokens`` > 0 applies the rule to every
    block of that many rows on its own (0: the rows are one block)."""
    T, H = h.shape
    V = w_head.shape[0]
    dev = h.device
    _check(h, "h", torch.bfloat16, (T, H))
    _check(w_head, "w_head", torch.bfloat16, (V, H), dev)
    _check(tokens, "tokens", torch.int32, (T,), dev)
    _check(argmax, "argmax", torch.int32, (T,), dev)
    _check(conf, "conf", torch.float32, (T,), dev)
    _check(n_committed, "n_committed", torch.int32, (1,), dev)
    need = bdm_head_workspace_bytes(T, H, V)
    if ws is None:
        ws = workspace(need, dev)
    layout = BDM_LAYOUT_MFMA_TILES if isinstance(w_head, Packed) else BDM_LAYOUT_ROW_MAJOR
    st = load().bdm_lm_head_unmask(_ptr(h), T, H, _ptr(w_head), V, layout, int(mask_id),
                                   float(threshold), int(fallback), int(block_tokens),
                                   _ptr(tokens), _ptr(argmax), _ptr(conf), _ptr(n_committed),
                                   _ptr(ws), ws.numel(), _stream(stream))
    _raise("bdm_lm_head_unmask", st)
    return tokens


BDM_VERIFY_EXACT = 0
BDM_VERIFY_THRESHOLD = 1
_VERIFY_RULES = {"exact": BDM_VERIFY_EXACT, "threshold": BDM_VERIFY_THRESHOLD}


def bdm_head_verify_workspace_bytes(T1, H, V) -> int:
    n = _c_size()
    _raise("bdm_head_verify_workspace_bytes",
           load().bdm_head_verify_workspace_bytes(T1, H, V, ctypes.byref(n)))
    return n.value


def bdm_lm_head_verify(h, w_head, cand, rule: str = "threshold", ratio: float = 0.9,
                       delta: float = 0.6, tokens_out=None, n_accepted=None, accept=None,
                       argmax=None, p_cand=None, entropy=None, ws=None, stream=None):
    """Verify epilogue over T1 = len(cand) + 1 causal hidden rows.  Returns
    (tokens_out [T1] int32, n_accepted [1] int32), both device tensors."""
    T1, H = h.shape
    V = w_head.shape[0]
    dev = h.device
    if rule not in _VERIFY_RULES:
        raise ValueError(f"rule must be one of {sorted(_VERIFY_RULES)}")
    _check(h, "h", torch.bfloat16, (T1, H))
    _check(w_head, "w_head", torch.bfloat16, (V, H), dev)
    _check(cand, "cand", torch.int32, (T1 - 1,), dev)
    if tokens_out is None:
        tokens_out = torch.empty(T1, dtype=torch.int32, device=dev)
    if n_accepted is None:
        n_accepted = torch.empty(1, dtype=torch.int32, device=dev)
    _check(tokens_out, "tokens_out", torch.int32, (T1,), dev)
    _check(n_accepted, "n_accepted", torch.int32, (1,), dev)
    _check(accept, "accept", torch.int32, (T1 - 1,), dev)
    _check(argmax, "argmax", torch.int32, (T1,), dev)
    _check(p_cand, "p_cand", torch.float32, (T1 - 1,), dev)
    _check(entropy, "entropy", torch.float32, (T1,), dev)
    need = bdm_head_verify_workspace_bytes(T1, H, V)
    if ws is None:
        ws = workspace(need, dev)
    layout = BDM_LAYOUT_MFMA_TILES if isinstance(w_head, Packed) else BDM_LAYOUT_ROW_MAJOR
    st = load().bdm_lm_head_verify(_ptr(h), T1, H, _ptr(w_head), V, layout,
                                   _ptr(cand) if T1 > 1 else None, _VERIFY_RULES[rule],
                                   float(ratio), float(delta), _ptr(tokens_out),
                                   _ptr(n_accepted), _ptr(accept), _ptr(argmax), _ptr(p_cand),
                                   _ptr(entropy), _ptr(ws), ws.numel(), _stream(stream))
    _raise("bdm_lm_head_verify", st)
    return tokens_out, n_accepted


def bdm_head_stat_parts() -> int:
    n = _c_int(0)
    _raise("bdm_head_stat_parts", load().bdm_head_stat_parts(ctypes.byref(n)))
    return n.value


def bdm_lm_head_stats(h, w_head, mask_id: int, stat_max, stat_sum, stat_arg, vocab_offset=0,
                      stream=None):
    """Phase 1 of the head over the vocabulary rows [vocab_offset, vocab_offset + V) of
    w_head; stat_* are [T][stride] views whose first bdm_head_stat_parts() columns are
    written (pass column slices of a wider array to place several shards)."""
    T, H = h.shape
    V = w_head.shape[0]
    dev = h.device
    _check(h, "h", torch.bfloat16, (T, H))
    _check(w_head, "w_head", torch.bfloat16, (V, H), dev)
    for t, nm, dt in ((stat_max, "stat_max", torch.float32), (stat_sum, "stat_sum", torch.float32),
                      (stat_arg, "stat_arg", torch.int32)):
        if t.dtype != dt or t.device != dev or t.dim() != 2 or t.shape[0] != T or t.stride(1) != 1:
            raise ValueError(f"{nm}: expected a [T][*] {dt} device view with unit column stride")
    stride = stat_max.stride(0)
    if stat_sum.stride(0) != stride or stat_arg.stride(0) != stride:
        raise ValueError("stat_*: row strides differ")
    layout = BDM_LAYOUT_MFMA_TILES if isinstance(w_head, Packed) else BDM_LAYOUT_ROW_MAJOR
    _raise("bdm_lm_head_stats", load().bdm_lm_head_stats(
        _ptr(h), T, H, _ptr(w_head), V, int(vocab_offset), layout, int(mask_id), _ptr(stat_max),
        _ptr(stat_sum), _ptr(stat_arg), stride, _stream(stream)))


def bdm_unmask_from_stats(stat_max, stat_sum, stat_arg, mask_id: int, threshold: float,
                          fallback: bool, tokens, argmax=None, conf=None, n_committed=None,
                          stream=None, block_tokens: int = 0):
    """Phase 2: merge the [T][parts] triples (all columns of the given views) and
    apply the commit rule to tokens."""
    T, parts = stat_max.shape
    dev = tokens.device
    _check(tokens, "tokens", torch.int32, (T,), dev)
    _check(argmax, "argmax", torch.int32, (T,), dev)
    _check(conf, "conf", torch.float32, (T,), dev)
    _check(n_committed, "n_committed", torch.int32, (1,), dev)
    stride = stat_max.stride(0)
    _raise("bdm_unmask_from_stats", load().bdm_unmask_from_stats(
        _ptr(stat_max), _ptr(stat_sum), _ptr(stat_arg), T, parts, stride, int(mask_id),
        float(threshold), int(fallback), int(block_tokens), _ptr(tokens), _ptr(argmax),
        _ptr(conf), _ptr(n_committed), _stream(stream)))
    return tokens


def bdm_rmsnorm(x, out, gamma=None, eps: float = 1e-6, stream=None):
    T, H = x.shape
    _check(x, "x", torch.bfloat16, (T, H))
    _check(out, "out", torch.bfloat16, (T, H), x.device)
    _check(gamma, "gamma", torch.float32, (H,), x.device)
    st = load().bdm_rmsnorm(_ptr(x), _ptr(gamma), float(eps), T, H, _ptr(out), _stream(stream))
    _raise("bdm_rmsnorm", st)
    return out
