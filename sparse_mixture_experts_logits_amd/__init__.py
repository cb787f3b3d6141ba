"""Python binding of libmoe_mi355x.so, the MI355X sparse-MoE layer.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels. PyTorch supplies device memory and the current stream. The library
must be built (``python -m sparse_mixture_experts_logits_amd.build``); if it is
missing, every call raises -- there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

__all__ = ["moe_forward", "workspace_bytes", "quantize_fp8_rows", "MoeError", "load_library", "LIB_PATH",
           "FLAG_FORCE_TILED", "FLAG_FORCE_SKINNY", "WEIGHTS_NATIVE", "WEIGHTS_FP8_E4M3", "WEIGHTS_MXFP4", "quantize_mxfp4_rows",
           "SCORE_SOFTMAX", "SCORE_SIGMOID", "SCORE_SPARSEMIXER", "TileBlocks", "pack_tile_blocks",
           "tile_blocks_bytes", "bf16_bits_to_tensor", "EXPORTS"]

# MOE_MI355X_LIB may point at another build of the same library (tuning builds)
LIB_PATH = os.environ.get("MOE_MI355X_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                             "libmoe_mi355x.so")

MOE_BF16 = 0
MOE_F32 = 1
FLAG_FORCE_TILED = 0x1
FLAG_FORCE_SKINNY = 0x2
WEIGHTS_NATIVE = 0
WEIGHTS_FP8_E4M3 = 1
WEIGHTS_MXFP4 = 2
SCORE_SOFTMAX = 0
SCORE_SIGMOID = 1
SCORE_SPARSEMIXER = 2
LAYOUT_ROWS = 0
LAYOUT_TILE_BLOCKS = 1
PACK_GATE_UP = 0
PACK_DOWN = 1
EXPORTS = ("moe_opts_init", "moe_workspace_bytes", "moe_forward", "moe_forward_noalloc", "moe_quantize_fp8_rows",
           "moe_quantize_mxfp4_rows", "moe_tile_blocks_bytes", "moe_pack_tile_blocks", "moe_last_error")
NOALLOC_SCRATCH_BYTES = 128 << 20  # MOE_NOALLOC_SCRATCH_BYTES
STAGES = ("router", "scan", "permute", "gate_up", "down", "shared_gate_up", "shared_down", "combine")
STAGE_EVENTS = len(STAGES) + 1

STATUS = {0: "MOE_OK", -1: "MOE_ERR_INVALID_ARG", -2: "MOE_ERR_UNSUPPORTED", -3: "MOE_ERR_WORKSPACE",
          -4: "MOE_ERR_ALIGNMENT", -5: "MOE_ERR_HIP"}


class MoeOpts(ctypes.Structure):
    """Mirror of ``moe_opts`` in include/moe_mi355x.h."""
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("dtype", ctypes.c_int32),
        ("routed_scale", ctypes.c_float),
        ("flags", ctypes.c_uint32),
        ("router_bias", ctypes.c_void_p),
        ("shared_gate_up", ctypes.c_void_p),
        ("shared_down", ctypes.c_void_p),
        ("shared_I", ctypes.c_int64),
        ("router_logits", ctypes.c_void_p),
        ("topk_ids", ctypes.c_void_p),
        ("topk_weights", ctypes.c_void_p),
        ("expert_counts", ctypes.c_void_p),
        ("expert_offsets", ctypes.c_void_p),
        ("perm", ctypes.c_void_p),
        ("inv_perm", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("stream", ctypes.c_void_p),
        ("stage_events", ctypes.c_void_p),
        ("weight_format", ctypes.c_int32),
        ("gate_up_scale", ctypes.c_void_p),
        ("down_scale", ctypes.c_void_p),
        ("stats_mask", ctypes.c_void_p),
        ("router_prob_mean", ctypes.c_void_p),
        ("expert_load", ctypes.c_void_p),
        ("aux_loss", ctypes.c_void_p),
        ("score_func", ctypes.c_int32),
        ("selection_bias", ctypes.c_void_p),
        ("n_group", ctypes.c_int32),
        ("topk_group", ctypes.c_int32),
        ("jitter_eps", ctypes.c_float),
        ("gate_up_block_scale", ctypes.c_void_p),
        ("down_block_scale", ctypes.c_void_p),
        ("weight_layout", ctypes.c_int32),
    ]


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def load_library():
    """Load the in-tree HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FileNotFoundError(
                f"{LIB_PATH} is missing; build it with `python -m sparse_mixture_experts_logits_amd.build`")
        try:  # bind to the HIP runtime torch ships (same soname) when torch is present
            import torch  # noqa: F401
        except ImportError:  # pragma: no cover
            pass
        lib = ctypes.CDLL(LIB_PATH)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        lib.moe_opts_init.argtypes = [ctypes.POINTER(MoeOpts)]
        lib.moe_opts_init.restype = None
        lib.moe_workspace_bytes.argtypes = [i64, i64, i64, i64, i32, ctypes.POINTER(MoeOpts)]
        lib.moe_workspace_bytes.restype = i64
        lib.moe_forward.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i32, ctypes.POINTER(MoeOpts), vp]
        lib.moe_forward.restype = ctypes.c_int
        lib.moe_forward_noalloc.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i32, ctypes.POINTER(MoeOpts), vp]
        lib.moe_forward_noalloc.restype = ctypes.c_int
        lib.moe_quantize_fp8_rows.argtypes = [vp, i64, i64, vp, vp, vp]
        lib.moe_quantize_fp8_rows.restype = ctypes.c_int
        lib.moe_quantize_mxfp4_rows.argtypes = [vp, i64, i64, vp, vp, vp]
        lib.moe_quantize_mxfp4_rows.restype = ctypes.c_int
        lib.moe_tile_blocks_bytes.argtypes = [i32, i64, i64, i64]
        lib.moe_tile_blocks_bytes.restype = i64
        lib.moe_pack_tile_blocks.argtypes = [i32, vp, i64, i64, i64, vp, vp]
        lib.moe_pack_tile_blocks.restype = ctypes.c_int
        lib.moe_last_error.argtypes = []
        lib.moe_last_error.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def new_opts() -> MoeOpts:
    o = MoeOpts()
    load_library().moe_opts_init(ctypes.byref(o))
    return o


def last_error() -> str:
    return load_library().moe_last_error().decode()


def workspace_bytes(T, H, I, E, k, dtype=MOE_BF16, shared_I=0, flags=0, weight_layout=LAYOUT_ROWS) -> int:
    o = new_opts()
    o.dtype = dtype
    o.shared_I = shared_I
    o.flags = flags
    o.weight_layout = weight_layout
    n = load_library().moe_workspace_bytes(T, H, I, E, k, ctypes.byref(o))
    if n < 0:
        raise MoeError(int(n), last_error())
    return int(n)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def bf16_bits_to_tensor(a: np.ndarray, device="cuda"):
    """uint16 bf16 bit patterns (or float32) -> torch tensor on ``device``."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def quantize_fp8_rows(w, stream=None):
    """Per-row FP8 E4M3 quantisation of a contiguous bf16 CUDA tensor viewed
    as [rows, cols] (cols = last dimension): returns (q uint8 of w's shape,
    scale fp32 of w's leading shape) with w ~= e4m3(q) * scale."""
    import torch
    if w.dtype != torch.bfloat16 or not w.is_contiguous() or not w.is_cuda:
        raise ValueError("w must be a contiguous bf16 CUDA tensor")
    cols = w.shape[-1]
    rows = w.numel() // cols if cols else 0
    q = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    scale = torch.empty(w.shape[:-1], dtype=torch.float32, device=w.device)
    if stream is None:
        stream = torch.cuda.current_stream(w.device)
    rc = load_library().moe_quantize_fp8_rows(_ptr(w), rows, cols, _ptr(q), _ptr(scale),
                                              ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise MoeError(rc, last_error())
    return q, scale


class TileBlocks:
    """Routed expert weights in tile blocks (MOE_LAYOUT_TILE_BLOCKS), as
    ``pack_tile_blocks`` writes them: ``data`` is a flat bf16 CUDA tensor;
    ``which`` is PACK_GATE_UP (from gate_up [E, 2I, H]) or PACK_DOWN (from
    down [E, H, I])."""

    def __init__(self, data, which: int, E: int, I: int, H: int):
        self.data, self.which, self.E, self.I, self.H = data, which, E, I, H

    def data_ptr(self):
        return self.data.data_ptr()


def tile_blocks_bytes(which: int, E: int, I: int, H: int) -> int:
    n = load_library().moe_tile_blocks_bytes(int(which), E, I, H)
    if n < 0:
        raise MoeError(int(n), last_error())
    return int(n)


def pack_tile_blocks(w, which: int, stream=None) -> TileBlocks:
    """Routed expert weights from the nn.Linear layout into tile blocks:
    ``which`` PACK_GATE_UP takes gate_up [E, 2I, H], PACK_DOWN takes down
    [E, H, I] (contiguous bf16 CUDA tensors). Done once per weight set; the
    layer then reads them with ``moe_forward(..., gate_up=<TileBlocks>,
    down=<TileBlocks>)``."""
    import torch
    if w.dtype != torch.bfloat16 or not w.is_contiguous() or not w.is_cuda or w.dim() != 3:
        raise ValueError("w must be a contiguous 3-D bf16 CUDA tensor")
    if which == PACK_GATE_UP:
        E, twoI, H = w.shape
        I = twoI // 2
        if twoI != 2 * I:
            raise ValueError("gate_up must be [E, 2I, H]")
    elif which == PACK_DOWN:
        E, H, I = w.shape
    else:
        raise ValueError("which must be PACK_GATE_UP or PACK_DOWN")
    n = tile_blocks_bytes(which, E, I, H)
    out = torch.empty((n // 2,), dtype=torch.bfloat16, device=w.device)
    if stream is None:
        stream = torch.cuda.current_stream(w.device)
    rc = load_library().moe_pack_tile_blocks(int(which), _ptr(w), E, I, H, _ptr(out),
                                             ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise MoeError(rc, last_error())
    return TileBlocks(out, which, E, I, H)


def quantize_mxfp4_rows(w, stream=None):
    """MXFP4 quantisation (OCP MX: E2M1 codes, one E8M0 scale per 32
    consecutive elements of a row) of a contiguous bf16 CUDA tensor viewed as
    [rows, cols], cols a multiple of 32: returns (q uint8 [..., cols/2], two
    codes per byte, low nibble first; scale uint8 [..., cols/32])."""
    import torch
    if w.dtype != torch.bfloat16 or not w.is_contiguous() or not w.is_cuda:
        raise ValueError("w must be a contiguous bf16 CUDA tensor")
    cols = w.shape[-1]
    rows = w.numel() // cols if cols else 0
    q = torch.empty(w.shape[:-1] + (cols // 2,), dtype=torch.uint8, device=w.device)
    scale = torch.empty(w.shape[:-1] + (cols // 32,), dtype=torch.uint8, device=w.device)
    if stream is None:
        stream = torch.cuda.current_stream(w.device)
    rc = load_library().moe_quantize_mxfp4_rows(_ptr(w), rows, cols, _ptr(q), _ptr(scale),
                                                ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise MoeError(rc, last_error())
    return q, scale


def moe_forward(hidden, router_w, gate_up, down, k: int, *, routed_scale: float = 1.0, router_bias=None,
                shared_gate_up=None, shared_down=None, flags: int = 0, return_routing: bool = False,
                out=None, workspace=None, stream=None, stage_events=None, gate_up_scale=None, down_scale=None,
                router_stats: bool = False, stats_mask=None, score_func: str = "softmax",
                selection_bias=None, n_group: int = 0, topk_group: int = 0, jitter_eps: float | None = None,
                gate_up_block_scale=None, down_block_scale=None, no_alloc: bool = False):
    """Run the MoE layer on torch tensors already on the GPU.

    hidden [T, H], router_w [E, H], gate_up [E, 2I, H], down [E, H, I] (all
    bf16 or all fp32, contiguous); router_bias [E] fp32; shared_gate_up
    [2Is, H], shared_down [H, Is]. FP8 expert weights: gate_up and down as
    uint8 E4M3 codes with gate_up_scale [E, 2I] and down_scale [E, H] (fp32,
    from quantize_fp8_rows); activations bf16. MXFP4 expert weights: gate_up
    [E, 2I, H/2] and down [E, H, I/2] uint8 (two E2M1 codes per byte) with
    gate_up_block_scale [E, 2I, H/32] and down_block_scale [E, H, I/32] uint8
    (from quantize_mxfp4_rows). Tile-block expert weights: gate_up and down
    as ``TileBlocks`` from ``pack_tile_blocks`` (bf16; every batch runs on the
    tiled kernels). ``no_alloc`` calls moe_forward_noalloc: the
    library's own scratch instead of a workspace (``workspace`` must be None;
    pass ``out`` so that nothing is allocated here either). ``router_stats`` adds the
    load-balancing statistics (prob_mean [E], load [E], aux_loss [1]) to the
    routing dict, over the tokens with ``stats_mask`` != 0 (int32 [T]; all
    tokens if None). ``score_func`` "sigmoid" scores experts by the sigmoid of
    their logits and weights them by the selected scores over their sum;
    ``selection_bias`` [E] fp32 is added to the scores for selection only;
    ``n_group`` > 1 with ``topk_group`` limits selection to the best
    topk_group of n_group equal expert groups. ``score_func`` "sparsemixer"
    is PhiMoE's router at inference: greedy by logit, each round's weight a
    softmax over the unchosen experts within the relative threshold
    2 * ``jitter_eps`` (default 0.01) of that round's winner. Returns out [T, H] (and a dict of routing tensors when
    ``return_routing`` or ``router_stats``). Work is enqueued on ``stream``
    (default: torch's current stream)."""
    import torch
    lib = load_library()
    T, H = hidden.shape
    blocks = isinstance(gate_up, TileBlocks)
    if blocks != isinstance(down, TileBlocks):
        raise ValueError("gate_up and down must both be TileBlocks or both tensors")
    if blocks:
        if (gate_up.which, down.which) != (PACK_GATE_UP, PACK_DOWN) or \
                (gate_up.E, gate_up.I, gate_up.H) != (down.E, down.I, down.H) or gate_up.H != H:
            raise ValueError("tile blocks: gate_up and down of one [E, I, H] weight set, H of hidden")
        E, I = gate_up.E, gate_up.I
        gu_shape, dn_shape = (E, 2 * I, H), (E, H, I)
        gate_up, down = gate_up.data, down.data
    else:
        E, twoI, _ = gate_up.shape
        I = twoI // 2
        gu_shape, dn_shape = tuple(gate_up.shape), tuple(down.shape)
    o = new_opts()
    if blocks:
        o.weight_layout = LAYOUT_TILE_BLOCKS
    if hidden.dtype == torch.bfloat16:
        o.dtype = MOE_BF16
    elif hidden.dtype == torch.float32:
        o.dtype = MOE_F32
    else:
        raise TypeError(f"unsupported dtype {hidden.dtype}")
    lowp = gate_up.dtype == torch.uint8  # FP8 or MXFP4 expert weights
    w4 = lowp and gate_up_block_scale is not None
    if lowp and not w4:
        if down.dtype != torch.uint8 or gate_up_scale is None or down_scale is None:
            raise ValueError("FP8 weights need uint8 gate_up and down plus gate_up_scale and down_scale")
        gate_up_scale = gate_up_scale.to(device=hidden.device, dtype=torch.float32).contiguous()
        down_scale = down_scale.to(device=hidden.device, dtype=torch.float32).contiguous()
        if gate_up_scale.shape != (E, 2 * I) or down_scale.shape != (E, H):
            raise ValueError("gate_up_scale must be [E, 2I] and down_scale [E, H]")
        o.weight_format = WEIGHTS_FP8_E4M3
        o.gate_up_scale = gate_up_scale.data_ptr()
        o.down_scale = down_scale.data_ptr()
    if w4:
        if down.dtype != torch.uint8 or down_block_scale is None:
            raise ValueError("MXFP4 weights need uint8 gate_up and down plus both block scales")
        gate_up_block_scale = gate_up_block_scale.to(device=hidden.device, dtype=torch.uint8).contiguous()
        down_block_scale = down_block_scale.to(device=hidden.device, dtype=torch.uint8).contiguous()
        if gate_up_block_scale.shape != (E, 2 * I, H // 32) or down_block_scale.shape != (E, H, I // 32):
            raise ValueError("block scales must be [E, 2I, H/32] and [E, H, I/32]")
        o.weight_format = WEIGHTS_MXFP4
        o.gate_up_block_scale = gate_up_block_scale.data_ptr()
        o.down_block_scale = down_block_scale.data_ptr()
    acts = [hidden, router_w] + [t for t in (shared_gate_up, shared_down) if t is not None]
    acts += [] if lowp else [gate_up, down]
    for t in acts + ([gate_up, down] if lowp else []):
        if not t.is_contiguous() or not t.is_cuda:
            raise ValueError("all tensors must be contiguous CUDA tensors")
    for t in acts:
        if t.dtype != hidden.dtype:
            raise ValueError("activations, router and native-format weights must share one dtype")
    wcols = 2 if w4 else 1  # MXFP4: two codes per byte
    if router_w.shape != (E, H) or gu_shape != (E, 2 * I, H // wcols) or \
            dn_shape != (E, H, I // wcols) or (w4 and (H % 32 or I % 32)):
        raise ValueError("shape mismatch among hidden, router_w, gate_up, down")
    o.routed_scale = float(routed_scale)
    o.flags = int(flags)
    funcs = {"softmax": SCORE_SOFTMAX, "sigmoid": SCORE_SIGMOID, "sparsemixer": SCORE_SPARSEMIXER}
    if score_func not in funcs:
        raise ValueError(f"score_func must be one of {sorted(funcs)}")
    o.score_func = funcs[score_func]
    if selection_bias is not None:
        selection_bias = selection_bias.to(device=hidden.device, dtype=torch.float32).contiguous()
        if selection_bias.shape != (E,):
            raise ValueError("selection_bias must be [E]")
        o.selection_bias = selection_bias.data_ptr()
    o.n_group = int(n_group)
    o.topk_group = int(topk_group)
    if jitter_eps is not None:
        o.jitter_eps = float(jitter_eps)
    if router_bias is not None:
        router_bias = router_bias.to(device=hidden.device, dtype=torch.float32).contiguous()
        if router_bias.shape != (E,):
            raise ValueError("router_bias must be [E]")
        o.router_bias = router_bias.data_ptr()
    if shared_gate_up is not None:
        Is = shared_gate_up.shape[0] // 2
        if shared_gate_up.shape != (2 * Is, H) or shared_down is None or shared_down.shape != (H, Is):
            raise ValueError("shared expert shapes must be [2Is, H] and [H, Is]")
        o.shared_gate_up = shared_gate_up.data_ptr()
        o.shared_down = shared_down.data_ptr()
        o.shared_I = Is
    dev = hidden.device
    if out is None:
        out = torch.empty((T, H), dtype=hidden.dtype, device=dev)
    elif out.shape != (T, H) or out.dtype != hidden.dtype or not out.is_contiguous() or not out.is_cuda:
        raise ValueError("out must be a contiguous CUDA tensor of hidden's dtype and shape [T, H]")
    routing = None
    return_routing = return_routing or router_stats
    if return_routing:
        routing = dict(
            logits=torch.empty((T, E), dtype=torch.float32, device=dev),
            ids=torch.empty((T, k), dtype=torch.int32, device=dev),
            weights=torch.empty((T, k), dtype=torch.float32, device=dev),
            counts=torch.empty((E,), dtype=torch.int32, device=dev),
            offsets=torch.empty((E + 1,), dtype=torch.int32, device=dev),
            perm=torch.empty((T * k,), dtype=torch.int32, device=dev),
            inv=torch.empty((T * k,), dtype=torch.int32, device=dev),
        )
        o.router_logits = routing["logits"].data_ptr()
        o.topk_ids = routing["ids"].data_ptr()
        o.topk_weights = routing["weights"].data_ptr()
        o.expert_counts = routing["counts"].data_ptr()
        o.expert_offsets = routing["offsets"].data_ptr()
        o.perm = routing["perm"].data_ptr()
        o.inv_perm = routing["inv"].data_ptr()
    if router_stats:
        routing["prob_mean"] = torch.empty((E,), dtype=torch.float32, device=dev)
        routing["load"] = torch.empty((E,), dtype=torch.float32, device=dev)
        routing["aux_loss"] = torch.empty((1,), dtype=torch.float32, device=dev)
        o.router_prob_mean = routing["prob_mean"].data_ptr()
        o.expert_load = routing["load"].data_ptr()
        o.aux_loss = routing["aux_loss"].data_ptr()
        if stats_mask is not None:
            stats_mask = stats_mask.to(device=dev, dtype=torch.int32).contiguous()
            if stats_mask.shape != (T,):
                raise ValueError("stats_mask must be [T]")
            o.stats_mask = stats_mask.data_ptr()
    need = lib.moe_workspace_bytes(T, H, I, E, k, ctypes.byref(o))
    if need < 0:
        raise MoeError(int(need), last_error())
    if no_alloc:
        if workspace is not None:
            raise ValueError("no_alloc uses the library's scratch: pass no workspace")
    elif workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    elif workspace.numel() * workspace.element_size() < need or not workspace.is_cuda:
        # a caller that passes a workspace relies on the call allocating nothing
        raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} bytes; "
                         f"{need} are needed (workspace_bytes with the same flags and dtype)")
    if not no_alloc:
        o.workspace = workspace.data_ptr()
        o.workspace_bytes = workspace.numel() * workspace.element_size()
    current = torch.cuda.current_stream(dev)
    if stream is None:
        stream = current
    if stream != current:
        # buffers allocated here belong to the current stream's pool
        for t in (router_bias, workspace, out, gate_up_scale, down_scale, stats_mask, selection_bias,
                  gate_up_block_scale, down_block_scale,
                  *(routing.values() if routing else ())):
            if t is not None:
                t.record_stream(stream)
    o.stream = stream.cuda_stream
    if stage_events is not None:
        o.stage_events = ctypes.cast(stage_events, ctypes.c_void_p)
    fn = lib.moe_forward_noalloc if no_alloc else lib.moe_forward
    rc = fn(_ptr(hidden), _ptr(router_w), _ptr(gate_up), _ptr(down), T, H, I, E, int(k), ctypes.byref(o), _ptr(out))
    if rc != 0:
        raise MoeError(rc, last_error())
    if return_routing:
        return out, routing
    return out
