"""Python binding of libmoe_fp4.so, the MI355X (gfx950) routed-MoE FFN layer
with block-scaled FP4 experts and sqrtsoftplus routing.

Thin ctypes marshalling over the C ABI in include/moe_fp4.h: tensors are
torch tensors on the GPU (torch supplies device memory and the current
stream); every step of the layer runs in the library's HIP kernels.  There is
no fallback: if the library is missing, importing this package raises.

Entry points mirror the C names: quant_act, route, expert_ffn, layer
(plus workspace_size and the Layer helper that keeps one workspace).
"""

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_fp4.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python block_scaled_fp4_sqrtsoftplus_amd/build.py` "
        "(hipcc, gfx950); this package has no non-HIP fallback")

lib = ctypes.CDLL(LIB_PATH)

MOE_OK = 0
STATUS_NAMES = ["MOE_OK", "MOE_ERR_NULL_ARG", "MOE_ERR_BAD_SHAPE", "MOE_ERR_MISALIGNED",
                "MOE_ERR_WORKSPACE_TOO_SMALL", "MOE_ERR_UNSUPPORTED", "MOE_ERR_ARCH", "MOE_ERR_HIP",
                "MOE_ERR_SCRATCH_TOO_SMALL"]
ROUTE_SQRTSOFTPLUS, ROUTE_HASH = 0, 1
EXPERTS_MXFP4, EXPERTS_FP8, EXPERTS_NVFP4, EXPERTS_W4AFP8 = 0, 1, 2, 3
OP_ROUTE, OP_EXPERT_FFN, OP_LAYER = 0, 1, 2


class MoeConfigC(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int64), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("route_scale", ctypes.c_float), ("swiglu_limit", ctypes.c_float),
                ("route_mode", ctypes.c_int32), ("out_fp32", ctypes.c_int32),
                ("hash_seed", ctypes.c_uint64), ("expert_format", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class MoeExpertWeightsC(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w1", "w1_scale", "w3", "w3_scale", "w2", "w2_scale")]


class MoeSharedWeightsC(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w1", "w3", "w2")]


class MoeRoutingC(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("topk_idx", "topk_w", "expert_offsets", "sorted_pairs", "pair_pos")]


_vp, _sz, _i64, _i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64, ctypes.c_int32
lib.moe_status_str.restype = ctypes.c_char_p
lib.moe_status_str.argtypes = [ctypes.c_int]
lib.moe_workspace_size.restype = _sz
lib.moe_workspace_size.argtypes = [ctypes.POINTER(MoeConfigC), ctypes.c_int]
lib.moe_quant_act.restype = ctypes.c_int
lib.moe_quant_act.argtypes = [_vp, _i64, _i32, _vp, _vp, _vp]
lib.moe_route.restype = ctypes.c_int
lib.moe_route.argtypes = [ctypes.POINTER(MoeConfigC), _vp, _vp, _vp, _vp, _vp, _vp,
                          ctypes.POINTER(MoeRoutingC), _vp, _sz, _vp]
lib.moe_expert_ffn.restype = ctypes.c_int
lib.moe_expert_ffn.argtypes = [ctypes.POINTER(MoeConfigC), _vp, _vp, ctypes.POINTER(MoeRoutingC),
                               ctypes.POINTER(MoeExpertWeightsC), _vp, _vp, _vp, _vp, _sz, _vp]
lib.moe_layer.restype = ctypes.c_int
lib.moe_layer.argtypes = [ctypes.POINTER(MoeConfigC), _vp, _vp, _vp, _vp,
                          ctypes.POINTER(MoeExpertWeightsC), ctypes.POINTER(MoeSharedWeightsC), _vp,
                          ctypes.POINTER(MoeRoutingC), _vp, _sz, _vp]
lib.moe_expert_cast_fp8.restype = ctypes.c_int
lib.moe_expert_cast_fp8.argtypes = [ctypes.POINTER(MoeConfigC), ctypes.POINTER(MoeExpertWeightsC),
                                    ctypes.POINTER(MoeExpertWeightsC), _vp]
lib.moe_layer_graph_create.restype = ctypes.c_int
lib.moe_layer_graph_create.argtypes = [ctypes.POINTER(MoeConfigC), _vp, _vp, _vp, _vp,
                                       ctypes.POINTER(MoeExpertWeightsC),
                                       ctypes.POINTER(MoeSharedWeightsC), _vp,
                                       ctypes.POINTER(MoeRoutingC), _vp, _sz,
                                       ctypes.POINTER(_vp)]
lib.moe_graph_launch.restype = ctypes.c_int
lib.moe_graph_launch.argtypes = [_vp, _vp]
lib.moe_graph_destroy.restype = ctypes.c_int
lib.moe_graph_destroy.argtypes = [_vp]
lib.moe_layer_noalloc.restype = ctypes.c_int
lib.moe_layer_noalloc.argtypes = [ctypes.POINTER(MoeConfigC), _vp, _vp, _vp, _vp,
                                  ctypes.POINTER(MoeExpertWeightsC), ctypes.POINTER(MoeSharedWeightsC),
                                  _vp, ctypes.POINTER(MoeRoutingC), _vp]
NOALLOC_SCRATCH_BYTES = 64 << 20    # MOE_NOALLOC_SCRATCH_BYTES


class MoeError(RuntimeError):
    def __init__(self, status):
        self.status = status
        super().__init__(lib.moe_status_str(status).decode())


def _check(status):
    if status != MOE_OK:
        raise MoeError(status)


@dataclass
class Config:
    tokens: int
    hidden: int
    inter: int
    n_experts: int
    top_k: int
    route_scale: float = 1.5
    swiglu_limit: float = 10.0
    route_mode: int = ROUTE_SQRTSOFTPLUS
    out_fp32: int = 1
    hash_seed: int = 0
    expert_format: int = 0          # EXPERTS_MXFP4, EXPERTS_FP8, EXPERTS_NVFP4 or EXPERTS_W4AFP8

    def c(self):
        return MoeConfigC(self.tokens, self.hidden, self.inter, self.n_experts, self.top_k,
                          self.route_scale, self.swiglu_limit, self.route_mode, self.out_fp32,
                          self.hash_seed & ((1 << 64) - 1), self.expert_format, 0)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to the HIP library must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the HIP library must be contiguous")
    if t.numel() == 0:
        # an empty view still points into its storage (NULL only if that is empty too)
        return t.untyped_storage().data_ptr() + t.storage_offset() * t.element_size() or None
    return t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def workspace_size(cfg: Config, op: int) -> int:
    c = cfg.c()
    return lib.moe_workspace_size(ctypes.byref(c), op)


def _workspace(cfg, op, device):
    n = workspace_size(cfg, op)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device), n


def _routing_tensors(T, k, E, device):
    # at least one element each, so that T == 0 still passes valid pointers
    P = T * k
    n = max(P, 1)
    return {
        "topk_idx": torch.empty(n, dtype=torch.int32, device=device)[:P].view(T, k),
        "topk_w": torch.empty(n, dtype=torch.float32, device=device)[:P].view(T, k),
        "expert_offsets": torch.empty(E + 1, dtype=torch.int32, device=device),
        "sorted_pairs": torch.empty(n, dtype=torch.int32, device=device)[:P],
        "pair_pos": torch.empty(n, dtype=torch.int32, device=device)[:P],
    }


def _routing_c(r):
    return MoeRoutingC(*(_ptr(r[n]) for n in ("topk_idx", "topk_w", "expert_offsets", "sorted_pairs", "pair_pos")))


def _weights_c(w):
    return MoeExpertWeightsC(*(_ptr(w[n]) for n in ("w1", "w1_scale", "w3", "w3_scale", "w2", "w2_scale")))


def _as_bits(t):
    return t.view(torch.int16) if t is not None and t.dtype == torch.bfloat16 else t


def quant_act(x):
    """x [rows, cols] bf16 -> (q [rows, cols] uint8 E4M3, scale [rows, cols/128] uint8 E8M0)."""
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    s = torch.empty((rows, cols // 128), dtype=torch.uint8, device=x.device)
    _check(lib.moe_quant_act(_ptr(x), rows, cols, _ptr(q), _ptr(s), _stream()))
    return q, s


def route(cfg: Config, x=None, w_gate=None, bias=None, token_ids=None, logits_in=None,
          want_logits=False, device=None):
    """Routing of cfg.tokens tokens; returns dict of routing tensors (+ 'logits')."""
    device = device or next(t.device for t in (x, token_ids, logits_in) if t is not None)
    r = _routing_tensors(cfg.tokens, cfg.top_k, cfg.n_experts, device)
    logits = None
    if want_logits and cfg.route_mode == ROUTE_SQRTSOFTPLUS:
        logits = torch.empty((cfg.tokens, cfg.n_experts), dtype=torch.float32, device=device)
    ws, n = _workspace(cfg, OP_ROUTE, device)
    c, rc = cfg.c(), _routing_c(r)
    _check(lib.moe_route(ctypes.byref(c), _ptr(x), _ptr(w_gate), _ptr(bias), _ptr(token_ids),
                         _ptr(logits_in), _ptr(logits), ctypes.byref(rc), _ptr(ws), n, _stream()))
    if logits is not None:
        r["logits"] = logits
    return r


def expert_ffn(cfg: Config, xq, xs, routing, weights, want_h=False):
    """Routed experts: returns dict with 'out' [P, H] (fp32 or bf16 per
    cfg.out_fp32, rows in sorted-pair order) and optionally 'hq', 'hs'."""
    P = cfg.tokens * cfg.top_k
    dev = xq.device
    out = torch.empty((P, cfg.hidden), dtype=torch.float32 if cfg.out_fp32 else torch.bfloat16, device=dev)
    hq = hs = None
    if want_h:
        hq = torch.empty((P, cfg.inter), dtype=torch.uint8, device=dev)
        hs = torch.empty((P, cfg.inter // 128), dtype=torch.uint8, device=dev)
    ws, n = _workspace(cfg, OP_EXPERT_FFN, dev)
    c, rc, wc = cfg.c(), _routing_c(routing), _weights_c(weights)
    _check(lib.moe_expert_ffn(ctypes.byref(c), _ptr(xq), _ptr(xs), ctypes.byref(rc), ctypes.byref(wc),
                              _ptr(out), _ptr(hq), _ptr(hs), _ptr(ws), n, _stream()))
    res = {"out": out}
    if want_h:
        res.update(hq=hq, hs=hs)
    return res


def expert_cast_fp8(cfg: Config, weights):
    """MXFP4 expert weights -> FP8 expert weights (moe_expert_cast_fp8):
    returns a dict with w1, w3 [E, I, H], w2 [E, H, I] E4M3 bytes and their
    per-128 E8M0 scales."""
    E, H, I = cfg.n_experts, cfg.hidden, cfg.inter
    dev = weights["w1"].device
    u8 = dict(dtype=torch.uint8, device=dev)
    out = {"w1": torch.empty((E, I, H), **u8), "w1_scale": torch.empty((E, I, H // 128), **u8),
           "w3": torch.empty((E, I, H), **u8), "w3_scale": torch.empty((E, I, H // 128), **u8),
           "w2": torch.empty((E, H, I), **u8), "w2_scale": torch.empty((E, H, I // 128), **u8)}
    c = cfg.c()
    _check(lib.moe_expert_cast_fp8(ctypes.byref(c), ctypes.byref(_weights_c(weights)),
                                   ctypes.byref(_weights_c(out)), _stream()))
    return out


class Layer:
    """Holds a config, its workspace and the weight pointers, and runs the
    whole layer (moe_layer) on the current stream."""

    def __init__(self, cfg: Config, weights, w_gate=None, bias=None, shared=None, device=None):
        self.cfg = cfg
        self.device = device or weights["w1"].device
        self.weights = weights
        self.w_gate, self.bias, self.shared = w_gate, bias, shared
        self._c = cfg.c()
        self._wc = _weights_c(weights)
        self._sc = MoeSharedWeightsC(*(_ptr(shared[n]) for n in ("w1", "w3", "w2"))) if shared else None
        self.ws, self.ws_bytes = _workspace(cfg, OP_LAYER, self.device)

    def __call__(self, x, token_ids=None, y=None, routing=None):
        if y is None:
            y = torch.empty((self.cfg.tokens, self.cfg.hidden), dtype=torch.bfloat16, device=self.device)
        rc = _routing_c(routing) if routing is not None else None
        _check(lib.moe_layer(ctypes.byref(self._c), _ptr(x), _ptr(self.w_gate), _ptr(self.bias),
                             _ptr(token_ids), ctypes.byref(self._wc),
                             ctypes.byref(self._sc) if self._sc is not None else None,
                             _ptr(y), ctypes.byref(rc) if rc is not None else None,
                             _ptr(self.ws), self.ws_bytes, _stream()))
        return y


class LayerGraph:
    """One moe_layer call recorded into a HIP graph (moe_layer_graph_create)
    with fixed buffers: update x (and token_ids) in place, then launch();
    y and the routing arrays receive the results.  Holds references to every
    buffer the graph reads or writes."""

    def __init__(self, layer: "Layer", x, token_ids=None, y=None, routing=None):
        cfg = layer.cfg
        if y is None:
            y = torch.empty((cfg.tokens, cfg.hidden), dtype=torch.bfloat16, device=layer.device)
        self.layer, self.x, self.token_ids, self.y, self.routing = layer, x, token_ids, y, routing
        rc = _routing_c(routing) if routing is not None else None
        h = _vp()
        _check(lib.moe_layer_graph_create(
            ctypes.byref(layer._c), _ptr(x), _ptr(layer.w_gate), _ptr(layer.bias), _ptr(token_ids),
            ctypes.byref(layer._wc), ctypes.byref(layer._sc) if layer._sc is not None else None,
            _ptr(y), ctypes.byref(rc) if rc is not None else None, _ptr(layer.ws), layer.ws_bytes,
            ctypes.byref(h)))
        self._h = h

    def launch(self):
        _check(lib.moe_graph_launch(self._h, _stream()))
        return self.y

    def close(self):
        if self._h:
            _check(lib.moe_graph_destroy(self._h))
            self._h = _vp()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def layer_noalloc(cfg: Config, x, weights, y, w_gate=None, bias=None, token_ids=None, shared=None,
                  routing=None):
    """moe_layer_noalloc: the whole layer on the library's static device
    scratch (no workspace, nothing allocated by the call); y [T, H] bf16 and
    the optional routing arrays are the caller's."""
    c = cfg.c()
    wc = _weights_c(weights)
    sc = MoeSharedWeightsC(*(_ptr(shared[n]) for n in ("w1", "w3", "w2"))) if shared else None
    rc = _routing_c(routing) if routing is not None else None
    _check(lib.moe_layer_noalloc(ctypes.byref(c), _ptr(x), _ptr(w_gate), _ptr(bias), _ptr(token_ids),
                                 ctypes.byref(wc), ctypes.byref(sc) if sc is not None else None,
                                 _ptr(y), ctypes.byref(rc) if rc is not None else None, _stream()))
    return y


def layer(cfg: Config, x, weights, w_gate=None, bias=None, token_ids=None, shared=None,
          want_routing=False):
    """One call of the whole layer; returns y [T, H] bf16 (and the routing)."""
    L = Layer(cfg, weights, w_gate, bias, shared, x.device)
    routing = _routing_tensors(cfg.tokens, cfg.top_k, cfg.n_experts, x.device) if want_routing else None
    y = L(x, token_ids, routing=routing)
    return (y, routing) if want_routing else y
