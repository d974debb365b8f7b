"""The C-ABI library on a host without a GPU: it loads, exports every entry
point include/moe_fp4.h declares, sizes workspaces, and rejects invalid
arguments with the documented status codes before making any HIP call."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_fp4.h")

moe = pytest.importorskip("block_scaled_fp4_sqrtsoftplus_amd",
                          reason="libmoe_fp4.so not built (run __graft_entry__.build())")
lib = moe.lib
C = moe.MoeConfigC


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:const char\*|size_t|moe_status)\s+(moe_\w+)\(", src, re.M)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert set(names) == {"moe_status_str", "moe_workspace_size", "moe_quant_act", "moe_route",
                          "moe_expert_ffn", "moe_layer", "moe_layer_graph_create",
                          "moe_graph_launch", "moe_graph_destroy", "moe_expert_cast_fp8",
                          "moe_layer_noalloc"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for i, name in enumerate(moe.STATUS_NAMES):
        assert lib.moe_status_str(i).decode().startswith(name)
    assert lib.moe_status_str(99)


def _cfg(**kw):
    d = dict(tokens=64, hidden=4096, inter=2048, n_experts=256, top_k=6, route_scale=1.5,
             swiglu_limit=10.0, route_mode=0, out_fp32=1, hash_seed=0)
    d.update(kw)
    return C(**d)


def test_workspace_sizes():
    c = _cfg()
    P, T, H, I, E = 384, 64, 4096, 2048, 256
    lay = lib.moe_workspace_size(ctypes.byref(c), moe.OP_LAYER)
    ffn = lib.moe_workspace_size(ctypes.byref(c), moe.OP_EXPERT_FFN)
    rt = lib.moe_workspace_size(ctypes.byref(c), moe.OP_ROUTE)
    assert ffn >= P * I + P * I // 128
    assert lay >= ffn + rt + P * H * 4 + T * H + T * I * 2 + T * H * 4
    assert rt >= T * E * 4
    assert lib.moe_workspace_size(None, moe.OP_LAYER) == 0
    bad = _cfg(hidden=100)
    assert lib.moe_workspace_size(ctypes.byref(bad), moe.OP_LAYER) == 0
    assert lib.moe_workspace_size(ctypes.byref(c), 7) == 0


def test_layer_workspace_holds_shared_split_partials():
    # decode-sized batches (T <= 64, H and I multiples of 512) add the shared
    # expert's split-K partial sums: max(H/512 * T * 2I, I/512 * T * H) floats
    base = dict(n_experts=8, top_k=2)
    for T, H, I in [(64, 4096, 2048), (1, 2048, 512), (37, 1024, 1536)]:
        with_part = lib.moe_workspace_size(ctypes.byref(_cfg(tokens=T, hidden=H, inter=I, **base)),
                                           moe.OP_LAYER)
        # the same sizes with I = 384 (not a multiple of 512) carve no partials
        no_part = lib.moe_workspace_size(ctypes.byref(_cfg(tokens=T, hidden=H, inter=I - 128, **base)),
                                         moe.OP_LAYER)
        part = max(H // 512 * T * 2 * I, I // 512 * T * H) * 4
        assert with_part >= part
        assert with_part - no_part >= part - 256 * 64   # I - 128 shrinks the other buffers a little
    # 65 tokens: the side-stream kernels, no partials
    a = lib.moe_workspace_size(ctypes.byref(_cfg(tokens=65, **base)), moe.OP_LAYER)
    b = lib.moe_workspace_size(ctypes.byref(_cfg(tokens=65, inter=1920, **base)), moe.OP_LAYER)
    assert a - b < 8 * 64 * 4096 * 4


@pytest.mark.parametrize("field,value", [
    ("tokens", -1), ("hidden", 0), ("hidden", 200), ("hidden", 32768), ("inter", 64),
    ("n_experts", 0), ("n_experts", 513), ("top_k", 0), ("top_k", 9), ("route_mode", 3),
    ("swiglu_limit", 0.0), ("swiglu_limit", float("nan")), ("route_scale", float("inf")),
    ("tokens", 1 << 29),  # tokens * top_k overflows int32
])
def test_bad_config_rejected(field, value):
    c = _cfg(**{field: value})
    st = lib.moe_layer(ctypes.byref(c), 16, 16, None, None, None, None, 16, None, None, 0, None)
    assert st == 2  # MOE_ERR_BAD_SHAPE
    ws = moe.MoeRoutingC(16, 16, 16, 16, 16)
    st = lib.moe_route(ctypes.byref(c), 16, 16, None, None, None, None, ctypes.byref(ws), 16, 1 << 40, None)
    assert st == 2


def _w(**kw):
    d = dict(w1=16, w1_scale=16, w3=16, w3_scale=16, w2=16, w2_scale=16)
    d.update(kw)
    return moe.MoeExpertWeightsC(**d)


def test_layer_argument_errors():
    c = _cfg()
    big = 1 << 40
    w = _w()
    # NULL weights / x / y / gate
    assert lib.moe_layer(ctypes.byref(c), 16, 16, None, None, None, None, 16, None, 16, big, None) == 1
    assert lib.moe_layer(ctypes.byref(c), 16, 16, None, None, ctypes.byref(_w(w2=None)), None, 16, None, 16, big, None) == 1
    assert lib.moe_layer(ctypes.byref(c), None, 16, None, None, ctypes.byref(w), None, 16, None, 16, big, None) == 1
    assert lib.moe_layer(ctypes.byref(c), 16, None, None, None, ctypes.byref(w), None, 16, None, 16, big, None) == 1
    # hash mode needs token ids, not the gate
    h = _cfg(route_mode=1)
    assert lib.moe_layer(ctypes.byref(h), 16, None, None, None, ctypes.byref(w), None, 16, None, 16, big, None) == 1
    # misaligned pointers
    assert lib.moe_layer(ctypes.byref(c), 18, 16, None, None, ctypes.byref(w), None, 16, None, 16, big, None) == 3
    assert lib.moe_layer(ctypes.byref(c), 16, 16, None, None, ctypes.byref(_w(w3_scale=17)), None, 16, None, 16, big, None) == 3
    # workspace too small
    need = lib.moe_workspace_size(ctypes.byref(c), moe.OP_LAYER)
    assert lib.moe_layer(ctypes.byref(c), 16, 16, None, None, ctypes.byref(w), None, 16, None, 16, need - 1, None) == 4
    # shared expert with a NULL part
    sh = moe.MoeSharedWeightsC(16, None, 16)
    assert lib.moe_layer(ctypes.byref(c), 16, 16, None, None, ctypes.byref(w), ctypes.byref(sh), 16, None, 16, big, None) == 1
    # incomplete routing_out
    r = moe.MoeRoutingC(16, 16, None, 16, 16)
    assert lib.moe_layer(ctypes.byref(c), 16, 16, None, None, ctypes.byref(w), None, 16, ctypes.byref(r), 16, big, None) == 1


def test_graph_argument_errors():
    c = _cfg()
    big = 1 << 40
    w = _w()
    h = ctypes.c_void_p(12345)
    # no place for the handle
    assert lib.moe_layer_graph_create(ctypes.byref(c), 16, 16, None, None, ctypes.byref(w), None, 16,
                                      None, 16, big, None) == 1
    # the layer's own argument errors, before any HIP call; the handle is cleared
    assert lib.moe_layer_graph_create(ctypes.byref(c), None, 16, None, None, ctypes.byref(w), None,
                                      16, None, 16, big, ctypes.byref(h)) == 1
    assert not h.value
    assert lib.moe_layer_graph_create(ctypes.byref(c), 18, 16, None, None, ctypes.byref(w), None,
                                      16, None, 16, big, ctypes.byref(h)) == 3
    need = lib.moe_workspace_size(ctypes.byref(c), moe.OP_LAYER)
    assert lib.moe_layer_graph_create(ctypes.byref(c), 16, 16, None, None, ctypes.byref(w), None,
                                      16, None, 16, need - 1, ctypes.byref(h)) == 4
    assert lib.moe_graph_launch(None, None) == 1
    assert lib.moe_graph_destroy(None) == 0


def test_expert_format_and_cast_argument_errors():
    c = _cfg()
    c.expert_format = 4
    assert lib.moe_workspace_size(ctypes.byref(c), moe.OP_LAYER) == 0
    assert lib.moe_layer(ctypes.byref(c), 16, 16, None, None, ctypes.byref(_w()), None, 16, None, 16,
                         1 << 40, None) == 2
    c.expert_format = 1
    assert lib.moe_workspace_size(ctypes.byref(c), moe.OP_LAYER) > 0
    # NVFP4 experts need K % 512 == 0 for both GEMMs
    n = _cfg(hidden=4096, inter=384)
    n.expert_format = 2
    assert lib.moe_layer(ctypes.byref(n), 16, 16, None, None, ctypes.byref(_w()), None, 16, None, 16,
                         1 << 40, None) == 5
    n.inter = 512
    assert lib.moe_workspace_size(ctypes.byref(n), moe.OP_LAYER) > 0
    # and so do W4AFP8 experts
    n = _cfg(hidden=640, inter=512)
    n.expert_format = moe.EXPERTS_W4AFP8
    assert lib.moe_layer(ctypes.byref(n), 16, 16, None, None, ctypes.byref(_w()), None, 16, None, 16,
                         1 << 40, None) == 5
    n.hidden = 1024
    assert lib.moe_workspace_size(ctypes.byref(n), moe.OP_LAYER) > 0
    # cast: NULL / misaligned source or destination arrays
    assert lib.moe_expert_cast_fp8(ctypes.byref(c), None, ctypes.byref(_w()), None) == 1
    assert lib.moe_expert_cast_fp8(ctypes.byref(c), ctypes.byref(_w()), ctypes.byref(_w(w2=None)), None) == 1
    assert lib.moe_expert_cast_fp8(ctypes.byref(c), ctypes.byref(_w(w1_scale=20)), ctypes.byref(_w()), None) == 3


def test_quant_act_argument_errors():
    assert lib.moe_quant_act(16, 4, 100, 16, 16, None) == 2
    assert lib.moe_quant_act(16, -1, 128, 16, 16, None) == 2
    assert lib.moe_quant_act(None, 4, 128, 16, 16, None) == 1
    assert lib.moe_quant_act(18, 4, 128, 16, 16, None) == 3
    assert lib.moe_quant_act(None, 0, 128, None, None, None) == 0   # empty: nothing to do


def test_expert_ffn_argument_errors():
    c = _cfg()
    big = 1 << 40
    r = moe.MoeRoutingC(None, None, 16, 16, None)       # only offsets and sorted pairs are read
    w = _w()
    assert lib.moe_expert_ffn(ctypes.byref(c), 16, 16, ctypes.byref(r), ctypes.byref(w), None, None, None, 16, big, None) == 1
    assert lib.moe_expert_ffn(ctypes.byref(c), 16, 16, ctypes.byref(r), ctypes.byref(w), 16, 16, None, 16, big, None) == 1
    assert lib.moe_expert_ffn(ctypes.byref(c), 16, 24, ctypes.byref(r), ctypes.byref(w), 16, None, None, 16, big, None) == 3
    need = lib.moe_workspace_size(ctypes.byref(c), moe.OP_EXPERT_FFN)
    assert lib.moe_expert_ffn(ctypes.byref(c), 16, 16, ctypes.byref(r), ctypes.byref(w), 16, None, None, 16, need - 1, None) == 4


def test_noalloc_rejects_beyond_scratch():
    # moe_layer_noalloc refuses a call whose workspace exceeds its static
    # scratch before any HIP call (4096 tokens of the V4-Flash layer need
    # ~0.5 GB), and checks its arguments like moe_layer
    big = _cfg(tokens=4096)
    assert lib.moe_workspace_size(ctypes.byref(big), moe.OP_LAYER) > moe.NOALLOC_SCRATCH_BYTES
    w = moe.MoeExpertWeightsC(*([16] * 6))
    st = lib.moe_layer_noalloc(ctypes.byref(big), 16, 16, None, None, ctypes.byref(w), None, 16,
                               None, None)
    assert moe.STATUS_NAMES[st] == "MOE_ERR_SCRATCH_TOO_SMALL"
    small = _cfg(tokens=64)
    assert lib.moe_workspace_size(ctypes.byref(small), moe.OP_LAYER) <= moe.NOALLOC_SCRATCH_BYTES
    assert lib.moe_layer_noalloc(ctypes.byref(small), None, 16, None, None, ctypes.byref(w), None,
                                 16, None, None) == 1          # x NULL
    assert lib.moe_layer_noalloc(ctypes.byref(small), 8, 16, None, None, ctypes.byref(w), None,
                                 16, None, None) == 3          # x misaligned
    bad = _cfg(hidden=100)
    assert lib.moe_layer_noalloc(ctypes.byref(bad), 16, 16, None, None, ctypes.byref(w), None,
                                 16, None, None) == 2
