"""The C ABI of include/moe.h without a GPU: the library loads, exports what the header declares, sizes
workspaces, and rejects bad arguments on the host before any launch (no device work is needed for that).
"""
import ctypes
import os
import re

import pytest

from sparse_mixture_experts_08_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="libmoe.so not built")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert _declared_functions() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol():
    # RTLD_NOW: every symbol the library needs (kernel launch stubs included) must resolve at load
    L = ctypes.CDLL(B.LIB_PATH, mode=os.RTLD_NOW)
    for name in _declared_functions():
        assert hasattr(L, name), name


PROBE_HEADER = os.path.join(ROOT, "include", "moe_probe.h")
PROBE_LIB = os.path.join(os.path.dirname(B.LIB_PATH), "libmoe_probe.so")


@pytest.mark.skipif(not os.path.exists(PROBE_LIB), reason="libmoe_probe.so not built")
def test_probe_library_exports_every_declared_symbol():
    # the measurement library of include/moe_probe.h (peaks, the quantisation self-check) likewise
    text = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(moe_probe_[a-z0-9_]+)\s*\(", text)))
    assert names == ["moe_probe_check_quant_division", "moe_probe_mfma", "moe_probe_stream_read"]
    L = ctypes.CDLL(PROBE_LIB, mode=os.RTLD_NOW)
    for name in names:
        assert hasattr(L, name), name


def _shape(**kw):
    base = dict(T=64, d=7168, E=256, k=8, inter=2048, inter_shared=2048, act_dtype=B.MOE_BF16, w_dtype=B.MOE_BF16)
    base.update(kw)
    return B.make_shape(**base)


def test_workspace_size_valid_shapes():
    assert B.moe_workspace_size(_shape()) > 0
    assert B.moe_workspace_size(_shape(T=0)) > 0
    assert B.moe_workspace_size(_shape(act_dtype=B.MOE_F32, w_dtype=B.MOE_F32, d=512, E=32, k=4, inter=256,
                                       inter_shared=256)) > 0
    assert 0 < B.moe_workspace_size(_shape(w_dtype=B.MOE_FP8_E4M3, T=32768)) < 8 << 30


@pytest.mark.parametrize("kw", [
    dict(k=0), dict(T=-1), dict(E=0), dict(k=9, E=8),                     # invalid
    dict(k=17, E=64), dict(E=1025), dict(d=7100), dict(inter=2000),       # unsupported
    dict(inter_shared=100), dict(act_dtype=B.MOE_F32),                    # (F32, BF16) pair
    dict(act_dtype=B.MOE_FP8_E4M3, w_dtype=B.MOE_FP8_E4M3), dict(act_dtype=7),
])
def test_workspace_size_rejects_bad_shapes(kw):
    assert B.moe_workspace_size(_shape(**kw)) == 0


def test_operands_beyond_32_bit_offsets_are_unsupported():
    # The GEMMs address x, h and one expert's weights with 32-bit byte offsets: a shape whose x or h
    # reaches 4 GB is refused (before any launch), one just below is accepted.
    assert B.moe_workspace_size(_shape(T=299594, d=7168)) == 0          # x: 299594 * 7168 * 2 B >= 4 GB
    assert B.moe_workspace_size(_shape(T=116509, k=8, inter=2048)) == 0  # h: T * 9 * 2048 * 2 B >= 4 GB
    assert B.moe_workspace_size(_shape(T=116508, k=8, inter=2048)) > 0   # the largest T below the h limit


def _call_forward(shape, ptrs=None, ws_bytes=1 << 30):
    L = B.lib()
    p = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(20)] if ptrs is None else ptrs
    return L.moe_forward(ctypes.byref(shape), *p, ctypes.c_size_t(ws_bytes), None)


def test_forward_argument_errors_are_host_side():
    s = _shape()
    # k > E, bad dtype pair, bad sizes: rejected before any pointer is touched
    assert _call_forward(_shape(k=9, E=8)) == 1
    assert _call_forward(_shape(d=7100)) == 2
    assert _call_forward(_shape(act_dtype=B.MOE_F32)) == 2
    # null required pointer
    p = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(20)]
    p[0] = None                                   # x
    assert _call_forward(s, p) == 1
    # y aliasing x
    p = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(20)]
    p[15] = p[0]
    assert _call_forward(s, p) == 1
    # misaligned weight pointer
    p = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(20)]
    p[3] = ctypes.c_void_p(0x1000 * 4 + 2)
    assert _call_forward(s, p) == 1
    # fp8 weights without scales
    p = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(20)]
    p[6] = None                                   # W1s
    assert _call_forward(_shape(w_dtype=B.MOE_FP8_E4M3), p) == 1
    # workspace too small, or misaligned
    assert _call_forward(s, ws_bytes=1024) == 3
    p = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(20)]
    p[19] = ctypes.c_void_p(0x1000 * 20 + 16)
    assert _call_forward(s, p) == 3


def test_empty_input_is_a_no_op():
    # T = 0: nothing to compute, nothing launched, any pointers accepted
    assert _call_forward(_shape(T=0), [None] * 20, ws_bytes=0) == 0
    L = B.lib()
    assert L.moe_route(ctypes.byref(_shape(T=0)), *([None] * 10), ctypes.c_size_t(0), None) == 0


def test_status_strings():
    for st in range(6):
        assert B.moe_status_string(st)
    assert "workspace" in B.moe_status_string(3)
    assert "scratch" in B.moe_status_string(5)


def _call_noalloc(shape, ptrs=None):
    # x, Wg, bias, W1, W3, W2, W1s, W3s, W2s, S1, S3, S2, S1s, S3s, S2s, y, idx, w, counts
    L = B.lib()
    p = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(19)] if ptrs is None else ptrs
    return L.moe_forward_noalloc(ctypes.byref(shape), *p, None)


def test_noalloc_host_side_errors():
    # Everything the no-allocation entry point refuses is refused on the host, before its first device call
    # (the lookup of its static scratch): shapes, pointers, and shapes whose workspace exceeds the scratch.
    assert B.NOALLOC_SCRATCH_BYTES == 64 << 20
    assert _call_noalloc(_shape(k=9, E=8)) == 1
    assert _call_noalloc(_shape(d=7100)) == 2
    p = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(19)]
    p[0] = None                                          # x
    assert _call_noalloc(_shape(), p) == 1
    p = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(19)]
    p[15] = p[0]                                         # y aliasing x
    assert _call_noalloc(_shape(), p) == 1
    p = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(19)]
    p[6] = None                                          # fp8 W1s
    assert _call_noalloc(_shape(w_dtype=B.MOE_FP8_E4M3), p) == 1
    # the decode configuration fits the 64 MiB scratch, a prefill-sized one does not
    assert B.moe_workspace_size(_shape(T=64)) <= B.NOALLOC_SCRATCH_BYTES
    assert B.moe_workspace_size(_shape(T=256)) <= B.NOALLOC_SCRATCH_BYTES
    assert B.moe_workspace_size(_shape(T=512)) > B.NOALLOC_SCRATCH_BYTES
    assert _call_noalloc(_shape(T=512)) == 5
    assert _call_noalloc(_shape(T=4096)) == 5
    assert _call_noalloc(_shape(T=0), [None] * 19) == 0


def _call_shard(shape, e0, e1, n_shared, ptrs=None, ws_bytes=1 << 30):
    # x, Wg, bias, allowed | W1, W3, W2, W1s, W3s, W2s, S1, S3, S2, S1s, S3s, S2s, y_partial, idx, w, counts, ws
    L = B.lib()
    p = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(21)] if ptrs is None else ptrs
    return L.moe_forward_shard(ctypes.byref(shape), *p[:4], e0, e1, n_shared, *p[4:], ctypes.c_size_t(ws_bytes), None,
                               None)


def test_shard_argument_errors_are_host_side():
    s = _shape()
    assert _call_shard(s, 0, 257, 2048) == 1            # e1 > E
    assert _call_shard(s, 9, 8, 2048) == 1              # e0 > e1
    assert _call_shard(s, -1, 8, 2048) == 1
    assert _call_shard(s, 0, 8, 4096) == 1              # more shared features than the expert has
    assert _call_shard(s, 0, 8, 100) == 2               # not a multiple of 128
    assert _call_shard(_shape(d=7100), 0, 8, 128) == 2
    p = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(21)]
    p[16] = None                                         # y_partial
    assert _call_shard(s, 0, 8, 128, p) == 1
    p = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(21)]
    p[4] = None                                          # W1 with a non-empty expert range
    assert _call_shard(s, 0, 8, 128, p) == 1
    p = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(21)]
    p[10] = None                                         # S1 with a shared slice
    assert _call_shard(s, 0, 8, 128, p) == 1
    p = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(21)]
    p[16] = p[0]                                         # y_partial aliasing x
    assert _call_shard(s, 0, 8, 128, p) == 1
    assert _call_shard(s, 0, 8, 128, ws_bytes=4096) == 3
    # T = 0 with empty ranges and no pointers: a no-op
    assert _call_shard(_shape(T=0), 0, 0, 0, [None] * 21, ws_bytes=0) == 0


def test_route_limited_and_utilization_argument_errors():
    L = B.lib()
    p = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(11)]
    p[3] = None                                          # allowed is required
    assert L.moe_route_limited(ctypes.byref(_shape()), *p, ctypes.c_size_t(1 << 30), None) == 1
    assert L.moe_route_limited(ctypes.byref(_shape(k=9, E=8)), *([ctypes.c_void_p(16)] * 11),
                               ctypes.c_size_t(1 << 30), None) == 1
    q = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(4)]
    assert L.moe_expert_utilization(0, *q, None) == 1
    assert L.moe_expert_utilization(-3, *q, None) == 1
    q[2] = None
    assert L.moe_expert_utilization(8, *q, None) == 1


def test_route_grouped_argument_errors():
    # Every case fails on the host, before any launch (the pointers are never dereferenced).
    L = B.lib()
    p = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(10)]

    def call(shape, n_group, ws_bytes=1 << 30):
        return L.moe_route_grouped(ctypes.byref(shape), n_group, *p, ctypes.c_size_t(ws_bytes), None)

    assert call(_shape(), 0) == 1                        # n_group < 1
    assert call(_shape(), -8) == 1
    assert call(_shape(k=9, E=8), 4) == 1                # the shape itself is invalid (k > E)
    assert call(_shape(E=256, k=8), 3) == 2              # n_group does not divide E
    assert call(_shape(E=256, k=7), 8) == 2              # odd k
    assert call(_shape(E=256, k=8), 2) == 2              # k / 2 groups more than there are
    assert call(_shape(E=16, k=4), 16) == 2              # one expert per group
    assert call(_shape(E=256, k=8), 32) == 2             # more groups than lanes per token (E <= 256: 16)
    assert call(_shape(E=512, k=8), 128) == 2            # ... (E > 256: 64)
    assert call(_shape(), 8, ws_bytes=16) == 3           # a valid grouping with too small a workspace
    assert call(_shape(T=0), 8, ws_bytes=0) == 0         # no tokens: a no-op (nothing is read or launched)


def test_quantize_e4m3_argument_errors():
    L = B.lib()
    x, q, s = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000), ctypes.c_void_p(0x3000)
    assert L.moe_quantize_e4m3(-1, 128, x, q, s, None) == 1
    assert L.moe_quantize_e4m3(4, 0, x, q, s, None) == 1
    assert L.moe_quantize_e4m3(4, 100, x, q, s, None) == 2         # cols not a multiple of 128
    assert L.moe_quantize_e4m3(4, 256, None, q, s, None) == 1
    assert L.moe_quantize_e4m3(4, 256, ctypes.c_void_p(0x1008), q, s, None) == 1   # x not 16-byte aligned
    assert L.moe_quantize_e4m3(4, 256, x, q, ctypes.c_void_p(0x3002), None) == 1   # scales not 4-byte aligned
    assert L.moe_quantize_e4m3(0, 256, None, None, None, None) == 0  # no rows: a no-op
