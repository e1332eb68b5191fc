"""ctypes wrapper for the CPU oracle (libmoe_oracle.so, built from moe_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the benchmark's CPU-baseline leg,
never by the product path.  All arrays are host numpy arrays; bf16 data travels as uint16 bit patterns
and E4M3 data as uint8 codes.
"""
import ctypes
import os

import numpy as np

from . import build as _build

F32, BF16, FP8_E4M3 = 0, 1, 2

_LIB = None


class OracleShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int64), ("E", ctypes.c_int64), ("k", ctypes.c_int64),
                ("inter", ctypes.c_int64), ("inter_shared", ctypes.c_int64),
                ("act_dtype", ctypes.c_int32), ("w_dtype", ctypes.c_int32)]


def lib():
    global _LIB
    if _LIB is None:
        path = os.environ.get("MOE_ORACLE_LIB")   # another build of the same source (the sanitizer build)
        if not path:
            path = _build.LIB
            if not os.path.exists(path):
                _build.build()
        L = ctypes.CDLL(path)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.oracle_round_bf16_from_double.restype = ctypes.c_float
        L.oracle_round_bf16_from_double.argtypes = [ctypes.c_double]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_encode.argtypes = [ctypes.c_double]
        L.oracle_e4m3_decode.restype = ctypes.c_double
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_quantize_rows_e4m3.argtypes = [i64, i64, vp, vp, vp]
        L.oracle_router_logits.argtypes = [i64, i64, i64, i32, vp, vp, vp, vp]
        L.oracle_route.argtypes = [i64, i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.oracle_forward.argtypes = [ctypes.POINTER(OracleShape)] + [vp] * 15 + [i64, vp, vp, vp]
        L.oracle_swiglu_rows.argtypes = [ctypes.POINTER(OracleShape)] + [vp] * 6 + [i64, i64, vp, vp]
        L.oracle_route_limited.argtypes = [i64, i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.oracle_route_grouped.argtypes = [i64, i64, i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.oracle_expert_utilization.argtypes = [i64, vp, vp, vp, vp]
        L.oracle_forward_shard.argtypes = [ctypes.POINTER(OracleShape)] + [vp] * 15 + [i64, i64, i64, i64, i64, vp, vp]
        L.oracle_num_threads.restype = ctypes.c_int
        _LIB = L
    return _LIB


def _p(a):
    """Pointer of a C-contiguous numpy array (None -> NULL)."""
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def num_threads() -> int:
    return lib().oracle_num_threads()


def round_bf16(v: float) -> float:
    return lib().oracle_round_bf16_from_double(float(v))


def e4m3_encode(v: float) -> int:
    return int(lib().oracle_e4m3_encode(float(v)))


def e4m3_decode(c: int) -> float:
    return float(lib().oracle_e4m3_decode(int(c)))


def quantize_rows_e4m3(v: np.ndarray):
    """Per 1x128-group E4M3 quantisation of an fp32 [rows, cols] matrix -> (codes uint8, scales fp32)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    rows, cols = v.shape
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows, cols // 128), np.float32)
    if lib().oracle_quantize_rows_e4m3(rows, cols, _p(v), _p(q), _p(s)):
        raise ValueError("cols must be a multiple of 128")
    return q, s


def router_logits(x: np.ndarray, Wg: np.ndarray, bias, act_dtype: int) -> np.ndarray:
    """fp32 logits [T, E] of x [T, d] under the gate weight Wg [E, d] (nn.Linear layout)."""
    x = np.ascontiguousarray(x)
    Wg = np.ascontiguousarray(Wg, dtype=np.float32)
    T, d = x.shape
    E = Wg.shape[0]
    L = np.empty((T, E), np.float32)
    lib().oracle_router_logits(T, d, E, act_dtype, _p(x), _p(Wg), _p(bias), _p(L))
    return L


def route(x: np.ndarray, Wg: np.ndarray, bias, k: int, act_dtype: int) -> dict:
    """Routing of every token: logits, idx/w [T,k], counts [E], offsets [E+1], sorted_slots, pos [T*k]."""
    x = np.ascontiguousarray(x)
    Wg = np.ascontiguousarray(Wg, dtype=np.float32)
    bias = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    T, d = x.shape
    E = Wg.shape[0]
    out = dict(logits=np.empty((T, E), np.float32), idx=np.empty((T, k), np.int32),
               w=np.empty((T, k), np.float32), counts=np.empty(E, np.int32),
               offsets=np.empty(E + 1, np.int32), sorted_slots=np.empty(T * k, np.int32),
               pos=np.empty(T * k, np.int32))
    rc = lib().oracle_route(T, d, E, k, act_dtype, _p(x), _p(Wg), _p(bias), _p(out["logits"]), _p(out["idx"]),
                            _p(out["w"]), _p(out["counts"]), _p(out["offsets"]), _p(out["sorted_slots"]),
                            _p(out["pos"]))
    if rc:
        raise ValueError(f"oracle_route failed ({rc})")
    return out


def route_limited(x: np.ndarray, Wg: np.ndarray, bias, allowed: np.ndarray, k: int, act_dtype: int) -> dict:
    """route() with the logits of experts where allowed[e] == 0 set to -inf before top-k."""
    x = np.ascontiguousarray(x)
    Wg = np.ascontiguousarray(Wg, dtype=np.float32)
    bias = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    allowed = np.ascontiguousarray(allowed, dtype=np.uint8)
    T, d = x.shape
    E = Wg.shape[0]
    out = dict(logits=np.empty((T, E), np.float32), idx=np.empty((T, k), np.int32),
               w=np.empty((T, k), np.float32), counts=np.empty(E, np.int32),
               offsets=np.empty(E + 1, np.int32), sorted_slots=np.empty(T * k, np.int32),
               pos=np.empty(T * k, np.int32))
    rc = lib().oracle_route_limited(T, d, E, k, act_dtype, _p(x), _p(Wg), _p(bias), _p(allowed), _p(out["logits"]),
                                    _p(out["idx"]), _p(out["w"]), _p(out["counts"]), _p(out["offsets"]),
                                    _p(out["sorted_slots"]), _p(out["pos"]))
    if rc:
        raise ValueError(f"oracle_route_limited failed ({rc})")
    return out


def route_grouped(x: np.ndarray, Wg: np.ndarray, bias, k: int, n_group: int, act_dtype: int) -> dict:
    """route() with group-limited selection: the k / 2 groups (of n_group) with the largest sums of their
    two best logits, two experts from each."""
    x = np.ascontiguousarray(x)
    Wg = np.ascontiguousarray(Wg, dtype=np.float32)
    bias = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    T, d = x.shape
    E = Wg.shape[0]
    out = dict(logits=np.empty((T, E), np.float32), idx=np.empty((T, k), np.int32),
               w=np.empty((T, k), np.float32), counts=np.empty(E, np.int32),
               offsets=np.empty(E + 1, np.int32), sorted_slots=np.empty(T * k, np.int32),
               pos=np.empty(T * k, np.int32))
    rc = lib().oracle_route_grouped(T, d, E, k, n_group, act_dtype, _p(x), _p(Wg), _p(bias), _p(out["logits"]),
                                    _p(out["idx"]), _p(out["w"]), _p(out["counts"]), _p(out["offsets"]),
                                    _p(out["sorted_slots"]), _p(out["pos"]))
    if rc:
        raise ValueError(f"oracle_route_grouped failed ({rc})")
    return out


def expert_utilization(counts: np.ndarray):
    """(utilization fp32 [E], flags int32 [E] (+1 over 2x mean, -1 under 0.1x mean), (n_over, n_under))."""
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    E = counts.shape[0]
    util = np.empty(E, np.float32)
    flags = np.empty(E, np.int32)
    summary = np.empty(2, np.int32)
    lib().oracle_expert_utilization(E, _p(counts), _p(util), _p(flags), _p(summary))
    return util, flags, (int(summary[0]), int(summary[1]))


def forward_shard(shape: dict, x, W1, W3, W2, S1, S3, S2, idx, w, e0, e1, s0, s1, tokens=None,
                  W1s=None, W3s=None, W2s=None, S1s=None, S3s=None, S2s=None):
    """fp32 partial output of one expert-parallel rank: experts [e0, e1) + shared features [s0, s1)."""
    sh = OracleShape(**shape)
    T, d = int(shape["T"]), int(shape["d"])
    toks = np.arange(T, dtype=np.int32) if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
    n = toks.shape[0]
    part = np.empty((n, d), np.float32)
    args = [np.ascontiguousarray(a) if a is not None else None
            for a in (x, W1, W3, W2, W1s, W3s, W2s, S1, S3, S2, S1s, S3s, S2s, idx, w)]
    rc = lib().oracle_forward_shard(ctypes.byref(sh), *[_p(a) for a in args], e0, e1, s0, s1, n, _p(toks), _p(part))
    if rc:
        raise ValueError(f"oracle_forward_shard failed ({rc})")
    return part


def forward(shape: dict, x, W1, W3, W2, S1, S3, S2, idx, w, tokens=None,
            W1s=None, W3s=None, W2s=None, S1s=None, S3s=None, S2s=None):
    """Layer output for the listed tokens (default: all).  Returns (out_f32 [n,d], y [n,d] act dtype)."""
    sh = OracleShape(**shape)
    T, d = int(shape["T"]), int(shape["d"])
    toks = np.arange(T, dtype=np.int32) if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
    n = toks.shape[0]
    out = np.empty((n, d), np.float32)
    y = np.empty((n, d), np.float32 if shape["act_dtype"] == F32 else np.uint16)
    args = [np.ascontiguousarray(a) if a is not None else None
            for a in (x, W1, W3, W2, W1s, W3s, W2s, S1, S3, S2, S1s, S3s, S2s, idx, w)]
    rc = lib().oracle_forward(ctypes.byref(sh), *[_p(a) for a in args], n, _p(toks), _p(out), _p(y))
    if rc:
        raise ValueError(f"oracle_forward failed ({rc})")
    return out, y


def swiglu_rows(shape: dict, xv: np.ndarray, w1, w3, w2, n_inter: int, s1=None, s3=None, s2=None):
    """One SwiGLU weight set applied to fp32 activation rows xv [rows, d] -> [rows, d] (act-dtype values)."""
    sh = OracleShape(**shape)
    xv = np.ascontiguousarray(xv, dtype=np.float32)
    rows = xv.shape[0]
    y = np.empty((rows, int(shape["d"])), np.float32)
    args = [np.ascontiguousarray(a) if a is not None else None for a in (w1, w3, w2, s1, s3, s2)]
    lib().oracle_swiglu_rows(ctypes.byref(sh), *[_p(a) for a in args], n_inter, rows, _p(xv), _p(y))
    return y
