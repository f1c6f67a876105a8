"""CPU oracle of the routed-expert MoE layer -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never loads it and
shares no code with it: the C source (``oracle.c``) restates the layer's
definition from the pages in plain loops (fp32 router in a fixed order, exact
top-k, fp64 FFN).  This wrapper only marshals numpy arrays.

Parity pins (what ties this oracle to the pages and to mathematics rather
than to itself) live in tests/test_oracle_pins.py; every function below has
at least one.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")

F32, BF16 = 0, 1
IQ2, Q2K, Q8, Q4K, MX4, VQ12, VQ13 = 1, 2, 3, 4, 5, 6, 7
_BW = {IQ2: 256, Q2K: 256, Q8: 32, Q4K: 256, MX4: 32}
_BB = {IQ2: 66, Q2K: 84, Q8: 34, Q4K: 144, MX4: 17}

_lib = None


def build() -> str:
    """Compile liboracle.so with gcc (no fast-math; IEEE fmaf and additions)."""
    tmp = "%s.%d.tmp" % (_SO, os.getpid())
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC",
                           "-Wall", "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _SO)
    return _SO


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_SO)
        P, I, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        L.orc_half.argtypes, L.orc_half.restype = [ctypes.c_uint16], ctypes.c_double
        L.orc_logit.argtypes, L.orc_logit.restype = [P, I, I64, P, I], ctypes.c_float
        L.orc_router_logits.argtypes = [P, I, I, I, P, I, P]
        L.orc_topk.argtypes = [P, I, I, I, P]
        L.orc_route_weights.argtypes = [P, P, I, I, I, P]
        L.orc_bucket.argtypes = [P, I, I, I, P, P, P, P]
        L.orc_dequant.argtypes, L.orc_dequant.restype = [I, P, I64, P, P], I
        L.orc_dequant_rows.argtypes, L.orc_dequant_rows.restype = [I, P, I64, I, P, P, P], I
        L.orc_e4m3.argtypes, L.orc_e4m3.restype = [I], ctypes.c_double
        L.orc_ffn.argtypes = [I, I, I, I, I, I, P, P, P, P, P, I, I, P, P, P, P, P, I, I, P, I, P, P, P]
        L.orc_ffn_grouped.argtypes = L.orc_ffn.argtypes
        L.orc_ffn_grouped.restype = I
        L.orc_sigmoid32.argtypes, L.orc_sigmoid32.restype = [ctypes.c_float], ctypes.c_float
        L.orc_bias_keys.argtypes = [P, I, I, P, P]
        L.orc_ffn.restype = I
        L.orc_threads.restype = I
        L.orc_set_threads.argtypes = [I]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _x(x, x_dtype):
    return _c(x, np.uint16 if x_dtype == BF16 else np.float32)


def threads() -> int:
    return lib().orc_threads()


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))


def half(bits: int) -> float:
    return lib().orc_half(bits)


def router_logits(x, x_dtype, W) -> np.ndarray:
    """z [T, E] fp32 in the fixed summation order (see oracle.c)."""
    x = _x(x, x_dtype)
    W = _c(W, np.float32)
    T, d = x.shape
    E = W.shape[0]
    z = np.empty((T, E), dtype=np.float32)
    lib().orc_router_logits(_p(x), x_dtype, T, d, _p(W), E, _p(z))
    return z


def topk(z, k) -> np.ndarray:
    z = _c(z, np.float32)
    T, E = z.shape
    idx = np.empty((T, k), dtype=np.int32)
    lib().orc_topk(_p(z), T, E, k, _p(idx))
    return idx


def route_weights(z, idx) -> np.ndarray:
    z = _c(z, np.float32)
    idx = _c(idx, np.int32)
    T, E = z.shape
    k = idx.shape[1]
    wt = np.empty((T, k), dtype=np.float32)
    lib().orc_route_weights(_p(z), _p(idx), T, E, k, _p(wt))
    return wt


def sigmoid32(z: float) -> float:
    """The fixed fp32 sigmoid of the biased selection keys (see oracle.c)."""
    return float(lib().orc_sigmoid32(float(z)))


def bias_keys(z, b) -> np.ndarray:
    """key[t, e] = sigmoid32(z[t, e]) + b[e] in fp32."""
    z = _c(z, np.float32)
    b = _c(b, np.float32)
    T, E = z.shape
    key = np.empty((T, E), dtype=np.float32)
    lib().orc_bias_keys(_p(z), T, E, _p(b), _p(key))
    return key


def route(x, x_dtype, W, k, bias=None):
    """(z, idx, wt) for every token of x; with a router bias the experts are
    selected on sigmoid32(z) + bias, the weights still come from z."""
    z = router_logits(x, x_dtype, W)
    idx = topk(z if bias is None else bias_keys(z, bias), k)
    return z, idx, route_weights(z, idx)


def bucket(idx, E):
    """(counts [E], offsets [E+1], perm [n], pos [n]) of the flat routes."""
    idx = _c(idx, np.int32)
    T, k = idx.shape
    n = T * k
    if n and (idx.min() < 0 or idx.max() >= E):
        raise ValueError("bucket: every key must lie in [0, E)")
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(n, np.int32)
    pos = np.empty(n, np.int32)
    lib().orc_bucket(_p(idx), T, k, E, _p(counts), _p(offsets), _p(perm), _p(pos))
    return counts, offsets, perm, pos


def dequant(fmt, blocks, grid=None) -> np.ndarray:
    """Every weight of consecutive blocks, exactly, as float64."""
    blocks = _c(blocks, np.uint8).reshape(-1)
    nb = blocks.size // _BB[fmt]
    assert nb * _BB[fmt] == blocks.size
    out = np.empty(nb * _BW[fmt], dtype=np.float64)
    g = None if grid is None else _c(grid, np.uint8)
    if fmt == IQ2 and g is None:
        raise ValueError("IQ2 needs a grid")
    rc = lib().orc_dequant(fmt, _p(blocks), nb, _p(g), _p(out))
    if rc != 0:
        raise ValueError("bad format")
    return out


def vq_row_bytes(fmt, K) -> int:
    """Bytes of one VQ row of K weights: fp16 gain, 12-bit stream, bit plane."""
    return 2 + 3 * K // 16 + (K // 64 if fmt == VQ13 else 0)


def e4m3(code: int) -> float:
    """The value of one E4M3 byte (nan for the two not-a-number codes)."""
    return lib().orc_e4m3(int(code))


def dequant_rows(fmt, rows, K, grid=None, codebook=None) -> np.ndarray:
    """Every weight of consecutive rows of K weights, exactly, as float64
    [n_rows, K] (block formats row by row; VQ rows with the codebook)."""
    rows = _c(rows, np.uint8).reshape(-1)
    rb = vq_row_bytes(fmt, K) if fmt in (VQ12, VQ13) else K // _BW[fmt] * _BB[fmt]
    n = rows.size // rb
    assert n * rb == rows.size
    out = np.empty((n, K), dtype=np.float64)
    g = None if grid is None else _c(grid, np.uint8)
    cb = None if codebook is None else _c(codebook, np.uint8)
    if lib().orc_dequant_rows(fmt, _p(rows), n, K, _p(g), _p(cb), _p(out)) != 0:
        raise ValueError("bad format or missing codebook")
    return out


def ffn(layer, x, x_dtype, idx, wt, tokens=None, grouped=False) -> np.ndarray:
    """Expert FFN + shared expert for the listed tokens (all if None).

    layer: a synth.Layer (canonical bytes).  Returns y [len(tokens), d] fp32.
    grouped: evaluate expert by expert (orc_ffn_grouped: each expert
    dequantised once, results bitwise those of the token-by-token loop).
    """
    s = layer.spec
    x = _x(x, x_dtype)
    T = x.shape[0]
    idx = _c(idx, np.int32)
    wt = _c(wt, np.float32)
    tok = None if tokens is None else _c(tokens, np.int32)
    n_tok = T if tok is None else tok.size
    y = np.empty((n_tok, s.d), dtype=np.float32)
    sh = s.has_shared
    k = idx.shape[1]  # routes per token as given (may differ from the layer's top_k)
    dg = getattr(layer, "down_gain", None)
    gain = None if dg is None else _c(dg, np.float32)
    cb = getattr(layer, "vq_codebook", None)
    fn = lib().orc_ffn_grouped if grouped else lib().orc_ffn
    rc = fn(s.E, s.d, s.f, k, s.fmt_gate_up, s.fmt_down, _p(_c(layer.w_gate, np.uint8)),
                       _p(_c(layer.w_up, np.uint8)), _p(_c(layer.w_down, np.uint8)), _p(_c(layer.grid, np.uint8)),
                       _p(None if cb is None else _c(cb, np.uint8)), int(sh), s.fmt_shared if sh else 0,
                       _p(_c(layer.s_gate, np.uint8)) if sh else None,
                       _p(_c(layer.s_up, np.uint8)) if sh else None,
                       _p(_c(layer.s_down, np.uint8)) if sh else None,
                       _p(gain), _p(x), x_dtype, T, _p(tok), n_tok, _p(idx), _p(wt), _p(y))
    if rc == -2:
        raise MemoryError("oracle ffn: out of host memory")
    if rc != 0:
        raise ValueError("oracle ffn: token or expert index out of range, or unusable format")
    return y


def layer_forward(layer, x, x_dtype, tokens=None):
    """Routing + FFN for the listed tokens: returns (y, idx, wt) for them."""
    x = _x(x, x_dtype)
    xs = x if tokens is None else x[np.asarray(tokens)]
    _, idx, wt = route(xs, x_dtype, layer.w_router, layer.spec.k, getattr(layer, "router_bias", None))
    return ffn(layer, xs, x_dtype, idx, wt), idx, wt
