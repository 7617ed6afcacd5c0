"""CPU oracle for the CSA / HCA hybrid compressed attention path.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only callers.  The product path
(``long_context_sparse_03_amd``) never imports this package, and this package
never imports the product: the two share no code.

The arithmetic lives in ``csa_oracle.c`` (plain C, fp64, OpenMP over
queries); this module builds it with gcc on first use and wraps each function
for numpy arrays.  ``oracle.layer`` composes the functions into whole layers.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csa_oracle.c")
_LIB = os.path.join(_HERE, "libcsa_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, IEEE semantics kept: no fast-math,
    no FMA contraction) into ``oracle/libcsa_oracle.so``."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
            "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wno-unknown-pragmas",
            _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        D = ctypes.c_double
        F = ctypes.c_float
        sig = {
            "orc_bf16_bits": (ctypes.c_uint16, [F]),
            "orc_bf16_value": (F, [ctypes.c_uint16]),
            "orc_bf16_bits_from_double": (ctypes.c_uint16, [D]),
            "orc_e4m3_decode": (D, [ctypes.c_uint8]),
            "orc_e4m3_encode": (ctypes.c_uint8, [F]),
            "orc_e2m1_decode": (D, [ctypes.c_uint8]),
            "orc_e2m1_encode": (ctypes.c_uint8, [F]),
            "orc_mx_scale_code": (I, [F]),
            "orc_mxfp4_pack": (None, [I, P, P, P]),
            "orc_mxfp4_unpack": (None, [I, P, P, P]),
            "orc_compress": (None, [I, I, I, I, P, P, P, P, P, P, P]),
            "orc_compress_weights": (None, [I, I, I, I, P, P, P, P, P]),
            "orc_rmsnorm": (None, [I, I, P, P, D, P]),
            "orc_rope": (None, [I, I, I, P, D, P]),
            "orc_index_scores": (None, [I, I, I, P, P, P, I, P, I, P, I]),
            "orc_topk": (None, [I, P, I, P, I, P]),
            "orc_attend": (None, [I, I, I, P, P, D, D, D, D, I, P, P, P]),
            "orc_attend_batch": (None, [I, I, I, I, P, P, D, P, D, D, P, P, I, P, P, I, P, P]),
            "orc_fp8_block_append": (None, [I, I, I, P, I, I, P]),
            "orc_fp8_block_decode": (None, [I, I, I, P, I, P]),
            "orc_num_threads": (I, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def num_threads() -> int:
    return int(lib().orc_num_threads())


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------

def bf16_bits(x) -> np.ndarray:
    """float32 array -> uint16 bf16 bit patterns (round to nearest even)."""
    x = _f32(x)
    f = lib().orc_bf16_bits
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.uint16).reshape(x.shape)


def bf16_round(x) -> np.ndarray:
    """Round float32 values to bf16 and return them as float32.  Vectorised
    form of ``orc_bf16_bits`` (same bit rule); checked against it in the pins."""
    u = _f32(x).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32)


def bf16_from_double(v: float) -> float:
    b = lib().orc_bf16_bits_from_double(float(v))
    return float(lib().orc_bf16_value(b))


def e4m3_encode(x) -> np.ndarray:
    x = _f32(x)
    f = lib().orc_e4m3_encode
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.uint8).reshape(x.shape)


def e4m3_decode(q) -> np.ndarray:
    q = np.asarray(q, dtype=np.uint8)
    f = lib().orc_e4m3_decode
    return np.array([f(int(v)) for v in q.ravel()], dtype=np.float64).reshape(q.shape)


def e2m1_encode(x) -> np.ndarray:
    x = _f32(x)
    f = lib().orc_e2m1_encode
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.uint8).reshape(x.shape)


def e2m1_decode(q) -> np.ndarray:
    q = np.asarray(q, dtype=np.uint8)
    f = lib().orc_e2m1_decode
    return np.array([f(int(v)) for v in q.ravel()], dtype=np.float64).reshape(q.shape)


def mx_scale_code(amax: float) -> int:
    return int(lib().orc_mx_scale_code(float(amax)))


def mxfp4_pack(x):
    """x [..., n] float32 (n multiple of 32) -> (codes uint8 [..., n/2], scales uint8 [..., n/32])."""
    x = _f32(x)
    n = x.shape[-1]
    rows = x.reshape(-1, n)
    codes = np.zeros((rows.shape[0], n // 2), np.uint8)
    scales = np.zeros((rows.shape[0], n // 32), np.uint8)
    f = lib().orc_mxfp4_pack
    for i in range(rows.shape[0]):
        r = np.ascontiguousarray(rows[i])
        cc = np.zeros(n // 2, np.uint8)
        ss = np.zeros(n // 32, np.uint8)
        f(n, _p(r), _p(cc), _p(ss))
        codes[i] = cc
        scales[i] = ss
    return codes.reshape(x.shape[:-1] + (n // 2,)), scales.reshape(x.shape[:-1] + (n // 32,))


def mxfp4_unpack(codes, scales) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    n = codes.shape[-1] * 2
    rc = codes.reshape(-1, n // 2)
    rs = scales.reshape(-1, n // 32)
    out = np.zeros((rc.shape[0], n), np.float64)
    f = lib().orc_mxfp4_unpack
    for i in range(rc.shape[0]):
        o = np.zeros(n, np.float64)
        f(n, _p(np.ascontiguousarray(rc[i])), _p(np.ascontiguousarray(rs[i])), _p(o))
        out[i] = o
    return out.reshape(codes.shape[:-1] + (n,))


# --------------------------------------------------------------------------
# method steps
# --------------------------------------------------------------------------

def compress(Ca, Cb, Za, Zb, Ba, Bb, m: int, overlap: bool) -> np.ndarray:
    """Compressed entries [floor(n/m), c] from projected rows [n, c]."""
    Ca, Za, Ba = _f64(Ca), _f64(Za), _f64(Ba)
    n, c = Ca.shape
    Cb = _f64(Cb) if Cb is not None else Ca
    Zb = _f64(Zb) if Zb is not None else Za
    Bb = _f64(Bb) if Bb is not None else Ba
    out = np.zeros((n // m, c), np.float64)
    lib().orc_compress(n, c, m, int(bool(overlap)), _p(Ca), _p(Cb), _p(Za), _p(Zb), _p(Ba), _p(Bb), _p(out))
    return out


def compress_weights(Za, Zb, Ba, Bb, m: int, overlap: bool) -> np.ndarray:
    """Softmax weights S [floor(n/m), 2m, c] of the compressor."""
    Za, Ba = _f64(Za), _f64(Ba)
    n, c = Za.shape
    Zb = _f64(Zb) if Zb is not None else Za
    Bb = _f64(Bb) if Bb is not None else Ba
    S = np.zeros((n // m, 2 * m, c), np.float64)
    lib().orc_compress_weights(n, c, m, int(bool(overlap)), _p(Za), _p(Zb), _p(Ba), _p(Bb), _p(S))
    return S


def rmsnorm(x, gamma, eps: float) -> np.ndarray:
    x = _f64(x)
    c = x.shape[-1]
    rows = x.reshape(-1, c)
    y = np.zeros_like(rows)
    lib().orc_rmsnorm(rows.shape[0], c, _p(rows), _p(_f64(gamma)), float(eps), _p(y))
    return y.reshape(x.shape)


def rope(x, pos, r: int, theta: float) -> np.ndarray:
    """Rotate the last r channels of each row of x [rows, c] at pos[rows]."""
    y = _f64(x).copy()
    c = y.shape[-1]
    rows = y.reshape(-1, c)
    p = _f64(np.broadcast_to(np.asarray(pos, np.float64), (rows.shape[0],)))
    lib().orc_rope(rows.shape[0], c, r, _p(p), float(theta), _p(rows))
    return rows.reshape(y.shape)


def index_scores(qI, w, n_vis, K, fmt: int) -> np.ndarray:
    """qI [T, nh, cI], w [T, nh], n_vis [T], K [E, cI] -> float32 [T, E]
    (entries at s >= n_vis stay NaN)."""
    qI, w, K = _f64(qI), _f64(w), _f64(K)
    T, nh, cI = qI.shape
    E = K.shape[0]
    out = np.full((T, max(E, 1)), np.nan, np.float32)
    nv = np.ascontiguousarray(n_vis, np.int32)
    lib().orc_index_scores(T, nh, cI, _p(qI), _p(w), _p(nv), E, _p(K), int(fmt), _p(out), out.shape[1])
    return out[:, :E]


def topk(scores, n_valid, k: int) -> np.ndarray:
    s = _f32(scores)
    T, ld = s.shape
    nv = np.ascontiguousarray(n_valid, np.int32)
    out = np.zeros((T, k), np.int32)
    lib().orc_topk(T, _p(s), ld, _p(nv), int(k), _p(out))
    return out


def attend(q_raw, gamma_q, eps, pos, theta, scale, X, sink, r: int) -> np.ndarray:
    """One query: q_raw [nh, c], rows X [nrows, c] -> o [nh, c]."""
    q_raw, X = _f64(q_raw), _f64(X).reshape(-1, np.shape(q_raw)[1])
    nh, c = q_raw.shape
    out = np.zeros((nh, c), np.float64)
    lib().orc_attend(nh, c, r, _p(q_raw), _p(_f64(gamma_q)), float(eps), float(pos), float(theta),
                     float(scale), X.shape[0], _p(X), _p(_f64(sink)), _p(out))
    return out


def attend_batch(q_raw, gamma_q, eps, pos, theta, scale, entries, sel, n_ent, win, n_win, sink, r):
    """Queries of one request.  q_raw [T, nh, c]; entries [E, c]; sel [T, k]
    (or None for dense: n_ent [T] entries each); win [n_tok, c] window rows."""
    q_raw = _f64(q_raw)
    T, nh, c = q_raw.shape
    entries = _f64(entries).reshape(-1, c)
    if entries.shape[0] == 0:
        entries = np.zeros((1, c))
    win = _f64(win).reshape(-1, c)
    posd = _f64(pos)
    out = np.zeros((T, nh, c), np.float64)
    if sel is not None:
        sel = np.ascontiguousarray(sel, np.int32)
        k = sel.shape[1]
        sel_p, ne_p = _p(sel), None
        ne = None
    else:
        k = 0
        ne = np.ascontiguousarray(n_ent, np.int32)
        sel_p, ne_p = None, _p(ne)
    lib().orc_attend_batch(T, nh, c, r, _p(q_raw), _p(_f64(gamma_q)), float(eps), _p(posd), float(theta),
                           float(scale), _p(entries), sel_p, k, ne_p, _p(win), int(n_win), _p(_f64(sink)),
                           _p(out))
    return out


def fp8_block_append(block: np.ndarray, c: int, r: int, epb: int, first: int, x) -> None:
    """In-place append of x [n_new, c] float32 into a mixed FP8/BF16 block."""
    x = _f32(x)
    assert block.dtype == np.uint8 and block.flags.c_contiguous
    lib().orc_fp8_block_append(c, r, epb, _p(block), int(first), x.shape[0], _p(x))


def fp8_block_decode(block: np.ndarray, c: int, r: int, epb: int, slot: int) -> np.ndarray:
    out = np.zeros(c, np.float64)
    lib().orc_fp8_block_decode(c, r, epb, _p(np.ascontiguousarray(block)), int(slot), _p(out))
    return out
