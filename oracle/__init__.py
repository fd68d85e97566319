"""CPU oracle for CSA / HCA attention -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check in __graft_entry__ and the cpu_baseline leg of
bench.py may import this package.  The product path (the HIP library and its
Python binding) never imports it, and this package imports nothing from the
product path: the two share no code.  The only module both sides read is the
seeded input generator, which holds none of the method's arithmetic.

The arithmetic lives in oracle.c (plain fp64 C, built as liboracle.so); this
file is a ctypes wrapper plus the orchestration of the per-layer steps in the
order the pages describe them (dsv4 book Ch.5-7).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

FMT_F32, FMT_BF16, FMT_FP8MIX, FMT_E4M3, FMT_FP4 = 0, 1, 2, 3, 4
FMT_BY_NAME = {"f32": FMT_F32, "bf16": FMT_BF16, "fp8mix": FMT_FP8MIX, "e4m3": FMT_E4M3, "fp4": FMT_FP4}


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (-O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB_PATH)
        P, I, I64, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        sig = {
            "orc_e4m3_decode": (D, [ctypes.c_uint8]),
            "orc_e4m3_encode": (ctypes.c_uint8, [D]),
            "orc_bf16_decode": (D, [ctypes.c_uint16]),
            "orc_bf16_encode": (ctypes.c_uint16, [D]),
            "orc_pow2_exponent": (I, [D]),
            "orc_encode_bf16_array": (None, [I64, P, P]),
            "orc_decode_bf16_array": (None, [I64, P, P]),
            "orc_decode_e4m3_array": (None, [I64, P, P]),
            "orc_e2m1_decode": (D, [ctypes.c_uint8]),
            "orc_e2m1_encode": (ctypes.c_uint8, [D]),
            "orc_fp4_block_exponent": (I, [D]),
            "orc_decode_e2m1_array": (None, [I64, P, P]),
            "orc_quantize_rows_e4m3": (None, [I64, I, P, P, P]),
            "orc_record_stride": (I64, [I, I, I]),
            "orc_page_bytes": (I64, [I, I, I, I]),
            "orc_store_entry": (None, [I, I, I, I, P, P, I64, P]),
            "orc_load_entry": (None, [I, I, I, I, P, P, I64, P]),
            "orc_rmsnorm": (None, [I, P, P, D, P]),
            "orc_rope": (None, [I, I, D, D, I, P]),
            "orc_compress_entry": (None, [I, I, I, I, P, P, P, P, P, P, P]),
            "orc_compress": (I64, [I64, I, I, I, P, P, P, P, P, P, P]),
            "orc_finish_store": (None, [I, I, I, I, P, P, I64, I64, P, P, D, D, I, I, I]),
            "orc_load_entries": (None, [I, I, I, I, P, P, I64, I64, P]),
            "orc_window_prep": (None, [I64, I, I, D, D, P, P, P, P]),
            "orc_index_scores": (I, [I64, I, I, I, P, P, P, P, I, I, P, P, I, P, I64, P, P]),
            "orc_topk": (None, [I64, I64, P, P, I, P, P]),
            "orc_attend": (I, [I64, I, I, I, D, D, D, P, P, P, P, I, I, P, P, I, P, I, I, P, P, I,
                              I, I, P, I, P, P, P]),
            "orc_num_threads": (I, []),
            "orc_set_num_threads": (None, [I]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def num_threads() -> int:
    return lib().orc_num_threads()


def set_num_threads(n: int) -> None:
    """Threads the oracle's parallel loops use from now on."""
    lib().orc_set_num_threads(int(n))


# ---------------------------------------------------------------- codecs
def e4m3_decode(codes) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape, np.float64)
    lib().orc_decode_e4m3_array(codes.size, _p(codes), _p(out))
    return out


def e4m3_encode_scalar(x: float) -> int:
    return int(lib().orc_e4m3_encode(float(x)))


def e2m1_decode(codes) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape, np.float64)
    lib().orc_decode_e2m1_array(codes.size, _p(codes), _p(out))
    return out


def e2m1_encode_scalar(x: float) -> int:
    return int(lib().orc_e2m1_encode(float(x)))


def fp4_block_exponent(amax: float) -> int:
    return int(lib().orc_fp4_block_exponent(float(amax)))


def bf16_encode(x) -> np.ndarray:
    x = _f64(x)
    out = np.empty(x.shape, np.uint16)
    lib().orc_encode_bf16_array(x.size, _p(x), _p(out))
    return out


def bf16_decode(bits) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, np.float64)
    lib().orc_decode_bf16_array(bits.size, _p(bits), _p(out))
    return out


def pow2_exponent(amax: float) -> int:
    return int(lib().orc_pow2_exponent(float(amax)))


def quantize_rows_e4m3(x):
    """Rows -> (e4m3 codes, per-row power-of-two exponent)."""
    x = _f64(x)
    c = x.shape[-1]
    n = x.size // c
    codes = np.empty(x.shape, np.uint8)
    exps = np.empty(x.shape[:-1], np.int32)
    lib().orc_quantize_rows_e4m3(n, c, _p(x), _p(codes), _p(exps))
    return codes, exps


def dequantize_rows_e4m3(codes, exps) -> np.ndarray:
    return e4m3_decode(codes) * np.ldexp(1.0, np.asarray(exps))[..., None]


# ---------------------------------------------------------------- layout
def record_stride(fmt: int, D: int, R: int) -> int:
    return int(lib().orc_record_stride(fmt, D, R))


def page_bytes(fmt: int, D: int, R: int, P: int) -> int:
    return int(lib().orc_page_bytes(fmt, D, R, P))


def finish_store(fmt, D, R, P, pool, pt_row, first, x, gain=None, eps=1e-6, base=1e4, ratio=1,
                 norm=True, rope=True):
    """Entry epilogue (RMSNorm -> RoPE at ratio*i) and encode into `pool` (uint8, modified in place)."""
    x = _f64(x).reshape(-1, D)
    g = _f64(np.ones(D) if gain is None else gain)
    pt_row = np.ascontiguousarray(pt_row, dtype=np.int32)
    assert pool.dtype == np.uint8 and pool.flags.c_contiguous
    lib().orc_finish_store(fmt, D, R, P, _p(pool), _p(pt_row), int(first), x.shape[0], _p(x), _p(g),
                           float(eps), float(base), int(ratio), int(norm), int(rope))


def load_entries(fmt, D, R, P, pool, pt_row, first, n) -> np.ndarray:
    out = np.empty((n, D), np.float64)
    pt_row = np.ascontiguousarray(pt_row, dtype=np.int32)
    lib().orc_load_entries(fmt, D, R, P, _p(pool), _p(pt_row), int(first), int(n), _p(out))
    return out


# ---------------------------------------------------------------- math steps
def rmsnorm(x, g=None, eps=1e-6) -> np.ndarray:
    x = _f64(x)
    g = _f64(np.ones(x.shape[-1]) if g is None else g)
    y = np.empty_like(x)
    lib().orc_rmsnorm(x.shape[-1], _p(x), _p(g), float(eps), _p(y))
    return y


def rope(x, R, pos, base=1e4, sign=1) -> np.ndarray:
    y = _f64(x).copy()
    lib().orc_rope(y.shape[-1], R, float(base), float(pos), int(sign), _p(y))
    return y


def compress_entry(m, overlap, has_prev, Ca, Za, Cb, Zb, Ba, Bb) -> np.ndarray:
    Ca, Za, Ba = _f64(Ca), _f64(Za), _f64(Ba)
    c = Ca.shape[-1]
    Cb = _f64(Cb) if Cb is not None else np.zeros_like(Ca)
    Zb = _f64(Zb) if Zb is not None else np.zeros_like(Za)
    Bb = _f64(Bb) if Bb is not None else np.zeros_like(Ba)
    out = np.empty(c, np.float64)
    lib().orc_compress_entry(c, m, int(overlap), int(has_prev), _p(Ca), _p(Za), _p(Cb), _p(Zb), _p(Ba),
                             _p(Bb), _p(out))
    return out


def compress(m, overlap, Ca, Za, Ba, Cb=None, Zb=None, Bb=None) -> np.ndarray:
    """All completed entries (floor(L/m)) of a sequence; no epilogue."""
    Ca, Za, Ba = _f64(Ca), _f64(Za), _f64(Ba)
    L, c = Ca.shape
    if overlap:
        Cb, Zb, Bb = _f64(Cb), _f64(Zb), _f64(Bb)
    out = np.empty((L // m, c), np.float64)
    lib().orc_compress(L, c, m, int(overlap), _p(Ca), _p(Za), _p(Cb), _p(Zb), _p(Ba), _p(Bb), _p(out))
    return out


def window_prep(raw, pos, R, gain=None, eps=1e-6, base=1e4) -> np.ndarray:
    raw = _f64(raw)
    n, D = raw.shape
    g = _f64(np.ones(D) if gain is None else gain)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    out = np.empty_like(raw)
    lib().orc_window_prep(n, D, R, float(base), float(eps), _p(raw), _p(g), _p(pos), _p(out))
    return out


def index_scores(qI, w, pos, m, idx_fmt, P, pool, page_table, n_avail, seq=None, n_cols=None):
    """Indexer scores [n_rows, n_cols] (only the first n_elig[r] of row r are defined; rest NaN)."""
    qI = _f64(qI)
    n_rows, nI, cI = qI.shape
    w = _f64(w)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    seq_a = None if seq is None else np.ascontiguousarray(seq, dtype=np.int32)
    page_table = np.ascontiguousarray(page_table, dtype=np.int32).reshape(-1, np.shape(page_table)[-1])
    n_avail = np.ascontiguousarray(n_avail, dtype=np.int64)
    if n_cols is None:
        n_cols = int(max(1, (pos // m).max()))
    scores = np.full((n_rows, n_cols), np.nan)
    n_elig = np.empty(n_rows, np.int64)
    rc = lib().orc_index_scores(n_rows, nI, cI, m, _p(qI), _p(w), _p(pos), _p(seq_a), idx_fmt, P, _p(pool),
                                _p(page_table), page_table.shape[1], _p(n_avail), n_cols, _p(scores),
                                _p(n_elig))
    if rc != 0:
        raise ValueError("indexer needs entries the cache does not hold")
    return scores, n_elig


def topk(scores, n_elig, k):
    scores = _f64(scores)
    n_rows, n_cols = scores.shape
    n_elig = np.ascontiguousarray(n_elig, dtype=np.int64)
    idx = np.empty((n_rows, k), np.int32)
    cnt = np.empty(n_rows, np.int32)
    lib().orc_topk(n_rows, n_cols, _p(scores), _p(n_elig), k, _p(idx), _p(cnt))
    return idx, cnt


def attend(q, pos, kv_fmt, P, pool, page_table, n_avail, mode, ratio, window, n_win, sink, R,
           gq=None, seq=None, idx=None, cnt=None, base=1e4, eps=1e-6, scale=None, want_lse=False):
    """Core attention rows (mode 0 = CSA over idx/cnt, 1 = HCA dense).

    window: stored window [S, W, D] as float32 (fp32 storage) or uint16 (bf16 bits).
    """
    q = _f64(q)
    n_rows, nh, D = q.shape
    gq = _f64(np.ones(D) if gq is None else gq)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    seq_a = None if seq is None else np.ascontiguousarray(seq, dtype=np.int32)
    page_table = np.ascontiguousarray(page_table, dtype=np.int32).reshape(-1, np.shape(page_table)[-1])
    n_avail = np.ascontiguousarray(n_avail, dtype=np.int64)
    if window.dtype == np.float32:
        win_fmt = 0
    elif window.dtype == np.uint16:
        win_fmt = 1
    else:
        raise TypeError("window must be float32 or bf16 bits (uint16)")
    window = np.ascontiguousarray(window)
    W = window.shape[1]
    sink = _f64(sink)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    if mode == 0:
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        cnt = np.ascontiguousarray(cnt, dtype=np.int32)
        k = idx.shape[1]
    else:
        k = 0
    out = np.empty((n_rows, nh, D), np.float64)
    lse = np.empty((n_rows, nh), np.float64) if want_lse else None
    rc = lib().orc_attend(n_rows, nh, D, R, float(base), float(scale), float(eps), _p(q), _p(gq), _p(pos),
                          _p(seq_a), kv_fmt, P, _p(pool), _p(page_table), page_table.shape[1], _p(n_avail),
                          int(mode), int(ratio), _p(idx), _p(cnt), int(k), int(n_win), win_fmt, _p(window), W,
                          _p(sink), _p(out), _p(lse))
    if rc != 0:
        raise ValueError("attention row needs an entry that is missing or not causally available")
    return (out, lse) if want_lse else out
