"""ctypes binding of libcsahca.so, the MI355X (gfx950) CSA / HCA attention library.

Argument marshalling only: every function below forwards device pointers of
torch tensors (and torch's current HIP stream) to the C entry point of the same
name in include/csahca.h and raises CAError on a non-zero status.  All
computation happens in the library's HIP kernels.  Importing this package
fails loudly when the library has not been built (see build.py).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsahca.so")

F32, BF16, FP8MIX, E4M3, FP4 = 0, 1, 2, 3, 4
STATUS_POS_RANGE = 1   # device status bit: a decode row's position outside [0, max_pos]
FORMATS = {"f32": F32, "bf16": BF16, "fp8mix": FP8MIX, "e4m3": E4M3, "fp4": FP4}


class CAError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"csahca error {code}: {msg}")
        self.code = code


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m long_context_attention_17_amd.build` "
                      "(or __graft_entry__.build()) before using the HIP path")
_lib = ctypes.CDLL(LIB_PATH)

_P, _I32, _I64, _F, _D, _SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double,
                               ctypes.c_size_t)


class _Cache(ctypes.Structure):
    _fields_ = [("format", _I32), ("dim", _I32), ("rope_dim", _I32), ("page_size", _I32), ("pool", _P),
                ("n_pages", _I64), ("page_table", _P), ("n_seqs", _I32), ("max_pages", _I32)]


class CompressParams(ctypes.Structure):
    _fields_ = [("ratio", _I32), ("overlap", _I32), ("in_format", _I32), ("apply_norm", _I32),
                ("apply_rope", _I32), ("eps", _F), ("rope_base", _D)]


class WindowParams(ctypes.Structure):
    _fields_ = [("dim", _I32), ("rope_dim", _I32), ("in_format", _I32), ("win_format", _I32), ("eps", _F),
                ("rope_base", _D)]


class IndexParams(ctypes.Structure):
    _fields_ = [("n_heads", _I32), ("dim", _I32), ("ratio", _I32), ("k", _I32), ("q_format", _I32),
                ("q_quant", _I32), ("status", _P)]


class AttendParams(ctypes.Structure):
    _fields_ = [("n_heads", _I32), ("dim", _I32), ("rope_dim", _I32), ("n_win", _I32), ("q_format", _I32),
                ("win_format", _I32), ("out_format", _I32), ("scale", _F), ("eps", _F), ("rope_base", _D),
                ("status", _P)]


_PC = ctypes.POINTER(_Cache)


class DecodeEntryJob(ctypes.Structure):
    _fields_ = [("params", CompressParams), ("new_rows", _P), ("tail", _P), ("Ba", _P), ("Bb", _P), ("gain", _P),
                ("cache", _PC)]


class DecodeState(ctypes.Structure):
    _fields_ = [("window", _P), ("W", _I32), ("S", _I32), ("win_dim", _I32), ("win_format", _I32),
                ("n_jobs", _I32), ("tail", _P * 2), ("tail_floats", _I64 * 2), ("cache", _PC * 2),
                ("ratio", _I32 * 2)]


class QueryProjParams(ctypes.Structure):
    _fields_ = [("d", _I32), ("d_c", _I32), ("n_q", _I32), ("n_qi", _I32), ("n_i", _I32), ("w_dq", _P), ("w_uq", _P),
                ("w_iuq", _P), ("w_w", _P)]


class OutProjParams(ctypes.Structure):
    _fields_ = [("n_h", _I32), ("c", _I32), ("d_g", _I32), ("d", _I32), ("w_o1", _P), ("w_o2", _P)]


_SIGS = {
    "ca_last_error": (ctypes.c_char_p, []),
    "ca_record_stride": (_I64, [_I32, _I32, _I32]),
    "ca_page_bytes": (_I64, [_I32, _I32, _I32, _I32]),
    "ca_store_entries": (ctypes.c_int, [_PC, _I32, _I64, _I64, _P, _P, _F, _I32, _D, _I32, _P]),
    "ca_compress_prefill": (ctypes.c_int, [ctypes.POINTER(CompressParams), _P, _P, _P, _P, _P, _P, _P, _I64, _I64,
                                           _I32, _PC, _P]),
    "ca_compress_decode": (ctypes.c_int, [ctypes.POINTER(CompressParams), _P, _P, _I32, _P, _P, _P, _P, _PC, _P]),
    "ca_window_append": (ctypes.c_int, [ctypes.POINTER(WindowParams), _P, _P, _P, _P, _I32, _P, _I32, _I32, _P]),
    "ca_decode_append": (ctypes.c_int, [ctypes.POINTER(WindowParams), _P, _P, _P, _I32, _P, _I32, _I32,
                                        ctypes.POINTER(DecodeEntryJob), _I32, _P]),
    "ca_index_topk_workspace": (_SZ, [ctypes.POINTER(IndexParams), _I32, _I64]),
    "ca_index_topk_prefill": (ctypes.c_int, [ctypes.POINTER(IndexParams), _P, _P, _I64, _I64, _I32, _PC, _P, _P, _P,
                                             _P, _I64, _P, _SZ, _P]),
    "ca_index_topk_decode": (ctypes.c_int, [ctypes.POINTER(IndexParams), _P, _P, _P, _I32, _I64, _PC, _P, _P, _P,
                                            _P, _I64, _P, _SZ, _P]),
    "ca_attend_workspace": (_SZ, [ctypes.POINTER(AttendParams), _I32, _I64, _I32, _I32]),
    "ca_csa_attend_prefill": (ctypes.c_int, [ctypes.POINTER(AttendParams), _P, _P, _PC, _I32, _P, _P, _I32, _I32,
                                             _P, _I32, _P, _I64, _I64, _P, _P, _P, _SZ, _P]),
    "ca_csa_attend_decode": (ctypes.c_int, [ctypes.POINTER(AttendParams), _P, _P, _PC, _P, _P, _I32, _I32, _P, _I32,
                                            _I64, _P, _I32, _P, _P, _P, _P, _SZ, _P]),
    "ca_hca_attend_prefill": (ctypes.c_int, [ctypes.POINTER(AttendParams), _P, _P, _PC, _I32, _I32, _P, _I32, _P,
                                             _I64, _I64, _P, _P, _P, _SZ, _P]),
    "ca_hca_attend_decode": (ctypes.c_int, [ctypes.POINTER(AttendParams), _P, _P, _PC, _I32, _P, _I32, _I64, _P,
                                            _I32, _P, _P, _P, _P, _SZ, _P]),
    "ca_csa_decode_step": (ctypes.c_int, [ctypes.POINTER(WindowParams), _P, _P, _P, _I32, _I32,
                                          ctypes.POINTER(DecodeEntryJob), ctypes.POINTER(IndexParams), _P, _P, _P, _P,
                                          _P, _SZ, ctypes.POINTER(AttendParams), _P, _P, _P, _I32, _I64, _P, _P, _P,
                                          _P, _SZ, _P]),
    "ca_hca_decode_step": (ctypes.c_int, [ctypes.POINTER(WindowParams), _P, _P, _P, _I32, _I32,
                                          ctypes.POINTER(DecodeEntryJob), ctypes.POINTER(AttendParams), _P, _P, _P,
                                          _I32, _I64, _P, _P, _P, _P, _SZ, _P]),
    "ca_attend_decode_plan": (ctypes.c_int, [ctypes.POINTER(AttendParams), _I64, ctypes.POINTER(_I32),
                                             ctypes.POINTER(_I32), ctypes.POINTER(_I32)]),
    "ca_static_scratch_bytes": (_SZ, []),
    "ca_hca_decode_step_noalloc": (ctypes.c_int, [ctypes.POINTER(WindowParams), _P, _P, _P, _I32, _I32,
                                                  ctypes.POINTER(DecodeEntryJob), ctypes.POINTER(AttendParams), _P,
                                                  _P, _P, _I32, _I64, _P, _P, _P, _P]),
    "ca_state_bytes": (_I64, [ctypes.POINTER(DecodeState), _I64]),
    "ca_state_save": (ctypes.c_int, [ctypes.POINTER(DecodeState), _I32, _I64, _P, _I64, _P]),
    "ca_state_load": (ctypes.c_int, [ctypes.POINTER(DecodeState), _I32, _I64, _P, _I64, _P]),
    "ca_query_proj_workspace": (_SZ, [ctypes.POINTER(QueryProjParams), _I64]),
    "ca_query_proj": (ctypes.c_int, [ctypes.POINTER(QueryProjParams), _P, _I64, _P, _P, _P, _P, _P, _SZ, _P]),
    "ca_out_proj_workspace": (_SZ, [ctypes.POINTER(OutProjParams), _I64]),
    "ca_out_proj": (ctypes.c_int, [ctypes.POINTER(OutProjParams), _P, _I64, _P, _P, _P, _SZ, _P]),
    "ca_timer_start": (ctypes.c_int, [ctypes.c_uint32, _I64]),
    "ca_timer_read": (ctypes.c_int, [_I32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_I64)]),
    "ca_timer_stop": (ctypes.c_int, []),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_SIGS)


def lib():
    return _lib


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(rc: int):
    if rc != 0:
        raise CAError(rc, _lib.ca_last_error().decode())


def record_stride(fmt: int, dim: int, rope_dim: int) -> int:
    return int(_lib.ca_record_stride(fmt, dim, rope_dim))


def page_bytes(fmt: int, dim: int, rope_dim: int, page_size: int) -> int:
    return int(_lib.ca_page_bytes(fmt, dim, rope_dim, page_size))


class Cache:
    """A paged compressed cache: a uint8 page pool plus an int32 page table [n_seqs, max_pages]."""

    def __init__(self, fmt: int, dim: int, rope_dim: int, page_size: int, pool: torch.Tensor,
                 page_table: torch.Tensor):
        if pool.dtype != torch.uint8 or page_table.dtype != torch.int32 or page_table.dim() != 2:
            raise TypeError("pool must be uint8 and page_table int32 [n_seqs, max_pages]")
        pb = page_bytes(fmt, dim, rope_dim, page_size)
        self.fmt, self.dim, self.rope_dim, self.page_size = fmt, dim, rope_dim, page_size
        self.pool, self.page_table = pool, page_table
        self.n_pages = pool.numel() // pb
        self.desc = _Cache(fmt, dim, rope_dim, page_size, pool.data_ptr(), self.n_pages, page_table.data_ptr(),
                           page_table.shape[0], page_table.shape[1])

    @classmethod
    def allocate(cls, fmt, dim, rope_dim, page_size, n_pages, page_table, device="cuda"):
        pool = torch.zeros(n_pages * page_bytes(fmt, dim, rope_dim, page_size), dtype=torch.uint8, device=device)
        return cls(fmt, dim, rope_dim, page_size, pool, page_table.to(device=device, dtype=torch.int32).contiguous())

    @property
    def ref(self):
        return ctypes.byref(self.desc)


def store_entries(cache: Cache, seq: int, first: int, src: torch.Tensor, gain=None, eps=1e-6, apply_rope=True,
                  rope_base=1e4, pos_stride=1, stream=None):
    assert src.dtype == torch.float32
    _check(_lib.ca_store_entries(cache.ref, seq, first, src.shape[0], _ptr(src), _ptr(gain), eps, int(apply_rope),
                                 rope_base, pos_stride, _stream(stream)))


def compress_prefill(p: CompressParams, Ca, Za, Cb, Zb, Ba, Bb, gain, L: int, seq: int, cache: Cache, stream=None,
                     t0: int = 0):
    """Rows hold positions t0..t0+L-1 (t0 > 0: continuing a prefix whose entries the cache holds)."""
    _check(_lib.ca_compress_prefill(ctypes.byref(p), _ptr(Ca), _ptr(Za), _ptr(Cb), _ptr(Zb), _ptr(Ba), _ptr(Bb),
                                    _ptr(gain), L, t0, seq, cache.ref, _stream(stream)))


def compress_decode(p: CompressParams, new_rows, pos, tail, Ba, Bb, gain, cache: Cache, stream=None):
    _check(_lib.ca_compress_decode(ctypes.byref(p), _ptr(new_rows), _ptr(pos), pos.shape[0], _ptr(tail), _ptr(Ba),
                                   _ptr(Bb), _ptr(gain), cache.ref, _stream(stream)))


def window_append(p: WindowParams, kv_raw, gain, window, pos=None, seq=None, stream=None):
    S, W = window.shape[0], window.shape[1]
    _check(_lib.ca_window_append(ctypes.byref(p), _ptr(kv_raw), _ptr(gain), _ptr(pos), _ptr(seq), kv_raw.shape[0],
                                 _ptr(window), W, S, _stream(stream)))


def decode_append(wp: WindowParams, kv_raw, w_gain, window, pos, jobs, stream=None):
    """Window append of row b's token (sequence b) plus the compressor steps of `jobs`, each
    (CompressParams, new_rows, tail, Ba, Bb, gain, Cache), in one launch."""
    S, W = window.shape[0], window.shape[1]
    _check(_lib.ca_decode_append(ctypes.byref(wp), _ptr(kv_raw), _ptr(w_gain), _ptr(pos), pos.shape[0],
                                 _ptr(window), W, S, _jobs_array(jobs), len(jobs), _stream(stream)))


def _jobs_array(jobs):
    arr = (DecodeEntryJob * len(jobs))()
    for q, (p, new_rows, tail, Ba, Bb, gain, cache) in enumerate(jobs):
        arr[q] = DecodeEntryJob(p, _ptr(new_rows), _ptr(tail), _ptr(Ba), _ptr(Bb), _ptr(gain),
                                ctypes.pointer(cache.desc))
    return arr


def csa_decode_step(wp: WindowParams, kv_raw, w_gain, window, jobs, ip: IndexParams, qI, wI, idx, cnt, iws,
                    ap: AttendParams, q, q_gain, pos, max_pos: int, sink, out, ws, lse=None, stream=None):
    """A CSA layer's decode step in one call (jobs: the main entry's and the indexer key's
    (CompressParams, new_rows, tail, Ba, Bb, gain, Cache)); the same results as
    decode_append + index_topk_decode + csa_attend_decode."""
    S, W = window.shape[0], window.shape[1]
    _check(_lib.ca_csa_decode_step(ctypes.byref(wp), _ptr(kv_raw), _ptr(w_gain), _ptr(window), W, S,
                                   _jobs_array(jobs), ctypes.byref(ip), _ptr(qI), _ptr(wI), _ptr(idx), _ptr(cnt),
                                   _ptr(iws), iws.numel(), ctypes.byref(ap), _ptr(q), _ptr(q_gain), _ptr(pos),
                                   pos.shape[0], max_pos, _ptr(sink), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(),
                                   _stream(stream)))


def hca_decode_step(wp: WindowParams, kv_raw, w_gain, window, job, ap: AttendParams, q, q_gain, pos, max_pos: int,
                    sink, out, ws, lse=None, stream=None):
    """An HCA layer's decode step in one call; the same results as decode_append +
    hca_attend_decode."""
    S, W = window.shape[0], window.shape[1]
    _check(_lib.ca_hca_decode_step(ctypes.byref(wp), _ptr(kv_raw), _ptr(w_gain), _ptr(window), W, S,
                                   _jobs_array([job]), ctypes.byref(ap), _ptr(q), _ptr(q_gain), _ptr(pos),
                                   pos.shape[0], max_pos, _ptr(sink), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(),
                                   _stream(stream)))


def static_scratch_bytes() -> int:
    return int(_lib.ca_static_scratch_bytes())


def hca_decode_step_noalloc(wp: WindowParams, kv_raw, w_gain, window, job, ap: AttendParams, q, q_gain, pos,
                            max_pos: int, sink, out, lse=None, stream=None):
    """hca_decode_step with the library's static device scratch instead of a workspace
    (nothing is allocated; calls that overlap on one GPU race)."""
    S, W = window.shape[0], window.shape[1]
    _check(_lib.ca_hca_decode_step_noalloc(ctypes.byref(wp), _ptr(kv_raw), _ptr(w_gain), _ptr(window), W, S,
                                           _jobs_array([job]), ctypes.byref(ap), _ptr(q), _ptr(q_gain), _ptr(pos),
                                           pos.shape[0], max_pos, _ptr(sink), _ptr(out), _ptr(lse),
                                           _stream(stream)))


def decode_state(window, win_format: int, jobs):
    """Descriptor of one layer's decode state: the window ring [S, W, dim] and, per job,
    (tail ring [S, span, narr, dim] fp32, Cache, ratio)."""
    st = DecodeState()
    st.window, st.S, st.W, st.win_dim, st.win_format = window.data_ptr(), window.shape[0], window.shape[1], \
        window.shape[2], win_format
    st.n_jobs = len(jobs)
    st._keep = [c for _, c, _ in jobs]
    for j, (tail, cache, ratio) in enumerate(jobs):
        st.tail[j] = tail.data_ptr()
        st.tail_floats[j] = tail[0].numel()
        st.cache[j] = ctypes.pointer(cache.desc)
        st.ratio[j] = ratio
    return st


def state_bytes(st: DecodeState, pos: int) -> int:
    n = int(_lib.ca_state_bytes(ctypes.byref(st), pos))
    if n < 0:
        raise CAError(-1, _lib.ca_last_error().decode())
    return n


def state_save(st: DecodeState, seq: int, pos: int, buffer, stream=None):
    _check(_lib.ca_state_save(ctypes.byref(st), seq, pos, _ptr(buffer), buffer.numel(), _stream(stream)))


def state_load(st: DecodeState, seq: int, pos: int, buffer, stream=None):
    _check(_lib.ca_state_load(ctypes.byref(st), seq, pos, _ptr(buffer), buffer.numel(), _stream(stream)))


def index_topk_workspace(p: IndexParams, n_rows: int, max_pos: int) -> int:
    return int(_lib.ca_index_topk_workspace(ctypes.byref(p), n_rows, max_pos))


def index_topk_prefill(p: IndexParams, qI, w, seq: int, idx_cache: Cache, out_idx, out_cnt, out_score=None,
                       all_scores=None, ws=None, stream=None, t0: int = 0):
    L = qI.shape[0]
    if ws is None:
        ws = torch.empty(max(1, index_topk_workspace(p, L, max(t0 + L - 1, 0))), dtype=torch.uint8,
                         device=qI.device)
    st = all_scores.shape[1] if all_scores is not None else 0
    _check(_lib.ca_index_topk_prefill(ctypes.byref(p), _ptr(qI), _ptr(w), L, t0, seq, idx_cache.ref, _ptr(out_idx),
                                      _ptr(out_cnt), _ptr(out_score), _ptr(all_scores), st, _ptr(ws),
                                      0 if ws is None else ws.numel(), _stream(stream)))


def index_topk_decode(p: IndexParams, qI, w, pos, max_pos: int, idx_cache: Cache, out_idx, out_cnt,
                      out_score=None, all_scores=None, ws=None, stream=None):
    B = qI.shape[0]
    if ws is None:   # also with all_scores: the long-row top-k state lives in the workspace
        ws = torch.empty(max(1, index_topk_workspace(p, B, max_pos)), dtype=torch.uint8, device=qI.device)
    st = all_scores.shape[1] if all_scores is not None else 0
    _check(_lib.ca_index_topk_decode(ctypes.byref(p), _ptr(qI), _ptr(w), _ptr(pos), B, max_pos, idx_cache.ref,
                                     _ptr(out_idx), _ptr(out_cnt), _ptr(out_score), _ptr(all_scores), st, _ptr(ws),
                                     0 if ws is None else ws.numel(), _stream(stream)))


def attend_decode_plan(p: AttendParams, total: int):
    """(chunk length, chunks, most chunks of any row up to `total` items) of the decode split plan."""
    ln, n, mx = _I32(0), _I32(0), _I32(0)
    _check(_lib.ca_attend_decode_plan(ctypes.byref(p), total, ctypes.byref(ln), ctypes.byref(n), ctypes.byref(mx)))
    return ln.value, n.value, mx.value


def attend_workspace(p: AttendParams, n_rows: int, max_pos: int, k: int, ratio: int) -> int:
    return int(_lib.ca_attend_workspace(ctypes.byref(p), n_rows, max_pos, k, ratio))


def csa_attend_prefill(p: AttendParams, q, q_gain, kv: Cache, seq: int, idx, cnt, ratio: int, window, sink, out,
                       lse=None, stream=None, t0: int = 0):
    L, k = q.shape[0], idx.shape[1]
    _check(_lib.ca_csa_attend_prefill(ctypes.byref(p), _ptr(q), _ptr(q_gain), kv.ref, seq, _ptr(idx), _ptr(cnt), k,
                                      ratio, _ptr(window), window.shape[1], _ptr(sink), L, t0, _ptr(out), _ptr(lse),
                                      None, 0, _stream(stream)))


def csa_attend_decode(p: AttendParams, q, q_gain, kv: Cache, idx, cnt, ratio: int, pos, max_pos: int, window, sink,
                      out, lse=None, ws=None, stream=None):
    B, k = q.shape[0], idx.shape[1]
    if ws is None:
        ws = torch.empty(max(1, attend_workspace(p, B, max_pos, k, ratio)), dtype=torch.uint8, device=q.device)
    _check(_lib.ca_csa_attend_decode(ctypes.byref(p), _ptr(q), _ptr(q_gain), kv.ref, _ptr(idx), _ptr(cnt), k, ratio,
                                     _ptr(pos), B, max_pos, _ptr(window), window.shape[1], _ptr(sink), _ptr(out),
                                     _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)))


def hca_attend_prefill(p: AttendParams, q, q_gain, kv: Cache, seq: int, ratio: int, window, sink, out, lse=None,
                       stream=None, t0: int = 0):
    L = q.shape[0]
    _check(_lib.ca_hca_attend_prefill(ctypes.byref(p), _ptr(q), _ptr(q_gain), kv.ref, seq, ratio, _ptr(window),
                                      window.shape[1], _ptr(sink), L, t0, _ptr(out), _ptr(lse), None, 0,
                                      _stream(stream)))


def hca_attend_decode(p: AttendParams, q, q_gain, kv: Cache, ratio: int, pos, max_pos: int, window, sink, out,
                      lse=None, ws=None, stream=None):
    B = q.shape[0]
    if ws is None:
        ws = torch.empty(max(1, attend_workspace(p, B, max_pos, 0, ratio)), dtype=torch.uint8, device=q.device)
    _check(_lib.ca_hca_attend_decode(ctypes.byref(p), _ptr(q), _ptr(q_gain), kv.ref, ratio, _ptr(pos), B, max_pos,
                                     _ptr(window), window.shape[1], _ptr(sink), _ptr(out), _ptr(lse), _ptr(ws),
                                     ws.numel(), _stream(stream)))


# ---------------------------------------------------------------- launch timing (diagnostics)
TIMED_CSA_ATTEND, TIMED_HCA_ATTEND, TIMED_INDEX_SCORES, TIMED_PROJ_GEMM = 0, 1, 2, 3


def timer_start(kernels, max_launches: int = 4096):
    """Bracket every later eager launch of the given kernels with HIP events on their stream."""
    mask = 0
    for k in kernels:
        mask |= 1 << k
    _check(_lib.ca_timer_start(mask, max_launches))


def timer_read(kernel: int):
    """(summed milliseconds, launch count) of the kernel's timed launches; waits for the last one."""
    ms, n = ctypes.c_double(0.0), ctypes.c_int64(0)
    _check(_lib.ca_timer_read(kernel, ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def timer_stop():
    _check(_lib.ca_timer_stop())


# ------------------------------------------------------------ sublayer projections
class QueryProj:
    """Weights of the low-rank query projections (bf16 [out, in] tensors on the device):
    w_dq [d_c, d], w_uq [n_h c, d_c], w_iuq [n_I c_I, d_c] and w_w [n_I, d] (the last two
    None for an HCA layer, which has no indexer)."""

    def __init__(self, w_dq, w_uq, w_iuq=None, w_w=None):
        self.w = (w_dq, w_uq, w_iuq, w_w)
        n_qi = 0 if w_iuq is None else w_iuq.shape[0]
        n_i = 0 if w_w is None else w_w.shape[0]
        self.p = QueryProjParams(w_dq.shape[1], w_dq.shape[0], w_uq.shape[0], n_qi, n_i, _ptr(w_dq), _ptr(w_uq),
                                 _ptr(w_iuq), _ptr(w_w))

    def workspace(self, T: int) -> int:
        return int(_lib.ca_query_proj_workspace(ctypes.byref(self.p), T))

    def __call__(self, h, c_q, q, q_i=None, w_i=None, ws=None, stream=None):
        T = h.shape[0]
        if ws is None:
            ws = torch.empty(max(1, self.workspace(T)), dtype=torch.uint8, device=h.device)
        _check(_lib.ca_query_proj(ctypes.byref(self.p), _ptr(h), T, _ptr(c_q), _ptr(q), _ptr(q_i), _ptr(w_i),
                                  _ptr(ws), ws.numel(), _stream(stream)))


class OutProj:
    """Weights of the grouped output projection: w_o1 [g, d_g, 8 c] and w_o2 [d, g d_g] (bf16)."""

    def __init__(self, w_o1, w_o2, c: int):
        self.w = (w_o1, w_o2)
        g, d_g, _ = w_o1.shape
        self.p = OutProjParams(8 * g, c, d_g, w_o2.shape[0], _ptr(w_o1), _ptr(w_o2))

    def workspace(self, T: int) -> int:
        return int(_lib.ca_out_proj_workspace(ctypes.byref(self.p), T))

    def __call__(self, o, u, y, ws=None, stream=None):
        T = o.shape[0]
        if ws is None:
            ws = torch.empty(max(1, self.workspace(T)), dtype=torch.uint8, device=o.device)
        _check(_lib.ca_out_proj(ctypes.byref(self.p), _ptr(o), T, _ptr(u), _ptr(y), _ptr(ws), ws.numel(),
                                _stream(stream)))
