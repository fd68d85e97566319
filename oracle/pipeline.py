"""Oracle orchestration of one CSA or HCA layer, prefill and decode -- TEST INFRASTRUCTURE ONLY.

The steps run in the order the dsv4 book gives them:
  CSA (Ch.5-6): compress main KV (overlapping 2m softmax pooling) -> RMSNorm ->
      RoPE at m*i -> store; compress indexer keys the same way (no norm, no
      RoPE) -> store; window tokens RMSNorm -> RoPE; indexer scores over
      s < floor(t/m); top-k; shared-KV attention over the selected entries
      plus the window with the sink; de-rotation of the output.
  HCA (Ch.7): disjoint m' pooling -> RMSNorm -> RoPE -> store; dense attention
      over i < floor(t/m') plus the window.
Inputs are torch tensors or numpy arrays straight from the seeded generator;
they are turned into float64 numpy arrays here.
"""
from __future__ import annotations

import numpy as np

from . import (FMT_BY_NAME, FMT_E4M3, FMT_F32, FMT_FP4, attend, bf16_encode, compress, compress_entry,
               dequantize_rows_e4m3, finish_store, index_scores, load_entries, page_bytes, quantize_rows_e4m3,
               topk, window_prep)


def f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float64).numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def take_rows(x, rows) -> np.ndarray:
    """float64 copy of x[rows] (rows selected before the conversion, so a large device
    tensor is never converted whole)."""
    if hasattr(x, "detach"):
        import torch
        idx = torch.as_tensor(np.asarray(rows, np.int64), device=x.device)
        return f64(x[idx])
    return f64(np.asarray(x)[np.asarray(rows)])


def store_window(values: np.ndarray, act: str) -> np.ndarray:
    """Round processed window rows to their storage format (fp32 or bf16 bits)."""
    if act == "f32":
        return values.astype(np.float32)
    return bf16_encode(values)


def indexer_query_values(qI: np.ndarray, idx_fmt: str, q_quant: str = "e4m3") -> np.ndarray:
    """The indexer query as the indexer sees it: e4m3 with one power-of-two
    scale per (token, head) for e4m3 and FP4 key pools (FP4 keys meet fp8
    queries, the mixed FP4 x FP8 product of the dsv4 book Ch.8 "FLOP
    comparison" note), unchanged for fp32 ones.  With q_quant "fp4" (FP4 keys
    only; Ch.6 "The lightning indexer" runs the whole indexer in FP4) every
    (token, head) row is quantized exactly as an FP4 key is stored: e2m1 codes
    with one power of two per 32 channels, encoded into an FP4 page and read
    back with the same codec."""
    if idx_fmt == "f32":
        return qI
    if q_quant == "fp4":
        assert idx_fmt == "fp4", "FP4 queries meet FP4 keys"
        shape = qI.shape
        rows = np.ascontiguousarray(qI, np.float64).reshape(-1, shape[-1])
        n, c = rows.shape
        P = 64
        pages = max(1, -(-n // P))
        pool = new_pool(pages, FMT_FP4, c, 0, P)
        pt = np.arange(pages, dtype=np.int32)
        if n:
            finish_store(FMT_FP4, c, 0, P, pool, pt, 0, rows, None, 0.0, 1.0, 1, False, False)
        return load_entries(FMT_FP4, c, 0, P, pool, pt, 0, n).reshape(shape)
    codes, exps = quantize_rows_e4m3(qI)
    return dequantize_rows_e4m3(codes, exps)


def new_pool(n_pages: int, fmt: int, D: int, R: int, P: int) -> np.ndarray:
    return np.zeros(n_pages * page_bytes(fmt, D, R, P), np.uint8)


def csa_prefill(cfg, inp: dict, pt_row, n_pool_pages: int, rows=None, idx_override=None, want_lse=False) -> dict:
    """One CSA prefill layer over a single sequence.  `rows` restricts the
    indexer / top-k / attention to a subset of query rows; `idx_override`
    (idx, cnt) replaces the oracle's own top-k in the attention step; with
    want_lse the result also holds each row's log softmax denominator "lse"."""
    L, D, R, P, m = inp["L"], cfg.D, cfg.R, cfg.page, cfg.m
    kv_fmt, idx_fmt = FMT_BY_NAME[cfg.kv], FMT_BY_NAME[cfg.idx]
    pt_row = np.asarray(pt_row, np.int32)
    res = {}
    E = compress(m, 1, f64(inp["Ca"]), f64(inp["Za"]), f64(inp["Ba"]), f64(inp["Cb"]), f64(inp["Zb"]),
                 f64(inp["Bb"]))
    pool = new_pool(n_pool_pages, kv_fmt, D, R, P)
    finish_store(kv_fmt, D, R, P, pool, pt_row, 0, E, f64(inp["g_kv"]), cfg.eps, cfg.rope_base, m, True, True)
    EI = compress(m, 1, f64(inp["ICa"]), f64(inp["IZa"]), f64(inp["IBa"]), f64(inp["ICb"]), f64(inp["IZb"]),
                  f64(inp["IBb"]))
    ipool = new_pool(n_pool_pages, idx_fmt, cfg.cI, 0, P)
    finish_store(idx_fmt, cfg.cI, 0, P, ipool, pt_row, 0, EI, None, cfg.eps, cfg.rope_base, m, False, False)
    res.update(entries_raw=E, pool=pool, ikeys_raw=EI, ipool=ipool, n_entries=E.shape[0])
    pos_all = np.arange(L, dtype=np.int64)
    win = store_window(window_prep(f64(inp["kv_raw"]), pos_all, R, f64(inp["g_w"]), cfg.eps, cfg.rope_base),
                       cfg.act)[None]
    res["window"] = win
    rows = pos_all if rows is None else np.asarray(rows, np.int64)
    res["rows"] = rows
    qI = indexer_query_values(take_rows(inp["qI"], rows), cfg.idx, getattr(cfg, "idx_q", "e4m3"))
    scores, n_elig = index_scores(qI, take_rows(inp["w"], rows), rows, m, idx_fmt, P, ipool, pt_row[None],
                                  [E.shape[0]], n_cols=max(1, E.shape[0]))
    idx, cnt = topk(scores, n_elig, cfg.k)
    res.update(scores=scores, n_elig=n_elig, idx=idx, cnt=cnt, qI=qI)
    a_idx, a_cnt = (idx, cnt) if idx_override is None else idx_override
    o = attend(take_rows(inp["q"], rows), rows, kv_fmt, P, pool, pt_row[None], [E.shape[0]], 0, m, win,
               cfg.n_win, f64(inp["sink"]), R, gq=f64(inp["g_q"]), idx=a_idx, cnt=a_cnt,
               base=cfg.rope_base, eps=cfg.eps, want_lse=want_lse)
    res["out"], res["lse"] = o if want_lse else (o, None)
    return res


def hca_prefill(cfg, inp: dict, pt_row, n_pool_pages: int, rows=None, want_lse=False) -> dict:
    L, D, R, P, m = inp["L"], cfg.D, cfg.R, cfg.page, cfg.m_hca
    kv_fmt = FMT_BY_NAME[cfg.kv]
    pt_row = np.asarray(pt_row, np.int32)
    E = compress(m, 0, f64(inp["C"]), f64(inp["Z"]), f64(inp["B"]))
    pool = new_pool(n_pool_pages, kv_fmt, D, R, P)
    finish_store(kv_fmt, D, R, P, pool, pt_row, 0, E, f64(inp["g_kv"]), cfg.eps, cfg.rope_base, m, True, True)
    pos_all = np.arange(L, dtype=np.int64)
    win = store_window(window_prep(f64(inp["kv_raw"]), pos_all, R, f64(inp["g_w"]), cfg.eps, cfg.rope_base),
                       cfg.act)[None]
    rows = pos_all if rows is None else np.asarray(rows, np.int64)
    o = attend(take_rows(inp["q"], rows), rows, kv_fmt, P, pool, pt_row[None], [E.shape[0]], 1, m, win, cfg.n_win,
               f64(inp["sink"]), R, gq=f64(inp["g_q"]), base=cfg.rope_base, eps=cfg.eps, want_lse=want_lse)
    out, lse = o if want_lse else (o, None)
    return dict(entries_raw=E, pool=pool, window=win, rows=rows, out=out, lse=lse, n_entries=E.shape[0])


def decode_state(cfg, inp: dict, seqs=None) -> dict:
    """Build the oracle's view of a decode layer's caches from the raw
    generator state: every stored entry gets the entry epilogue and is encoded
    through the page table; window rows for positions t-n_win+1..t are
    normalized, rotated and stored at slot position mod n_win."""
    D, R, P = cfg.D, cfg.R, cfg.page
    layer, ratio = inp["layer"], inp["ratio"]
    kv_fmt = FMT_BY_NAME[cfg.kv]
    pt = np.asarray(inp["page_table"].cpu() if hasattr(inp["page_table"], "cpu") else inp["page_table"], np.int32)
    B = pt.shape[0]
    seqs = range(B) if seqs is None else seqs
    offs = inp["entry_offsets"]
    pool = new_pool(inp["n_pool_pages"], kv_fmt, D, R, P)
    g_kv = f64(inp["g_kv"])
    ipool = None
    if layer == "csa":
        idx_fmt = FMT_BY_NAME[cfg.idx]
        ipool = new_pool(inp["n_pool_pages"], idx_fmt, cfg.cI, 0, P)
    for b in seqs:
        a, e = offs[b], offs[b + 1]
        if e > a:
            finish_store(kv_fmt, D, R, P, pool, pt[b], 0, f64(inp["entries"][a:e]), g_kv, cfg.eps, cfg.rope_base,
                         ratio, True, True)
            if ipool is not None:
                finish_store(FMT_BY_NAME[cfg.idx], cfg.cI, 0, P, ipool, pt[b], 0, f64(inp["ikeys"][a:e]), None,
                             cfg.eps, cfg.rope_base, ratio, False, False)
    pos = np.asarray(inp["pos"], np.int64)
    W = cfg.n_win
    raw = f64(inp["kv_raw"])
    g_w = f64(inp["g_w"])
    win_vals = np.zeros((B, W, D))
    for b in seqs:
        p = pos[b] - W + 1 + np.arange(W)
        ok = p >= 0
        vals = window_prep(raw[b][ok], p[ok], R, g_w, cfg.eps, cfg.rope_base)
        win_vals[b, p[ok] % W] = vals
    return dict(pool=pool, ipool=ipool, page_table=pt, window=store_window(win_vals, cfg.act),
                n_avail=np.asarray(inp["n_entries"], np.int64), pos=pos)


def decode_compress(cfg, inp: dict, b: int):
    """The entry the new token of sequence b completes (None if it completes
    none), computed from the tail ring plus the new token's rows.  Returns
    (entry index, main entry values before the epilogue, indexer key values)."""
    layer, ratio = inp["layer"], inp["ratio"]
    t = int(inp["pos"][b])
    if (t + 1) % ratio:
        return None
    i = (t + 1) // ratio - 1
    tail = f64(inp["tail"][b])            # [span, narr, D]
    new = f64(inp["new_rows"][b])         # [narr, D]
    span = tail.shape[0]

    def rows(arr, first, n, tl, nw):
        out = []
        for p in range(first, first + n):
            out.append(nw[arr] if p == t else tl[p % span, arr])
        return np.stack(out)

    if layer == "csa":
        # ring arrays per slot: 0 = C^a, 1 = C^b, 2 = Z^a, 3 = Z^b
        m = ratio
        e_main = compress_entry(m, 1, i > 0, rows(0, m * i, m, tail, new), rows(2, m * i, m, tail, new),
                                rows(1, m * (i - 1), m, tail, new) if i > 0 else None,
                                rows(3, m * (i - 1), m, tail, new) if i > 0 else None,
                                f64(inp["Ba"]), f64(inp["Bb"]))
        itail, inew = f64(inp["itail"][b]), f64(inp["new_irows"][b])
        e_idx = compress_entry(m, 1, i > 0, rows(0, m * i, m, itail, inew), rows(2, m * i, m, itail, inew),
                               rows(1, m * (i - 1), m, itail, inew) if i > 0 else None,
                               rows(3, m * (i - 1), m, itail, inew) if i > 0 else None,
                               f64(inp["IBa"]), f64(inp["IBb"]))
        return i, e_main, e_idx
    m = ratio
    e_main = compress_entry(m, 0, False, rows(0, m * i, m, tail, new), rows(1, m * i, m, tail, new), None, None,
                            f64(inp["B"]), None)
    return i, e_main, None


def csa_decode_step(cfg, inp: dict, state: dict, seqs=None, idx_override=None, want_lse=False) -> dict:
    """Indexer, top-k and attention for the new token of each sequence
    (`idx_override` (idx, cnt) replaces the oracle's own top-k in the attention)."""
    B = state["page_table"].shape[0]
    seqs = np.arange(B) if seqs is None else np.asarray(seqs)
    pos = state["pos"][seqs]
    qI = indexer_query_values(f64(inp["qI"])[seqs], cfg.idx, getattr(cfg, "idx_q", "e4m3"))
    n_cols = int(max(1, state["n_avail"].max()))
    scores, n_elig = index_scores(qI, f64(inp["w"])[seqs], pos, cfg.m, FMT_BY_NAME[cfg.idx], cfg.page,
                                  state["ipool"], state["page_table"], state["n_avail"], seq=seqs, n_cols=n_cols)
    idx, cnt = topk(scores, n_elig, cfg.k)
    a_idx, a_cnt = (idx, cnt) if idx_override is None else idx_override
    o = attend(f64(inp["q"])[seqs], pos, FMT_BY_NAME[cfg.kv], cfg.page, state["pool"], state["page_table"],
               state["n_avail"], 0, cfg.m, state["window"], cfg.n_win, f64(inp["sink"]), cfg.R,
               gq=f64(inp["g_q"]), seq=seqs, idx=a_idx, cnt=a_cnt, base=cfg.rope_base, eps=cfg.eps,
               want_lse=want_lse)
    out, lse = o if want_lse else (o, None)
    return dict(scores=scores, n_elig=n_elig, idx=idx, cnt=cnt, out=out, lse=lse, seqs=seqs, qI=qI)


def hca_decode_step(cfg, inp: dict, state: dict, seqs=None, want_lse=False) -> dict:
    B = state["page_table"].shape[0]
    seqs = np.arange(B) if seqs is None else np.asarray(seqs)
    pos = state["pos"][seqs]
    o = attend(f64(inp["q"])[seqs], pos, FMT_BY_NAME[cfg.kv], cfg.page, state["pool"], state["page_table"],
               state["n_avail"], 1, cfg.m_hca, state["window"], cfg.n_win, f64(inp["sink"]), cfg.R,
               gq=f64(inp["g_q"]), seq=seqs, base=cfg.rope_base, eps=cfg.eps, want_lse=want_lse)
    out, lse = o if want_lse else (o, None)
    return dict(out=out, lse=lse, seqs=seqs)


__all__ = ["f64", "take_rows", "csa_prefill", "hca_prefill", "decode_state", "decode_compress", "csa_decode_step",
           "hca_decode_step", "indexer_query_values", "store_window", "new_pool", "FMT_E4M3", "FMT_F32"]
