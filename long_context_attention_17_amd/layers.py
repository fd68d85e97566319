"""One CSA or HCA layer, prefill and decode, as a sequence of library calls.

The order follows the dsv4 book: CSA (Ch.5-6) compresses the main KV stream
and the indexer keys (overlapping 2m pooling), normalizes/rotates the window
tokens, scores the eligible blocks with the lightning indexer, keeps the top-k
and attends over them plus the window; HCA (Ch.7) compresses with disjoint m'
blocks and attends densely.  Every step is a call into libcsahca.so; this
module only allocates outputs (torch) and passes pointers.
"""
from __future__ import annotations

import math

import torch

from . import binding as ca
from .configs import Config, get


def act_format(cfg: Config) -> int:
    return ca.F32 if cfg.act == "f32" else ca.BF16


def act_dtype(cfg: Config):
    return torch.float32 if cfg.act == "f32" else torch.bfloat16


def attend_params(cfg: Config) -> ca.AttendParams:
    a = act_format(cfg)
    return ca.AttendParams(cfg.n_h, cfg.D, cfg.R, cfg.n_win, a, a, a, 1.0 / math.sqrt(cfg.D), cfg.eps, cfg.rope_base)


def compress_params(cfg: Config, ratio: int, overlap: bool, main: bool) -> ca.CompressParams:
    return ca.CompressParams(ratio, int(overlap), act_format(cfg), int(main), int(main), cfg.eps, cfg.rope_base)


def window_params(cfg: Config) -> ca.WindowParams:
    a = act_format(cfg)
    return ca.WindowParams(cfg.D, cfg.R, a, a, cfg.eps, cfg.rope_base)


def index_params(cfg: Config) -> ca.IndexParams:
    return ca.IndexParams(cfg.nI, cfg.cI, cfg.m, cfg.k, act_format(cfg), ca.FP4 if cfg.idx_q == "fp4" else 0)


def main_cache(cfg: Config, page_table: torch.Tensor, n_pages: int, device="cuda") -> ca.Cache:
    return ca.Cache.allocate(ca.FORMATS[cfg.kv], cfg.D, cfg.R, cfg.page, n_pages, page_table, device)


def index_cache(cfg: Config, page_table: torch.Tensor, n_pages: int, device="cuda") -> ca.Cache:
    return ca.Cache.allocate(ca.FORMATS[cfg.idx], cfg.cI, 0, cfg.page, n_pages, page_table, device)


# ------------------------------------------------------------------ prefill
class CSAPrefill:
    """CSA prefill of one sequence; each stage can run on its own, over all rows or
    over positions [t0, t1) (continuing a prefix whose entries the cache holds)."""

    def __init__(self, cfg, inp: dict, page_table: torch.Tensor, n_pages: int):
        self.cfg = cfg = get(cfg)
        self.inp, self.L = inp, inp["L"]
        dev = inp["q"].device
        self.kv = main_cache(cfg, page_table, n_pages, dev)
        self.ik = index_cache(cfg, page_table, n_pages, dev)
        self.window = torch.empty(1, self.L, cfg.D, dtype=act_dtype(cfg), device=dev)
        self.idx = torch.empty(self.L, cfg.k, dtype=torch.int32, device=dev)
        self.cnt = torch.empty(self.L, dtype=torch.int32, device=dev)
        self.out = torch.empty(self.L, cfg.n_h, cfg.D, dtype=act_dtype(cfg), device=dev)
        self.ws = torch.empty(max(1, ca.index_topk_workspace(index_params(cfg), self.L, max(self.L - 1, 0))),
                              dtype=torch.uint8, device=dev)
        self.ap, self.ip = attend_params(cfg), index_params(cfg)

    def compress(self, t0: int = 0, t1: int | None = None):
        """Entries whose pooling window lies in rows [t0, t1) (all of them for t0 = 0)."""
        c, i = self.cfg, self.inp
        t1 = self.L if t1 is None else t1
        r = slice(t0, t1)
        ca.compress_prefill(compress_params(c, c.m, True, True), i["Ca"][r], i["Za"][r], i["Cb"][r], i["Zb"][r],
                            i["Ba"], i["Bb"], i["g_kv"], t1 - t0, 0, self.kv, t0=t0)
        ca.compress_prefill(compress_params(c, c.m, True, False), i["ICa"][r], i["IZa"][r], i["ICb"][r], i["IZb"][r],
                            i["IBa"], i["IBb"], None, t1 - t0, 0, self.ik, t0=t0)

    def window_append(self, t0: int = 0, t1: int | None = None):
        _window_rows(self, t0, t1)

    def index_topk(self, out_score=None, all_scores=None, t0: int = 0, t1: int | None = None):
        t1 = self.L if t1 is None else t1
        r = slice(t0, t1)
        ca.index_topk_prefill(self.ip, self.inp["qI"][r], self.inp["w"][r], 0, self.ik, self.idx[r], self.cnt[r],
                              out_score, all_scores, self.ws if all_scores is None else None, t0=t0)

    def attend(self, idx=None, cnt=None, lse=None, t0: int = 0, t1: int | None = None):
        t1 = self.L if t1 is None else t1
        r = slice(t0, t1)
        ca.csa_attend_prefill(self.ap, self.inp["q"][r], self.inp["g_q"], self.kv, 0,
                              (self.idx if idx is None else idx)[r], (self.cnt if cnt is None else cnt)[r], self.cfg.m,
                              self.window, self.inp["sink"], self.out[r], lse, t0=t0)

    def run(self):
        self.compress()
        self.window_append()
        self.index_topk()
        self.attend()
        return self.out


def _window_rows(layer, t0, t1):
    """Window rows of positions [t0, t1) (all positions by default) into the layer's window."""
    t1 = layer.L if t1 is None else t1
    raw = layer.inp["kv_raw"]
    if t0 == 0 and t1 == layer.L:
        ca.window_append(window_params(layer.cfg), raw, layer.inp["g_w"], layer.window)
        return
    pos = torch.arange(t0, t1, dtype=torch.int32, device=raw.device)
    ca.window_append(window_params(layer.cfg), raw[t0:t1], layer.inp["g_w"], layer.window, pos=pos)


class HCAPrefill:
    def __init__(self, cfg, inp: dict, page_table: torch.Tensor, n_pages: int):
        self.cfg = cfg = get(cfg)
        self.inp, self.L = inp, inp["L"]
        dev = inp["q"].device
        self.kv = main_cache(cfg, page_table, n_pages, dev)
        self.window = torch.empty(1, self.L, cfg.D, dtype=act_dtype(cfg), device=dev)
        self.out = torch.empty(self.L, cfg.n_h, cfg.D, dtype=act_dtype(cfg), device=dev)
        self.ap = attend_params(cfg)

    def compress(self, t0: int = 0, t1: int | None = None):
        c, i = self.cfg, self.inp
        t1 = self.L if t1 is None else t1
        r = slice(t0, t1)
        ca.compress_prefill(compress_params(c, c.m_hca, False, True), i["C"][r], i["Z"][r], None, None, i["B"], None,
                            i["g_kv"], t1 - t0, 0, self.kv, t0=t0)

    def window_append(self, t0: int = 0, t1: int | None = None):
        _window_rows(self, t0, t1)

    def attend(self, lse=None, t0: int = 0, t1: int | None = None):
        t1 = self.L if t1 is None else t1
        r = slice(t0, t1)
        ca.hca_attend_prefill(self.ap, self.inp["q"][r], self.inp["g_q"], self.kv, 0, self.cfg.m_hca, self.window,
                              self.inp["sink"], self.out[r], lse, t0=t0)

    def run(self):
        self.compress()
        self.window_append()
        self.attend()
        return self.out


# ------------------------------------------------------------------ decode
class DecodeLayer:
    """Decode state of one CSA or HCA layer for a batch, built from the raw
    generator state (cache entries get the entry epilogue on the GPU), and one
    decode step for the new token of every sequence."""

    def __init__(self, cfg, inp: dict, device="cuda"):
        self.cfg = cfg = get(cfg)
        self.inp = inp
        self.layer, self.ratio = inp["layer"], inp["ratio"]
        self.B = B = inp["q"].shape[0]
        dev = torch.device(device)
        self.pos = inp["pos"].to(device=dev, dtype=torch.int32)
        self.max_pos = int(inp["pos"].max())
        self.seq_ids = torch.arange(B, dtype=torch.int32, device=dev)
        pt = inp["page_table"].to(dev)
        self.kv = main_cache(cfg, pt, inp["n_pool_pages"], dev)
        offs = inp["entry_offsets"]
        for b in range(B):
            a, e = offs[b], offs[b + 1]
            if e > a:
                ca.store_entries(self.kv, b, 0, inp["entries"][a:e], inp["g_kv"], cfg.eps, True, cfg.rope_base,
                                 self.ratio)
        self.ik = None
        if self.layer == "csa":
            self.ik = index_cache(cfg, pt, inp["n_pool_pages"], dev)
            for b in range(B):
                a, e = offs[b], offs[b + 1]
                if e > a:
                    ca.store_entries(self.ik, b, 0, inp["ikeys"][a:e], None, cfg.eps, False, cfg.rope_base, 1)
        # window ring: positions t-n_win+1 .. t-1 now; the step appends t
        W = cfg.n_win
        self.window = torch.zeros(B, W, cfg.D, dtype=act_dtype(cfg), device=dev)
        rel = torch.arange(W - 1, device=dev, dtype=torch.int32)
        wpos = (self.pos[:, None] - (W - 1) + rel[None, :])
        wseq = self.seq_ids[:, None].expand(B, W - 1)
        keep = (wpos >= 0).reshape(-1)
        raw = inp["kv_raw"][:, :W - 1].reshape(B * (W - 1), cfg.D)[keep].contiguous()
        ca.window_append(window_params(cfg), raw, inp["g_w"], self.window,
                         pos=wpos.reshape(-1)[keep].contiguous(), seq=wseq.reshape(-1)[keep].contiguous())
        self.new_kv = inp["kv_raw"][:, W - 1].contiguous()
        self.tail = inp["tail"].to(dev).contiguous()
        self.new_rows = inp["new_rows"].contiguous()
        if self.layer == "csa":
            self.itail = inp["itail"].to(dev).contiguous()
            self.new_irows = inp["new_irows"].contiguous()
            self.idx = torch.empty(B, cfg.k, dtype=torch.int32, device=dev)
            self.cnt = torch.empty(B, dtype=torch.int32, device=dev)
            self.ip = index_params(cfg)
            self.iws = torch.empty(max(1, ca.index_topk_workspace(self.ip, B, self.max_pos)), dtype=torch.uint8,
                                   device=dev)
        self.ap = attend_params(cfg)
        k = cfg.k if self.layer == "csa" else 0
        self.aws = torch.empty(max(1, ca.attend_workspace(self.ap, B, self.max_pos, k, self.ratio)),
                               dtype=torch.uint8, device=dev)
        self.out = torch.empty(B, cfg.n_h, cfg.D, dtype=act_dtype(cfg), device=dev)

    # individual stages
    def _append_jobs(self):
        c, i = self.cfg, self.inp
        if self.layer == "csa":
            return [(compress_params(c, c.m, True, True), self.new_rows, self.tail, i["Ba"], i["Bb"], i["g_kv"],
                     self.kv),
                    (compress_params(c, c.m, True, False), self.new_irows, self.itail, i["IBa"], i["IBb"], None,
                     self.ik)]
        return [(compress_params(c, c.m_hca, False, True), self.new_rows, self.tail, i["B"], None, i["g_kv"],
                 self.kv)]

    def append(self):
        """The new token's window append and compressor step(s) in one launch: the same
        results, bit for bit, as append_token() followed by compress()."""
        ca.decode_append(window_params(self.cfg), self.new_kv, self.inp["g_w"], self.window, self.pos,
                         self._append_jobs())

    def fused_step(self):
        """The whole decode step in one library call (ca_csa_decode_step / ca_hca_decode_step):
        the same results as step(), with the query preparation and the top-k state clearing
        folded into the append launch."""
        c, i = self.cfg, self.inp
        jobs = self._append_jobs()
        if self.layer == "csa":
            ca.csa_decode_step(window_params(c), self.new_kv, i["g_w"], self.window, jobs, self.ip, i["qI"], i["w"],
                               self.idx, self.cnt, self.iws, self.ap, i["q"], i["g_q"], self.pos, self.max_pos,
                               i["sink"], self.out, self.aws)
        else:
            ca.hca_decode_step(window_params(c), self.new_kv, i["g_w"], self.window, jobs[0], self.ap, i["q"],
                               i["g_q"], self.pos, self.max_pos, i["sink"], self.out, self.aws)
        return self.out

    def fused_step_noalloc(self):
        """HCA only: fused_step() with the library's static device scratch instead of the
        layer's attention workspace (ca_hca_decode_step_noalloc)."""
        c, i = self.cfg, self.inp
        assert self.layer == "hca", "the allocation-free step is the HCA layer's"
        ca.hca_decode_step_noalloc(window_params(c), self.new_kv, i["g_w"], self.window, self._append_jobs()[0],
                                   self.ap, i["q"], i["g_q"], self.pos, self.max_pos, i["sink"], self.out)
        return self.out

    def state(self):
        """Descriptor of this layer's decode state (ca_state_save / ca_state_load)."""
        jobs = [(self.tail, self.kv, self.ratio)]
        if self.layer == "csa":
            jobs.append((self.itail, self.ik, self.ratio))
        return ca.decode_state(self.window, act_format(self.cfg), jobs)

    def append_token(self):
        ca.window_append(window_params(self.cfg), self.new_kv, self.inp["g_w"], self.window, pos=self.pos,
                         seq=self.seq_ids)

    def compress(self):
        c, i = self.cfg, self.inp
        if self.layer == "csa":
            ca.compress_decode(compress_params(c, c.m, True, True), self.new_rows, self.pos, self.tail, i["Ba"],
                               i["Bb"], i["g_kv"], self.kv)
            ca.compress_decode(compress_params(c, c.m, True, False), self.new_irows, self.pos, self.itail, i["IBa"],
                               i["IBb"], None, self.ik)
        else:
            ca.compress_decode(compress_params(c, c.m_hca, False, True), self.new_rows, self.pos, self.tail, i["B"],
                               None, i["g_kv"], self.kv)

    def index_topk(self, out_score=None, all_scores=None):
        ca.index_topk_decode(self.ip, self.inp["qI"], self.inp["w"], self.pos, self.max_pos, self.ik, self.idx,
                             self.cnt, out_score, all_scores, self.iws if all_scores is None else None)

    def attend(self, idx=None, cnt=None, lse=None):
        if self.layer == "csa":
            ca.csa_attend_decode(self.ap, self.inp["q"], self.inp["g_q"], self.kv, self.idx if idx is None else idx,
                                 self.cnt if cnt is None else cnt, self.cfg.m, self.pos, self.max_pos, self.window,
                                 self.inp["sink"], self.out, lse, self.aws)
        else:
            ca.hca_attend_decode(self.ap, self.inp["q"], self.inp["g_q"], self.kv, self.cfg.m_hca, self.pos,
                                 self.max_pos, self.window, self.inp["sink"], self.out, lse, self.aws)

    def step(self):
        self.append()
        if self.layer == "csa":
            self.index_topk()
        self.attend()
        return self.out
