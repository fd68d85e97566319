"""Seeded synthetic inputs shaped like the workloads (random draws only).

This module holds none of the attention method's arithmetic: it draws
Gaussian tensors, casts them to the preset's storage dtype, draws context
lengths and page permutations, and nothing else.  Both the HIP path and the
CPU oracle consume what it returns.

Recipe (every tensor has its own stable id; the torch generator for a tensor
is seeded with seed * 1000 + id on the device the tensor is made on):
  projections C*, Z*, biases B*, queries q, raw window KV, raw decode entries:
      N(0,1)/sqrt(D)
  indexer projections / queries / raw keys: N(0,1)/sqrt(c_I)
  indexer combiner weights w: N(0,1)/sqrt(n_I);  attention sinks: N(0,1)
  RMSNorm gains: 1
  sublayer: hidden states h and attention outputs o: N(0,1); every projection
      weight ([out, in]): N(0,1)/sqrt(in); all bf16
  decode contexts: uniform integers in [ctx_lo, ctx_hi] (the new token sits at
      t = ctx); page tables: a random permutation of a pool holding the
      needed pages plus 10%.
"""
from __future__ import annotations

import math

import torch

from .configs import Config, get

_IDS = {
    "Ca": 1, "Cb": 2, "Za": 3, "Zb": 4, "Ba": 5, "Bb": 6,
    "ICa": 7, "ICb": 8, "IZa": 9, "IZb": 10, "IBa": 11, "IBb": 12,
    "kv_raw": 13, "q": 14, "qI": 15, "w": 16, "sink": 17,
    "C": 18, "Z": 19, "B": 20,
    "entries": 21, "ikeys": 22, "ctx": 23, "pages": 24,
    "tail": 25, "itail": 26, "new_rows": 27, "new_irows": 28,
    "h": 29, "w_dq": 30, "w_uq": 31, "w_iuq": 32, "w_w": 33, "w_o1": 34, "w_o2": 35, "o": 36,
}


def _gen(seed: int, name: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000 + _IDS[name])
    return g


def act_dtype(cfg: Config):
    return torch.float32 if cfg.act == "f32" else torch.bfloat16


def normal(shape, std, seed, name, device, dtype=torch.float32, salt: int = 0):
    g = _gen(seed + salt, name, device)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    x.mul_(std)
    return x.to(dtype)


def page_table(n_entries, page: int, seed: int, device="cpu"):
    """Page table [B, max_pages] (int32, -1 where unused) and pool size in pages."""
    need = [max(1, math.ceil(n / page)) for n in n_entries]
    total = sum(need)
    n_pool = total + max(1, total // 10)
    g = _gen(seed, "pages", "cpu")
    perm = torch.randperm(n_pool, generator=g)
    max_pages = max(need)
    pt = torch.full((len(need), max_pages), -1, dtype=torch.int32)
    o = 0
    for b, k in enumerate(need):
        pt[b, :k] = perm[o:o + k].to(torch.int32)
        o += k
    return pt.to(device), n_pool


def prefill_layer(cfg, layer: str, device, L: int | None = None) -> dict:
    """Inputs of one prefill layer ("csa" or "hca") of a single sequence."""
    cfg = get(cfg)
    L = cfg.L if L is None else L
    D, s = cfg.D, cfg.seed + (0 if layer == "csa" else 500)
    ad = act_dtype(cfg)
    sd = 1.0 / math.sqrt(D)
    out = {"L": L, "layer": layer}
    if layer == "csa":
        for n in ("Ca", "Cb", "Za", "Zb"):
            out[n] = normal((L, D), sd, s, n, device, ad)
        out["Ba"] = normal((cfg.m, D), sd, s, "Ba", device)
        out["Bb"] = normal((cfg.m, D), sd, s, "Bb", device)
        si = 1.0 / math.sqrt(cfg.cI)
        for n in ("ICa", "ICb", "IZa", "IZb"):
            out[n] = normal((L, cfg.cI), si, s, n, device, ad)
        out["IBa"] = normal((cfg.m, cfg.cI), si, s, "IBa", device)
        out["IBb"] = normal((cfg.m, cfg.cI), si, s, "IBb", device)
        out["qI"] = normal((L, cfg.nI, cfg.cI), si, s, "qI", device, ad)
        out["w"] = normal((L, cfg.nI), 1.0 / math.sqrt(cfg.nI), s, "w", device)
    else:
        out["C"] = normal((L, D), sd, s, "C", device, ad)
        out["Z"] = normal((L, D), sd, s, "Z", device, ad)
        out["B"] = normal((cfg.m_hca, D), sd, s, "B", device)
    out["kv_raw"] = normal((L, D), sd, s, "kv_raw", device, ad)
    out["q"] = normal((L, cfg.n_h, D), sd, s, "q", device, ad)
    out["sink"] = normal((cfg.n_h,), 1.0, s, "sink", device)
    ones = torch.ones(D, device=device, dtype=torch.float32)
    out["g_kv"], out["g_q"], out["g_w"] = ones, ones.clone(), ones.clone()
    return out


def decode_contexts(cfg) -> torch.Tensor:
    cfg = get(cfg)
    if cfg.ctx_lo == cfg.ctx_hi:
        return torch.full((cfg.B,), cfg.ctx_lo, dtype=torch.int64)
    g = _gen(cfg.seed, "ctx", "cpu")
    return torch.randint(cfg.ctx_lo, cfg.ctx_hi + 1, (cfg.B,), generator=g, dtype=torch.int64)


def decode_layer(cfg, layer: str, device, ctx: torch.Tensor | None = None) -> dict:
    """State and step inputs of one decode layer for a batch of sequences.

    The new token of sequence b sits at t_b = ctx_b.  The cache holds every
    entry completed by tokens 0..t_b-1 (as raw pre-epilogue vectors here), the
    window rows cover positions t_b-n_win+1..t_b (the last one is the new
    token), and the compressor tail ring holds the projection rows of the
    preceding tokens at slot position mod span.
    """
    cfg = get(cfg)
    ctx = decode_contexts(cfg) if ctx is None else ctx
    D, B = cfg.D, cfg.B
    s = cfg.seed + (0 if layer == "csa" else 500)
    ad = act_dtype(cfg)
    sd = 1.0 / math.sqrt(D)
    ratio = cfg.m if layer == "csa" else cfg.m_hca
    n_ent = [int(t) // ratio for t in ctx.tolist()]
    out = {"layer": layer, "ctx": ctx, "pos": ctx.clone(), "n_entries": n_ent, "ratio": ratio}
    offs = [0]
    for n in n_ent:
        offs.append(offs[-1] + n)
    out["entry_offsets"] = offs
    out["entries"] = normal((offs[-1], D), sd, s, "entries", device)
    # one spare slot per sequence for the entry the new token may complete
    pt, n_pool = page_table([n + 1 for n in n_ent], cfg.page, s, device)
    out["page_table"], out["n_pool_pages"] = pt, n_pool
    if layer == "csa":
        si = 1.0 / math.sqrt(cfg.cI)
        out["ikeys"] = normal((offs[-1], cfg.cI), si, s, "ikeys", device)
        out["qI"] = normal((B, cfg.nI, cfg.cI), si, s, "qI", device, ad)
        out["w"] = normal((B, cfg.nI), 1.0 / math.sqrt(cfg.nI), s, "w", device)
        span, narr = 2 * cfg.m, 4
        out["itail"] = normal((B, span, narr, cfg.cI), si, s, "itail", device)
        out["new_irows"] = normal((B, narr, cfg.cI), si, s, "new_irows", device, ad)
        out["IBa"] = normal((cfg.m, cfg.cI), si, s, "IBa", device)
        out["IBb"] = normal((cfg.m, cfg.cI), si, s, "IBb", device)
        out["Ba"] = normal((cfg.m, D), sd, s, "Ba", device)
        out["Bb"] = normal((cfg.m, D), sd, s, "Bb", device)
    else:
        span, narr = cfg.m_hca, 2
        out["B"] = normal((cfg.m_hca, D), sd, s, "B", device)
    out["tail"] = normal((B, span, narr, D), sd, s, "tail", device)
    out["new_rows"] = normal((B, narr, D), sd, s, "new_rows", device, ad)
    out["kv_raw"] = normal((B, cfg.n_win, D), sd, s, "kv_raw", device, ad)
    out["q"] = normal((B, cfg.n_h, D), sd, s, "q", device, ad)
    out["sink"] = normal((cfg.n_h,), 1.0, s, "sink", device)
    ones = torch.ones(D, device=device, dtype=torch.float32)
    out["g_kv"], out["g_q"], out["g_w"] = ones, ones.clone(), ones.clone()
    return out


def sublayer_weights(dims, seed: int, device, indexer: bool = True) -> dict:
    """Random projection weights of the attention sublayer, bf16 [out, in] (see configs.SublayerDims)."""
    d = dims
    bf = torch.bfloat16
    w = {"w_dq": normal((d.d_c, d.d), 1.0 / math.sqrt(d.d), seed, "w_dq", device, bf),
         "w_uq": normal((d.n_h * d.c, d.d_c), 1.0 / math.sqrt(d.d_c), seed, "w_uq", device, bf),
         "w_o1": normal((d.g, d.d_g, 8 * d.c), 1.0 / math.sqrt(8 * d.c), seed, "w_o1", device, bf),
         "w_o2": normal((d.d, d.g * d.d_g), 1.0 / math.sqrt(d.g * d.d_g), seed, "w_o2", device, bf)}
    if indexer:
        w["w_iuq"] = normal((d.n_i * d.c_i, d.d_c), 1.0 / math.sqrt(d.d_c), seed, "w_iuq", device, bf)
        w["w_w"] = normal((d.n_i, d.d), 1.0 / math.sqrt(d.d), seed, "w_w", device, bf)
    return w


def hidden(T: int, width: int, seed: int, device, name: str = "h") -> torch.Tensor:
    """T rows of N(0,1) activations (bf16): hidden states ("h") or attention outputs ("o")."""
    return normal((T, width), 1.0, seed, name, device, torch.bfloat16)
