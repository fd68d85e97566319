"""Decode top-k over long rows (more candidates than one workgroup holds in
LDS): the multi-workgroup histogram / gather / resolve path, against the
oracle's sort, including planted ties that straddle the selection boundary."""
import numpy as np
import pytest
import torch

import oracle
from oracle import pipeline as opl
from gpu_util import check_topk, f64, gpu_cache_from, log, to_np

pytestmark = pytest.mark.gpu


def _run(ctx, k, dup=None, seed=11, idx="e4m3", idx_q="e4m3"):
    from long_context_attention_17_amd import binding as ca, synth
    from long_context_attention_17_amd.configs import Config
    cfg = Config(name="topk_long", phase="decode", D=512, R=64, n_h=64, act="bf16", kv="fp8mix", m=4, k=k, n_win=128,
                 nI=8, cI=64, idx=idx, idx_q=idx_q, B=len(ctx), ctx_lo=min(ctx), ctx_hi=max(ctx), seed=seed)
    fmt = oracle.FMT_BY_NAME[idx]
    ctx = torch.tensor(ctx, dtype=torch.int64)
    n_e = [int(t) // cfg.m for t in ctx]
    pt, n_pool = synth.page_table([n + 1 for n in n_e], cfg.page, seed)
    keys = synth.normal((sum(n_e), cfg.cI), 1 / 8, seed, "ikeys", "cpu")
    offs = np.concatenate([[0], np.cumsum(n_e)])
    if dup is not None:
        for b in range(len(n_e)):
            a, lo, hi = offs[b], dup[0], min(dup[1], n_e[b])
            keys[a + lo:a + hi] = keys[a + dup[2]]
    pool = opl.new_pool(n_pool, fmt, cfg.cI, 0, cfg.page)
    for b in range(len(n_e)):
        oracle.finish_store(fmt, cfg.cI, 0, cfg.page, pool, to_np(pt)[b], 0, f64(keys[offs[b]:offs[b + 1]]),
                            norm=False, rope=False)
    qI = synth.normal((len(n_e), cfg.nI, cfg.cI), 1 / 8, seed, "qI", "cpu").to(torch.bfloat16)
    w = synth.normal((len(n_e), cfg.nI), 0.35, seed, "w", "cpu").abs()     # positive weights: ties stay ties
    pos = ctx.numpy()
    qv = opl.indexer_query_values(f64(qI), idx, idx_q)
    sc, ne = oracle.index_scores(qv, f64(w), pos, cfg.m, fmt, cfg.page, pool, to_np(pt), n_e,
                                 seq=np.arange(len(n_e)), n_cols=max(n_e))
    oidx, ocnt = oracle.topk(sc, ne, k)
    ik = gpu_cache_from(pool, to_np(pt), fmt, cfg.cI, 0, cfg.page)
    from long_context_attention_17_amd import layers
    ip = layers.index_params(cfg)
    B = len(n_e)
    gidx = torch.empty(B, k, dtype=torch.int32, device="cuda")
    gcnt = torch.empty(B, dtype=torch.int32, device="cuda")
    gsc = torch.empty(B, k, dtype=torch.float32, device="cuda")
    posd = torch.from_numpy(pos.astype(np.int32)).cuda()
    ws = torch.empty(ca.index_topk_workspace(ip, B, int(pos.max())), dtype=torch.uint8, device="cuda")
    ca.index_topk_decode(ip, qI.cuda(), w.cuda(), posd, int(pos.max()), ik, gidx, gcnt, gsc, ws=ws)
    torch.cuda.synchronize()
    # the scores the kernel used live at the start of the workspace
    stride = (max(int(pos.max()) // cfg.m, 1) + 63) // 64 * 64
    all_s = ws[:B * stride * 4].view(torch.float32).view(B, stride).cpu().numpy()
    swaps = check_topk(to_np(gidx), to_np(gcnt), oidx, ocnt, all_s, sc, k)
    log(f"  long top-k rows={n_e} k={k}: {swaps} boundary swaps")
    g = to_np(gidx)
    for b in range(B):
        np.testing.assert_array_equal(to_np(gsc)[b], all_s[b][g[b]])
    return g, oidx, all_s


def test_long_rows_random():
    _run([70001, 99999, 131072], 1024)


def test_long_rows_k2048_million():
    _run([1 << 20], 2048, seed=5)


def test_long_rows_planted_ties_across_boundary():
    """9000 identical keys (more than the resolve pass holds in LDS) that include the k-th
    score: the kept ones must be the lowest-index copies."""
    g, o, s = _run([120000], 1024, dup=(1000, 10000, 5))
    row = s[0]
    sel = set(g[0].tolist())
    tied = [5] + list(range(1000, 10000))
    chosen = [t for t in tied if t in sel]
    assert chosen == tied[:len(chosen)]


def test_long_rows_small_tie_group():
    g, o, s = _run([90000], 512, dup=(3000, 3500, 7))
    sel = set(g[0].tolist())
    tied = [7] + list(range(3000, 3500))
    chosen = [t for t in tied if t in sel]
    assert chosen == tied[:len(chosen)]


def test_long_rows_fp4_keys():
    """FP4 indexer keys (e2m1 + E8M0 scale per 32 channels) through the scaled MFMA and the long top-k."""
    _run([70000, 123457, 200003], 2048, seed=23, idx="fp4")


def test_long_rows_fp4_queries():
    """FP4 queries against FP4 keys (e2m1 x e2m1 MFMA) through the long top-k."""
    _run([70000, 123457, 200003], 2048, seed=29, idx="fp4", idx_q="fp4")
