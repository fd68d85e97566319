"""GPU parity of the attention sublayer around CSA / HCA: the low-rank query
projections and the grouped output projection (HIP MFMA GEMMs through the C-ABI)
against the oracle (oracle/sublayer.py), element by element.

Each GEMM stage is compared with the oracle applied to that stage's own GPU input
(h for the latent and the combiner weights, the GPU's stored latent for q / q^I, the
GPU's stored u for y), under the bound
    |gpu - oracle| <= one storage step at the larger magnitude + 2^-14 M,
M = sum_k |a_k w_k| (the MFMA's fp32 accumulation error, as for the indexer scores),
and the rel-L2 of the difference within half a bf16 step (2^-9; fp32 outputs 2^-16).
Chained stages are also compared end to end, with the latent's one-ulp rounding
differences added to the bound (2^-7 M of the second stage)."""
import numpy as np
import pytest
import torch

from oracle import sublayer as osl
from gpu_util import f64, log, to_np

pytestmark = pytest.mark.gpu


def _small_dims(**kw):
    from long_context_attention_17_amd.configs import SublayerDims
    base = dict(name="small", d=2240, d_c=192, n_h=16, c=64, n_i=8, c_i=32, g=2, d_g=192)
    base.update(kw)
    return SublayerDims(**base)


def check_gemm(gpu, a, w, ref, out, what, extra=0.0, quiet=False):
    """gpu, ref [rows, N]; a [rows, K], w [N, K] (fp64 values of the stage's operands)."""
    gpu = np.asarray(gpu, np.float64)
    M = np.abs(a) @ np.abs(w).T
    big = np.maximum(np.abs(gpu), np.abs(ref))
    if out == "bf16":
        step = 2.0 ** (np.floor(np.log2(np.maximum(big, 1e-30))) - 7)
        rel_max = 2.0 ** -9
    else:
        step = big * 2.0 ** -23
        rel_max = 2.0 ** -16
    bound = step + 2.0 ** -14 * M + extra * M + 1e-30
    d = np.abs(gpu - ref)
    assert np.isfinite(gpu).all(), f"{what}: non-finite values"
    worst = float((d / bound).max()) if d.size else 0.0
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-30))
    if not quiet:
        log(f"  {what}: worst {worst:.3f} of the bound, rel-L2 {rel:.2e}, {float((d > 0).mean()):.3%} differ")
    bad = d > bound
    if bad.any():
        r, c = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} elements beyond the bound, e.g. [{r}, {c}] gpu {gpu[r, c]:.8g} "
                             f"oracle {ref[r, c]:.8g} bound {bound[r, c]:.3g}")
    assert rel <= rel_max, f"{what}: rel-L2 {rel:.3e} > {rel_max:.1e}"


def run_query(dims, T, rows=None, seed=11):
    from long_context_attention_17_amd import binding as ca, synth
    w = synth.sublayer_weights(dims, seed, "cuda")
    h = synth.hidden(T, dims.d, seed, "cuda")
    qp = ca.QueryProj(w["w_dq"], w["w_uq"], w["w_iuq"], w["w_w"])
    c_q = torch.empty(T, dims.d_c, dtype=torch.bfloat16, device="cuda")
    q = torch.empty(T, dims.n_h * dims.c, dtype=torch.bfloat16, device="cuda")
    q_i = torch.empty(T, dims.n_i * dims.c_i, dtype=torch.bfloat16, device="cuda")
    w_i = torch.empty(T, dims.n_i, dtype=torch.float32, device="cuda")
    qp(h, c_q, q, q_i, w_i)
    torch.cuda.synchronize()
    rows = np.arange(T) if rows is None else rows
    ridx = torch.from_numpy(rows).cuda()
    W = {k: f64(v) for k, v in w.items()}
    hv, cg = f64(h[ridx]), f64(c_q[ridx])
    log(f"[query proj] {dims.name} T={T} ({len(rows)} rows compared) ws={qp.workspace(T)} B")
    orc = osl.low_rank_query(hv, W["w_dq"], W["w_uq"], W["w_iuq"], W["w_w"], act="bf16")
    check_gemm(cg, hv, W["w_dq"], orc["c"], "bf16", "latent c^Q = h W^DQ")
    check_gemm(f64(w_i[ridx]), hv, W["w_w"], orc["w"], "f32", "combiner weights w^I = h W^w")
    st = {"q": osl.project(cg, W["w_uq"], "bf16"), "qI": osl.project(cg, W["w_iuq"], "bf16")}
    check_gemm(f64(q[ridx]), cg, W["w_uq"], st["q"], "bf16", "queries q = c^Q W^UQ (GPU latent)")
    check_gemm(f64(q_i[ridx]), cg, W["w_iuq"], st["qI"], "bf16", "indexer queries q^I = c^Q W^IUQ (GPU latent)")
    # end to end from h: the two sides' latents may differ by one bf16 ulp (<= 2^-7 |c|)
    check_gemm(f64(q[ridx]), orc["c"], W["w_uq"], orc["q"], "bf16", "queries end to end", extra=2.0 ** -7)
    check_gemm(f64(q_i[ridx]), orc["c"], W["w_iuq"], orc["qI"], "bf16", "indexer queries end to end",
               extra=2.0 ** -7)


def run_out(dims, T, rows=None, seed=12):
    from long_context_attention_17_amd import binding as ca, synth
    w = synth.sublayer_weights(dims, seed, "cuda", indexer=False)
    o = synth.hidden(T, dims.n_h * dims.c, seed, "cuda", name="o")
    op = ca.OutProj(w["w_o1"], w["w_o2"], dims.c)
    u = torch.empty(T, dims.g * dims.d_g, dtype=torch.bfloat16, device="cuda")
    y = torch.empty(T, dims.d, dtype=torch.bfloat16, device="cuda")
    op(o, u, y)
    torch.cuda.synchronize()
    rows = np.arange(T) if rows is None else rows
    ridx = torch.from_numpy(rows).cuda()
    w1, w2 = f64(w["w_o1"]), f64(w["w_o2"])
    ov, ug = f64(o[ridx]), f64(u[ridx])
    log(f"[out proj] {dims.name} T={T} ({len(rows)} rows compared) ws={op.workspace(T)} B")
    orc = osl.grouped_out_proj(ov, w1, w2, act="bf16")
    width = 8 * dims.c
    for j in range(dims.g):
        blk = slice(j * dims.d_g, (j + 1) * dims.d_g)
        check_gemm(ug[:, blk], ov[:, j * width:(j + 1) * width], w1[j], orc["u"][:, blk], "bf16",
                   f"group {j}: u_j = o_j W1_j", quiet=0 < j < dims.g - 1)
    check_gemm(f64(y[ridx]), ug, w2, osl.project(ug, w2, "bf16"), "bf16", "y = u W2 (GPU u)")
    check_gemm(f64(y[ridx]), orc["u"], w2, orc["y"], "bf16", "y end to end", extra=2.0 ** -7)


def sample(T, n):
    return np.unique(np.concatenate([np.arange(min(T, 64)), np.arange(max(0, T - 64), T),
                                     np.linspace(0, T - 1, n).astype(np.int64)]))


@pytest.mark.parametrize("T", [1, 5, 33, 300, 2100])
def test_query_proj_small_ragged(T):
    """Several M / N / K tiles with ragged edges: d = 2240 (35 K tiles, split 8 ways at small T),
    d_c = 192 (1.5 N tiles), 8 combiner weights (one partial tile), T from 1 to 2100 (both tile
    shapes: 32 and 128 rows)."""
    run_query(_small_dims(), T)


@pytest.mark.parametrize("T", [5, 300])
def test_query_proj_widths_off_the_store_granule(T):
    """Output widths that are not multiples of 8 (100 query channels, 60 indexer channels, 3
    weights): rows of C are not 16-byte aligned, and each row ends in a partial 8-column run."""
    run_query(_small_dims(n_h=1, c=100, n_i=3, c_i=20), T)


def test_big_tiles_with_ragged_edges():
    """Shapes large enough for the 256 x 256 tiles (at least 1,024 of them) with ragged edges in
    M (8,200 rows) and N (8,480 query channels; group width 300)."""
    rows = sample(8200, 48)
    run_query(_small_dims(n_h=16, c=530), 8200, rows=rows)
    run_out(_small_dims(n_h=128, c=64, g=16, d_g=300), 8200, rows=rows)


@pytest.mark.parametrize("T", [1, 5, 33, 300, 2100])
def test_out_proj_small_ragged(T):
    run_out(_small_dims(), T)


def test_query_proj_flash_prefill_32k():
    from long_context_attention_17_amd.configs import SUBLAYERS
    run_query(SUBLAYERS["flash"], 32768, rows=sample(32768, 256))


def test_out_proj_flash_prefill_32k():
    from long_context_attention_17_amd.configs import SUBLAYERS
    run_out(SUBLAYERS["flash"], 32768, rows=sample(32768, 256))


@pytest.mark.parametrize("T", [8, 64])
def test_sublayer_pro_decode(T):
    from long_context_attention_17_amd.configs import SUBLAYERS
    run_query(SUBLAYERS["pro"], T)
    run_out(SUBLAYERS["pro"], T)


def test_sublayer_pro_prefill_ragged():
    from long_context_attention_17_amd.configs import SUBLAYERS
    T = 4096 + 37
    run_query(SUBLAYERS["pro"], T, rows=sample(T, 32))
    run_out(SUBLAYERS["pro"], T, rows=sample(T, 32))


def test_sublayer_around_csa_prefill():
    """The layers wired as the pages describe them: h -> low-rank queries (q as [L, n_h, c],
    q^I as [L, n_I, c_I], w^I) -> CSA prefill (compressors, indexer, top-k, attention) ->
    grouped output projection of the heads concatenated in head order.  Each stage is compared
    with the oracle on its GPU input; the attention at the top-k rule and 2e-2."""
    from long_context_attention_17_amd import binding as ca, layers, synth
    from long_context_attention_17_amd.configs import Config
    import oracle
    from oracle import pipeline as opl
    from gpu_util import check_out, check_topk
    from test_gpu_small import check_swapped_rows_prefill
    cfg = Config(name="sublayer_csa", phase="prefill", D=512, R=64, n_h=64, act="bf16", kv="bf16", csa=True, m=4,
                 k=64, n_win=128, nI=8, cI=64, idx="e4m3", hca=False, L=777, seed=5151)
    dims = _small_dims(d=1024, d_c=256, n_h=64, c=512, n_i=8, c_i=64, g=8, d_g=256)
    L = cfg.L
    w = synth.sublayer_weights(dims, 21, "cuda")
    h = synth.hidden(L, dims.d, 21, "cuda")
    qp = ca.QueryProj(w["w_dq"], w["w_uq"], w["w_iuq"], w["w_w"])
    c_q = torch.empty(L, dims.d_c, dtype=torch.bfloat16, device="cuda")
    q = torch.empty(L, dims.n_h * dims.c, dtype=torch.bfloat16, device="cuda")
    q_i = torch.empty(L, dims.n_i * dims.c_i, dtype=torch.bfloat16, device="cuda")
    w_i = torch.empty(L, dims.n_i, dtype=torch.float32, device="cuda")
    qp(h, c_q, q, q_i, w_i)
    inp = synth.prefill_layer(cfg, "csa", "cuda")
    inp["q"], inp["qI"], inp["w"] = q.view(L, cfg.n_h, cfg.D), q_i.view(L, cfg.nI, cfg.cI), w_i
    pt, n_pool = synth.page_table([L // cfg.m], cfg.page, cfg.seed)
    gp = layers.CSAPrefill(cfg, inp, pt.cuda(), n_pool)
    gp.run()
    op = ca.OutProj(w["w_o1"], w["w_o2"], dims.c)
    u = torch.empty(L, dims.g * dims.d_g, dtype=torch.bfloat16, device="cuda")
    y = torch.empty(L, dims.d, dtype=torch.bfloat16, device="cuda")
    op(gp.out.view(L, cfg.n_h * cfg.D), u, y)
    torch.cuda.synchronize()
    log(f"[sublayer + csa prefill] L={L} d={dims.d} d_c={dims.d_c}")
    W = {k: f64(v) for k, v in w.items()}
    hv, cg = f64(h), f64(c_q)
    orc_q = osl.low_rank_query(hv, W["w_dq"], W["w_uq"], W["w_iuq"], W["w_w"], act="bf16")
    check_gemm(cg, hv, W["w_dq"], orc_q["c"], "bf16", "latent")
    check_gemm(f64(q), cg, W["w_uq"], osl.project(cg, W["w_uq"], "bf16"), "bf16", "queries (GPU latent)")
    check_gemm(f64(q_i), cg, W["w_iuq"], osl.project(cg, W["w_iuq"], "bf16"), "bf16", "indexer queries (GPU latent)")
    check_gemm(f64(w_i), hv, W["w_w"], orc_q["w"], "f32", "combiner weights")
    rows = sample(L, 96)
    orc = opl.csa_prefill(cfg, inp, to_np(pt)[0], n_pool, rows=rows)
    ridx = torch.from_numpy(rows).cuda()
    swaps = check_topk(to_np(gp.idx[ridx]), to_np(gp.cnt[ridx]), orc["idx"], orc["cnt"], orc["scores"],
                       orc["scores"], cfg.k)
    same = np.array([np.array_equal(to_np(gp.idx[r]), orc["idx"][i]) for i, r in enumerate(rows)])
    check_out(f64(gp.out[ridx])[same], orc["out"][same], "bf16", f"attention on the projected queries ({swaps} swaps)")
    check_swapped_rows_prefill(cfg, inp, pt, n_pool, gp, same, rows=rows)
    ov = f64(gp.out.view(L, cfg.n_h * cfg.D)[ridx])
    orc_o = osl.grouped_out_proj(ov, f64(w["w_o1"]), W["w_o2"], act="bf16")
    check_gemm(f64(y[ridx]), orc_o["u"], W["w_o2"], orc_o["y"], "bf16", "sublayer output y (GPU attention output)",
               extra=2.0 ** -7)
