"""Benchmark of the CSA + HCA hot path on one MI355X.

Default workload: the million-token decode step (batch 8, context 2^20, 128
query heads, D = 512, fp8-mixed pages): one CSA layer step (window append and
compressor tail updates in one launch, lightning indexer + top-k over 262,144
compressed entries, gathered attention over 2,048 + 128 items) and one HCA
layer step (window append and compressor tail update in one launch, dense
attention over 8,192 + 128 items).  Other presets: --workload decode_mixed | prefill_csa_32k |
prefill_hca_128k | tiny, the million-token decode with FP4 indexer keys
(decode_1m_fp4idx) or FP4 keys and queries (decode_1m_fp4qk), and prefills
that continue a stored prefix (prefill_csa_32k_after_16k,
prefill_hca_128k_after_64k).  The attention sublayer's projections (low-rank
queries, grouped output projection) have workloads of their own:
sublayer_pro_decode_b8, sublayer_flash_decode_b64, sublayer_flash_prefill_32k,
sublayer_pro_prefill_32k.

Prints ONE JSON line.  Inputs are resident in HBM before the timed region; the
timed region rotates independent replicas of every cache (so the per-step
working set is not served from the 256 MB Infinity Cache).  Per-stage times
come from HIP events recorded on the stream the kernels run on.
"""
from __future__ import annotations

import argparse
import copy
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CSA+HCA attention tokens/s (prefill, decode) at 128K–1M ctx; % HBM/MFMA peak"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
# workload -> config number, or (config number, overrides): decode_1m_fp4idx is the million-token
# decode with the indexer keys stored in FP4 (e2m1 + E8M0 per 32 channels) instead of e4m3, and
# decode_1m_fp4qk the same with the indexer queries in FP4 too
WORKLOADS = {"decode_1m": 5, "decode_mixed": 4, "prefill_csa_32k": 2, "prefill_hca_128k": 3, "tiny": 1,
             "decode_1m_fp4idx": (5, {"idx": "fp4", "name": "million_decode_b8_fp4idx"}),
             "decode_1m_fp4qk": (5, {"idx": "fp4", "idx_q": "fp4", "name": "million_decode_b8_fp4_indexer"}),
             # prefills that continue a stored prefix (its entries reloaded; the unfinished block,
             # the window and the new rows computed)
             "prefill_csa_32k_after_16k": (2, {"prefix": 16384, "name": "csa_prefill_32k_after_16k_prefix"}),
             "prefill_hca_128k_after_64k": (3, {"prefix": 65536, "name": "hca_prefill_128k_after_64k_prefix"})}
# the attention sublayer's projections (low-rank queries, grouped output projection) at the
# Flash / Pro widths: name -> (widths, tokens per step)
SUBLAYER_WORKLOADS = {"sublayer_pro_decode_b8": ("pro", 8), "sublayer_flash_decode_b64": ("flash", 64),
                      "sublayer_flash_prefill_32k": ("flash", 32768), "sublayer_pro_prefill_32k": ("pro", 32768)}
SUBLAYER_METRIC = "attention sublayer projections (low-rank q + grouped output) tokens/s; % HBM/MFMA peak"
# sources that define each timed kernel (its counter readings go stale when they change)
KERNEL_SOURCES = {"attend_mx_kernel": ["attend.hip", "common.h", "kernels.h"],
                  "index_scores_fp8_kernel": ["indexer.hip", "common.h", "kernels.h"],
                  "index_scores_fp4_kernel": ["indexer.hip", "common.h", "kernels.h"],
                  "gemm_nt_kernel": ["proj.hip", "common.h", "kernels.h"],
                  "gemm_skinny_kernel": ["proj.hip", "common.h", "kernels.h"]}


def hca_dense_units(cfg, max_pos):
    """Whether the HCA decode attention launch of this batch numbers its units densely: the
    library does so for up to 64 rows when the padded unit space (rows x the most chunks
    a row up to max_pos can get, in blocks of 8, per 64-head group) exceeds the CUs."""
    from long_context_attention_17_amd import binding as ca, layers
    if cfg.B > 64:
        return False
    max_chunks = ca.attend_decode_plan(layers.attend_params(cfg), max_pos // cfg.m_hca + cfg.n_win)[2]
    units = (cfg.B * max_chunks + 7) // 8 * 8 * (cfg.n_h // 64)
    return max_chunks > 1 and units > torch.cuda.get_device_properties(0).multi_processor_count


def progress(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash(symbol: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[symbol.split("<")[0]]:
        with open(os.path.join(ROOT, "long_context_attention_17_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------------ algorithmic work
def index_key_bytes(cfg):
    """Bytes of one indexer key in its page: e4m3 codes + fp32 scale, e2m1 codes + one
    E8M0 byte per 32 channels, or fp32."""
    return {"e4m3": cfg.cI + 4, "fp4": cfg.cI // 2 + cfg.cI // 32, "f32": 4 * cfg.cI}[cfg.idx]


def index_kernel_symbol(cfg, qpw):
    if cfg.idx_q == "fp4":
        return f"index_scores_fp4_kernel<{qpw}>"
    return f"index_scores_fp8_kernel<{qpw}, {4 if cfg.idx == 'fp4' else 3}>"


def kernel_roofline(bound, units, symbol, launch_ms):
    """Achieved rate of one timed kernel against its peak (HBM bytes or bf16 MFMA flops)."""
    if bound == "hbm":
        achieved, peak, unit = units / (launch_ms / 1e3) / 1e9, PEAK_HBM_GBS, "GB/s"
    else:
        achieved, peak, unit = units / (launch_ms / 1e3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
    return {"kernel": symbol, "bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "launch_ms": round(launch_ms, 5), "work_per_launch": units}


def decode_work(cfg, pos):
    """Per-step algorithmic bytes / flops of each stage, summed over the batch."""
    D, R, nh = cfg.D, cfg.R, cfg.n_h
    rec = 584 if cfg.kv == "fp8mix" else (2 * D if cfg.kv == "bf16" else 4 * D)
    w = {"index_bytes": 0, "index_flops": 0, "csa_flops": 0, "csa_bytes": 0, "hca_flops": 0, "hca_bytes": 0}
    for t in pos:
        ne = t // cfg.m
        nw = min(t + 1, cfg.n_win)
        w["index_bytes"] += ne * index_key_bytes(cfg)
        w["index_flops"] += 2 * cfg.nI * cfg.cI * ne
        sel = min(ne, cfg.k)
        w["csa_flops"] += 4 * nh * D * (sel + nw)
        w["csa_bytes"] += sel * rec + nw * 2 * D + 2 * (2 * nh * D)
        nh_e = t // cfg.m_hca
        w["hca_flops"] += 4 * nh * D * (nh_e + nw)
        w["hca_bytes"] += nh_e * rec + nw * 2 * D + 2 * (2 * nh * D)
    return w


def prefill_work(cfg):
    """Flops of the rows a prefill computes (positions prefix..L-1)."""
    L, D, nh = cfg.L, cfg.D, cfg.n_h
    t = torch.arange(cfg.prefix, L, dtype=torch.float64)
    nw = torch.clamp(t + 1, max=cfg.n_win)
    w = {}
    if cfg.csa:
        ne = torch.floor(t / cfg.m)
        w["csa_flops"] = float((4 * nh * D * (torch.clamp(ne, max=cfg.k) + nw)).sum())
        w["index_flops"] = float((2 * cfg.nI * cfg.cI * ne).sum())
    if cfg.hca:
        w["hca_flops"] = float((4 * nh * D * (torch.floor(t / cfg.m_hca) + nw)).sum())
    return w


# ------------------------------------------------------------------ timing helpers
class StageTimer:
    """HIP events around each stage, on the current (kernel) stream."""

    def __init__(self):
        self.pairs = {}

    def run(self, name, fn):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        self.pairs.setdefault(name, []).append((s, e))

    def means_ms(self):
        return {k: sum(s.elapsed_time(e) for s, e in v) / len(v) for k, v in self.pairs.items()}


def time_kernels(run, kernels, reps):
    """Average launch duration (ms) of library kernels, from the HIP events that the library
    records around each eager launch on the launch stream (ca_timer_*).  The timed passes are
    queued behind a GPU spin so that their kernels run back to back, as in the graph replays;
    `queued` reports whether the spin outlasted the host's enqueueing."""
    from long_context_attention_17_amd import binding as ca
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    run(0)
    host_s = time.perf_counter() - h0                  # host enqueue time of one pass
    torch.cuda.synchronize()
    ca.timer_start(list(kernels.values()), max_launches=8 * reps)
    try:
        torch.cuda._sleep(int((2.0 * reps * host_s + 0.005) * 2.4e9))
        spin_end = torch.cuda.Event()
        spin_end.record()
        for i in range(reps):
            run(i)
        queued = not spin_end.query()
        raw = {name: ca.timer_read(k) for name, k in kernels.items()}
    finally:
        ca.timer_stop()
    return {name: (ms / n if n else float("nan"), n / reps) for name, (ms, n) in raw.items()}, queued


def replicate_decode_layer(dl, n):
    """Independent copies of a decode layer's caches and state (same values, new memory)."""
    from long_context_attention_17_amd import binding as ca
    reps = [dl]
    for _ in range(n - 1):
        r = copy.copy(dl)
        r.kv = ca.Cache(dl.kv.fmt, dl.kv.dim, dl.kv.rope_dim, dl.kv.page_size, dl.kv.pool.clone(), dl.kv.page_table)
        if dl.ik is not None:
            r.ik = ca.Cache(dl.ik.fmt, dl.ik.dim, dl.ik.rope_dim, dl.ik.page_size, dl.ik.pool.clone(),
                            dl.ik.page_table)
        r.window = dl.window.clone()
        r.tail = dl.tail.clone()
        if dl.layer == "csa":
            r.itail = dl.itail.clone()
        reps.append(r)
    return reps


# ------------------------------------------------------------------ workloads
def bench_decode(cfg, steps, warmup, replicas, args):
    from long_context_attention_17_amd import layers, synth
    ctx = synth.decode_contexts(cfg)
    layer_objs = {}
    for name in ("csa", "hca"):
        progress(f"building {name} decode state")
        inp = synth.decode_layer(cfg, name, "cuda", ctx)
        dl = layers.DecodeLayer(cfg, inp)
        torch.cuda.synchronize()
        del inp["entries"]
        inp.pop("ikeys", None)
        layer_objs[name] = replicate_decode_layer(dl, replicas)
        torch.cuda.empty_cache()
    torch.cuda.synchronize()

    def stages_of(i):
        c = layer_objs["csa"][i % replicas]
        h = layer_objs["hca"][i % replicas]
        # append: the new token's window append and compressor step(s) in one launch
        return [("csa_append", c.append), ("csa_index_topk", c.index_topk), ("csa_attend", c.attend),
                ("hca_append", h.append), ("hca_attend", h.attend)]

    def step(i):
        # each layer's step is one library call (ca_csa_decode_step / ca_hca_decode_step): the
        # stages above, with the query preparation and top-k state clearing in the append launch
        layer_objs["csa"][i % replicas].fused_step()
        layer_objs["hca"][i % replicas].fused_step()

    progress("warmup (eager)")
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # One HIP graph per replica for the whole step (the library only enqueues kernels on the
    # current stream, never allocates or synchronizes, so its calls capture as they are).
    progress("capturing step graphs")
    graphs = []
    for i in range(replicas):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(i)
        graphs.append(g)
    for i in range(warmup):
        graphs[i % replicas].replay()
    torch.cuda.synchronize()
    progress("timed steps")
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    t0.record()
    for i in range(steps):
        graphs[i % replicas].replay()
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = t0.elapsed_time(t1) / steps
    # per-stage device time: each stage captured on its own, replayed back to back between
    # two events on the stream the kernels run on (rotating replicas like the step)
    progress("per-stage timing")
    names = [n for n, _ in stages_of(0)]
    stage_graphs = {n: [] for n in names}
    for i in range(replicas):
        for n, fn in stages_of(i):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn()
            stage_graphs[n].append(g)
    st = {}
    reps = max(steps, 20)
    for n in names:
        for i in range(replicas):
            stage_graphs[n][i].replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            stage_graphs[n][i % replicas].replay()
        e1.record()
        torch.cuda.synchronize()
        st[n] = e0.elapsed_time(e1) / reps
    # the stages leave the caches exactly as the step does (idempotent at a fixed position)
    pos = [int(x) for x in ctx.tolist()]
    work = decode_work(cfg, pos)
    value = cfg.B / (ms_step / 1e3)
    # per-kernel launch durations and the dominant kernel's roofline
    from long_context_attention_17_amd import binding as ca
    progress("kernel timing")
    kt, queued = time_kernels(step, {"csa_attend": ca.TIMED_CSA_ATTEND, "hca_attend": ca.TIMED_HCA_ATTEND,
                                     "index_scores": ca.TIMED_INDEX_SCORES}, max(steps, 20))
    fmt = 2 if cfg.kv == "fp8mix" else 1
    dense = "true" if hca_dense_units(cfg, max(pos)) else "false"
    roof_of = {   # algorithmic work of one launch (the launch covers the whole batch)
        "index_scores": ("hbm", work["index_bytes"], index_kernel_symbol(cfg, 1)),
        "csa_attend": ("mfma", work["csa_flops"], f"attend_mx_kernel<{fmt}, 0, true, false>"),
        "hca_attend": ("mfma", work["hca_flops"], f"attend_mx_kernel<{fmt}, 1, true, {dense}>"),
    }
    dom = max(roof_of, key=lambda k: kt[k][0] * kt[k][1])
    bound, units, symbol = roof_of[dom]
    launch_ms = kt[dom][0]
    if bound == "hbm":
        achieved, peak, unit = units / (launch_ms / 1e3) / 1e9, PEAK_HBM_GBS, "GB/s"
    else:
        achieved, peak, unit = units / (launch_ms / 1e3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
    step_bytes = work["index_bytes"] + work["csa_bytes"] + work["hca_bytes"]
    extra = {
        "stages_ms": {k: round(v, 5) for k, v in st.items()},
        "step_hbm_bytes_algorithmic": step_bytes,
        "step_hbm_frac_of_peak": round(step_bytes / (ms_step / 1e3) / (PEAK_HBM_GBS * 1e9), 4),
        "stage_rooflines": {
            "csa_index_topk": {"bound": "hbm", "achieved_GBs": round(work["index_bytes"] / st["csa_index_topk"] / 1e6, 1)},
            "csa_attend": {"bound": "mfma", "achieved_TFLOPs": round(work["csa_flops"] / st["csa_attend"] / 1e9, 2)},
            "hca_attend": {"bound": "mfma", "achieved_TFLOPs": round(work["hca_flops"] / st["hca_attend"] / 1e9, 2)},
        },
        "kernel_launch_ms": {k: round(v[0], 5) for k, v in kt.items()},
        "kernel_rooflines": {k: kernel_roofline(*roof_of[k], kt[k][0]) for k in roof_of},
        "kernel_timing_queued": queued,
        "wall_s_timed": round(wall, 4),
        "timing": "whole step: HIP-graph replays (one graph per cache replica) of one ca_csa_decode_step "
                  "and one ca_hca_decode_step call; stages: the separate calls (append, index_topk, attend), "
                  "per-stage graphs replayed back to back between HIP events; kernels: HIP events recorded by "
                  "the library around each eager launch on its stream",
    }
    config = {"workload": f"{cfg.name}: decode step of one CSA + one HCA layer, batch {cfg.B}, "
                          f"context {cfg.ctx_lo}-{cfg.ctx_hi}, {cfg.n_h} heads, D={cfg.D}, kv {cfg.kv}, "
                          f"k={cfg.k}, window {cfg.n_win}, m={cfg.m}, m'={cfg.m_hca}",
              "batch": cfg.B, "context": [min(pos), max(pos)], "replicas": replicas}
    roof = {"kernel": symbol, "stage": dom, "bound": bound, "achieved": round(achieved, 3), "peak": peak,
            "unit": unit, "frac": round(achieved / peak, 4), "launch_ms": round(launch_ms, 5),
            "work_per_launch": units}
    return value, ms_step, config, roof, extra, (ctx, layer_objs)


def bench_prefill(cfg, steps, warmup, replicas, args):
    from long_context_attention_17_amd import layers, synth
    objs = []
    if cfg.csa:
        inp = synth.prefill_layer(cfg, "csa", "cuda")
        pt, n_pool = synth.page_table([cfg.L // cfg.m], cfg.page, cfg.seed)
        objs.append(("csa", layers.CSAPrefill(cfg, inp, pt.cuda(), n_pool)))
    if cfg.hca:
        inp = synth.prefill_layer(cfg, "hca", "cuda")
        pt, n_pool = synth.page_table([cfg.L // cfg.m_hca], cfg.page, cfg.seed)
        objs.append(("hca", layers.HCAPrefill(cfg, inp, pt.cuda(), n_pool)))

    P = cfg.prefix

    def first_row(name):
        """First projection row a continuation needs: the block the first missing entry pools from."""
        if P == 0:
            return 0
        ratio = cfg.m if name == "csa" else cfg.m_hca
        E = P // ratio
        return ratio * max(E - 1, 0) if name == "csa" else ratio * E

    if P > 0:   # the stored prefix: its entries are in the cache before the timed prefill
        for name, o in objs:
            o.compress(0, P)
        torch.cuda.synchronize()

    def step(timer=None):
        for name, o in objs:
            stages = [(f"{name}_compress", lambda o=o, name=name: o.compress(first_row(name), cfg.L)),
                      (f"{name}_window_append", lambda o=o: o.window_append(max(0, P - cfg.n_win + 1) if P else 0,
                                                                           cfg.L))]
            if name == "csa":
                stages.append(("csa_index_topk", lambda o=o: o.index_topk(t0=P, t1=cfg.L)))
            stages.append((f"{name}_attend", lambda o=o: o.attend(t0=P, t1=cfg.L)))
            for sname, fn in stages:
                timer.run(sname, fn) if timer else fn()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    t0.record()
    for _ in range(steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = t0.elapsed_time(t1) / steps
    timer = StageTimer()
    for _ in range(steps):
        step(timer)
    torch.cuda.synchronize()
    st = timer.means_ms()
    work = prefill_work(cfg)
    value = (cfg.L - P) / (ms_step / 1e3)
    # per-kernel launch durations (library-recorded HIP events) and the dominant kernel's roofline
    from long_context_attention_17_amd import binding as ca
    progress("kernel timing")
    kernels = {}
    if cfg.csa:
        kernels["csa_attend"] = ca.TIMED_CSA_ATTEND
    if cfg.hca:
        kernels["hca_attend"] = ca.TIMED_HCA_ATTEND
    kt, queued = time_kernels(lambda i: step(), kernels, max(steps, 3))
    dom = max(kt, key=lambda k: kt[k][0] * kt[k][1])
    flops = work["csa_flops"] if dom == "csa_attend" else work["hca_flops"]
    launch_ms = kt[dom][0]
    achieved = flops / (launch_ms / 1e3) / 1e12
    fmt = 2 if cfg.kv == "fp8mix" else 1
    roof = {"kernel": f"attend_mx_kernel<{fmt}, {0 if dom == 'csa_attend' else 1}, false, false>", "stage": dom,
            "bound": "mfma",
            "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "launch_ms": round(launch_ms, 5), "work_per_launch": flops}
    extra = {"stages_ms": {k: round(v, 4) for k, v in st.items()},
             "kernel_launch_ms": {k: round(v[0], 5) for k, v in kt.items()}, "kernel_timing_queued": queued,
             "wall_s_timed": round(wall, 4), "algorithmic_flops": work}
    config = {"workload": f"{cfg.name}: prefill of {'CSA' if cfg.csa else ''}{'+' if cfg.csa and cfg.hca else ''}"
                          f"{'HCA' if cfg.hca else ''}, L={cfg.L}, {cfg.n_h} heads, D={cfg.D}, kv {cfg.kv}"
                          + (f", continuing a stored prefix of {P} tokens (rows {P}..{cfg.L - 1})" if P else ""),
              "seq_len": cfg.L}
    if P:
        config["prefix"] = P
    return value, ms_step, config, roof, extra, objs


def bench_sublayer(name, steps, warmup, replicas):
    """One step = ca_query_proj + ca_out_proj for T tokens (synthetic weights of the model's
    widths; `replicas` weight sets used in turn so that no step finds its weights in cache)."""
    from long_context_attention_17_amd import binding as ca, synth
    from long_context_attention_17_amd.configs import SUBLAYERS
    dname, T = SUBLAYER_WORKLOADS[name]
    d = SUBLAYERS[dname]
    bf = torch.bfloat16
    sets = []
    for i in range(replicas):
        w = synth.sublayer_weights(d, 100 + i, "cuda")
        sets.append((w, ca.QueryProj(w["w_dq"], w["w_uq"], w["w_iuq"], w["w_w"]), ca.OutProj(w["w_o1"], w["w_o2"], d.c)))
    h = synth.hidden(T, d.d, 7, "cuda")
    o = synth.hidden(T, d.n_h * d.c, 7, "cuda", name="o")
    c_q = torch.empty(T, d.d_c, dtype=bf, device="cuda")
    q = torch.empty(T, d.n_h * d.c, dtype=bf, device="cuda")
    qi = torch.empty(T, d.n_i * d.c_i, dtype=bf, device="cuda")
    wi = torch.empty(T, d.n_i, dtype=torch.float32, device="cuda")
    u = torch.empty(T, d.g * d.d_g, dtype=bf, device="cuda")
    y = torch.empty(T, d.d, dtype=bf, device="cuda")
    ws = torch.empty(max(1, sets[0][1].workspace(T), sets[0][2].workspace(T)), dtype=torch.uint8, device="cuda")

    def step(i):
        _, qp, op = sets[i % replicas]
        qp(h, c_q, q, qi, wi, ws=ws)
        op(o, u, y, ws=ws)

    graphs = []
    step(0)
    torch.cuda.synchronize()
    for i in range(replicas):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(i)
        graphs.append(g)
    for i in range(warmup):
        graphs[i % replicas].replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        graphs[i % replicas].replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    kt, queued = time_kernels(step, {"gemm": ca.TIMED_PROJ_GEMM}, max(steps, 10))
    launch_ms, per_step = kt["gemm"]
    flops = 2.0 * T * (d.d * (d.d_c + d.n_i) + d.d_c * (d.n_h * d.c + d.n_i * d.c_i)
                       + d.n_h * d.c * d.d_g + d.g * d.d_g * d.d)
    wbytes = 2 * sum(int(v.numel()) for v in sets[0][0].values())
    abytes = T * (2 * (d.d + d.d_c + d.n_h * d.c + d.n_i * d.c_i + d.n_h * d.c + d.g * d.d_g + d.d) + 4 * d.n_i)
    abytes += T * 2 * (d.d_c + d.g * d.d_g)             # the latent and u, read back by the second stages
    gemm_ms = launch_ms * per_step
    # the step's GEMM launches: gemm_skinny_kernel for M <= 32, else gemm_nt_kernel with 128 x 128
    # or 256 x 256 tiles (by the output's tile count); the roofline sums them all
    symbol = "gemm_skinny_kernel<2, 1>" if T <= 32 else "gemm_nt_kernel"
    if T <= 256:
        roof = kernel_roofline("hbm", wbytes + abytes, symbol, gemm_ms)
        roof["work_unit"] = "bytes of weights and activations per step (all GEMM launches of the step)"
    else:
        roof = kernel_roofline("mfma", flops, symbol, gemm_ms)
        roof["work_unit"] = "flops per step (all GEMM launches of the step)"
    roof["launch_ms"] = round(launch_ms, 5)
    roof["launches_per_step"] = per_step
    roof["stage"] = "sublayer"
    config = {"workload": f"{name}: low-rank query projections (d={d.d} -> d_c={d.d_c} -> {d.n_h}x{d.c} queries, "
                          f"{d.n_i}x{d.c_i} indexer queries, {d.n_i} combiner weights) and grouped output projection "
                          f"({d.g} groups of 8 heads -> d_g={d.d_g} -> d={d.d}) for {T} tokens, bf16, synthetic weights",
              "tokens": T, "replicas": replicas}
    extra = {"metric_note": SUBLAYER_METRIC, "kernel_timing_queued": queued,
             "step_flops": flops, "step_weight_bytes": wbytes,
             "timing": "whole step: HIP-graph replays (one graph per weight set); kernel: HIP events recorded by "
                       "the library around each eager GEMM launch, summed over the step's launches"}
    return T / (ms / 1e3), ms, config, roof, extra, (sets, graphs)


def cpu_baseline_sublayer(name, budget_s=10.0):
    """The oracle's sublayer (numpy fp64 matmuls) on a sample of rows, all host threads, then one thread."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import sublayer as osl
    from long_context_attention_17_amd import synth
    from long_context_attention_17_amd.configs import SUBLAYERS
    dname, T = SUBLAYER_WORKLOADS[name]
    d = SUBLAYERS[dname]
    w = {k: v.double().numpy() for k, v in synth.sublayer_weights(d, 100, "cpu").items()}
    n = min(T, 64)
    h = synth.hidden(n, d.d, 7, "cpu").double().numpy()
    o = synth.hidden(n, d.n_h * d.c, 7, "cpu", name="o").double().numpy()

    def run(rows):
        osl.low_rank_query(h[:rows], w["w_dq"], w["w_uq"], w["w_iuq"], w["w_w"], act="bf16")
        osl.grouped_out_proj(o[:rows], w["w_o1"], w["w_o2"], act="bf16")

    reps, t = 0, 0.0
    while t < budget_s and reps < 20:
        t0 = time.perf_counter()
        run(n)
        t += time.perf_counter() - t0
        reps += 1
    threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    with threadpool_limits(1):
        t0 = time.perf_counter()
        run(max(1, n // 8))
        t1 = time.perf_counter() - t0
    return {"value": round(n * reps / t, 4), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "host_threads": os.cpu_count(),
            "sample": f"{n} of {T} rows, {reps} repeat(s), {t:.1f} s (numpy fp64 matmuls on {threads} BLAS threads)",
            "one_thread": {"value": round(max(1, n // 8) / t1, 4), "unit": "tokens/s",
                           "sample": f"{max(1, n // 8)} rows, {t1:.1f} s"}}


# ------------------------------------------------------------------ CPU baseline (oracle)
def cpu_baseline_decode(cfg, ctx_state, budget_s=12.0):
    """The oracle's decode step (indexer + top-k + CSA attention + HCA attention) for a
    sample of the batch's sequences, timed on the host cores."""
    import oracle
    from oracle import pipeline as opl
    from long_context_attention_17_amd import synth
    ctx, _ = ctx_state
    seqs = [0, 1] if cfg.B >= 2 else [0]
    states = {}
    progress("cpu baseline: building the oracle's state for the sampled sequences")
    for name in ("csa", "hca"):
        # draw on the GPU (fast), keep only the sampled sequences' cache rows on the host
        inp = synth.decode_layer(cfg, name, "cuda", ctx)
        last = inp["entry_offsets"][len(seqs)]
        host = {}
        for key, v in inp.items():
            if key in ("entries", "ikeys"):
                host[key] = v[:last].cpu()
            elif isinstance(v, torch.Tensor):
                host[key] = v.cpu()
            else:
                host[key] = v
        del inp
        torch.cuda.empty_cache()
        states[name] = (host, opl.decode_state(cfg, host, seqs=seqs))
    reps, t_total = 0, 0.0
    progress("cpu baseline: timing the oracle")
    while t_total < budget_s or reps == 0:
        t0 = time.perf_counter()
        opl.csa_decode_step(cfg, states["csa"][0], states["csa"][1], seqs=seqs)
        opl.hca_decode_step(cfg, states["hca"][0], states["hca"][1], seqs=seqs)
        t_total += time.perf_counter() - t0
        reps += 1
        if reps >= 50:
            break
    tok_s = len(seqs) * reps / t_total
    cores = oracle.num_threads()
    # the same step for one sequence on one thread (a few repeats)
    progress("cpu baseline: one thread")
    oracle.set_num_threads(1)
    try:
        reps1, t1 = 0, 0.0
        while t1 < 3.0 and reps1 < 5:
            t0 = time.perf_counter()
            opl.csa_decode_step(cfg, states["csa"][0], states["csa"][1], seqs=seqs[:1])
            opl.hca_decode_step(cfg, states["hca"][0], states["hca"][1], seqs=seqs[:1])
            t1 += time.perf_counter() - t0
            reps1 += 1
    finally:
        oracle.set_num_threads(cores)
    return {"value": round(tok_s, 4), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(), "host_threads": os.cpu_count(),
            "sample": f"{len(seqs)} of {cfg.B} sequences (both layers' indexer, top-k and attention), {reps} repeat(s), "
                      f"{t_total:.1f} s; the oracle's loops run on {cores} threads (over keys in the indexer, "
                      f"over heads in attention)",
            "one_thread": {"value": round(reps1 / t1, 4), "unit": "tokens/s",
                           "sample": f"sequence 0 only, {reps1} repeat(s), {t1:.1f} s"}}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_prefill(cfg, budget_s=12.0):
    import numpy as np
    import oracle
    from oracle import pipeline as opl
    from long_context_attention_17_amd import synth
    rows = np.unique(np.linspace(cfg.L // 2, cfg.L - 1, 64).astype(np.int64))
    t_total, n_rows = 0.0, 0
    for name in (["csa"] if cfg.csa else []) + (["hca"] if cfg.hca else []):
        inp = synth.prefill_layer(cfg, name, "cpu")
        ratio = cfg.m if name == "csa" else cfg.m_hca
        pt, n_pool = synth.page_table([cfg.L // ratio], cfg.page, cfg.seed)
        t0 = time.perf_counter()
        (opl.csa_prefill if name == "csa" else opl.hca_prefill)(cfg, inp, pt.numpy()[0], n_pool, rows=rows)
        t_total += time.perf_counter() - t0
    n_rows = len(rows)
    cores = oracle.num_threads()
    rows1 = rows[::8]
    oracle.set_num_threads(1)
    try:
        t1 = 0.0
        for name in (["csa"] if cfg.csa else []) + (["hca"] if cfg.hca else []):
            inp = synth.prefill_layer(cfg, name, "cpu")
            ratio = cfg.m if name == "csa" else cfg.m_hca
            pt, n_pool = synth.page_table([cfg.L // ratio], cfg.page, cfg.seed)
            t0 = time.perf_counter()
            (opl.csa_prefill if name == "csa" else opl.hca_prefill)(cfg, inp, pt.numpy()[0], n_pool, rows=rows1)
            t1 += time.perf_counter() - t0
    finally:
        oracle.set_num_threads(cores)
    return {"value": round(n_rows / t_total, 4), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(), "host_threads": os.cpu_count(),
            "sample": f"{n_rows} query rows from the second half of the sequence (compression of the whole "
                      f"sequence included), {t_total:.1f} s on {cores} threads",
            "one_thread": {"value": round(len(rows1) / t1, 4), "unit": "tokens/s",
                           "sample": f"{len(rows1)} of those rows (compression included), {t1:.1f} s"}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_1m", choices=sorted(WORKLOADS) + sorted(SUBLAYER_WORKLOADS))
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run a plain device-to-device copy of this many MiB (3 times), the reference "
                         "kernel for scaling HBM counter readings")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the workload and runs on one GPU only (--gpus 1); "
              "the library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    from long_context_attention_17_amd.configs import CONFIGS
    torch.cuda.set_device(0)
    if args.workload in SUBLAYER_WORKLOADS:
        value, ms, config, roof, extra, state = bench_sublayer(args.workload, args.steps, args.warmup,
                                                               max(args.replicas, 3))
        roof["traffic"] = None
        line = {"metric": SUBLAYER_METRIC, "value": round(value, 3), "unit": "tokens/s", "n_gpus": 1,
                "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
                "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic", "config": config,
                "roofline": roof}
        del state
        torch.cuda.empty_cache()
        if not args.no_cpu_baseline:
            line["cpu_baseline"] = cpu_baseline_sublayer(args.workload)
        line.update(extra)
        line["kernel_source_hash"] = kernel_source_hash(roof["kernel"])
        print(json.dumps(line), flush=True)
        return
    wl = WORKLOADS[args.workload]
    cfg = CONFIGS[wl] if isinstance(wl, int) else dataclasses.replace(CONFIGS[wl[0]], **wl[1])
    if args.copy_calibration_mib > 0:
        src = torch.empty(args.copy_calibration_mib << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()
    if cfg.phase == "decode":
        value, ms, config, roof, extra, state = bench_decode(cfg, args.steps, args.warmup, args.replicas, args)
    else:
        value, ms, config, roof, extra, state = bench_prefill(cfg, args.steps, args.warmup, args.replicas, args)
    # HBM traffic of the dominant kernel from committed rocprofv3 counter runs (null if stale)
    traffic = None
    tpath = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tpath):
        with open(tpath) as f:
            tj = json.load(f)
        ent = tj.get(args.workload, {}).get(roof["kernel"])
        if ent and ent.get("source_hash") == kernel_source_hash(roof["kernel"]):
            traffic = ent.get("bytes_per_launch")
    roof["traffic"] = traffic
    line = {"metric": METRIC, "value": round(value, 3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic", "config": config, "roofline": roof}
    del state
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = (cpu_baseline_decode(cfg, (synth_ctx(cfg), None)) if cfg.phase == "decode"
                                else cpu_baseline_prefill(cfg))
    line.update(extra)
    line["kernel_source_hash"] = kernel_source_hash(roof["kernel"])
    print(json.dumps(line), flush=True)


def synth_ctx(cfg):
    from long_context_attention_17_amd import synth
    return synth.decode_contexts(cfg)


if __name__ == "__main__":
    main()
