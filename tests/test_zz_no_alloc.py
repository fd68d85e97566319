"""The allocation-free HCA decode step (ca_hca_decode_step_noalloc) against the
workspace step (ca_hca_decode_step) it varies: bitwise the same outputs and caches,
on two calls in a row, the second with a smaller input than the first."""
import ctypes

import pytest
import torch

from gpu_util import log

pytestmark = pytest.mark.gpu


def _case(name, n_h, B, lo, hi, seed):
    from long_context_attention_17_amd.configs import Config
    return Config(name=name, phase="decode", D=512, R=64, n_h=n_h, act="bf16", kv="fp8mix", m=4, k=64, n_win=128,
                  nI=8, cI=64, hca=True, m_hca=128, B=B, ctx_lo=lo, ctx_hi=hi, seed=seed)


def test_no_alloc_step_matches_the_workspace_step():
    from long_context_attention_17_amd import binding as ca, layers, synth
    lib = ca.lib()
    assert lib.ca_static_scratch_bytes() == 64 << 20
    for cfg in (_case("noalloc_big", 128, 6, 20000, 60000, 8101), _case("noalloc_small", 64, 2, 300, 1500, 8102)):
        ctx = synth.decode_contexts(cfg)
        dl = layers.DecodeLayer(cfg, synth.decode_layer(cfg, "hca", "cuda", ctx))
        need = ca.attend_workspace(dl.ap, cfg.B, dl.max_pos, 0, cfg.m_hca)
        log(f"[no-alloc] {cfg.name}: B={cfg.B} n_h={cfg.n_h} ctx={ctx.tolist()} scratch needed {need} bytes")
        state = {"window": dl.window, "tail": dl.tail, "kv": dl.kv.pool}
        before = {k: v.clone() for k, v in state.items()}
        dl.fused_step()                                   # the workspace step
        torch.cuda.synchronize()
        ref = {k: v.clone() for k, v in state.items()}
        ref["out"] = dl.out.view(torch.int16).clone()
        for k, v in state.items():
            v.copy_(before[k])
        dl.out.fill_(7.0)
        dl.fused_step_noalloc()                           # the static-scratch step
        torch.cuda.synchronize()
        got = dict(state, out=dl.out.view(torch.int16))
        for k, v in ref.items():
            assert torch.equal(got[k], v), f"{cfg.name}: the allocation-free step differs in {k}"
