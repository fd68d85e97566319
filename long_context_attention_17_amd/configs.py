"""The five workload presets (shapes, ratios, storage formats).

Each preset is a single-GPU workload of compressed sparse attention (CSA) and
heavily compressed attention (HCA) as described in the dsv4 book (Ch.5-8):
head dimension D with the last R channels rotary, n_h query heads over one
shared key=value head, CSA ratio m with an n_I x c_I lightning indexer and
top-k, HCA ratio m', and a sliding window of n_win raw tokens.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Config:
    name: str
    phase: str                 # "prefill" or "decode"
    D: int                     # entry / query head dimension
    R: int                     # rotary channels (the last R of D)
    n_h: int                   # query heads
    act: str                   # storage of q, projections and window: "f32" | "bf16"
    kv: str                    # compressed-entry record: "f32" | "bf16" | "fp8mix"
    csa: bool = True
    m: int = 4                 # CSA compression ratio
    k: int = 0                 # CSA top-k (entries)
    n_win: int = 128           # window of raw tokens (both layers)
    nI: int = 0                # indexer heads
    cI: int = 0                # indexer head dim
    idx: str = "e4m3"          # indexer storage: "f32" | "e4m3" | "fp4" (e2m1 + E8M0 scale per 32 channels)
    idx_q: str = "e4m3"        # indexer queries for e4m3 / fp4 keys: "e4m3", or "fp4" (fp4 keys only)
    hca: bool = False
    m_hca: int = 128           # HCA compression ratio
    L: int = 0                 # prefill length
    B: int = 0                 # decode batch
    ctx_lo: int = 0            # decode context range (inclusive); the new token sits at t = ctx
    ctx_hi: int = 0
    page: int = 64             # entries per cache page
    eps: float = 1e-6
    rope_base: float = 10000.0
    seed: int = 0
    prefix: int = 0            # prefill only: positions 0..prefix-1 are a stored prefix (their entries are
                               # in the cache); the prefill computes positions prefix..L-1
    notes: str = field(default="", compare=False)

    def __post_init__(self):
        if self.idx_q not in ("e4m3", "fp4") or (self.idx_q == "fp4" and self.idx != "fp4"):
            raise ValueError(f"idx_q={self.idx_q!r} with idx={self.idx!r}: fp4 queries need fp4 keys")


CONFIGS = {
    1: Config(name="tiny_f32", phase="prefill", D=64, R=8, n_h=8, act="f32", kv="f32",
              csa=True, m=4, k=64, n_win=64, nI=4, cI=32, idx="f32", hca=True, m_hca=64, L=1024,
              seed=1001, notes="CSA + HCA single layer each, fp32, L=1024"),
    2: Config(name="csa_prefill_32k", phase="prefill", D=512, R=64, n_h=64, act="bf16", kv="bf16",
              csa=True, m=4, k=1024, n_win=128, nI=8, cI=64, idx="e4m3", hca=False, L=32768,
              seed=1002, notes="CSA prefill, bf16, L=32768"),
    3: Config(name="hca_prefill_128k", phase="prefill", D=512, R=64, n_h=64, act="bf16", kv="bf16",
              csa=False, hca=True, m_hca=128, n_win=128, L=131072,
              seed=1003, notes="HCA prefill, bf16, L=131072"),
    4: Config(name="mixed_decode_b64", phase="decode", D=512, R=64, n_h=64, act="bf16", kv="fp8mix",
              csa=True, m=4, k=1024, n_win=128, nI=8, cI=64, idx="e4m3", hca=True, m_hca=128,
              B=64, ctx_lo=16384, ctx_hi=131072, seed=1004,
              notes="decode, B=64, ctx ~ U{16384..131072}, CSA layer + HCA layer, fp8 pages"),
    5: Config(name="million_decode_b8", phase="decode", D=512, R=64, n_h=128, act="bf16", kv="fp8mix",
              csa=True, m=4, k=2048, n_win=128, nI=8, cI=64, idx="e4m3", hca=True, m_hca=128,
              B=8, ctx_lo=1 << 20, ctx_hi=1 << 20, seed=1005,
              notes="decode, B=8, ctx=2^20, CSA layer + HCA layer, fp8 pages"),
}


def get(cfg) -> Config:
    return CONFIGS[cfg] if isinstance(cfg, int) else cfg


@dataclass(frozen=True)
class SublayerDims:
    """Widths of the attention sublayer's projections (dsv4 book Ch.6 "Low-rank query
    generation", "Grouped output projections"): hidden d, query latent d_c, n_h heads of
    c, n_i indexer heads of c_i, g groups of 8 heads each projected to d_g."""
    name: str
    d: int
    d_c: int
    n_h: int
    c: int
    n_i: int
    c_i: int
    g: int
    d_g: int


SUBLAYERS = {
    "flash": SublayerDims("flash", d=4096, d_c=1024, n_h=64, c=512, n_i=64, c_i=128, g=8, d_g=1024),
    "pro": SublayerDims("pro", d=7168, d_c=1536, n_h=128, c=512, n_i=64, c_i=128, g=16, d_g=1024),
}
