"""Oracle of the attention sublayer around CSA / HCA -- TEST INFRASTRUCTURE ONLY
(same rules as the rest of this package: only tests/, the smoke check and the
cpu_baseline leg of bench.py use it).

dsv4 book Ch.6 "Low-rank query generation": the hidden state h_t (width d) is
projected down to a shared query latent c^Q_t (width d_c); the main queries q_t
(n_h heads of c) and the indexer queries q^I_t (n_I heads of c_I) are both expanded
from that latent, while the indexer's per-head combiner weights w^I_t come from
h_t directly ("The lightning indexer").

dsv4 book Ch.6 "Grouped output projections" (and Ch.4 "Query head scaling and
grouped output projections"): the n_h head outputs are split into g groups of 8
heads; each group's 8 c concatenated channels are projected to d_g, and the g
results, concatenated, are projected to d.  No nonlinearity sits between the two.

The equations themselves did not survive the pages' extraction; the readings taken:
  - every projection is a plain linear map, x -> x W, no bias, no normalization of
    the latent (none is named);
  - group j holds heads 8j .. 8j+7 (contiguous), its input is their outputs
    concatenated in head order;
  - weights are given as [out, in] arrays (the transpose of the pages' x W form:
    W^{DQ} as [d_c, d], W^{UQ} as [n_h c, d_c], W^{IUQ} as [n_I c_I, d_c],
    W^w as [n_I, d], the group projections as [g, d_g, 8 c], the final one as
    [d, g d_g]);
  - the latent c^Q and the group outputs u are stored in the activation format
    (`act`: "bf16" rounds them to bfloat16, round to nearest even, as the stored
    queries are; "f64" keeps them exact), q and q^I are stored in `act`, w^I in
    fp32, the sublayer output y in `act`.

Every product is numpy's fp64 matmul (a library primitive) of the given values;
nothing is blocked, fused or reordered.
"""
from __future__ import annotations

import numpy as np

from . import bf16_decode, bf16_encode

HEADS_PER_GROUP = 8


def store(x, act: str) -> np.ndarray:
    """The value a tensor holds once stored in `act` ("bf16" | "f32" | "f64")."""
    x = np.asarray(x, np.float64)
    if act == "bf16":
        return bf16_decode(bf16_encode(x))
    if act == "f32":
        return x.astype(np.float32).astype(np.float64)
    if act == "f64":
        return x
    raise ValueError(act)


def project(x, w, act):
    """One linear map of the sublayer, x [T, in] -> x W (w given as [out, in]), stored in act."""
    return store(np.asarray(x, np.float64) @ np.asarray(w, np.float64).T, act)


def low_rank_query(h, w_dq, w_uq, w_iuq, w_w, act="bf16"):
    """Ch.6 "Low-rank query generation" and "The lightning indexer".
    h [T, d]; returns c^Q [T, d_c], q [T, n_h c], q^I [T, n_I c_I], w^I [T, n_I]."""
    c = project(h, w_dq, act)                                     # shared latent
    return {"c": c,
            "q": project(c, w_uq, act),                           # main queries from the latent
            "qI": project(c, w_iuq, act),                         # indexer queries from the same latent
            "w": project(h, w_w, "f32" if act != "f64" else "f64")}   # from h itself


def group_proj(o, w_o1, act="bf16"):
    """The first stage of Ch.6 "Grouped output projections": o [T, n_h c] (heads in head
    order), w_o1 [g, d_g, 8 c]; group j maps heads 8j .. 8j+7 to block j of u [T, g d_g]."""
    o = np.asarray(o, np.float64)
    w_o1 = np.asarray(w_o1, np.float64)
    g, d_g, width = w_o1.shape
    assert o.shape[1] == g * width, "the heads must split into g groups of the projection's width"
    u = np.empty((o.shape[0], g * d_g))
    for j in range(g):
        u[:, j * d_g:(j + 1) * d_g] = o[:, j * width:(j + 1) * width] @ w_o1[j].T
    return store(u, act)


def grouped_out_proj(o, w_o1, w_o2, act="bf16"):
    """Ch.6 "Grouped output projections".  o [T, n_h c]; w_o1 [g, d_g, 8 c]; w_o2 [d, g d_g].
    Returns u [T, g d_g] (the g group outputs, concatenated) and y [T, d]."""
    u = group_proj(o, w_o1, act)
    return {"u": u, "y": project(u, w_o2, act)}


def weight_shapes(d, d_c, n_h, c, n_i, c_i, g, d_g):
    """Shapes of the sublayer's weights in the [out, in] layout above."""
    assert n_h == HEADS_PER_GROUP * g, "8 heads per group"
    return {"w_dq": (d_c, d), "w_uq": (n_h * c, d_c), "w_iuq": (n_i * c_i, d_c), "w_w": (n_i, d),
            "w_o1": (g, d_g, HEADS_PER_GROUP * c), "w_o2": (d, g * d_g)}
