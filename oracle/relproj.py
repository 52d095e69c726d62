"""Projection of the relative-position embeddings into the per-head tables,
float64 numpy.

TEST INFRASTRUCTURE: only tests, the smoke entry and the benchmark's CPU
baseline may import this module. The product path never does.

What it computes. The tables qr and kr that the disentangled scores read
are per-head projections of one relative-embedding table shared by the
batch (a DeBERTa-v3-base-shaped encoder projects a 512 x 768 table). In
DeBERTa-v2/v3 (the models the DisentangledFlash README's "Attribution"
section names) the projections are the attention layer's own query and key
linear maps, and the kernels-community layer reuses the host encoder's
projection modules rather than copying them. With E the [n_rel, hidden]
relative embeddings, nn.Linear-style weights W ([out = H*d, in = hidden])
and biases b:

    qr = E Wq^T + bq,    kr = E Wk^T + bk          ([n_rel, H*d])

Head h of a row is columns h*d .. h*d+d-1, as in the forward. A missing
bias is zero.
"""

from __future__ import annotations

import numpy as np


def rel_proj(E, Wq, Wk, bq=None, bk=None):
    """(qr, kr) in float64."""
    E = np.asarray(E, dtype=np.float64)
    out = []
    for W, b in ((Wq, bq), (Wk, bk)):
        W = np.asarray(W, dtype=np.float64)
        y = E @ W.T
        if b is not None:
            y = y + np.asarray(b, dtype=np.float64)[None, :]
        out.append(y)
    return out[0], out[1]


def abs_bound(E, W):
    """sum_i |E[r, i]| |W[o, i]| for every output: the scale that bounds the
    rounding error of any fp32-accumulated evaluation of the product."""
    return np.abs(np.asarray(E, np.float64)) @ np.abs(np.asarray(W, np.float64)).T
