"""The dense projections on either side of the attention path, composed from
the library's GEMM calls (argument marshalling only: every product runs in
``csa_linear`` / ``csa_grouped_linear``).

Sources (page title, section): "DeepSeek-V4 内部机制" §1.2 Step 2 (query side:
c^Q_t = h_t . W^DQ, indexer queries from c^Q) and Step 3 (grouped output
projection: g groups of head outputs, each projected to d_g, concatenated,
projected to d; V4-Pro g = 16, d_g = 1024); m.admirer.cn article, CSA section
(the query side drops to d_c = 1024 first).

Weights are stored one row per output ([N x K]); the low-rank query c^Q and
the grouped intermediate z are kept in bf16 between the two products.
"""
from __future__ import annotations

import torch

from . import abi


def query_path(h, W_DQ, W_UQ, W_UQI, W_w, stream=None):
    """h [T x d] bf16 -> (q [T x n_h*c] bf16, q_idx [T x n_hI*c_I] bf16,
    w [T x n_hI] fp32): c^Q = h W_DQ^T (bf16), q = c^Q W_UQ^T,
    q_idx = c^Q W_UQI^T, w = h W_w^T."""
    T = h.shape[0]
    bf = abi.ACT_BF16
    cq = torch.empty((T, W_DQ.shape[0]), dtype=torch.bfloat16, device=h.device)
    abi.linear(bf, bf, h, W_DQ, cq, stream=stream)
    q = torch.empty((T, W_UQ.shape[0]), dtype=torch.bfloat16, device=h.device)
    abi.linear(bf, bf, cq, W_UQ, q, stream=stream)
    q_idx = torch.empty((T, W_UQI.shape[0]), dtype=torch.bfloat16, device=h.device)
    abi.linear(bf, bf, cq, W_UQI, q_idx, stream=stream)
    w = torch.empty((T, W_w.shape[0]), dtype=torch.float32, device=h.device)
    abi.linear(bf, abi.ACT_F32, h, W_w, w, stream=stream)
    return q, q_idx, w


def output_projection(o, W_G, W_O, out_fmt=abi.ACT_BF16, stream=None):
    """o [T x n_h*c] bf16 (the heads in order), W_G [g x d_g x (n_h*c/g)],
    W_O [d x g*d_g] -> y [T x d]: z = concat_g(o_g W_G[g]^T) (bf16), y = z W_O^T."""
    T, g = o.shape[0], W_G.shape[0]
    bf = abi.ACT_BF16
    z = torch.empty((T, g * W_G.shape[1]), dtype=torch.bfloat16, device=o.device)
    abi.grouped_linear(bf, bf, g, o, W_G, z, stream=stream)
    y = torch.empty((T, W_O.shape[0]), dtype=torch.bfloat16 if out_fmt == abi.ACT_BF16 else torch.float32,
                    device=o.device)
    abi.linear(bf, out_fmt, z, W_O, y, stream=stream)
    return y
