"""Layer descriptors of the workloads the pages describe (shapes only).

Sources (page title, section): "DeepSeek-V4 内部机制" §1.3 (m = 4, m' = 128),
§1.4 table (n_win = 128, RoPE on the last 64 channels), §1.5 (FP8 + BF16 KV),
§6.2 (FP4 indexer, BF16 scores); m.admirer.cn CSA section (top-k 512 for the
Flash shape, 1024 for the Pro shape; block of 128 raw tokens).
"""
from __future__ import annotations

from .abi import (ACT_BF16, ACT_F32, IDX_BF16, IDX_F32, IDX_MXFP4, KIND_CSA, KIND_HCA, KV_BF16, KV_F32, KV_FP8,
                  LayerDesc)


def layer(kind, m, c, r, n_heads, n_idx_heads=0, c_idx=0, top_k=0, n_win=128, win_cap=128, block_tokens=128,
          kv_fmt=KV_F32, idx_fmt=IDX_F32, score_fmt=ACT_F32, act_fmt=ACT_F32, out_fmt=ACT_F32,
          rope_theta=10000.0, norm_eps=1e-6, flags=0) -> LayerDesc:
    return LayerDesc(kind=kind, m=m, c=c, rope_dim=r, n_heads=n_heads, n_idx_heads=n_idx_heads, c_idx=c_idx,
                     top_k=top_k, n_win=n_win, win_cap=win_cap, block_tokens=block_tokens, kv_fmt=kv_fmt,
                     idx_fmt=idx_fmt, score_fmt=score_fmt, act_fmt=act_fmt, out_fmt=out_fmt,
                     rope_theta=rope_theta, norm_eps=norm_eps, flags=flags)


def tiny_csa_fp32(win_cap=128) -> LayerDesc:
    """Tiny CSA layer, fp32 throughout: c=128 (RoPE 32), m=4, 8 heads,
    indexer 4 x 64, top-64, 128-token window (hidden width 512)."""
    return layer(KIND_CSA, 4, 128, 32, 8, 4, 64, 64, win_cap=win_cap)


def hca_bf16(win_cap=128) -> LayerDesc:
    """HCA layer, bf16 activations and KV, fp32 output: c=256 (RoPE 64),
    m'=128, 16 heads (hidden width 1024)."""
    return layer(KIND_HCA, 128, 256, 64, 16, kv_fmt=KV_BF16, act_fmt=ACT_BF16, out_fmt=ACT_F32, win_cap=win_cap)


def csa_flash_decode(win_cap=128) -> LayerDesc:
    """CSA decode, Flash-like: c=512 (64 RoPE channels in bf16, 448 in fp8 with
    a per-block scale), m=4, 64 heads, indexer 64 x 128 bf16, top-512."""
    return layer(KIND_CSA, 4, 512, 64, 64, 64, 128, 512, kv_fmt=KV_FP8, idx_fmt=IDX_BF16, score_fmt=ACT_BF16,
                 act_fmt=ACT_BF16, out_fmt=ACT_BF16, win_cap=win_cap)


def csa_pro(win_cap=128, idx_fmt=IDX_BF16) -> LayerDesc:
    """CSA, Pro-like: as the Flash shape with 128 heads and top-1024."""
    return layer(KIND_CSA, 4, 512, 64, 128, 64, 128, 1024, kv_fmt=KV_FP8, idx_fmt=idx_fmt, score_fmt=ACT_BF16,
                 act_fmt=ACT_BF16, out_fmt=ACT_BF16, win_cap=win_cap)


def hca_pro(win_cap=128) -> LayerDesc:
    """HCA, Pro-like: c=512 fp8/bf16 KV, m'=128, 128 heads."""
    return layer(KIND_HCA, 128, 512, 64, 128, kv_fmt=KV_FP8, act_fmt=ACT_BF16, out_fmt=ACT_BF16, win_cap=win_cap)


# hidden widths used for the compressor projection of each shape
D_TINY, D_HCA, D_FLASH, D_PRO = 512, 1024, 4096, 7168
