"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module draws random numbers and lays out bookkeeping arrays (block
tables, positions).  It holds none of the method's arithmetic, and neither the
HIP library nor the oracle is imported here.

Generator: numpy PCG64 seeded per case.  Hidden states and the raw rows that
stand in for compressed entries / indexer keys are N(0, 1); projection
weights are N(0, 1/sqrt(fan_in)); position biases and sink logits are N(0, 1);
the indexer head weights w are N(0, 1) / sqrt(n_hI).  RMSNorm gains are 1.
"""
from __future__ import annotations

import numpy as np


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def normal(g: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    return (g.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def weights(g: np.random.Generator, fan_in: int, fan_out: int) -> np.ndarray:
    return normal(g, (fan_in, fan_out), 1.0 / np.sqrt(fan_in))


def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """Round float32 data to bf16 with torch's CPU cast and return float32
    values: used only to build inputs that are bf16 by definition."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


def block_table(g: np.random.Generator, n_req: int, blocks_per_req: int, extra: int = 0) -> np.ndarray:
    """A random placement of every request's logical blocks in one physical
    pool of n_req*blocks_per_req + extra blocks (int32 [n_req, blocks_per_req])."""
    total = n_req * blocks_per_req + extra
    perm = g.permutation(total).astype(np.int32)
    return perm[: n_req * blocks_per_req].reshape(n_req, blocks_per_req)


def csa_weights(g: np.random.Generator, d: int, c: int, m: int, c_I: int = 0):
    """Compressor parameters of one CSA layer: W [d, 4c] = [aKV|bKV|aZ|bZ],
    B^a, B^b [m, c], and the indexer's own W_I [d, 4c_I], B^a_I, B^b_I."""
    out = {
        "W": weights(g, d, 4 * c),
        "Ba": normal(g, (m, c)),
        "Bb": normal(g, (m, c)),
    }
    if c_I:
        out["W_I"] = weights(g, d, 4 * c_I)
        out["BaI"] = normal(g, (m, c_I))
        out["BbI"] = normal(g, (m, c_I))
    return out


def hca_weights(g: np.random.Generator, d: int, c: int, m: int):
    """Compressor parameters of one HCA layer: W [d, 2c] = [KV|Z], B [m, c]."""
    return {"W": weights(g, d, 2 * c), "Ba": normal(g, (m, c))}


def queries(g: np.random.Generator, T: int, n_h: int, c: int, n_hI: int = 0, c_I: int = 0):
    """Raw attention queries [T, n_h, c], indexer queries [T, n_hI, c_I] and
    indexer head weights [T, n_hI]."""
    out = {"q": normal(g, (T, n_h, c))}
    if n_hI:
        out["qI"] = normal(g, (T, n_hI, c_I))
        out["w"] = normal(g, (T, n_hI), 1.0 / np.sqrt(n_hI))
    return out


def sinks(g: np.random.Generator, n_h: int) -> np.ndarray:
    return normal(g, (n_h,))
