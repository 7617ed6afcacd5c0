"""Whole-layer composition of the oracle's steps (TEST INFRASTRUCTURE ONLY).

Every function here strings together the fp64 steps of ``csa_oracle.c`` in
the order the pages give them; nothing is blocked, fused or reordered.

Sources (page title, section):
  [DD] "DeepSeek-V4 内部机制" deep dive: §1.2 Step 1 (compressor), Step 2
       (indexer, top-k), §1.3 (HCA), §1.4 table (Q/KV RMSNorm, partial RoPE,
       128-token window, sink equation), §1.5 (BF16 RoPE dims + FP8 rest),
       §6.2 (FP4 indexer QK, BF16 scores), §7 (state cache + paged cache whose
       block holds lcm(m, m') raw tokens).
  [YP] yunpan.plus explainer, eqs. (6)-(11).
  [AD] m.admirer.cn article, CSA/HCA section.

Readings where the pages are silent (listed in the design doc as well):
  * the compressor softmax runs over the 2m window rows, per channel;
  * entry 0 has no previous block and soft-maxes over its m own rows only;
  * entry i is visible to the query at t iff m*(i+1)-1 <= t;
  * entry i carries RoPE position m*i; the query at t position t; the output
    is rotated back at -t; RoPE pairs are interleaved over the last r
    channels with theta = 10000;
  * RMSNorm eps = 1e-6 on q heads, compressed entries and window rows; the
    indexer keys and queries get neither norm nor RoPE;
  * window rows are the rows C^a_j (CSA) / C_j (HCA) of the compressor's own
    projection, normalised and rotated at j, for j in [t-n_win+1, t];
  * the softmax scale is 1/sqrt(c); the sink logit is unscaled.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

import oracle as O

KV_F32, KV_BF16, KV_FP8 = "f32", "bf16", "fp8"
IDX_F32, IDX_BF16, IDX_MXFP4 = "f32", "bf16", "mxfp4"


@dataclass
class Spec:
    kind: str            # "csa" | "hca"
    m: int               # compression ratio (4 CSA, 128 HCA)
    c: int               # compressed KV width
    r: int               # RoPE channels (the last r of c)
    n_h: int             # query heads
    n_hI: int = 0        # indexer heads (CSA)
    c_I: int = 0         # indexer key width (CSA)
    top_k: int = 0       # CSA
    n_win: int = 128
    block_tokens: int = 128
    kv_fmt: str = KV_F32
    idx_fmt: str = IDX_F32
    score_fmt: str = "f32"
    win_fmt: str = "f32"
    theta: float = 10000.0
    eps: float = 1e-6

    @property
    def overlap(self) -> bool:
        return self.kind == "csa"

    @property
    def epb(self) -> int:
        return self.block_tokens // self.m

    @property
    def scale(self) -> float:
        return 1.0 / np.sqrt(self.c)


# ---------------------------------------------------------------------------
# a1: projection + compressor + entry / window-row normalisation
# ---------------------------------------------------------------------------

def project(H, W):
    """The compressor's projections H . W in fp64 (a plain matmul)."""
    return np.asarray(H, np.float64) @ np.asarray(W, np.float64)


def query_path(H, W_DQ, W_UQ, W_UQI, W_w, round_mid: bool = True):
    """[DD] §1.2 Step 2 query side; [AD] d_c = 1024: c^Q = H W_DQ^T (stored in
    bf16 unless round_mid is False), q = c^Q W_UQ^T, q^I = c^Q W_UQI^T, and
    the indexer head weights w = H W_w^T (reading: a projection of the
    token's hidden state).  Weights one row per output."""
    H = np.asarray(H, np.float64)
    cq = H @ np.asarray(W_DQ, np.float64).T
    if round_mid:
        cq = O.bf16_round(cq).astype(np.float64)
    return (cq @ np.asarray(W_UQ, np.float64).T, cq @ np.asarray(W_UQI, np.float64).T,
            H @ np.asarray(W_w, np.float64).T)


def grouped_output(Oh, W_G, W_O, round_mid: bool = True):
    """[DD] §1.2 Step 3: the head outputs (concatenated in head order, width
    n_h*c) split into g equal groups; group j is projected by W_G[j]
    (d_g x n_h*c/g) to d_g; the g results, concatenated in group order (bf16
    unless round_mid is False), are projected by W_O (d x g*d_g) to d."""
    Oh = np.asarray(Oh, np.float64)
    g = W_G.shape[0]
    K = Oh.shape[1] // g
    z = np.concatenate([Oh[:, j * K:(j + 1) * K] @ np.asarray(W_G[j], np.float64).T for j in range(g)], axis=1)
    if round_mid:
        z = O.bf16_round(z).astype(np.float64)
    return z @ np.asarray(W_O, np.float64).T


def compress_layer(spec: Spec, H, W, Ba, Bb=None, gamma=None, W_I=None, BaI=None, BbI=None, pos0: int = 0):
    """Entries, indexer keys and window rows of one request's tokens 0..n-1
    (the sequence may start at position pos0, a multiple of m: entry i is then
    rotated at pos0 + m*i and window row j at pos0 + j; its first entry has no
    previous block).

    CSA: W = [W^aKV | W^bKV | W^aZ | W^bZ] (d x 4c), W_I likewise (d x 4c_I).
    HCA: W = [W^KV | W^Z] (d x 2c).
    Returns (entries [n/m, c] normalised+rotated, keys [n/m, c_I] raw,
    window rows [n, c] normalised+rotated), all fp64.
    """
    c, m = spec.c, spec.m
    P = project(H, W)
    n = P.shape[0]
    if spec.overlap:
        Ca, Cb, Za, Zb = (P[:, j * c:(j + 1) * c] for j in range(4))
        E = O.compress(Ca, Cb, Za, Zb, Ba, Bb, m, True)
    else:
        Ca, Za = P[:, :c], P[:, c:2 * c]
        E = O.compress(Ca, None, Za, None, Ba, None, m, False)
    ne = E.shape[0]
    g = np.ones(c) if gamma is None else np.asarray(gamma, np.float64)
    assert pos0 % m == 0
    Ehat = O.rope(O.rmsnorm(E, g, spec.eps), pos0 + m * np.arange(ne, dtype=np.float64), spec.r, spec.theta)
    R = O.rope(O.rmsnorm(Ca, g, spec.eps), pos0 + np.arange(n, dtype=np.float64), spec.r, spec.theta)
    K = None
    if spec.kind == "csa" and W_I is not None:
        cI = spec.c_I
        PI = project(H, W_I)
        CaI, CbI, ZaI, ZbI = (PI[:, j * cI:(j + 1) * cI] for j in range(4))
        K = O.compress(CaI, CbI, ZaI, ZbI, BaI, BbI, m, True)
    return Ehat, K, R


# ---------------------------------------------------------------------------
# a2: storage rounding and block layout
# ---------------------------------------------------------------------------

def kv_record_bytes(spec: Spec) -> int:
    if spec.kv_fmt == KV_F32:
        return 4 * spec.c
    if spec.kv_fmt == KV_BF16:
        return 2 * spec.c
    return (spec.c - spec.r) + 2 * spec.r


def kv_block_bytes(spec: Spec) -> int:
    hdr = 64 if spec.kv_fmt == KV_FP8 else 0
    return hdr + spec.epb * kv_record_bytes(spec)


def idx_block_bytes(spec: Spec) -> int:
    cI = spec.c_I
    if spec.idx_fmt == IDX_F32:
        return spec.epb * cI * 4
    if spec.idx_fmt == IDX_BF16:
        return spec.epb * cI * 2
    return spec.epb * (cI // 2 + cI // 32)


def store_entries(spec: Spec, entries32, calls):
    """Logical block bytes of a request's entries and their dequantised fp64
    values.  entries32 [ne, c] float32; calls is a list of (first, count)
    entry ranges appended together (the fp8 block-scale rule is applied per
    call and block).  Returns (blocks uint8 [nb, block_bytes], deq [ne, c])."""
    c, r, epb = spec.c, spec.r, spec.epb
    x = np.ascontiguousarray(entries32, np.float32).reshape(-1, c)
    ne = x.shape[0]
    nb = (ne + epb - 1) // epb
    bb = kv_block_bytes(spec)
    blocks = np.zeros((max(nb, 1), bb), np.uint8)
    deq = np.zeros((ne, c), np.float64)
    if spec.kv_fmt == KV_F32:
        for i in range(ne):
            blocks[i // epb, (i % epb) * 4 * c:(i % epb + 1) * 4 * c] = x[i].view(np.uint8)
        deq[:] = x
    elif spec.kv_fmt == KV_BF16:
        xb = O.bf16_round(x)
        for i in range(ne):
            blocks[i // epb, (i % epb) * 2 * c:(i % epb + 1) * 2 * c] = (
                xb[i].view(np.uint32) >> 16).astype(np.uint16).view(np.uint8)
        deq[:] = xb
    else:
        for first, count in calls:
            e = first
            while e < first + count:
                b = e // epb
                stop = min(first + count, (b + 1) * epb)
                blk = np.ascontiguousarray(blocks[b])
                O.fp8_block_append(blk, c, r, epb, e - b * epb, x[e:stop])
                blocks[b] = blk
                e = stop
        for i in range(ne):
            deq[i] = O.fp8_block_decode(blocks[i // epb], c, r, epb, i % epb)
    return blocks[:nb], deq


def store_keys(spec: Spec, keys32):
    """Logical indexer-key block bytes and dequantised keys (fp64)."""
    cI, epb = spec.c_I, spec.epb
    x = np.ascontiguousarray(keys32, np.float32).reshape(-1, cI)
    ne = x.shape[0]
    nb = (ne + epb - 1) // epb
    blocks = np.zeros((max(nb, 1), idx_block_bytes(spec)), np.uint8)
    if spec.idx_fmt == IDX_F32:
        for i in range(ne):
            blocks[i // epb, (i % epb) * 4 * cI:(i % epb + 1) * 4 * cI] = x[i].view(np.uint8)
        deq = x.astype(np.float64)
    elif spec.idx_fmt == IDX_BF16:
        xb = O.bf16_round(x)
        for i in range(ne):
            blocks[i // epb, (i % epb) * 2 * cI:(i % epb + 1) * 2 * cI] = (
                xb[i].view(np.uint32) >> 16).astype(np.uint16).view(np.uint8)
        deq = xb.astype(np.float64)
    else:
        codes, scales = O.mxfp4_pack(x)
        for i in range(ne):
            b, s = i // epb, i % epb
            blocks[b, s * (cI // 2):(s + 1) * (cI // 2)] = codes[i]
            off = epb * (cI // 2)
            blocks[b, off + s * (cI // 32):off + (s + 1) * (cI // 32)] = scales[i]
        deq = O.mxfp4_unpack(codes, scales)
    return blocks[:nb], deq


def round_rows(fmt: str, rows32) -> np.ndarray:
    """Window rows as stored (fp32 or bf16), returned as fp64."""
    x = np.ascontiguousarray(rows32, np.float32)
    if fmt == "bf16":
        return O.bf16_round(x).astype(np.float64)
    return x.astype(np.float64)


def quantize_index_queries(spec: Spec, qI32) -> np.ndarray:
    """The indexer query as the QK product consumes it: fp32 or bf16 values as
    given, or MXFP4 (32-element blocks along c_I) for the FP4 indexer path."""
    q = np.ascontiguousarray(qI32, np.float32)
    if spec.idx_fmt == IDX_MXFP4:
        codes, scales = O.mxfp4_pack(q)
        return O.mxfp4_unpack(codes, scales)
    return q.astype(np.float64)


# ---------------------------------------------------------------------------
# a3-a6 for the queries of one request
# ---------------------------------------------------------------------------

def visible(spec: Spec, pos) -> np.ndarray:
    """Number of compressed entries whose last raw token is <= t."""
    return ((np.asarray(pos, np.int64) + 1) // spec.m).astype(np.int32)


def scores(spec: Spec, qI_deq, w, pos, keys_deq):
    fmt = 1 if spec.score_fmt == "bf16" else 0
    return O.index_scores(qI_deq, w, visible(spec, pos), keys_deq, fmt)


def attend(spec: Spec, q_raw, gamma_q, pos, entries_deq, win_deq, sinks, sel=None):
    """Sparse (sel given) or dense (HCA: all visible entries) MQA + window + sink."""
    g = np.ones(spec.c) if gamma_q is None else gamma_q
    n_ent = None if sel is not None else visible(spec, pos)
    return O.attend_batch(q_raw, g, spec.eps, np.asarray(pos, np.float64), spec.theta, spec.scale,
                          entries_deq, sel, n_ent, win_deq, spec.n_win, sinks, spec.r)


def csa_queries(spec: Spec, q_raw, qI32, w, pos, keys_deq, entries_deq, win_deq, sinks, gamma_q=None):
    """Full CSA path for the queries of one request; returns (scores, sel, o)."""
    qd = quantize_index_queries(spec, qI32)
    sc = scores(spec, qd, w, pos, keys_deq)
    sc_safe = np.nan_to_num(sc, nan=0.0)
    sel = O.topk(sc_safe, visible(spec, pos), spec.top_k)
    o = attend(spec, q_raw, gamma_q, pos, entries_deq, win_deq, sinks, sel)
    return sc, sel, o
