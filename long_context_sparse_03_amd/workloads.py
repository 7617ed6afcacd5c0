"""Synthetic decode workloads on the GPU: caches, state and the decode step.

A workload is a stack of layers (CSA and/or HCA) and n_req requests, each
with ctx tokens already in the caches.  The caches are filled through the
library itself (cache_append), from fp32 rows that a caller-supplied source
produces, so the stored bytes follow the library's own formats.  One decode
step runs, for every layer in order, the library's calls for one new token
per request (compress_append, or compress_kv and cache_append); all buffers
are allocated up front, so a step allocates nothing and can be captured in a
HIP graph.  Positions live in two device buffers that alternate: a step reads
one, and its first layer's compress call writes the advanced positions into
the other (csa_batch.next_start_pos), so no other work advances them; a graph
holds steps of both parities.
"""
from __future__ import annotations

import numpy as np
import torch

from . import abi
from .layer import LayerState, make_batch


def torch_rows(seed: int):
    """Row source drawing N(0, 1) fp32 rows on the GPU (torch generator)."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)

    def rows(layer: int, req: int, kind: str, start: int, n: int, width: int) -> torch.Tensor:
        return torch.randn((n, width), generator=gen, device="cuda", dtype=torch.float32)
    return rows


class DecodeWorkload:
    def __init__(self, descs, d_model: int, n_req: int, ctx: int, max_steps: int, rows, seed: int = 0,
                 weight_std: float | None = None, fill_chunk: int = 1 << 16, fused_append: bool = True,
                 fused_topk: bool = True):
        self.descs = list(descs)
        self.fused_append = fused_append
        self.fused_topk = fused_topk
        self.d = d_model
        self.n_req = n_req
        self.ctx = ctx
        self.max_steps = max_steps
        self.dev = "cuda"
        max_ctx = ctx + max_steps
        self.max_ctx = max_ctx
        self.blocks_per_req = (max_ctx + 127) // 128 + 1
        g = np.random.Generator(np.random.PCG64(seed))
        # one block table per request, shared by every layer (each layer has its own pool)
        perm = g.permutation(n_req * self.blocks_per_req).astype(np.int32)
        self.block_table = torch.from_numpy(perm.reshape(n_req, self.blocks_per_req)).to(self.dev)
        self.layers = []
        std = weight_std if weight_std is not None else 1.0 / np.sqrt(d_model)
        for li, desc in enumerate(self.descs):
            assert desc.block_tokens == 128
            st = LayerState(desc, n_req, n_req * self.blocks_per_req, device=self.dev)
            ncols = st.sizes.proj_cols
            n_main = 4 * desc.c if st.is_csa else 2 * desc.c
            Wt = (torch.randn((ncols, d_model), device=self.dev) * std).to(torch.bfloat16)
            P = {
                "W": Wt[:n_main].contiguous(),
                "W_idx": Wt[n_main:].contiguous() if st.is_csa else None,
                "B_a": torch.randn((desc.m, desc.c), device=self.dev),
                "B_b": torch.randn((desc.m, desc.c), device=self.dev) if st.is_csa else None,
                "B_a_idx": torch.randn((desc.m, desc.c_idx), device=self.dev) if st.is_csa else None,
                "B_b_idx": torch.randn((desc.m, desc.c_idx), device=self.dev) if st.is_csa else None,
                "gamma": torch.ones(desc.c, device=self.dev),
                "q_gamma": torch.ones(desc.c, device=self.dev),
                "sinks": torch.randn(desc.n_heads, device=self.dev),
            }
            self.layers.append((st, P))
            self._fill(li, st, desc, rows, fill_chunk)
        self._alloc_step_buffers()

    # ------------------------------------------------------------------
    def _batch(self, start, n_new, max_new, max_ctx, n_tokens):
        cu = torch.tensor(np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32), device=self.dev)
        sp = torch.tensor(np.asarray(start, np.int32), device=self.dev)
        return make_batch(cu, sp, self.block_table, max_new, max_ctx, n_tokens)

    def _fill(self, li, st, desc, rows, chunk):
        n_req, ctx, m = self.n_req, self.ctx, desc.m
        E = ctx // m
        # compressed entries (and indexer keys) of every request
        for e0 in range(0, E, chunk):
            n = min(chunk, E - e0)
            ents = torch.cat([rows(li, r, "entries", e0, n, desc.c) for r in range(n_req)])
            keys = (torch.cat([rows(li, r, "keys", e0, n, desc.c_idx) for r in range(n_req)]) if st.is_csa else None)
            meta = torch.tensor(np.stack([np.repeat(np.arange(n_req), n), np.tile(np.arange(e0, e0 + n), n_req)],
                                         1).astype(np.int32), device=self.dev)
            cnt = torch.tensor([n * n_req], dtype=torch.int32, device=self.dev)
            bi = self._batch(np.zeros(n_req), np.zeros(n_req, np.int64), 0, m * (e0 + n), 0)
            st.append(bi, 0, ents, keys, meta, cnt, n * n_req, None)
        # window rows of the last n_win - 1 tokens
        nw = min(desc.n_win - 1, ctx)
        if nw > 0:
            win = torch.cat([rows(li, r, "window", ctx - nw, nw, desc.c) for r in range(n_req)])
            bi = self._batch(np.full(n_req, ctx - nw), np.full(n_req, nw), nw, ctx, nw * n_req)
            st.append(bi, nw * n_req, None, None, None, None, 0, win)
        # compressor tail: project the hidden rows of the last 2m tokens
        nt = min(2 * m, ctx)
        if nt > 0:
            _, P = self.layers[li]
            H = torch.cat([rows(li, r, "hidden", ctx - nt, nt, self.d) for r in range(n_req)]).to(torch.bfloat16)
            bi = self._batch(np.full(n_req, ctx - nt), np.full(n_req, nt), nt, ctx, nt * n_req)
            max_e = n_req * (ctx // m - (ctx - nt) // m)
            st.compress(bi, nt * n_req, H, P["W"], P["W_idx"], P["B_a"], P["B_b"], P["B_a_idx"], P["B_b_idx"],
                        P["gamma"], max_e)
        torch.cuda.synchronize()

    def _alloc_step_buffers(self):
        n, dev = self.n_req, self.dev
        self.cu_new = torch.arange(n + 1, dtype=torch.int32, device=dev)
        # two position buffers: a step of parity p reads pos[p]; its first
        # layer's compress call writes the next positions into pos[1 - p]
        self.pos = [torch.full((n,), self.ctx, dtype=torch.int32, device=dev) for _ in range(2)]
        self.bi_adv = [make_batch(self.cu_new, self.pos[p], self.block_table, 1, self.max_ctx, n,
                                  next_start_pos=self.pos[1 - p]) for p in range(2)]
        self.bis = [make_batch(self.cu_new, self.pos[p], self.block_table, 1, self.max_ctx, n) for p in range(2)]
        self.parity = 0
        self.bi = self.bis[0]
        self.H = torch.randn((n, self.d), device=dev).to(torch.bfloat16)
        self.bufs = []
        for st, P in self.layers:
            desc = st.desc
            b = {
                "entries": torch.empty((n, desc.c), device=dev),
                "keys": torch.empty((n, max(desc.c_idx, 1)), device=dev),
                "meta": torch.empty((n, 2), dtype=torch.int32, device=dev),
                "count": torch.zeros(1, dtype=torch.int32, device=dev),
                "win": torch.empty((n, desc.c), device=dev),
                "ws_c": st.workspace("compress", abi.workspace_size(desc, abi.OP_COMPRESS, n)),
                "q": torch.randn((n, desc.n_heads, desc.c), device=dev).to(torch.bfloat16),
                "out": torch.empty((n, desc.n_heads, desc.c),
                                   dtype=torch.bfloat16 if desc.out_fmt == abi.ACT_BF16 else torch.float32,
                                   device=dev),
            }
            rows = (desc.top_k if st.is_csa else self.max_ctx // desc.m) + desc.n_win
            b["ws_a"] = st.workspace("attn", abi.workspace_size(desc, abi.OP_ATTENTION, n, rows))
            if st.is_csa:
                self.ld = (self.max_ctx // desc.m + 63) // 64 * 64
                b["qI"] = torch.randn((n, desc.n_idx_heads, desc.c_idx), device=dev).to(torch.bfloat16)
                b["w"] = torch.randn((n, desc.n_idx_heads), device=dev) / np.sqrt(desc.n_idx_heads)
                b["scores"] = torch.empty((n, self.ld), dtype=torch.bfloat16 if desc.score_fmt == abi.ACT_BF16
                                          else torch.float32, device=dev)
                b["n_valid"] = torch.empty(n, dtype=torch.int32, device=dev)
                b["sel"] = torch.empty((n, desc.top_k), dtype=torch.int32, device=dev)
                b["ws_t"] = st.workspace("topk", abi.workspace_size(desc, abi.OP_TOPK, n, self.ld, desc.top_k))
                b["ws_it"] = st.workspace("index_topk", abi.workspace_size(desc, abi.OP_INDEX_TOPK, n, self.ld))
                b["ld"] = self.ld
            self.bufs.append(b)

    # ------------------------------------------------------------------
    def layer_calls(self, li: int, parity: int = 0):
        """The library calls of layer li for one decode token per request, at
        the positions of buffer `parity` (layer 0 also advances them into the
        other buffer)."""
        st, P = self.layers[li]
        b = self.bufs[li]
        desc, n, bi = st.desc, self.n_req, self.bis[parity]
        bic = self.bi_adv[parity] if li == 0 else bi
        s = None
        keys = b["keys"] if st.is_csa else None
        if self.fused_append:
            abi.compress_append(desc, bic.batch, n, self.d, self.H, P["W"], P["W_idx"], P["B_a"], P["B_b"],
                                P["B_a_idx"], P["B_b_idx"], P["gamma"], st.state, b["entries"], keys, b["meta"],
                                b["count"], n, b["win"], st.kv, st.idx, b["ws_c"], stream=s)
        else:
            abi.compress_kv(desc, bic.batch, n, self.d, self.H, P["W"], P["W_idx"], P["B_a"], P["B_b"],
                            P["B_a_idx"], P["B_b_idx"], P["gamma"], st.state, b["entries"], keys, b["meta"],
                            b["count"], n, b["win"], b["ws_c"], stream=s)
            abi.cache_append(desc, bi.batch, n, b["entries"], keys, b["meta"], b["count"], n, b["win"], st.kv,
                             st.idx, st.state, stream=s)
        if st.is_csa:
            if self.fused_topk:
                abi.index_topk(desc, bi.batch, n, b["qI"], b["w"], st.idx, b["scores"], b["ld"], b["n_valid"],
                               b["sel"], b["ws_it"], stream=s)
            else:
                abi.index_scores(desc, bi.batch, n, b["qI"], b["w"], st.idx, b["scores"], b["ld"], b["n_valid"],
                                 stream=s)
                abi.topk_select(desc.score_fmt, n, b["scores"], b["ld"], b["n_valid"], desc.top_k, b["sel"],
                                b["ws_t"], stream=s)
            abi.sparse_mqa(desc, bi.batch, n, b["q"], P["q_gamma"], b["sel"], st.kv, st.state, P["sinks"], b["out"],
                           b["ws_a"], stream=s)
        else:
            abi.hca_attention(desc, bi.batch, n, b["q"], P["q_gamma"], st.kv, st.state, P["sinks"], b["out"],
                              b["ws_a"], stream=s)

    def index_call(self, li: int):
        """Only the index_scores call of CSA layer li (same buffers as the step)."""
        st, _ = self.layers[li]
        b = self.bufs[li]
        abi.index_scores(st.desc, self.bis[self.parity].batch, self.n_req, b["qI"], b["w"], st.idx, b["scores"],
                         b["ld"], b["n_valid"])

    def step(self, parity: int | None = None):
        """One decode step through every layer at the positions of buffer
        `parity` (default: the workload's current one, which then flips); the
        first layer writes the next positions into the other buffer."""
        p = self.parity if parity is None else parity
        for li in range(len(self.layers)):
            self.layer_calls(li, parity=p)
        if parity is None:
            self.parity ^= 1
