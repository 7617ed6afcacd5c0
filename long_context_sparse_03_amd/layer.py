"""Device buffers of one attention layer and the order of its calls.

``LayerState`` owns a layer's paged KV pool, its indexer-key pool (CSA), the
per-request state slots (window ring + compressor tail) and the workspaces,
all as torch device tensors; its methods call the library in the order the
method runs: compress_kv -> cache_append -> index_scores -> topk_select ->
sparse_mqa (CSA), or compress_kv -> cache_append -> hca_attention (HCA).
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass, field

import torch

from . import abi
from .abi import Batch, LayerDesc


@dataclass
class BatchInfo:
    batch: Batch
    n_tokens: int
    cu_new: torch.Tensor
    start_pos: torch.Tensor
    block_table: torch.Tensor
    next_start_pos: torch.Tensor | None = None
    keep: list = field(default_factory=list)


def make_batch(cu_new: torch.Tensor, start_pos: torch.Tensor, block_table: torch.Tensor, max_new: int,
               max_ctx: int, n_tokens: int, next_start_pos: torch.Tensor | None = None) -> BatchInfo:
    """Wrap int32 device tensors (cu_new [n_req+1], start_pos [n_req],
    block_table [n_req, max_blocks], optionally next_start_pos [n_req]) and
    host bounds into a csa_batch."""
    assert cu_new.dtype == torch.int32 and start_pos.dtype == torch.int32 and block_table.dtype == torch.int32
    cu_new, start_pos, block_table = cu_new.contiguous(), start_pos.contiguous(), block_table.contiguous()
    if next_start_pos is not None:
        assert next_start_pos.dtype == torch.int32 and next_start_pos.is_contiguous()
    b = Batch(n_req=start_pos.numel(), max_new=int(max_new), max_ctx=int(max_ctx),
              max_blocks=block_table.shape[1], cu_new=cu_new.data_ptr(), start_pos=start_pos.data_ptr(),
              block_table=block_table.data_ptr(),
              next_start_pos=None if next_start_pos is None else next_start_pos.data_ptr())
    return BatchInfo(b, int(n_tokens), cu_new, start_pos, block_table, next_start_pos)


class LayerState:
    def __init__(self, desc: LayerDesc, n_slots: int, pool_blocks: int, device="cuda"):
        self.desc = desc
        self.sizes = abi.layer_sizes(desc)
        self.device = device
        self.kv = torch.zeros(pool_blocks * self.sizes.kv_block_bytes, dtype=torch.uint8, device=device)
        self.idx = (torch.zeros(pool_blocks * self.sizes.idx_block_bytes, dtype=torch.uint8, device=device)
                    if self.sizes.idx_block_bytes else None)
        self.state = torch.zeros(n_slots * self.sizes.state_bytes, dtype=torch.uint8, device=device)
        self._ws = {}

    @property
    def is_csa(self) -> bool:
        return self.desc.kind == abi.KIND_CSA

    def workspace(self, key: str, nbytes: int) -> torch.Tensor | None:
        if nbytes == 0:
            return None
        t = self._ws.get(key)
        if t is None or t.numel() < nbytes:
            t = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
            self._ws[key] = t
        return t[:nbytes]

    # -- a1 ---------------------------------------------------------------
    def compress(self, bi: BatchInfo, n_tokens: int, H, W, W_idx, B_a, B_b, B_a_idx, B_b_idx, gamma,
                 max_entries: int, stream=None):
        d = self.desc
        c = d.c
        out_e = torch.empty((max(max_entries, 1), c), dtype=torch.float32, device=self.device)
        out_k = (torch.empty((max(max_entries, 1), d.c_idx), dtype=torch.float32, device=self.device)
                 if self.is_csa else None)
        meta = torch.empty((max(max_entries, 1), 2), dtype=torch.int32, device=self.device)
        count = torch.zeros(1, dtype=torch.int32, device=self.device)
        win = torch.empty((max(n_tokens, 1), c), dtype=torch.float32, device=self.device)
        ws = self.workspace("compress", abi.workspace_size(d, abi.OP_COMPRESS, n_tokens))
        abi.compress_kv(d, bi.batch, n_tokens, H.shape[1] if H is not None else W.shape[1], H, W, W_idx, B_a, B_b,
                        B_a_idx, B_b_idx, gamma, self.state, out_e, out_k, meta, count, max_entries, win, ws,
                        stream=stream)
        return out_e, out_k, meta, count, win

    def compress_append(self, bi: BatchInfo, n_tokens: int, H, W, W_idx, B_a, B_b, B_a_idx, B_b_idx, gamma,
                        max_entries: int, stream=None):
        """compress() and then append() of its outputs, in one library call."""
        d = self.desc
        c = d.c
        out_e = torch.empty((max(max_entries, 1), c), dtype=torch.float32, device=self.device)
        out_k = (torch.empty((max(max_entries, 1), d.c_idx), dtype=torch.float32, device=self.device)
                 if self.is_csa else None)
        meta = torch.empty((max(max_entries, 1), 2), dtype=torch.int32, device=self.device)
        count = torch.zeros(1, dtype=torch.int32, device=self.device)
        win = torch.empty((max(n_tokens, 1), c), dtype=torch.float32, device=self.device)
        ws = self.workspace("compress", abi.workspace_size(d, abi.OP_COMPRESS, n_tokens))
        abi.compress_append(d, bi.batch, n_tokens, H.shape[1] if H is not None else W.shape[1], H, W, W_idx, B_a,
                            B_b, B_a_idx, B_b_idx, gamma, self.state, out_e, out_k, meta, count, max_entries, win,
                            self.kv, self.idx, ws, stream=stream)
        return out_e, out_k, meta, count, win

    # -- a2 ---------------------------------------------------------------
    def append(self, bi: BatchInfo, n_tokens: int, entries, keys, meta, count, max_entries: int, win, stream=None):
        abi.cache_append(self.desc, bi.batch, n_tokens, entries, keys, meta, count, max_entries, win, self.kv,
                         self.idx, self.state, stream=stream)

    # -- a3 / a4 ------------------------------------------------------------
    def index(self, bi: BatchInfo, n_tokens: int, q_idx, w, scores, ld, n_valid, stream=None):
        abi.index_scores(self.desc, bi.batch, n_tokens, q_idx, w, self.idx, scores, ld, n_valid, stream=stream)

    def index_topk(self, bi: BatchInfo, n_tokens: int, q_idx, w, scores, ld, n_valid, out_idx, stream=None):
        ws = self.workspace("index_topk", abi.workspace_size(self.desc, abi.OP_INDEX_TOPK, n_tokens, ld))
        abi.index_topk(self.desc, bi.batch, n_tokens, q_idx, w, self.idx, scores, ld, n_valid, out_idx, ws,
                       stream=stream)

    def topk(self, n_rows: int, scores, ld: int, n_valid, out_idx, stream=None):
        d = self.desc
        ws = self.workspace("topk", abi.workspace_size(d, abi.OP_TOPK, n_rows, ld, d.top_k))
        abi.topk_select(d.score_fmt, n_rows, scores, ld, n_valid, d.top_k, out_idx, ws, stream=stream)

    # -- a5 / a6 ------------------------------------------------------------
    def attend(self, bi: BatchInfo, n_tokens: int, q, q_gamma, sinks, out, sel=None, stream=None):
        d = self.desc
        rows = (d.top_k if sel is not None else bi.batch.max_ctx // d.m) + d.n_win
        ws = self.workspace("attn", abi.workspace_size(d, abi.OP_ATTENTION, n_tokens, rows))
        if sel is not None:
            abi.sparse_mqa(d, bi.batch, n_tokens, q, q_gamma, sel, self.kv, self.state, sinks, out, ws, stream=stream)
        else:
            abi.hca_attention(d, bi.batch, n_tokens, q, q_gamma, self.kv, self.state, sinks, out, ws, stream=stream)

    # ---- prefix reuse (host-memory tier)
    def save_prefix(self, block_ids: torch.Tensor, slot: int, stream=None):
        """Blocks block_ids (device int32) and state slot `slot` into new
        pinned host tensors (blocks, state)."""
        n = int(block_ids.numel())
        blocks = torch.empty(abi.prefix_bytes(self.desc, n), dtype=torch.uint8, pin_memory=True)
        state = torch.empty(self.sizes.state_bytes, dtype=torch.uint8, pin_memory=True)
        abi.prefix_blocks(self.desc, n, block_ids, self.kv, self.idx, blocks, abi.TO_HOST, stream=stream)
        abi.prefix_state(self.desc, self.state.data_ptr() + slot * self.sizes.state_bytes, state, abi.TO_HOST,
                         stream=stream)
        return blocks, state

    def load_prefix(self, block_ids: torch.Tensor, slot: int, blocks: torch.Tensor, state: torch.Tensor,
                    stream=None):
        """The reverse of save_prefix, into blocks block_ids and slot `slot`."""
        abi.prefix_blocks(self.desc, int(block_ids.numel()), block_ids, self.kv, self.idx, blocks, abi.FROM_HOST,
                          stream=stream)
        abi.prefix_state(self.desc, self.state.data_ptr() + slot * self.sizes.state_bytes, state, abi.FROM_HOST,
                         stream=stream)
