"""ctypes binding of libcsa.so: the same calls as include/csa.h, taking torch
tensors (device memory) and the current HIP stream.  Argument marshalling
only; every step runs in the library's kernels."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcsa.so")

KIND_CSA, KIND_HCA = 0, 1
KV_F32, KV_BF16, KV_FP8 = 0, 1, 2
IDX_F32, IDX_BF16, IDX_MXFP4 = 0, 1, 2
ACT_F32, ACT_BF16 = 0, 1
OP_COMPRESS, OP_TOPK, OP_ATTENTION, OP_INDEX_TOPK = 0, 1, 2, 3
FLAG_BATCH_INVARIANT = 1
TO_HOST, FROM_HOST = 0, 1


class CSAError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed ({code}): {msg}")
        self.code = code


class LayerDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "kind", "m", "c", "rope_dim", "n_heads", "n_idx_heads", "c_idx", "top_k", "n_win", "win_cap",
        "block_tokens", "kv_fmt", "idx_fmt", "score_fmt", "act_fmt", "out_fmt")] + [
        ("rope_theta", ctypes.c_float), ("norm_eps", ctypes.c_float), ("flags", ctypes.c_int32)]

    @property
    def epb(self) -> int:
        return self.block_tokens // self.m


class Batch(ctypes.Structure):
    _fields_ = [("n_req", ctypes.c_int32), ("max_new", ctypes.c_int32), ("max_ctx", ctypes.c_int32),
                ("max_blocks", ctypes.c_int32), ("cu_new", ctypes.c_void_p), ("start_pos", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("next_start_pos", ctypes.c_void_p)]


class Sizes(ctypes.Structure):
    _fields_ = [("kv_block_bytes", ctypes.c_size_t), ("idx_block_bytes", ctypes.c_size_t),
                ("state_bytes", ctypes.c_size_t), ("entries_per_block", ctypes.c_int32),
                ("proj_cols", ctypes.c_int32)]


_lib = None


def lib():
    """Load libcsa.so; raise ImportError if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m long_context_sparse_03_amd.build` "
                              "(or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        LP, BP = ctypes.POINTER(LayerDesc), ctypes.POINTER(Batch)
        sig = {
            "csa_abi_version": (I, []),
            "csa_last_error": (ctypes.c_char_p, []),
            "csa_layer_sizes": (I, [LP, ctypes.POINTER(Sizes)]),
            "csa_workspace_size": (I, [LP, I, I, I, I, ctypes.POINTER(ctypes.c_size_t)]),
            "csa_compress_kv": (I, [P, LP, BP, I, I, P, P, P, P, P, P, P, P, P, P, P, P, P, I, P, P, Z]),
            "csa_cache_append": (I, [P, LP, BP, I, P, P, P, P, I, P, P, P, P]),
            "csa_compress_append": (I, [P, LP, BP, I, I, P, P, P, P, P, P, P, P, P, P, P, P, P, I, P, P, P, P, Z]),
            "csa_index_scores": (I, [P, LP, BP, I, P, P, P, P, I, P]),
            "csa_index_topk": (I, [P, LP, BP, I, P, P, P, P, I, P, P, P, Z]),
            "csa_topk_select": (I, [P, I, I, P, I, P, I, P, P, Z]),
            "csa_topk_select_static": (I, [P, I, I, P, I, P, I, P]),
            "csa_sparse_mqa": (I, [P, LP, BP, I, P, P, P, P, P, P, P, P, Z]),
            "csa_hca_attention": (I, [P, LP, BP, I, P, P, P, P, P, P, P, Z]),
            "csa_linear": (I, [P, I, I, I, I, I, P, P, P]),
            "csa_grouped_linear": (I, [P, I, I, I, I, I, I, P, P, P]),
            "csa_prefix_bytes": (I, [LP, I, ctypes.POINTER(ctypes.c_size_t)]),
            "csa_prefix_blocks": (I, [P, LP, I, P, P, P, P, I]),
            "csa_prefix_state": (I, [P, LP, P, P, I]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        raise CSAError(fn, rc, lib().csa_last_error().decode())


def _ptr(t) -> int | None:
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream=None) -> int | None:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def abi_version() -> int:
    return lib().csa_abi_version()


def layer_sizes(desc: LayerDesc) -> Sizes:
    out = Sizes()
    _check("csa_layer_sizes", lib().csa_layer_sizes(ctypes.byref(desc), ctypes.byref(out)))
    return out


def workspace_size(desc: LayerDesc, op: int, n_rows: int, max_cols: int = 0, top_k: int = 1) -> int:
    out = ctypes.c_size_t(0)
    _check("csa_workspace_size", lib().csa_workspace_size(ctypes.byref(desc), op, n_rows, max_cols, top_k,
                                                          ctypes.byref(out)))
    return out.value


def compress_kv(desc, batch, n_tokens, d, H, W, W_idx, B_a, B_b, B_a_idx, B_b_idx, gamma, state,
                out_entries, out_keys, out_meta, out_count, max_entries, out_win, ws, stream=None):
    _check("csa_compress_kv", lib().csa_compress_kv(
        _stream(stream), ctypes.byref(desc), ctypes.byref(batch), n_tokens, d, _ptr(H), _ptr(W), _ptr(W_idx),
        _ptr(B_a), _ptr(B_b), _ptr(B_a_idx), _ptr(B_b_idx), _ptr(gamma), _ptr(state), _ptr(out_entries),
        _ptr(out_keys), _ptr(out_meta), _ptr(out_count), max_entries, _ptr(out_win), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size()))


def cache_append(desc, batch, n_tokens, entries, keys, meta, count, max_entries, win, kv_cache, idx_cache, state,
                 stream=None):
    _check("csa_cache_append", lib().csa_cache_append(
        _stream(stream), ctypes.byref(desc), ctypes.byref(batch), n_tokens, _ptr(entries), _ptr(keys), _ptr(meta),
        _ptr(count), max_entries, _ptr(win), _ptr(kv_cache), _ptr(idx_cache), _ptr(state)))


def compress_append(desc, batch, n_tokens, d, H, W, W_idx, B_a, B_b, B_a_idx, B_b_idx, gamma, state,
                    out_entries, out_keys, out_meta, out_count, max_entries, out_win, kv_cache, idx_cache, ws,
                    stream=None):
    """compress_kv and then cache_append of its outputs, in one call."""
    _check("csa_compress_append", lib().csa_compress_append(
        _stream(stream), ctypes.byref(desc), ctypes.byref(batch), n_tokens, d, _ptr(H), _ptr(W), _ptr(W_idx),
        _ptr(B_a), _ptr(B_b), _ptr(B_a_idx), _ptr(B_b_idx), _ptr(gamma), _ptr(state), _ptr(out_entries),
        _ptr(out_keys), _ptr(out_meta), _ptr(out_count), max_entries, _ptr(out_win), _ptr(kv_cache),
        _ptr(idx_cache), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size()))


def index_scores(desc, batch, n_tokens, q_idx, w, idx_cache, scores, ld, n_valid, stream=None):
    _check("csa_index_scores", lib().csa_index_scores(
        _stream(stream), ctypes.byref(desc), ctypes.byref(batch), n_tokens, _ptr(q_idx), _ptr(w), _ptr(idx_cache),
        _ptr(scores), ld, _ptr(n_valid)))


def index_topk(desc, batch, n_tokens, q_idx, w, idx_cache, scores, ld, n_valid, out_idx, ws, stream=None):
    """index_scores and topk_select (k = desc.top_k) in one call."""
    _check("csa_index_topk", lib().csa_index_topk(
        _stream(stream), ctypes.byref(desc), ctypes.byref(batch), n_tokens, _ptr(q_idx), _ptr(w), _ptr(idx_cache),
        _ptr(scores), ld, _ptr(n_valid), _ptr(out_idx), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size()))


def topk_select(score_fmt, n_rows, scores, ld, n_valid, k, out_idx, ws, stream=None):
    _check("csa_topk_select", lib().csa_topk_select(
        _stream(stream), score_fmt, n_rows, _ptr(scores), ld, _ptr(n_valid), k, _ptr(out_idx), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size()))


def topk_select_static(score_fmt, n_rows, scores, ld, n_valid, k, out_idx, stream=None):
    """topk_select with the library's static scratch array instead of a workspace."""
    _check("csa_topk_select_static", lib().csa_topk_select_static(
        _stream(stream), score_fmt, n_rows, _ptr(scores), ld, _ptr(n_valid), k, _ptr(out_idx)))


def sparse_mqa(desc, batch, n_tokens, q, q_gamma, sel, kv_cache, state, sinks, out, ws, stream=None):
    _check("csa_sparse_mqa", lib().csa_sparse_mqa(
        _stream(stream), ctypes.byref(desc), ctypes.byref(batch), n_tokens, _ptr(q), _ptr(q_gamma), _ptr(sel),
        _ptr(kv_cache), _ptr(state), _ptr(sinks), _ptr(out), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size()))


def hca_attention(desc, batch, n_tokens, q, q_gamma, kv_cache, state, sinks, out, ws, stream=None):
    _check("csa_hca_attention", lib().csa_hca_attention(
        _stream(stream), ctypes.byref(desc), ctypes.byref(batch), n_tokens, _ptr(q), _ptr(q_gamma),
        _ptr(kv_cache), _ptr(state), _ptr(sinks), _ptr(out), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size()))


def prefix_bytes(desc, n_blocks: int) -> int:
    out = ctypes.c_size_t(0)
    _check("csa_prefix_bytes", lib().csa_prefix_bytes(ctypes.byref(desc), n_blocks, ctypes.byref(out)))
    return out.value


def prefix_blocks(desc, n_blocks, block_ids, kv_cache, idx_cache, host, direction, stream=None):
    """Blocks block_ids (device int32) of the caches to (TO_HOST) or from
    (FROM_HOST) the pinned host tensor `host`."""
    _check("csa_prefix_blocks", lib().csa_prefix_blocks(
        _stream(stream), ctypes.byref(desc), n_blocks, _ptr(block_ids), _ptr(kv_cache), _ptr(idx_cache), _ptr(host),
        direction))


def prefix_state(desc, state_slot_ptr: int, host, direction, stream=None):
    """One state slot (device address) to or from the pinned host tensor `host`."""
    _check("csa_prefix_state", lib().csa_prefix_state(
        _stream(stream), ctypes.byref(desc), state_slot_ptr, _ptr(host), direction))


def grouped_linear(act_fmt, out_fmt, groups, X, W, Y, stream=None):
    """Y[:, g*N:(g+1)*N] = X[:, g*K:(g+1)*K] . W[g]^T for every group g
    (X [rows x groups*K], W [groups x N x K], Y [rows x groups*N])."""
    K = X.shape[-1] // groups
    N = W.shape[-2]
    _check("csa_grouped_linear", lib().csa_grouped_linear(
        _stream(stream), act_fmt, out_fmt, X.shape[0], groups, K, N, _ptr(X), _ptr(W), _ptr(Y)))


def linear(act_fmt, out_fmt, X, W, Y, stream=None):
    """Y = X . W^T (X [rows x K], W [N x K], Y [rows x N])."""
    _check("csa_linear", lib().csa_linear(
        _stream(stream), act_fmt, out_fmt, X.shape[0], X.shape[1], W.shape[0], _ptr(X), _ptr(W), _ptr(Y)))

