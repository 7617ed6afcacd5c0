"""Batch invariance of a layer flagged CSA_FLAG_BATCH_INVARIANT ([YP] "批无关性 &
计算确定性"; [DD] §6.3): a request's outputs are bit-identical whether its calls
carry it alone or together with other requests.

Request A runs a prefill chunk and then decode steps twice, on separate
caches filled the same way: once alone, once with other requests in every
call (longer and shorter contexts, several new tokens per call, so the
calls take other kernels and split counts).  Every output of A is compared
bit for bit: compressed entries, indexer keys, window rows, index scores,
selected entries and the attention output.  Request 0's outputs are also
checked against the oracle (every call, a sample of the prefill chunk's
queries), so the flagged kernels (fixed attention splits with the ordered
merge, the small-row projection) are held to the same tolerances as the
unflagged ones.
"""
import numpy as np
import pytest
import torch

import synth
from harness import assert_close, decode_fp8_blocks, kv_block_bytes_of, reconcile_fp8_blocks, spec_of, tol_of
from long_context_sparse_03_amd import abi, presets
from long_context_sparse_03_amd.layer import LayerState
from oracle import layer as OL
from test_gpu_layers import Params, QueryOracle, compare_csa_queries, gpu_layer_call

pytestmark = pytest.mark.gpu

INV = abi.FLAG_BATCH_INVARIANT


def _desc(kind):
    if kind == "csa":     # Flash shape: FP8 + bf16 KV, bf16 indexer, 64 heads
        return presets.layer(abi.KIND_CSA, 4, 512, 64, 64, 64, 128, 512, win_cap=4096, kv_fmt=abi.KV_FP8,
                             idx_fmt=abi.IDX_BF16, score_fmt=abi.ACT_BF16, act_fmt=abi.ACT_BF16,
                             out_fmt=abi.ACT_BF16, flags=INV)
    return presets.layer(abi.KIND_HCA, 128, 512, 64, 128, win_cap=4096, kv_fmt=abi.KV_FP8, act_fmt=abi.ACT_BF16,
                         out_fmt=abi.ACT_BF16, flags=INV)


def _rows(d, n_tok, g, desc):
    """Per-token inputs of one request: H, q, qI, w."""
    H = synth.to_bf16_values(synth.normal(g, (n_tok, d)))
    qd = synth.queries(g, n_tok, desc.n_heads, desc.c, max(desc.n_idx_heads, 1), max(desc.c_idx, 1))
    return dict(H=H, q=synth.to_bf16_values(qd["q"]), qI=synth.to_bf16_values(qd["qI"]), w=qd["w"])


def _cat(parts, key, spans):
    return np.concatenate([p[key][a:b] for p, (a, b) in zip(parts, spans)])


def _run(desc, P, reqs, calls, n_blocks):
    """Run `calls` (per call: list of (request, first token, count)) over
    requests `reqs` (token inputs); returns, per call, A's (request 0's)
    outputs."""
    n = len(reqs)
    bt = np.arange(n * n_blocks, dtype=np.int32).reshape(n, n_blocks)
    st = LayerState(desc, n, bt.size)
    outs = []
    for call in calls:
        start = [s for _, s, _ in call]
        cnt = [c for _, _, c in call]
        rows = [reqs[r] for r, _, _ in call]
        spans = [(s, s + c) for _, s, c in call]
        sub_bt = bt[[r for r, _, _ in call]]
        qI = _cat(rows, "qI", spans) if desc.kind == abi.KIND_CSA else None
        w = _cat(rows, "w", spans) if desc.kind == abi.KIND_CSA else None
        got = gpu_layer_call(st, desc, P, start, cnt, sub_bt, _cat(rows, "H", spans), _cat(rows, "q", spans), qI, w)
        # request 0 is the first request of every call
        a_rows = slice(0, cnt[0])
        ent = got["meta"][:got["count"], 0] == 0
        o = {"entries": got["entries"][:got["count"]][ent], "win": got["win"][a_rows], "out": got["out"][a_rows]}
        if desc.kind == abi.KIND_CSA:
            V = (start[0] + np.arange(cnt[0]) + 1) // desc.m
            o["keys"] = got["keys"][:got["count"]][ent]
            o["scores"] = [got["scores"][j, :V[j]] for j in range(cnt[0])]
            o["sel"] = got["sel"][a_rows]
        outs.append(o)
    return outs, st, bt


def oracle_check_request(desc, P, x, calls, outs, max_queries=48, st=None, bt_row=None):
    """Outputs of one request against the oracle.  x: the request's token
    inputs (H, q, qI, w); calls: (first position, count) of each of its calls
    from position 0; outs: per call its outputs (entries and keys the call
    completed, window rows, selections, scores, attention output) or None
    (not checked).  The cache state a call's queries see is the oracle's
    storage of every entry completed up to and including that call, appended
    call by call (the FP8 block-scale rule applies per call).  At most
    max_queries queries of a call are checked (evenly spaced, first and last
    included).  With st and bt_row (the request's cache and block-table row)
    and FP8 entries, the oracle's stored bytes are first reconciled with the
    GPU's at rounding near-ties (harness.reconcile_fp8_blocks), so that a code
    the two sides legitimately round differently does not count as an
    attention error."""
    spec = spec_of(desc)
    m, csa = desc.m, desc.kind == abi.KIND_CSA
    n = calls[-1][0] + calls[-1][1]
    E, K, R = OL.compress_layer(spec, x["H"][:n], P.W, P.Ba, P.Bb, P.gamma, P.W_I, P.BaI, P.BbI)
    tol = tol_of(desc)
    ecalls_all = [(s // m, (s + c) // m - s // m) for s, c in calls if (s + c) // m > s // m]
    n_e = n // m
    rec_deq = None
    if st is not None and spec.kv_fmt == "fp8" and n_e > 0:
        o_blocks, _ = OL.store_entries(spec, E[:n_e].astype(np.float32), ecalls_all)
        g_blocks = kv_block_bytes_of(st, bt_row, o_blocks.shape[0])
        blocks, taken = reconcile_fp8_blocks(spec, o_blocks, g_blocks, E[:n_e].astype(np.float32))
        rec_deq = decode_fp8_blocks(spec, blocks, n_e)
        print(f"  oracle: {taken} stored values rounded the other way at near-ties, taken from the GPU", flush=True)
    ecalls = []
    for ci, ((s, c), o) in enumerate(zip(calls, outs)):
        i0, i1 = s // m, (s + c) // m
        if i1 > i0:
            ecalls.append((i0, i1 - i0))
        if o is None or c == 0:
            continue
        if i1 > i0:
            assert_close(o["entries"], E[i0:i1], 1e-3, f"call {ci} entries")
            if csa:
                assert_close(o["keys"], K[i0:i1], 1e-3, f"call {ci} keys")
        assert_close(o["win"], R[s:s + c], 1e-3, f"call {ci} window rows")
        if rec_deq is not None and i1 % spec.epb == 0:
            edeq = rec_deq[:i1]                   # every block complete: final, reconciled bytes
        else:
            _, edeq = OL.store_entries(spec, E[:i1].astype(np.float32), ecalls)
            if rec_deq is not None:
                full = (i1 // spec.epb) * spec.epb
                edeq[:full] = rec_deq[:full]
        wdeq = OL.round_rows(spec.win_fmt, R[:s + c].astype(np.float32))
        rows = np.arange(c) if c <= max_queries else np.unique(np.linspace(0, c - 1, max_queries).astype(int))
        pos = s + rows
        if csa:
            kdeq = OL.store_keys(spec, K[:i1].astype(np.float32))[1]
            qo = QueryOracle(spec, x["q"][pos], x["qI"][pos], x["w"][pos], pos, kdeq, edeq, wdeq, P.sinks,
                             P.q_gamma)
            V = (pos + 1) // m
            sc = np.full((len(rows), max(1, int(V.max()))), np.nan, np.float32)
            for j, rj in enumerate(rows):
                sc[j, :V[j]] = o["scores"][rj]
            sub = {"scores": sc, "sel": o["sel"][rows], "out": o["out"][rows]}
            e, msame = compare_csa_queries(desc, sub, 0, qo, f"call {ci}")
        else:
            want = OL.attend(spec, x["q"][pos], P.q_gamma, pos, edeq, wdeq, P.sinks)
            e = assert_close(o["out"][rows], want, tol, f"call {ci} attention")
        print(f"  oracle: call {ci} ({len(rows)} of {c} queries) attention err {e:.2e}", flush=True)


def _same(a, b, what):
    if isinstance(a, list):
        for j, (x, y) in enumerate(zip(a, b)):
            _same(x, y, f"{what}[{j}]")
        return
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape, f"{what}: shapes {a.shape} vs {b.shape}"
    assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                          b.view(np.uint32) if b.dtype == np.float32 else b), f"{what} differs"


@pytest.mark.parametrize("kind", ["csa", "hca"])
def test_batch_invariant_request(kind):
    desc = _desc(kind)
    d = presets.D_FLASH
    g = synth.rng(300)
    P = Params(g, desc, d)
    # request 0: 2944-token prefill (23 whole blocks) + 5 decode steps; the others only share
    # its calls (a request keeps its position in every call: its state slot)
    lens = [2949, 18000, 1900, 700]
    reqs = [_rows(d, n, g, desc) for n in lens]
    n_blocks = (max(lens) + 127) // 128 + 1
    alone = [[(0, 0, 2944)]] + [[(0, 2944 + i, 1)] for i in range(5)]
    # with company: a neighbour that grows by 3000 tokens per call (by the
    # last call its HCA rows need more splits than request 0's), and several
    # new tokens per request (other compressor and indexer launches)
    shared = [[(0, 0, 2944), (1, 0, 3000), (2, 0, 1890), (3, 0, 600)]]
    shared += [[(0, 2944 + i, 1), (1, 3000 * (i + 1), 3000), (2, 1890 + 2 * i, 2), (3, 600 + 20 * i, 20)]
               for i in range(5)]
    print(f"batch invariance {kind}", flush=True)
    a, st_a, bt_a = _run(desc, P, reqs, alone, n_blocks)
    b, _, _ = _run(desc, P, reqs, shared, n_blocks)
    for i, (x, y) in enumerate(zip(a, b)):
        for key in x:
            _same(x[key], y[key], f"call {i} {key}")
    print(f"  request 0 bit-identical over {len(a)} calls", flush=True)
    oracle_check_request(desc, P, reqs[0], [(s, c) for [(_, s, c)] in alone], a, st=st_a, bt_row=bt_a[0])
