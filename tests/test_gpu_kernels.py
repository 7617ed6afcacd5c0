"""Per-kernel parity of the HIP path against the CPU oracle (needs an MI355X).

Every test feeds both sides the same seeded inputs and isolates one call:
cache_append is compared byte for byte, top-k index sets bit-exactly (on the
oracle's own scores), index scores to one bf16 step (or the fp32 tolerance),
compressor and attention outputs with the acceptance metric
|g - r| <= rtol * (|r| + RMS(r)) at the tolerance of the path.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from harness import (append_entries, append_window, assert_close, batch, f32_of, i32, idx_block_bytes_of,
                     kv_block_bytes_of, rel_err, ring_rows, spec_of, to_dev, tol_of)
from long_context_sparse_03_amd import abi, presets
from long_context_sparse_03_amd.layer import LayerState
from oracle import layer as OL

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(msg, flush=True)


# ---------------------------------------------------------------------------
# a2: cache_append, byte-exact
# ---------------------------------------------------------------------------

APPEND_CASES = {
    "f32": presets.tiny_csa_fp32(),
    "bf16_hca": presets.hca_bf16(),
    "fp8_bf16idx": presets.csa_flash_decode(),
    "fp8_mxfp4idx": presets.csa_pro(idx_fmt=abi.IDX_MXFP4),
    "fp8_hca": presets.hca_pro(),
}


@pytest.mark.parametrize("name", list(APPEND_CASES))
def test_cache_append_bytes(name):
    desc = APPEND_CASES[name]
    spec = spec_of(desc)
    _flush(f"cache_append {name}")
    g = synth.rng(100)
    n_req, epb = 3, desc.block_tokens // desc.m
    # ragged call schedule crossing block boundaries; later calls larger in
    # magnitude so the fp8 block scale is raised and earlier slots re-encoded
    sched = [[5, 0, 33], [20, 7, 31], [40, 2, 64]]
    if epb == 1:
        sched = [[1, 0, 2], [3, 1, 1], [2, 4, 1]]
    tot = np.sum(sched, axis=0)
    nb = [(t + epb - 1) // epb for t in tot]
    bt = synth.block_table(g, n_req, max(nb), extra=5)
    st = LayerState(desc, n_req, bt.size + 5)
    ents = [synth.normal(g, (int(tot[r]), desc.c)) for r in range(n_req)]
    keys = [synth.normal(g, (int(tot[r]), desc.c_idx)) for r in range(n_req)] if desc.c_idx else None
    for r in range(n_req):
        ents[r][sched[0][r]:] *= 3.0
        ents[r][sched[0][r] + sched[1][r]:] *= 2.0
    done = [0] * n_req
    for call in sched:
        pe = [ents[r][done[r]:done[r] + call[r]] for r in range(n_req)]
        pk = [keys[r][done[r]:done[r] + call[r]] for r in range(n_req)] if keys else None
        append_entries(st, desc, bt, pe, list(done), pk)
        done = [done[r] + call[r] for r in range(n_req)]
    torch.cuda.synchronize()
    for r in range(n_req):
        calls, f = [], 0
        for call in sched:
            calls.append((f, call[r]))
            f += call[r]
        blocks, _ = OL.store_entries(spec, ents[r], calls)
        got = kv_block_bytes_of(st, bt[r], nb[r])
        rec = OL.kv_record_bytes(spec)
        hdr = 64 if spec.kv_fmt == "fp8" else 0
        for b in range(nb[r]):
            used = min(epb, int(tot[r]) - b * epb)
            lim = hdr + used * rec
            assert np.array_equal(got[b, :lim], blocks[b, :lim]), f"{name}: request {r} block {b} differs"
        if keys:
            kb, _ = OL.store_keys(spec, keys[r])
            gk = idx_block_bytes_of(st, bt[r], nb[r])
            if spec.idx_fmt == "mxfp4":
                half = epb * desc.c_idx // 2
                for b in range(nb[r]):
                    used = min(epb, int(tot[r]) - b * epb)
                    assert np.array_equal(gk[b, :used * desc.c_idx // 2], kb[b, :used * desc.c_idx // 2])
                    assert np.array_equal(gk[b, half:half + used * desc.c_idx // 32],
                                          kb[b, half:half + used * desc.c_idx // 32])
            else:
                kr = OL.idx_block_bytes(spec) // epb
                for b in range(nb[r]):
                    used = min(epb, int(tot[r]) - b * epb)
                    assert np.array_equal(gk[b, :used * kr], kb[b, :used * kr])


def test_window_ring_rows():
    desc = presets.csa_flash_decode(win_cap=200)
    _flush("window ring")
    g = synth.rng(101)
    bt = synth.block_table(g, 2, 10)
    st = LayerState(desc, 2, bt.size)
    sp = [0, 1000]
    rows = [synth.normal(g, (150, 512)), synth.normal(g, (73, 512))]
    append_window(st, desc, bt, sp, rows)
    torch.cuda.synchronize()
    for r in range(2):
        got = ring_rows(st, desc, r, np.arange(sp[r], sp[r] + rows[r].shape[0]))
        want = OL.round_rows("bf16", rows[r])
        assert np.array_equal(got, want.astype(np.float32))


# ---------------------------------------------------------------------------
# a4: top-k, bit-exact on given scores
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fmt,V,k,levels", [("bf16", [32768, 32768, 32000, 40957], 512, 64),
                                            ("bf16", [32768, 32768, 32000, 40957], 512, 6),
                                            ("bf16", [32768, 20000, 4000], 1024, 300)])
def test_topk_quantised_scores(fmt, V, k, levels):
    """Scores on a few levels: long tie runs at the threshold (the lower-bound
    pass keeps few or very many keys)."""
    _flush(f"topk quantised {fmt} k={k} V={V} levels={levels}")
    g = synth.rng(103)
    ld = max(V)
    sc = O.bf16_round(g.integers(0, levels, size=(len(V), ld)).astype(np.float32) / 4)
    nv = np.array(V, np.int32)
    want = O.topk(sc, nv, k)
    scores = to_dev(sc, torch.bfloat16)
    out = torch.full((len(V), k), -7, dtype=torch.int32, device="cuda")
    desc = presets.csa_flash_decode()
    ws = torch.empty(max(abi.workspace_size(desc, abi.OP_TOPK, len(V), ld, k), 1), dtype=torch.uint8, device="cuda")
    abi.topk_select(abi.ACT_BF16, len(V), scores, ld, i32(nv), k, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for t in range(len(V)):
        assert np.array_equal(got[t], want[t]), f"row {t} (V={V[t]}) differs"


@pytest.mark.parametrize("fmt,V,k", [("bf16", [0, 5, 512, 513, 4096, 32768, 100000, 1000], 512),
                                     ("f32", [64, 63, 1, 0, 700, 70000], 64),
                                     ("bf16", [262144, 33000, 1024, 1025], 1024),
                                     ("bf16", [3, 2000], 2048),
                                     ("bf16", [32768, 32768, 32768, 20000], 512),
                                     ("bf16", [40957, 40000, 32784, 7], 512),
                                     ("f32", [20000, 15000, 9000, 20000], 256),
                                     ("f32", [40000 - 37 * i for i in range(128)], 256)])
def test_topk_exact(fmt, V, k):
    _flush(f"topk {fmt} k={k} V={V}")
    g = synth.rng(102)
    ld = max(V) + 3
    T = len(V)
    sc = synth.normal(g, (T, ld))
    if fmt == "bf16":
        sc = O.bf16_round(sc)
        sc[0, ::7] = sc[0, 0]                        # ties
    else:
        sc = np.round(sc * 50).astype(np.float32) / 50   # many ties
    if T > 2:
        sc[2, :] = 1.0                               # tie storm
    nv = np.array(V, np.int32)
    want = O.topk(sc, nv, k)
    dt = torch.bfloat16 if fmt == "bf16" else torch.float32
    scores = to_dev(sc, dt)
    out = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    desc = presets.csa_flash_decode() if fmt == "bf16" else presets.tiny_csa_fp32()
    nbytes = abi.workspace_size(desc, abi.OP_TOPK, T, ld, k)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    abi.topk_select(abi.ACT_BF16 if fmt == "bf16" else abi.ACT_F32, T, scores, ld, i32(nv), k, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for t in range(T):
        assert np.array_equal(got[t], want[t]), f"row {t} (V={V[t]}) differs"


def test_topk_exact_rows_past_2_18():
    """The 1M decode shape: rows of up to 262,208 bf16 scores (ld 262,208,
    k 1024), which the standalone selector splits into 17 chunks merged by
    its 24-keys-per-thread instance; selections equal the oracle's."""
    V = [262208, 262145, 200000, 262207]
    ld, k = 262208, 1024
    _flush(f"topk bf16 k={k} ld={ld} V={V}")
    g = synth.rng(103)
    sc = O.bf16_round(synth.normal(g, (len(V), ld)))
    sc[1, ::5] = sc[1, 3]                            # ties
    nv = np.array(V, np.int32)
    want = O.topk(sc, nv, k)
    desc = presets.csa_pro()
    nbytes = abi.workspace_size(desc, abi.OP_TOPK, len(V), ld, k)
    assert nbytes == len(V) * 17 * k * 8
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.full((len(V), k), -7, dtype=torch.int32, device="cuda")
    abi.topk_select(abi.ACT_BF16, len(V), to_dev(sc, torch.bfloat16), ld, i32(nv), k, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for t in range(len(V)):
        assert np.array_equal(got[t], want[t]), f"row {t} (V={V[t]}) differs"


def test_topk_f32_keys_at_the_top_of_the_key_range():
    """fp32 scores whose order-preserving keys crowd the top of the 32-bit
    range (+NaN bit patterns with payloads up to 0x7FFFFFFF, keys up to
    0xFFFFFFFF), so the threshold's range narrowing works at the very top,
    where a bin's upper end would pass 2^32 without the clamp.  The oracle
    compares floats and does not order NaNs, so the expected sets come from
    the selector's documented total order: the sign-magnitude key of the bit
    pattern descending (-0 and +0 alike, keys 0 and 1 alike), then the lower
    position."""
    _flush("topk f32 keys near 0xFFFFFFFF")
    g = synth.rng(107)
    ld, k = 4096, 1500
    bits = np.empty((4, ld), np.uint32)
    bits[0] = synth.normal(g, (ld,)).astype(np.float32).view(np.uint32)
    bits[0, :3000] = 0x7FFFF000 + g.integers(0, 4096, size=3000).astype(np.uint32)
    bits[1] = 0x7FFFFF00 + g.integers(0, 256, size=ld).astype(np.uint32)   # 256 keys, long tie runs
    bits[1, ::97] = 0x7FFFFFFF                                              # the largest key
    bits[2] = synth.normal(g, (ld,)).astype(np.float32).view(np.uint32)
    bits[2, ::3] = 0xFFFFFFFF                                               # the smallest key
    bits[2, 1::3] = 0x7FFFFFFF
    bits[3] = 0x7FFFFFF0 + g.integers(0, 16, size=ld).astype(np.uint32)
    nv = np.array([ld, ld, ld - 5, 1000], np.int32)
    key = np.where(bits >> 31 == 1, ~bits, bits | np.uint32(0x80000000)).astype(np.uint64)
    key[(bits & 0x7FFFFFFF) == 0] = 0x80000000
    key = np.maximum(key, 1)      # keys 0 and 1 (two negative NaNs) share a rank, as the selector documents
    want = np.full((4, k), -1, np.int32)
    for t in range(4):
        V = int(nv[t])
        order = sorted(range(V), key=lambda s: (-int(key[t, s]), s))[:min(k, V)]
        want[t, :len(order)] = np.sort(order)
    scores = torch.from_numpy(bits.view(np.float32).copy()).cuda()
    out = torch.full((4, k), -7, dtype=torch.int32, device="cuda")
    desc = presets.tiny_csa_fp32()
    ws = torch.empty(max(abi.workspace_size(desc, abi.OP_TOPK, 4, ld, k), 1), dtype=torch.uint8, device="cuda")
    abi.topk_select(abi.ACT_F32, 4, scores, ld, i32(nv), k, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for t in range(4):
        assert np.array_equal(got[t], want[t]), f"row {t} (V={nv[t]}) differs"


# ---------------------------------------------------------------------------
# a3: index scores
# ---------------------------------------------------------------------------

INDEX_CASES = {
    "f32": presets.tiny_csa_fp32(),
    "bf16": presets.csa_flash_decode(),
    "mxfp4": presets.csa_pro(idx_fmt=abi.IDX_MXFP4),
    "bf16_prefill": presets.csa_flash_decode(win_cap=256),
    # prefill launch with fp32 scores, and with 40 heads (a partial third head tile)
    "bf16_prefill_f32scores": presets.layer(abi.KIND_CSA, 4, 512, 64, 64, 64, 128, 512, win_cap=256,
                                            kv_fmt=abi.KV_FP8, idx_fmt=abi.IDX_BF16, score_fmt=abi.ACT_F32,
                                            act_fmt=abi.ACT_BF16, out_fmt=abi.ACT_BF16),
    "bf16_prefill_40h": presets.layer(abi.KIND_CSA, 4, 512, 64, 64, 40, 128, 512, win_cap=256,
                                      kv_fmt=abi.KV_FP8, idx_fmt=abi.IDX_BF16, score_fmt=abi.ACT_BF16,
                                      act_fmt=abi.ACT_BF16, out_fmt=abi.ACT_BF16),
}


def check_score_row(desc, a, b, qdq, kdeq, w, what):
    """GPU scores a against the oracle's b for one query: fp32 scores to
    1e-4; bf16 scores within one bf16 step of b plus the worst-case error of
    fp32 sums over the channels and the heads, (c_I + n_hI) 2^-24
    sum_h |w_h| sum_c |q_hc k_c| on the dequantised operands (scores of heads
    with weights of both signs can cancel far below the size of their
    terms), and at least 97 % of them identical."""
    if desc.score_fmt != abi.ACT_BF16:
        assert_close(a, b, 1e-4, f"scores {what}")
        return
    V = len(b)
    qa = np.abs(np.asarray(qdq, np.float64)).reshape(desc.n_idx_heads, -1)
    ka = np.abs(np.asarray(kdeq[:V], np.float64))
    acc = (desc.c_idx + desc.n_idx_heads) * 2.0 ** -24 * (np.abs(np.asarray(w, np.float64)) @ (qa @ ka.T))
    ulp = np.maximum(np.abs(b), 1e-30) * 2.0 ** -7
    bad = np.abs(a - b) > ulp + acc + 1e-30
    assert not bad.any(), f"{what}: {bad.sum()} scores off by more than one bf16 step"
    assert V == 0 or np.mean(a == b) > 0.97


def _fill_keys(st, desc, bt, E_per_req, g):
    keys = [synth.normal(g, (E, desc.c_idx)) for E in E_per_req]
    ents = [synth.normal(g, (E, desc.c)) for E in E_per_req]
    append_entries(st, desc, bt, ents, [0] * len(E_per_req), keys)
    return ents, keys


@pytest.mark.parametrize("name", list(INDEX_CASES))
def test_index_scores(name):
    desc = INDEX_CASES[name]
    spec = spec_of(desc)
    _flush(f"index_scores {name}")
    g = synth.rng(103)
    E = [1000, 257, 4096]
    epb = desc.block_tokens // desc.m
    nb = [(e + epb - 1) // epb for e in E]
    bt = synth.block_table(g, 3, max(nb))
    st = LayerState(desc, 3, bt.size)
    ents, keys = _fill_keys(st, desc, bt, E, g)
    # queries: request 0 two tokens, request 1 one token early (V small), request 2 three;
    # the prefill shape runs ragged multi-token chunks (query groups of eight, partial last groups)
    start = [4 * 1000 - 2, 7, 4 * 4096 - 5]
    n_new = [2, 1, 3]
    if "prefill" in name:
        start = [4 * 1000 - 40, 0, 4 * 4096 - 21]
        n_new = [40, 30, 19]
    pos = [np.arange(s, s + n) for s, n in zip(start, n_new)]
    bi = batch(start, n_new, bt)
    T = sum(n_new)
    qd = synth.queries(g, T, 1, 1, desc.n_idx_heads, desc.c_idx)
    qI, w = qd["qI"], qd["w"]
    if desc.act_fmt == abi.ACT_BF16:
        qI = synth.to_bf16_values(qI)
    ld = 4 * 4096 // desc.m + 8
    sdt = torch.bfloat16 if desc.score_fmt == abi.ACT_BF16 else torch.float32
    scores = torch.full((T, ld), float("nan"), dtype=sdt, device="cuda")
    nvalid = torch.zeros(T, dtype=torch.int32, device="cuda")
    st.index(bi, T, to_dev(qI, torch.bfloat16 if desc.act_fmt == abi.ACT_BF16 else torch.float32), to_dev(w),
             scores, ld, nvalid)
    torch.cuda.synchronize()
    got = scores.float().cpu().numpy()
    gv = nvalid.cpu().numpy()
    row = 0
    for r in range(3):
        _, kdeq = OL.store_keys(spec, keys[r])
        qdq = OL.quantize_index_queries(spec, qI[row:row + n_new[r]])
        want = OL.scores(spec, qdq, w[row:row + n_new[r]], pos[r], kdeq)
        for j in range(n_new[r]):
            V = (pos[r][j] + 1) // desc.m
            assert gv[row + j] == V
            check_score_row(desc, got[row + j, :V], want[j, :V], qdq[j], kdeq[:V], w[row + j], f"row {row + j}")
            assert np.all(np.isnan(got[row + j, V:V + 8]))
        row += n_new[r]


def test_index_scores_many_requests():
    """More than 1024 requests with uneven new-token counts (0 to 3 per
    request): the decode launches look each query's request up in global
    memory (the LDS copy of cu_new holds at most 1024 requests); every score
    of a sample of requests against the oracle, bf16 and MXFP4 keys."""
    for desc in (presets.csa_flash_decode(), presets.csa_pro(idx_fmt=abi.IDX_MXFP4)):
        spec = spec_of(desc)
        _flush(f"index_scores 1100 requests idx_fmt={desc.idx_fmt}")
        g = synth.rng(108)
        n_req = 1100
        n_new = g.integers(0, 4, n_req)
        n_new[1050] = 3
        E = g.integers(1, 64, n_req)                 # entries cached per request (at most 2 blocks)
        start = [4 * int(e) + int(g.integers(0, 4)) for e in E]
        epb = desc.block_tokens // desc.m
        bt = synth.block_table(g, n_req, 3)
        st = LayerState(desc, n_req, bt.size)
        E_all = [(s + n) // desc.m for s, n in zip(start, n_new)]
        ents, keys = _fill_keys(st, desc, bt, E_all, g)
        bi = batch(start, n_new, bt)
        T = int(n_new.sum())
        qd = synth.queries(g, T, 1, 1, desc.n_idx_heads, desc.c_idx)
        qI, w = synth.to_bf16_values(qd["qI"]), qd["w"]
        ld = 72
        scores = torch.full((T, ld), float("nan"), dtype=torch.bfloat16, device="cuda")
        nvalid = torch.zeros(T, dtype=torch.int32, device="cuda")
        st.index(bi, T, to_dev(qI, torch.bfloat16), to_dev(w), scores, ld, nvalid)
        torch.cuda.synchronize()
        got = scores.float().cpu().numpy()
        gv = nvalid.cpu().numpy()
        cu = np.concatenate([[0], np.cumsum(n_new)])
        for r in list(range(0, n_req, 37)) + [1023, 1024, 1050, n_req - 1]:
            if n_new[r] == 0:
                continue
            pos = np.arange(start[r], start[r] + n_new[r])
            _, kdeq = OL.store_keys(spec, keys[r])
            qdq = OL.quantize_index_queries(spec, qI[cu[r]:cu[r + 1]])
            want = OL.scores(spec, qdq, w[cu[r]:cu[r + 1]], pos, kdeq)
            for j in range(n_new[r]):
                V = (pos[j] + 1) // desc.m
                assert gv[cu[r] + j] == V
                check_score_row(desc, got[cu[r] + j, :V], want[j, :V], qdq[j], kdeq[:V], w[cu[r] + j],
                                f"request {r} token {j}")
                assert np.all(np.isnan(got[cu[r] + j, V:]))


def test_index_prefill_matches_decode():
    """The prefill-shaped launch (eight queries per workgroup) and the decode
    launch split the channels into the same MFMA steps and sum in the same
    order: a query's scores are bit-identical whichever launch scores it."""
    desc = presets.csa_flash_decode(win_cap=256)
    _flush("index prefill vs decode")
    g = synth.rng(107)
    E = 4096
    epb = desc.block_tokens // desc.m
    bt = synth.block_table(g, 1, (E + epb - 1) // epb)
    st = LayerState(desc, 1, bt.size)
    _fill_keys(st, desc, bt, [E], g)
    T, s0 = 40, 4 * E - 40
    qd = synth.queries(g, T, 1, 1, desc.n_idx_heads, desc.c_idx)
    qI = to_dev(synth.to_bf16_values(qd["qI"]), torch.bfloat16)
    w = to_dev(qd["w"])
    ld = E + 8
    one = torch.full((T, ld), float("nan"), dtype=torch.bfloat16, device="cuda")
    nv = torch.zeros(T, dtype=torch.int32, device="cuda")
    st.index(batch([s0], [T], bt), T, qI, w, one, ld, nv)             # one call, 40 new tokens
    each = torch.full((T, ld), float("nan"), dtype=torch.bfloat16, device="cuda")
    nv1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    for j in range(T):                                                 # one call per token
        st.index(batch([s0 + j], [1], bt), 1, qI[j:j + 1], w[j:j + 1], each[j:j + 1], ld, nv1)
    torch.cuda.synchronize()
    a = one.view(torch.int16).cpu().numpy()
    b = each.view(torch.int16).cpu().numpy()
    for j in range(T):
        V = (s0 + j + 1) // desc.m
        assert np.array_equal(a[j, :V], b[j, :V]), f"token {j}: prefill and decode scores differ"


# ---------------------------------------------------------------------------
# a5 / a6: attention with window and sink, on shared inputs
# ---------------------------------------------------------------------------

def _invariant(d):
    d.flags = abi.FLAG_BATCH_INVARIANT
    return d


ATTN_CASES = {
    "f32_sparse": (presets.tiny_csa_fp32(win_cap=512), [[600, 2], [130, 1], [2050, 40]]),
    "bf16_hca": (presets.hca_bf16(win_cap=1024), [[8192, 3], [700, 2], [127, 1]]),
    "fp8_sparse_64h": (presets.csa_flash_decode(), [[40000, 1], [9000, 1], [131072, 1], [100, 1]]),
    "fp8_sparse_128h_prefill": (presets.csa_pro(win_cap=512), [[5000, 33]]),
    "fp8_hca_128h": (presets.hca_pro(), [[70000, 1], [20000, 1]]),
    # sinks of -inf (the ordinary softmax) and queries that see no compressed
    # entry yet (V = 0: window rows only; V = 1), 128 heads, FP8 entries
    "fp8_sparse_128h_sink_neg_inf": (presets.csa_pro(win_cap=256), [[0, 1], [2, 1], [3, 1], [130, 1], [5000, 2]],
                                     "-inf"),
    # batch-invariant HCA over 5,120 entries: 41 fixed 128-row splits (two
    # load batches in the combine), the shorter request's later splits empty
    "fp8_hca_128h_invariant_41_splits": (_invariant(presets.hca_pro()), [[655360, 1], [40000, 1]]),
}


@pytest.mark.parametrize("name", list(ATTN_CASES))
def test_attention(name):
    desc, reqs = ATTN_CASES[name][:2]
    sink_mode = ATTN_CASES[name][2] if len(ATTN_CASES[name]) > 2 else None
    spec = spec_of(desc)
    _flush(f"attention {name}")
    g = synth.rng(104)
    n_req = len(reqs)
    ctx = [s + n for s, n in reqs]
    E = [c // desc.m for c in ctx]
    epb = desc.block_tokens // desc.m
    nb = [max(1, (e + epb - 1) // epb) for e in E]
    bt = synth.block_table(g, n_req, max(nb))
    st = LayerState(desc, n_req, bt.size)
    ents = [synth.normal(g, (e, desc.c)) for e in E]
    keys = [synth.normal(g, (e, desc.c_idx)) for e in E] if desc.c_idx else None
    append_entries(st, desc, bt, ents, [0] * n_req, keys)
    # window rows for positions [max(0, start - n_win + 1), ctx)
    wstart = [max(0, s - desc.n_win + 1) for s, n in reqs]
    wrows = [synth.normal(g, (ctx[r] - wstart[r], desc.c)) for r in range(n_req)]
    # one call per request block of rows keeps within win_cap
    append_window(st, desc, bt, wstart, wrows)
    start = [s for s, n in reqs]
    n_new = [n for s, n in reqs]
    bi = batch(start, n_new, bt)
    T = sum(n_new)
    q = synth.normal(g, (T, desc.n_heads, desc.c))
    if desc.act_fmt == abi.ACT_BF16:
        q = synth.to_bf16_values(q)
    sinks = synth.sinks(g, desc.n_heads)
    if sink_mode == "-inf":
        sinks = np.full(desc.n_heads, -np.inf, np.float32)
    gq = synth.normal(g, (desc.c,)) * 0.1 + 1.0
    sel = None
    if desc.kind == abi.KIND_CSA:
        sel = np.full((T, desc.top_k), -1, np.int32)
        row = 0
        for r in range(n_req):
            for j in range(n_new[r]):
                V = (start[r] + j + 1) // desc.m
                kk = min(desc.top_k, V)
                sel[row, :kk] = np.sort(g.choice(V, kk, replace=False))
                row += 1
    out = torch.zeros((T, desc.n_heads, desc.c), dtype=torch.bfloat16 if desc.out_fmt == abi.ACT_BF16 else torch.float32,
                      device="cuda")
    adt = torch.bfloat16 if desc.act_fmt == abi.ACT_BF16 else torch.float32
    st.attend(bi, T, to_dev(q, adt), to_dev(gq), to_dev(sinks), out, sel=None if sel is None else i32(sel))
    torch.cuda.synchronize()
    got = f32_of(out)
    row = 0
    tol = tol_of(desc)
    for r in range(n_req):
        calls = [(i, min(epb, E[r] - i)) for i in range(0, E[r], epb)]
        _, edeq = OL.store_entries(spec, ents[r], calls)
        win = np.zeros((ctx[r], desc.c))
        win[wstart[r]:] = OL.round_rows(spec.win_fmt, wrows[r])
        pos = np.arange(start[r], start[r] + n_new[r])
        want = OL.attend(spec, q[row:row + n_new[r]], gq, pos, edeq, win, sinks,
                         None if sel is None else sel[row:row + n_new[r]])
        assert_close(got[row:row + n_new[r]], want, tol, f"{name} request {r}")
        row += n_new[r]


# ---------------------------------------------------------------------------
# a1: compressor (projection + merge + norm/RoPE + window rows), stateful
# ---------------------------------------------------------------------------

def _compress_run(desc, d, H_per_req, sched, W, Wi, Ba, Bb, BaI, BbI, gamma):
    """Run compress_kv over a call schedule (list of per-request token counts);
    returns per-request lists of (entry index -> entry, key) and window rows."""
    n_req = len(H_per_req)
    ctx = [h.shape[0] for h in H_per_req]
    epb = desc.block_tokens // desc.m
    bt = np.arange(n_req * 4, dtype=np.int32).reshape(n_req, 4)
    st = LayerState(desc, n_req, bt.size)
    adt = torch.bfloat16 if desc.act_fmt == abi.ACT_BF16 else torch.float32
    dW = to_dev(W.T.copy(), adt)
    dWi = to_dev(Wi.T.copy(), adt) if Wi is not None else None
    dBa, dBb = to_dev(Ba), to_dev(Bb) if Bb is not None else None
    dBaI = to_dev(BaI) if BaI is not None else None
    dBbI = to_dev(BbI) if BbI is not None else None
    dg = to_dev(gamma)
    done = [0] * n_req
    ent = [dict() for _ in range(n_req)]
    win = [np.zeros((ctx[r], desc.c), np.float32) for r in range(n_req)]
    for call in sched:
        Hc = np.concatenate([H_per_req[r][done[r]:done[r] + call[r]] for r in range(n_req)])
        bi = batch(done, call, bt, max_ctx=max(done[r] + call[r] for r in range(n_req)))
        T = int(sum(call))
        max_e = sum((done[r] + call[r]) // desc.m - done[r] // desc.m for r in range(n_req))
        e, k, meta, cnt, w = st.compress(bi, T, to_dev(Hc, adt) if T else None, dW, dWi, dBa, dBb, dBaI, dBbI, dg,
                                         max_e)
        torch.cuda.synchronize()
        assert int(cnt.item()) == max_e
        ee, mm = e.cpu().numpy(), meta.cpu().numpy()
        kk = k.cpu().numpy() if k is not None else None
        for j in range(max_e):
            r, i = int(mm[j, 0]), int(mm[j, 1])
            ent[r][i] = (ee[j], None if kk is None else kk[j])
        ww = w.cpu().numpy()
        row = 0
        for r in range(n_req):
            win[r][done[r]:done[r] + call[r]] = ww[row:row + call[r]]
            row += call[r]
        done = [done[r] + call[r] for r in range(n_req)]
    return ent, win


@pytest.mark.parametrize("name", ["tiny_fp32", "hca_bf16"])
def test_compress_kv_chunked_and_decode(name):
    _flush(f"compress_kv {name}")
    g = synth.rng(105)
    if name == "tiny_fp32":
        desc, d = presets.tiny_csa_fp32(win_cap=2048), presets.D_TINY
        ctx = [2056, 301]
        sched = [[1000, 0], [1048, 300], [1, 1]] + [[1, 0]] * 7
        w_ = synth.csa_weights(g, d, desc.c, desc.m, desc.c_idx)
        W, Wi, Ba, Bb, BaI, BbI = w_["W"], w_["W_I"], w_["Ba"], w_["Bb"], w_["BaI"], w_["BbI"]
        tol = 1e-4
    else:
        desc, d = presets.hca_bf16(win_cap=4224), presets.D_HCA
        ctx = [8192, 5000]
        # a 60-row call (four 16-row blocks, the last ragged) and one-token
        # calls take the projection in four partial products, which the
        # merge, window and tail kernels (several new tokens) and the fused
        # decode kernel (at most one) add; the long calls take the 128 x 128 tiles
        sched = [[3000, 4000], [40, 20], [1, 1], [1, 0], [4000, 979], [1150, 0]]
        w_ = synth.hca_weights(g, d, desc.c, desc.m)
        W, Wi, Ba, Bb, BaI, BbI = w_["W"], None, w_["Ba"], None, None, None
        W = synth.to_bf16_values(W)
        tol = 1e-3
    spec = spec_of(desc)
    gamma = (synth.normal(g, (desc.c,)) * 0.1 + 1.0).astype(np.float32)
    H = [synth.normal(g, (n, d)) for n in ctx]
    if desc.act_fmt == abi.ACT_BF16:
        H = [synth.to_bf16_values(h) for h in H]
    if Wi is not None and desc.act_fmt == abi.ACT_BF16:
        Wi = synth.to_bf16_values(Wi)
    ent, win = _compress_run(desc, d, H, sched, W, Wi, Ba, Bb, BaI, BbI, gamma)
    for r in range(len(ctx)):
        Ehat, K, R = OL.compress_layer(spec, H[r], W, Ba, Bb, gamma, Wi, BaI, BbI)
        assert len(ent[r]) == Ehat.shape[0]
        ge = np.stack([ent[r][i][0] for i in range(Ehat.shape[0])])
        e1 = assert_close(ge, Ehat, tol, f"entries r{r}")
        e2 = assert_close(win[r], R, tol, f"window rows r{r}")
        msg = f"{name} r{r}: entries {e1:.2e} window {e2:.2e}"
        if K is not None:
            gk = np.stack([ent[r][i][1] for i in range(K.shape[0])])
            e3 = assert_close(gk, K, tol, f"keys r{r}")
            msg += f" keys {e3:.2e}"
        _flush(msg)
