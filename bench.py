"""Decode throughput of the CSA / HCA hot path on one MI355X.

A step is one decode token for every request through every layer of the
workload: compress_kv, cache_append, index_scores, topk_select and
sparse_mqa per CSA layer; compress_kv, cache_append and hca_attention per HCA
layer.  Inputs (caches, window rings, compressor tails, weights, queries) are
synthetic, resident in HBM before timing starts, and the cache is rotated
over several replicas so that the 256 MB last-level cache cannot hold a
step's working set.  One HIP graph holds two steps of every replica in
rotation order, one per position buffer (each step's first compress call
writes the next positions into the other buffer), single-step graphs time a
remainder, and the graphs are replayed.  Prints one JSON line.

Workloads:
  csa_decode_128k  16 requests x 131072 cached tokens, one CSA layer
                   (c=512: 448 fp8 + 64 bf16 channels, per-block scale; m=4;
                   64 heads; indexer 64 x 128 bf16; top-512; window 128; d=4096)
  hybrid_decode_1m 4 requests x 1048576 cached tokens, layers CSA, HCA, CSA,
                   HCA (CSA: 128 heads, MXFP4 indexer, top-1024; HCA: m'=128;
                   c=512 fp8/bf16 KV; window 128; d=7168)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA, published


def workload_def(name: str):
    from long_context_sparse_03_amd import abi, presets
    if name == "csa_decode_128k":
        return dict(descs=[presets.csa_flash_decode()], d=presets.D_FLASH, n_req=16, ctx=131072, replicas=3)
    if name == "hybrid_decode_1m":
        return dict(descs=[presets.csa_pro(idx_fmt=abi.IDX_MXFP4), presets.hca_pro(),
                           presets.csa_pro(idx_fmt=abi.IDX_MXFP4), presets.hca_pro()],
                    d=presets.D_PRO, n_req=4, ctx=1 << 20, replicas=4)
    raise SystemExit(f"unknown workload {name}")


def algorithmic_bytes(wd) -> dict:
    """Bytes the method must move per decode step (no re-reads), by part."""
    from long_context_sparse_03_amd import abi
    n, ctx = wd["n_req"], wd["ctx"]
    tot = {"index_keys": 0, "kv_rows": 0, "weights": 0, "q_out": 0, "other": 0}
    idx_launch = 0
    for desc in wd["descs"]:
        c, r = desc.c, desc.rope_dim
        rec = (c - r) + 2 * r if desc.kv_fmt == abi.KV_FP8 else c * (2 if desc.kv_fmt == abi.KV_BF16 else 4)
        ncols = 4 * c + 4 * desc.c_idx if desc.kind == abi.KIND_CSA else 2 * c
        tot["weights"] += ncols * wd["d"] * 2
        tot["q_out"] += n * desc.n_heads * c * 2 * 2
        if desc.kind == abi.KIND_CSA:
            E = (ctx + 1) // desc.m
            kb = desc.c_idx * 2 if desc.idx_fmt == abi.IDX_BF16 else desc.c_idx // 2 + desc.c_idx // 32
            keys = n * E * kb
            qw = n * desc.n_idx_heads * (desc.c_idx * 2 + 4)
            sc = n * E * 2
            tot["index_keys"] += keys
            tot["kv_rows"] += n * (desc.top_k * (rec + 4) + desc.n_win * c * 2)
            tot["other"] += qw + sc
            idx_launch = keys + qw + sc
        else:
            E = (ctx + 1) // desc.m
            tot["kv_rows"] += n * (E * (rec + 4) + desc.n_win * c * 2)
    tot["total"] = sum(tot.values())
    tot["index_launch"] = idx_launch
    return tot


def _oracle_spec(desc):
    from oracle import layer as OL
    from long_context_sparse_03_amd import abi
    kv = {abi.KV_F32: "f32", abi.KV_BF16: "bf16", abi.KV_FP8: "fp8"}[desc.kv_fmt]
    idx = {abi.IDX_F32: "f32", abi.IDX_BF16: "bf16", abi.IDX_MXFP4: "mxfp4"}[desc.idx_fmt]
    fmt = {abi.ACT_F32: "f32", abi.ACT_BF16: "bf16"}
    return OL.Spec("csa" if desc.kind == abi.KIND_CSA else "hca", m=desc.m, c=desc.c, r=desc.rope_dim,
                   n_h=desc.n_heads, n_hI=desc.n_idx_heads, c_I=desc.c_idx, top_k=desc.top_k, n_win=desc.n_win,
                   kv_fmt=kv, idx_fmt=idx, score_fmt=fmt[desc.score_fmt], win_fmt=fmt[desc.act_fmt])


def _oracle_cache(spec, g, E, synth, OL):
    """Dequantised synthetic entries (and CSA keys) as the oracle stores them."""
    ents = synth.normal(g, (E, spec.c))
    _, edeq = OL.store_entries(spec, ents, [(i, min(spec.epb, E - i)) for i in range(0, E, spec.epb)])
    kdeq = OL.store_keys(spec, synth.normal(g, (E, spec.c_I)))[1] if spec.kind == "csa" else None
    return edeq, kdeq


def cpu_baseline(wd, n_tok: int, seed: int = 11) -> dict:
    """The oracle (fp64, as it stands) on a bounded sample of a decode
    workload.  One CSA layer (128K): n_tok consecutive decode tokens of one
    request through the projection of the new tokens, index scores, top-k
    and attention (the oracle runs a request's queries in parallel).  The
    hybrid 1M workload: one decode step of one request through all four
    layers (projection, then index scores, top-k and attention for CSA,
    dense attention for HCA)."""
    import oracle as O
    from oracle import layer as OL
    import synth
    from long_context_sparse_03_amd import abi
    g = synth.rng(seed)
    ctx, d = wd["ctx"], wd["d"]
    if len(wd["descs"]) == 1:
        desc = wd["descs"][0]
        spec = _oracle_spec(desc)
        E = (ctx + n_tok) // desc.m
        W = synth.weights(g, d, 4 * desc.c + 4 * desc.c_idx)
        edeq, kdeq = _oracle_cache(spec, g, E, synth, OL)
        win = np.zeros((ctx + n_tok, desc.c))
        win[ctx - 127:] = OL.round_rows("bf16", synth.normal(g, (n_tok + 127, desc.c)))
        qd = synth.queries(g, n_tok, desc.n_heads, desc.c, desc.n_idx_heads, desc.c_idx)
        H = synth.normal(g, (n_tok, d))
        sinks = synth.sinks(g, desc.n_heads)
        pos = np.arange(ctx, ctx + n_tok)
        t0 = time.perf_counter()
        OL.project(H, W)
        OL.csa_queries(spec, qd["q"], qd["qI"], qd["w"], pos, kdeq, edeq, win, sinks)
        elapsed = time.perf_counter() - t0
        return {"value": round(n_tok / elapsed, 3), "unit": "tokens/s", "cores": O.num_threads(), "kind": "oracle",
                "sample": f"{n_tok} consecutive decode tokens of one request at {ctx} cached tokens, first CSA "
                          f"layer ({E} entries): new-token projection, index scores, top-{desc.top_k}, attention; "
                          f"fp64; {elapsed:.1f} s"}
    # one request, one step through every layer (the two CSA layers, and
    # the two HCA layers, share one synthetic cache each)
    caches, parts = {}, []
    for desc in wd["descs"]:
        spec = _oracle_spec(desc)
        key = (desc.kind, desc.m)
        if key not in caches:
            E = (ctx + 1) // desc.m
            edeq, kdeq = _oracle_cache(spec, g, E, synth, OL)
            win = np.zeros((ctx + 1, desc.c))
            win[ctx - 127:] = OL.round_rows("bf16", synth.normal(g, (128, desc.c)))
            ncols = 4 * desc.c + 4 * desc.c_idx if desc.kind == abi.KIND_CSA else 2 * desc.c
            caches[key] = (edeq, kdeq, win, synth.weights(g, d, ncols))
        qd = synth.queries(g, 1, desc.n_heads, desc.c, desc.n_idx_heads, desc.c_idx)
        parts.append((desc, spec, qd, synth.sinks(g, desc.n_heads), synth.normal(g, (1, d))))
    pos = np.array([ctx])
    t0 = time.perf_counter()
    for desc, spec, qd, sinks, H in parts:
        edeq, kdeq, win, W = caches[(desc.kind, desc.m)]
        OL.project(H, W)
        if desc.kind == abi.KIND_CSA:
            OL.csa_queries(spec, qd["q"], qd["qI"], qd["w"], pos, kdeq, edeq, win, sinks)
        else:
            OL.attend(spec, qd["q"], None, pos, edeq, win, sinks)
    elapsed = time.perf_counter() - t0
    return {"value": round(1.0 / elapsed, 4), "unit": "tokens/s", "cores": O.num_threads(), "kind": "oracle",
            "sample": f"one decode step of one request at {ctx} cached tokens through all {len(parts)} layers "
                      f"(projection; CSA: index scores over {(ctx + 1) // 4} entries, top-k, attention; HCA: "
                      f"dense attention); fp64; {elapsed:.1f} s (whole-job rate of one request)"}


def cpu_baseline_prefill(n_q: int = 32, seed: int = 12) -> dict:
    """The oracle on a stratified sample of n_q of the 4096 chunk queries at
    1,048,576 cached tokens (index scores over ~262K entries, top-1024,
    attention), extrapolated to the chunk."""
    import oracle as O
    from oracle import layer as OL
    import synth
    from long_context_sparse_03_amd import presets
    desc = presets.csa_pro()
    spec = _oracle_spec(desc)
    g = synth.rng(seed)
    ctx, T = 1 << 20, 4096
    E = (ctx + T) // desc.m
    edeq, kdeq = _oracle_cache(spec, g, E, synth, OL)
    win = np.zeros((ctx + T, desc.c))
    win[ctx - 127:] = OL.round_rows("bf16", synth.normal(g, (T + 127, desc.c)))
    rows = np.linspace(0, T - 1, n_q).astype(int)
    qd = synth.queries(g, n_q, desc.n_heads, desc.c, desc.n_idx_heads, desc.c_idx)
    sinks = synth.sinks(g, desc.n_heads)
    t0 = time.perf_counter()
    OL.csa_queries(spec, qd["q"], qd["qI"], qd["w"], ctx + rows, kdeq, edeq, win, sinks)
    elapsed = time.perf_counter() - t0
    per_chunk = elapsed * T / n_q
    return {"value": round(T / per_chunk, 3), "unit": "tokens/s", "cores": O.num_threads(), "kind": "oracle",
            "sample": f"{n_q} stratified queries of the 4096-token chunk at {ctx} cached tokens (index scores, "
                      f"top-{desc.top_k}, attention), {elapsed:.1f} s, extrapolated x{T // n_q} to the chunk "
                      f"(compressor projection excluded)", "extrapolated": True}


def cpu_baseline_small(name: str) -> dict:
    """The oracle on a whole small workload: the tiny fp32 CSA layer
    (prefill 2048 + 8 decode tokens) or the HCA bf16 layer (2 x 8192)."""
    import oracle as O
    from oracle import layer as OL
    import synth
    from long_context_sparse_03_amd import presets
    if name == "tiny_csa":
        desc, d, reqs = presets.tiny_csa_fp32(), presets.D_TINY, [2056]
    else:
        desc, d, reqs = presets.hca_bf16(), presets.D_HCA, [8192, 8192]
    spec = _oracle_spec(desc)
    g = synth.rng(13)
    w = synth.csa_weights(g, d, desc.c, desc.m, desc.c_idx) if desc.c_idx else synth.hca_weights(g, d, desc.c,
                                                                                               desc.m)
    ins = [(synth.normal(g, (n, d)), synth.queries(g, n, desc.n_heads, desc.c, desc.n_idx_heads, desc.c_idx))
           for n in reqs]
    sinks = synth.sinks(g, desc.n_heads)
    t0 = time.perf_counter()
    for H, qd in ins:
        pos = np.arange(H.shape[0])
        E, K, R = OL.compress_layer(spec, H, w["W"], w["Ba"], w.get("Bb"), None, w.get("W_I"), w.get("BaI"),
                                    w.get("BbI"))
        _, edeq = OL.store_entries(spec, E.astype(np.float32), [(0, E.shape[0])])
        win = OL.round_rows(spec.win_fmt, R.astype(np.float32))
        if desc.c_idx:
            kdeq = OL.store_keys(spec, K.astype(np.float32))[1]
            OL.csa_queries(spec, qd["q"], qd["qI"], qd["w"], pos, kdeq, edeq, win, sinks)
        else:
            OL.attend(spec, qd["q"], None, pos, edeq, win, sinks)
    elapsed = time.perf_counter() - t0
    n = sum(reqs)
    return {"value": round(n / elapsed, 1), "unit": "tokens/s", "cores": O.num_threads(), "kind": "oracle",
            "sample": f"the whole workload ({' + '.join(map(str, reqs))} tokens: compressor, storage, "
                      f"{'index scores, top-k, ' if desc.c_idx else ''}attention); fp64; {elapsed:.2f} s"}


def profiled_traffic(kernel: str, workload: str):
    """HBM bytes per launch of a kernel from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, each scaled by the same counter on a copy of
    known size), or None when there is none or the kernel sources changed
    since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for ln in open(path):
        if ":" in ln and not ln.startswith(" "):
            k, v = ln.split(":", 1)
            vals[k.strip()] = v.strip().split()[0] if v.strip() else ""
    h = hashlib.sha256()
    for f in ("index.hip", "common.hpp", "kernels.hpp"):
        with open(os.path.join(ROOT, "long_context_sparse_03_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if vals.get("sources_sha256") != h.hexdigest():
        return None
    return int(float(vals["traffic_bytes_per_launch"]))


def time_decode(name, steps, warmup, replicas=0, graph=True, fused_append=True, fused_topk=True):
    """Decode throughput of one workload; returns a dict of measurements."""
    import torch
    from long_context_sparse_03_amd import abi
    from long_context_sparse_03_amd.workloads import DecodeWorkload, torch_rows

    wd = workload_def(name)
    reps = replicas or wd["replicas"]
    total_steps = warmup + steps + 2 * reps + 64
    t_build = time.time()
    wls = [DecodeWorkload(wd["descs"], wd["d"], wd["n_req"], wd["ctx"], max_steps=total_steps,
                          rows=torch_rows(1000 + i), seed=i, fused_append=fused_append, fused_topk=fused_topk)
           for i in range(reps)]
    torch.cuda.synchronize()
    build_s = time.time() - t_build

    stream = torch.cuda.Stream()
    # the order of steps: every replica at position buffer 0, then every
    # replica at buffer 1 (each step's first layer writes the advanced
    # positions into the other buffer), so 2 * reps steps return every
    # replica to buffer 0
    seq = [(r, p) for p in (0, 1) for r in range(reps)]
    with torch.cuda.stream(stream):
        for r, p in seq:
            wls[r].step(parity=p)
        stream.synchronize()

    # One graph holds 2 * reps consecutive steps (the launch of the graph is
    # shared by them, as a serving loop that captures several steps would
    # share it); single-step graphs time the steps before and after whole
    # replays.
    gph, gph_one = None, {}
    if graph:
        gph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gph, stream=stream):
            for r, p in seq:
                wls[r].step(parity=p)
        for r, p in seq:
            g1 = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g1, stream=stream):
                wls[r].step(parity=p)
            gph_one[(r, p)] = g1
        torch.cuda.synchronize()

    done = [0]

    def one(i):
        r, p = seq[i % len(seq)]
        if gph is not None:
            gph_one[(r, p)].replay()
        else:
            wls[r].step(parity=p)

    def run_steps(n):
        L = len(seq)
        while n > 0 and done[0] % L != 0:
            one(done[0])
            done[0] += 1
            n -= 1
        full, rem = divmod(n, L)
        for _ in range(full):
            if gph is not None:
                gph.replay()
            else:
                for r, p in seq:
                    wls[r].step(parity=p)
        done[0] += full * L
        for _ in range(rem):
            one(done[0])
            done[0] += 1

    with torch.cuda.stream(stream):
        run_steps(warmup)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        run_steps(steps)
        t1.record(stream)
        torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    # Per-launch time of the index scan, on the launch stream, right after
    # the timed steps: HIP events cannot be recorded inside a captured graph
    # here (torch on ROCm refuses external events), so csa_index_scores
    # launches (the same kernel without the fused top-k's counts) run back to
    # back over every CSA layer of every cache replica in turn, between one
    # pair of events.  The key sets visited in turn (replicas x CSA layers:
    # 3 x 135.5 MB at 128K, 8 x 73.4 MB at 1M) exceed the 256 MB last-level
    # cache, so every launch reads its keys from HBM.
    csa_layers = [i for i, (st, _) in enumerate(wls[0].layers) if st.is_csa]
    li = csa_layers[0]
    sets = [(r, l) for l in csa_layers for r in range(reps)]
    n_idx = 12 * len(sets)
    with torch.cuda.stream(stream):
        for r, l in sets:
            wls[r].index_call(l)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for j in range(n_idx):
            r, l = sets[j % len(sets)]
            wls[r].index_call(l)
        e1.record(stream)
        torch.cuda.synchronize()
    idx_avg_ms = e0.elapsed_time(e1) / n_idx
    key_set_bytes = algorithmic_bytes(wd)["index_launch"] * len(sets)
    ab = algorithmic_bytes(wd)
    kname = "index_decode_fp4_kernel" if wls[0].layers[li][0].desc.idx_fmt == abi.IDX_MXFP4 else "index_decode_kernel"
    roof = None
    if idx_avg_ms:
        achieved = ab["index_launch"] / (idx_avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": profiled_traffic(kname, name),
                "launch_ms": round(idx_avg_ms, 5), "algorithmic_bytes_per_launch": ab["index_launch"],
                "rotated_key_sets": len(sets), "rotated_bytes": key_set_bytes}
    step_gbs = ab["total"] / (ms * 1e-3) / 1e9
    del wls, gph, gph_one
    torch.cuda.empty_cache()
    return {"workload": name, "tokens_per_s": round(wd["n_req"] / (ms * 1e-3), 1), "ms_per_step": round(ms, 5),
            "requests": wd["n_req"], "ctx": wd["ctx"], "layers": len(wd["descs"]), "d": wd["d"],
            "replicas": reps, "graph": graph, "step_hbm_gbs": round(step_gbs, 1),
            "step_hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4), "step_algorithmic_bytes": ab, "roofline": roof,
            "setup_s": round(build_s, 1)}


def time_prefill(steps, warmup):
    """One 4096-token chunk on top of 1,048,576 cached tokens (Pro shape):
    compress_kv, cache_append, the fused index_topk, sparse_mqa.  The
    roofline times the index scan alone (csa_index_scores, the same kernel
    without the fused selection's per-chunk counts) right after the steps;
    the standalone selector (csa_topk_select) on the same scores is timed
    too, for comparison."""
    import torch
    from long_context_sparse_03_amd import abi, presets
    from long_context_sparse_03_amd import abi
    from long_context_sparse_03_amd.workloads import DecodeWorkload, torch_rows
    from long_context_sparse_03_amd.layer import make_batch

    desc = presets.csa_pro(win_cap=4352)
    T, ctx, d = 4096, 1 << 20, presets.D_PRO
    wl = DecodeWorkload([desc], d, 1, ctx, max_steps=T + 256, rows=torch_rows(77), seed=5)
    st, P = wl.layers[0]
    dev = "cuda"
    cu = torch.tensor([0, T], dtype=torch.int32, device=dev)
    sp = torch.tensor([ctx], dtype=torch.int32, device=dev)
    bi = make_batch(cu, sp, wl.block_table, T, ctx + T, T)
    H = torch.randn((T, d), device=dev).to(torch.bfloat16)
    q = torch.randn((T, desc.n_heads, desc.c), device=dev).to(torch.bfloat16)
    qI = torch.randn((T, desc.n_idx_heads, desc.c_idx), device=dev).to(torch.bfloat16)
    w = torch.randn((T, desc.n_idx_heads), device=dev) / 8.0
    n_e = T // desc.m
    ent = torch.empty((n_e, desc.c), device=dev)
    keys = torch.empty((n_e, desc.c_idx), device=dev)
    meta = torch.empty((n_e, 2), dtype=torch.int32, device=dev)
    cnt = torch.zeros(1, dtype=torch.int32, device=dev)
    win = torch.empty((T, desc.c), device=dev)
    ws_c = torch.empty(abi.workspace_size(desc, abi.OP_COMPRESS, T), dtype=torch.uint8, device=dev)
    ld = ((ctx + T) // desc.m + 63) // 64 * 64
    scores = torch.empty((T, ld), dtype=torch.bfloat16, device=dev)
    nv = torch.empty(T, dtype=torch.int32, device=dev)
    sel = torch.empty((T, desc.top_k), dtype=torch.int32, device=dev)
    ws_t = torch.empty(max(1, abi.workspace_size(desc, abi.OP_TOPK, T, ld, desc.top_k)), dtype=torch.uint8, device=dev)
    out = torch.empty((T, desc.n_heads, desc.c), dtype=torch.bfloat16, device=dev)
    ws_a = torch.empty(max(1, abi.workspace_size(desc, abi.OP_ATTENTION, T, desc.top_k + desc.n_win)),
                       dtype=torch.uint8, device=dev)
    ws_it = torch.empty(max(1, abi.workspace_size(desc, abi.OP_INDEX_TOPK, T, ld)), dtype=torch.uint8, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]

    def step():
        ev[0].record()
        abi.compress_kv(desc, bi.batch, T, d, H, P["W"], P["W_idx"], P["B_a"], P["B_b"], P["B_a_idx"], P["B_b_idx"],
                        P["gamma"], st.state, ent, keys, meta, cnt, n_e, win, ws_c)
        abi.cache_append(desc, bi.batch, T, ent, keys, meta, cnt, n_e, win, st.kv, st.idx, st.state)
        ev[1].record()
        abi.index_topk(desc, bi.batch, T, qI, w, st.idx, scores, ld, nv, sel, ws_it)
        ev[2].record()
        abi.sparse_mqa(desc, bi.batch, T, q, P["q_gamma"], sel, st.kv, st.state, P["sinks"], out, ws_a)
        ev[3].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    parts = np.zeros(3)
    tot = 0.0
    for _ in range(steps):
        step()
        torch.cuda.synchronize()
        parts += [ev[i].elapsed_time(ev[i + 1]) for i in range(3)]
        tot += ev[0].elapsed_time(ev[3])
    parts /= steps
    ms = tot / steps
    # the index scan alone (roofline) and the standalone selector, each
    # timed over `steps` launches on the scores the last step left
    ev[4].record()
    for _ in range(steps):
        abi.index_scores(desc, bi.batch, T, qI, w, st.idx, scores, ld, nv)
    ev[5].record()
    torch.cuda.synchronize()
    ms_index = ev[4].elapsed_time(ev[5]) / steps
    ev[4].record()
    for _ in range(steps):
        abi.topk_select(desc.score_fmt, T, scores, ld, nv, desc.top_k, sel, ws_t)
    ev[5].record()
    torch.cuda.synchronize()
    ms_topk_standalone = ev[4].elapsed_time(ev[5]) / steps
    E = ctx // desc.m
    sumV = sum((ctx + t + 1) // desc.m for t in range(T))
    idx_flop = 2.0 * desc.n_idx_heads * desc.c_idx * sumV
    attn_flop = 4.0 * desc.n_heads * desc.c * T * (desc.top_k + desc.n_win)
    proj_flop = 2.0 * T * d * (4 * desc.c + 4 * desc.c_idx)
    idx_tfs = idx_flop / (ms_index * 1e-3) / 1e12
    del wl
    torch.cuda.empty_cache()
    return {"workload": "csa_prefill_1m", "tokens_per_s": round(T / (ms * 1e-3), 1), "ms_per_chunk": round(ms, 3),
            "chunk": T, "ctx": ctx, "d": d,
            "ms_compress_append": round(parts[0], 3), "ms_index_topk": round(parts[1], 3),
            "ms_attention": round(parts[2], 3), "ms_index": round(ms_index, 3),
            "ms_topk_standalone": round(ms_topk_standalone, 3),
            "tflops_total": round((idx_flop + attn_flop + proj_flop) / (ms * 1e-3) / 1e12, 1),
            "roofline": {"bound": "mfma", "kernel": "index_prefill_kernel", "achieved": round(idx_tfs, 1),
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(idx_tfs / BF16_PEAK_TFLOPS, 4),
                         "traffic": None, "algorithmic_flop_per_launch": idx_flop},
            "attention_tflops": round(attn_flop / (parts[2] * 1e-3) / 1e12, 1)}


def time_small(name: str, reps: int = 5):
    """The two small workloads end to end on the GPU (launch-bound; absolute
    times): the tiny fp32 CSA layer (one request: a 2048-token prefill call,
    then 8 one-token decode calls) and the HCA bf16 layer (one call with 2
    requests x 8192 tokens).  Every call runs compress_kv, cache_append and
    the attention (CSA: index_topk in between)."""
    import torch
    from long_context_sparse_03_amd import abi, presets
    from long_context_sparse_03_amd.layer import LayerState, make_batch
    dev = "cuda"
    gen = torch.Generator(device=dev).manual_seed(21)
    if name == "tiny_csa":
        desc, d, n_req, sched = presets.tiny_csa_fp32(win_cap=2304), presets.D_TINY, 1, [(0, 2048)] + [
            (2048 + i, 1) for i in range(8)]
    else:
        desc, d, n_req, sched = presets.hca_bf16(win_cap=8320), presets.D_HCA, 2, [(0, 8192)]
    adt = torch.bfloat16 if desc.act_fmt == abi.ACT_BF16 else torch.float32
    csa = desc.kind == abi.KIND_CSA
    ncols = 4 * desc.c + 4 * desc.c_idx if csa else 2 * desc.c
    n_main = 4 * desc.c if csa else 2 * desc.c

    def rnd(*shape, std=1.0, dt=torch.float32):
        return (torch.randn(*shape, generator=gen, device=dev) * std).to(dt)
    Wt = rnd(ncols, d, std=d ** -0.5, dt=adt)
    P = dict(W=Wt[:n_main].contiguous(), W_idx=Wt[n_main:].contiguous() if csa else None, B_a=rnd(desc.m, desc.c),
             B_b=rnd(desc.m, desc.c) if csa else None, B_a_idx=rnd(desc.m, desc.c_idx) if csa else None,
             B_b_idx=rnd(desc.m, desc.c_idx) if csa else None, gamma=torch.ones(desc.c, device=dev),
             sinks=rnd(desc.n_heads))
    nb = (max(s + n for s, n in sched) + desc.block_tokens - 1) // desc.block_tokens + 1
    bt = torch.arange(n_req * nb, dtype=torch.int32, device=dev).view(n_req, nb)
    st = LayerState(desc, n_req, n_req * nb)
    calls = []
    for s0, n in sched:
        T = n * n_req
        cu = torch.arange(n_req + 1, dtype=torch.int32, device=dev) * n
        sp = torch.full((n_req,), s0, dtype=torch.int32, device=dev)
        bi = make_batch(cu, sp, bt, n, s0 + n, T)
        max_e = n_req * ((s0 + n) // desc.m - s0 // desc.m)
        ld = ((s0 + n) // desc.m + 7) // 8 * 8 + 8
        b = dict(bi=bi, T=T, max_e=max_e, ld=ld, H=rnd(T, d, dt=adt), q=rnd(T, desc.n_heads, desc.c, dt=adt),
                 out=torch.empty((T, desc.n_heads, desc.c), dtype=torch.float32 if desc.out_fmt == abi.ACT_F32
                                 else torch.bfloat16, device=dev))
        if csa:
            b.update(qI=rnd(T, desc.n_idx_heads, desc.c_idx, dt=adt), w=rnd(T, desc.n_idx_heads, std=0.125),
                     sc=torch.empty((T, ld), dtype=torch.float32, device=dev),
                     nv=torch.empty(T, dtype=torch.int32, device=dev),
                     sel=torch.empty((T, desc.top_k), dtype=torch.int32, device=dev))
        calls.append(b)

    def run():
        for b in calls:
            st.compress_append(b["bi"], b["T"], b["H"], P["W"], P["W_idx"], P["B_a"], P["B_b"], P["B_a_idx"],
                               P["B_b_idx"], P["gamma"], max(b["max_e"], 1))
            if csa:
                st.index_topk(b["bi"], b["T"], b["qI"], b["w"], b["sc"], b["ld"], b["nv"], b["sel"])
            st.attend(b["bi"], b["T"], b["q"], P["gamma"], P["sinks"], b["out"], sel=b["sel"] if csa else None)
    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    n_tok = sum(n for _, n in sched) * n_req
    del st
    torch.cuda.empty_cache()
    return {"workload": name, "tokens": n_tok, "calls": len(sched), "ms": round(ms, 3),
            "tokens_per_s": round(n_tok / (ms * 1e-3), 1),
            "note": "launch-bound parity workload; absolute time, no roofline"}


def time_prefix(reps=3):
    """Prefix reuse, host-memory tier: the blocks of a 1,048,576-token CSA
    prefix (Pro shape, 8192 blocks of KV and indexer keys) to and from pinned
    host memory, one launch each way."""
    import torch
    from long_context_sparse_03_amd import abi, presets
    from long_context_sparse_03_amd.layer import LayerState

    desc = presets.csa_pro()
    n_blocks = (1 << 20) // desc.block_tokens
    st = LayerState(desc, 1, n_blocks)
    ids = torch.arange(n_blocks, dtype=torch.int32, device="cuda")
    host = torch.empty(abi.prefix_bytes(desc, n_blocks), dtype=torch.uint8, pin_memory=True)
    nbytes = host.numel()
    res = {}
    for name, direction in (("save", abi.TO_HOST), ("restore", abi.FROM_HOST)):
        abi.prefix_blocks(desc, n_blocks, ids, st.kv, st.idx, host, direction)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            abi.prefix_blocks(desc, n_blocks, ids, st.kv, st.idx, host, direction)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res[name] = {"ms": round(ms, 3), "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1)}
    del st, host
    torch.cuda.empty_cache()
    return {"workload": "csa_prefix_1m_host", "blocks": n_blocks, "bytes": nbytes, **res,
            "note": "kernel reads / writes pinned host memory over PCIe"}


def time_projections(reps=20):
    """The dense projections around the path at the Pro shape for one decode
    step of 16 requests: the low-rank query path (d 7168 -> d_c 1024 -> 128
    heads x 512 and 64 indexer heads x 128, plus the 64 head weights) and the
    grouped output projection (16 groups of 8 heads -> 1024 each -> 7168).
    Weight-streaming: bytes are the bf16 weights read once."""
    import torch
    from long_context_sparse_03_amd import abi
    from long_context_sparse_03_amd.projections import output_projection, query_path

    T, d, dc, nqc, nic, nhi, ng, dg = 16, 7168, 1024, 128 * 512, 64 * 128, 64, 16, 1024
    gen = torch.Generator(device="cuda").manual_seed(7)

    def w(*shape):
        return (torch.randn(*shape, device="cuda", generator=gen) / shape[-1] ** 0.5).to(torch.bfloat16)

    h, o = w(T, d), w(T, nqc)
    W_DQ, W_UQ, W_UQI, W_w = w(dc, d), w(nqc, dc), w(nic, dc), w(nhi, d)
    W_G, W_O = w(ng, dg, nqc // ng), w(d, ng * dg)
    qb = 2 * (W_DQ.numel() + W_UQ.numel() + W_UQI.numel() + W_w.numel())
    ob = 2 * (W_G.numel() + W_O.numel())
    res = {}
    for name, fn, nbytes in (("query_path", lambda: query_path(h, W_DQ, W_UQ, W_UQI, W_w), qb),
                             ("output_projection", lambda: output_projection(o, W_G, W_O), ob)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1000
        res[name] = {"us": round(us, 1), "weight_bytes": nbytes, "gbs": round(nbytes / (us * 1e-6) / 1e9, 1)}
    return {"workload": "pro_projections_decode", "rows": T, **res,
            "note": "the same weights in every repetition: the query path's 167 MB fit the 256 MB last-level "
                    "cache, the output projection's 369 MB do not"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="csa_decode_128k", choices=["csa_decode_128k", "hybrid_decode_1m"])
    ap.add_argument("--replicas", type=int, default=0, help="cache replicas rotated between steps (0: workload default)")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the 1M decode and 1M prefill sub-results")
    ap.add_argument("--cpu-tokens", type=int, default=640, help="decode tokens in the CPU-oracle sample (0: skip)")
    ap.add_argument("--separate-append", action="store_true",
                    help="decode steps call compress_kv and cache_append instead of compress_append")
    ap.add_argument("--separate-topk", action="store_true",
                    help="decode steps call index_scores and topk_select instead of the fused index_topk")
    ap.add_argument("--copy-probe", action="store_true", help="also run a 1 GiB device copy (HBM counter scale)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        raise SystemExit(2)

    import torch
    if args.copy_probe:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    fused = not args.separate_append
    ftk = not args.separate_topk
    prim = time_decode(args.workload, args.steps, args.warmup, args.replicas, not args.no_graph, fused, ftk)
    extras = {}
    if not args.no_extras:
        other = "hybrid_decode_1m" if args.workload == "csa_decode_128k" else "csa_decode_128k"
        extras[other] = time_decode(other, max(20, args.steps // 2), args.warmup, 0, not args.no_graph, fused, ftk)
        extras["csa_prefill_1m"] = time_prefill(max(2, min(5, args.steps // 40)), 1)
        extras["csa_prefix_1m_host"] = time_prefix()
        extras["pro_projections_decode"] = time_projections()
        for small in ("tiny_csa", "hca_bf16"):
            extras[small] = time_small(small)
        # warm: one cache replica, whose step working set stays in the 256 MB
        # last-level cache between steps (the primary number rotates
        # replicas so that it does not)
        w = time_decode(args.workload, max(20, args.steps // 2), args.warmup, 1, not args.no_graph, fused, ftk)
        extras[args.workload + "_warm"] = {
            "workload": args.workload, "replicas": 1, "tokens_per_s": w["tokens_per_s"],
            "ms_per_step": w["ms_per_step"], "index_launch_ms": w["roofline"]["launch_ms"],
            "index_achieved_gbs": w["roofline"]["achieved"],
            "note": "keys partly served from the last-level cache; not an HBM rate"}
    wd = workload_def(args.workload)
    cpu = cpu_baseline(wd, args.cpu_tokens) if args.cpu_tokens > 0 else None
    if args.cpu_tokens > 0 and not args.no_extras:
        other = "hybrid_decode_1m" if args.workload == "csa_decode_128k" else "csa_decode_128k"
        extras[other]["cpu_baseline"] = cpu_baseline(workload_def(other), args.cpu_tokens)
        extras["csa_prefill_1m"]["cpu_baseline"] = cpu_baseline_prefill()
        for small in ("tiny_csa", "hca_bf16"):
            extras[small]["cpu_baseline"] = cpu_baseline_small(small)
    line = {
        "metric": "CSA decode tokens/s @128K & 1M ctx; achieved HBM GB/s and MFMA % of peak",
        "value": prim["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": prim["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16/fp8 storage, fp32 accumulate", "data": "synthetic",
        "config": {"workload": args.workload, "requests": prim["requests"], "ctx": prim["ctx"],
                   "layers": prim["layers"], "d": prim["d"], "replicas": prim["replicas"], "graph": prim["graph"],
                   "compress_append": fused, "index_topk": ftk},
        "step_hbm_gbs": prim["step_hbm_gbs"], "step_hbm_frac": prim["step_hbm_frac"],
        "step_algorithmic_bytes": prim["step_algorithmic_bytes"],
        "roofline": prim["roofline"],
        "cpu_baseline": cpu,
        "extra": extras,
        "setup_s": prim["setup_s"],
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
