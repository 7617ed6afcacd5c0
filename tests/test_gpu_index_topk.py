"""The fused index + top-k (csa_index_topk) against csa_index_scores followed
by csa_topk_select on the same inputs: scores, visible counts and selections
bit for bit.  The whole-layer tests (test_gpu_layers, test_gpu_invariance,
test_gpu_prefix) run the same comparison inside every CSA call and check the
selections against the oracle end to end; the cases here add what those do
not reach: tie storms (keys with few distinct values, so many scores are
equal at the threshold), rows with fewer visible entries than k (and none),
rows longer than one pass of the selection kernel (the multi-pass path),
ragged multi-token calls (the prefill-shaped indexer launch) and every key
format."""
import numpy as np
import pytest
import torch

import synth
from harness import append_entries, batch, to_dev
from long_context_sparse_03_amd import abi, presets
from long_context_sparse_03_amd.layer import LayerState

pytestmark = pytest.mark.gpu

CASES = {
    # name: (layer, per request (cached entries, start position, new tokens), tie storm)
    "flash_bf16_decode": (presets.csa_flash_decode(), [(32768, 131072, 1), (5000, 20003, 1), (100, 403, 1),
                                                       (0, 2, 1), (513, 2053, 1)], False),
    "flash_bf16_ties": (presets.csa_flash_decode(), [(9000, 36000, 1), (2000, 8001, 2), (700, 2801, 3)], True),
    "flash_bf16_prefill": (presets.csa_flash_decode(win_cap=512), [(3000, 11900, 100), (600, 2390, 33)], False),
    "flash_bf16_prefill_ties": (presets.csa_flash_decode(win_cap=512), [(5000, 19950, 64)], True),
    "pro_mxfp4_decode": (presets.csa_pro(idx_fmt=abi.IDX_MXFP4), [(60000, 240000, 1), (1023, 4093, 1),
                                                                  (2048, 8190, 2), (0, 0, 1)], False),
    "pro_mxfp4_ties": (presets.csa_pro(idx_fmt=abi.IDX_MXFP4), [(50000, 200001, 1), (3000, 12000, 3)], True),
    "pro_bf16_long_rows": (presets.csa_pro(), [(90000, 360000, 1), (45000, 180002, 2)], False),
    "tiny_fp32": (presets.tiny_csa_fp32(), [(512, 2050, 1), (40, 163, 2), (3, 14, 1)], False),
}


@pytest.mark.parametrize("name", list(CASES))
def test_index_topk_equals_two_calls(name):
    desc, reqs, ties = CASES[name]
    print(f"index_topk {name}", flush=True)
    g = synth.rng(400)
    n_req = len(reqs)
    E = [e for e, _, _ in reqs]
    start = [s for _, s, _ in reqs]
    n_new = [n for _, _, n in reqs]
    E_all = [(s + n) // desc.m for s, n in zip(start, n_new)]
    epb = desc.block_tokens // desc.m
    nb = max(max(1, (e + epb - 1) // epb) for e in E_all)
    bt = synth.block_table(g, n_req, nb)
    st = LayerState(desc, n_req, bt.size)
    keys = [synth.normal(g, (e, desc.c_idx)) for e in E_all]
    if ties:                                   # few distinct key values: many equal scores
        keys = [np.round(k) for k in keys]
    ents = [np.zeros((e, desc.c), np.float32) for e in E_all]
    append_entries(st, desc, bt, ents, [0] * n_req, keys)
    bi = batch(start, n_new, bt)
    T = sum(n_new)
    qd = synth.queries(g, T, 1, 1, desc.n_idx_heads, desc.c_idx)
    qI, w = qd["qI"], qd["w"]
    if ties:
        qI, w = np.round(qI), np.round(w * 8) / 8
    adt = torch.bfloat16 if desc.act_fmt == abi.ACT_BF16 else torch.float32
    qI_d, w_d = to_dev(qI, adt), to_dev(w)
    ld = (bi.batch.max_ctx // desc.m + 7) // 8 * 8 + 8
    sdt = torch.bfloat16 if desc.score_fmt == abi.ACT_BF16 else torch.float32
    k = desc.top_k
    sc1, sc2 = torch.zeros((T, ld), dtype=sdt, device="cuda"), torch.zeros((T, ld), dtype=sdt, device="cuda")
    nv1, nv2 = torch.empty(T, dtype=torch.int32, device="cuda"), torch.empty(T, dtype=torch.int32, device="cuda")
    sel1 = torch.full((T, k), -5, dtype=torch.int32, device="cuda")
    sel2 = torch.full((T, k), -6, dtype=torch.int32, device="cuda")
    st.index(bi, T, qI_d, w_d, sc1, ld, nv1)
    st.topk(T, sc1, ld, nv1, sel1)
    st.index_topk(bi, T, qI_d, w_d, sc2, ld, nv2, sel2)
    torch.cuda.synchronize()
    iv = torch.int16 if sdt == torch.bfloat16 else torch.int32
    assert torch.equal(nv1, nv2)
    assert torch.equal(sc1.view(iv), sc2.view(iv))
    s1, s2 = sel1.cpu().numpy(), sel2.cpu().numpy()
    nv = nv1.cpu().numpy()
    for r in range(T):
        assert np.array_equal(s1[r], s2[r]), f"row {r} (V={nv[r]}): selections differ"
        cnt = min(k, int(nv[r]))
        assert np.all(np.diff(s2[r, :cnt]) > 0) and np.all(s2[r, cnt:] == -1)
    if ties:
        # the threshold really was tied: some row's k-th score equals the (k+1)-th
        sc = sc1.float().cpu().numpy()
        tied = 0
        for r in range(T):
            V = int(nv[r])
            if V > k:
                srt = np.sort(sc[r, :V])[::-1]
                tied += srt[k - 1] == srt[k]
        assert tied > 0
    print(f"  {T} queries: identical scores and selections (V up to {nv.max()})", flush=True)


def test_index_topk_rejects_misaligned_rows():
    desc = presets.csa_flash_decode()
    bt = np.zeros((1, 4), np.int32)
    st = LayerState(desc, 1, 4)
    bi = batch([100], [1], bt)
    sc = torch.zeros((1, 36), dtype=torch.bfloat16, device="cuda")
    nv = torch.empty(1, dtype=torch.int32, device="cuda")
    sel = torch.empty((1, desc.top_k), dtype=torch.int32, device="cuda")
    q = torch.zeros((1, desc.n_idx_heads, desc.c_idx), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((1, desc.n_idx_heads), device="cuda")
    with pytest.raises(abi.CSAError) as e:
        st.index_topk(bi, 1, q, w, sc, 36, nv, sel)            # ld % 8 != 0
    assert e.value.code == -1
