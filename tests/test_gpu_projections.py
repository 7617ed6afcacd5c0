"""The dense projections around the path (csa_linear, csa_grouped_linear and
their compositions: the low-rank query path and the grouped output
projection, [DD] §1.2 Steps 2-3) against the oracle, on the GPU."""
import numpy as np
import pytest
import torch

import synth
from harness import assert_close, to_dev
from long_context_sparse_03_amd import abi
from long_context_sparse_03_amd.projections import output_projection, query_path
from oracle import layer as OL

pytestmark = pytest.mark.gpu

# T rows, d hidden, dc low rank, n_h*c, n_hI*c_I, n_hI, g groups, d_g
SHAPES = {
    "tiny": (5, 512, 256, 1024, 256, 4, 2, 256),
    "pro_decode": (16, 7168, 1024, 65536, 8192, 64, 16, 1024),
    "rows_200": (200, 1024, 256, 2048, 512, 8, 4, 256),
}


def _w(g, n, k):
    return synth.to_bf16_values((synth.normal(g, (n, k)) / np.sqrt(k)).astype(np.float32))


@pytest.mark.parametrize("name", list(SHAPES))
def test_query_path_and_grouped_output(name):
    T, d, dc, nqc, nic, nhi, ng, dg = SHAPES[name]
    print(f"projections {name}", flush=True)
    g = synth.rng(400)
    H = synth.to_bf16_values(synth.normal(g, (T, d)))
    W_DQ, W_UQ, W_UQI, W_w = _w(g, dc, d), _w(g, nqc, dc), _w(g, nic, dc), _w(g, nhi, d)
    Oh = synth.to_bf16_values(synth.normal(g, (T, nqc)))
    W_G = np.stack([_w(g, dg, nqc // ng) for _ in range(ng)])
    W_O = _w(g, d, ng * dg)
    bf = torch.bfloat16
    q, qI, w = query_path(to_dev(H, bf), to_dev(W_DQ, bf), to_dev(W_UQ, bf), to_dev(W_UQI, bf), to_dev(W_w, bf))
    y = output_projection(to_dev(Oh, bf), to_dev(W_G, bf), to_dev(W_O, bf), out_fmt=abi.ACT_F32)
    torch.cuda.synchronize()
    rq, rqI, rw = OL.query_path(H, W_DQ, W_UQ, W_UQI, W_w)
    ry = OL.grouped_output(Oh, W_G, W_O)
    e = [assert_close(q.float().cpu().numpy(), rq, 2e-2, "q"), assert_close(qI.float().cpu().numpy(), rqI, 2e-2, "qI"),
         assert_close(w.cpu().numpy(), rw, 2e-2, "w"), assert_close(y.cpu().numpy(), ry, 2e-2, "y")]
    print(f"  errors q {e[0]:.2e} qI {e[1]:.2e} w {e[2]:.2e} y {e[3]:.2e}", flush=True)


@pytest.mark.parametrize("rows", [3, 130])
def test_linear_fp32(rows):
    """fp32 inputs (fp32 MFMA products, fp32 accumulation): 1e-4 of the
    oracle, single and grouped, fp32 and bf16 outputs."""
    g = synth.rng(401)
    K, N, G = 256, 48, 3
    X = synth.normal(g, (rows, G * K)).astype(np.float32)
    W = (synth.normal(g, (G, N, K)) / np.sqrt(K)).astype(np.float32)
    Y = torch.empty((rows, G * N), device="cuda")
    abi.grouped_linear(abi.ACT_F32, abi.ACT_F32, G, to_dev(X), to_dev(W), Y)
    Y1 = torch.empty((rows, N), dtype=torch.bfloat16, device="cuda")
    abi.linear(abi.ACT_F32, abi.ACT_BF16, to_dev(X[:, :K].copy()), to_dev(W[0]), Y1)
    torch.cuda.synchronize()
    want = np.concatenate([X[:, j * K:(j + 1) * K].astype(np.float64) @ W[j].T.astype(np.float64) for j in range(G)], 1)
    assert_close(Y.cpu().numpy(), want, 1e-4, "grouped fp32")
    assert_close(Y1.float().cpu().numpy(), want[:, :N], 2e-2, "linear bf16 out")


@pytest.mark.parametrize("groups,M,K,N", [(1, 2333, 1024, 1999), (2, 2333, 1024, 1999), (1, 600, 1152, 700)])
def test_linear_bf16_many_rows(groups, M, K, N):
    """bf16 operands, more than 64 rows: the LDS-staged 256 x 160 tiles when
    the output has at least 128 of them, else the 128 x 128 tiles; rows and
    columns that end inside a tile, against the fp64 product of the same bf16
    values; fp32 out at 1e-4, bf16 out at 2e-2."""
    print(f"linear bf16 many rows, {groups} group(s), {M} x {K} x {N}", flush=True)
    g = synth.rng(402)
    X = synth.to_bf16_values(synth.normal(g, (M, groups * K)))
    W = np.stack([_w(g, N, K) for _ in range(groups)])
    bf = torch.bfloat16
    Y = torch.empty((M, groups * N), device="cuda")
    abi.grouped_linear(abi.ACT_BF16, abi.ACT_F32, groups, to_dev(X, bf), to_dev(W, bf), Y)
    Yb = torch.empty((M, groups * N), dtype=bf, device="cuda")
    abi.grouped_linear(abi.ACT_BF16, abi.ACT_BF16, groups, to_dev(X, bf), to_dev(W, bf), Yb)
    torch.cuda.synchronize()
    want = np.concatenate([X[:, j * K:(j + 1) * K].astype(np.float64) @ W[j].T.astype(np.float64)
                           for j in range(groups)], 1)
    e = assert_close(Y.cpu().numpy(), want, 1e-4, "fp32 out")
    eb = assert_close(Yb.float().cpu().numpy(), want, 2e-2, "bf16 out")
    print(f"  errors fp32 {e:.2e} bf16 {eb:.2e}", flush=True)
