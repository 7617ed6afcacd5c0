"""Pins of the CPU oracle against facts fixed outside it (CPU only).

Each test checks an oracle function against something the oracle does not
compute itself: a hand-derived worked example (tests/golden), a closed form,
an invariant of the mathematics, a special case that reduces to a textbook
computation done here by brute force in numpy, or torch's CPU dtype casts.
They are chosen so that a dropped term, a wrong sign or index, or a
transposed operand in the oracle fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from oracle import layer as L

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------

def test_bf16_matches_torch_cast():
    g = np.random.default_rng(1)
    x = np.concatenate([
        g.standard_normal(20000).astype(np.float32) * 10.0,
        np.float32([0.0, -0.0, 1.0, 1.00390625, 1.0078125, 1.01171875, 3.4e38, 1e-40, -1e-40, 65504.0]),
        (g.standard_normal(2000) * 1e-39).astype(np.float32),
    ]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.bf16_bits(x), ref)
    assert np.array_equal(O.bf16_round(x).view(np.uint32) >> 16, ref.astype(np.uint32))


def test_bf16_from_double_is_nearest_even():
    g = np.random.default_rng(2)
    for v in list(g.standard_normal(3000) * 7.0) + [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5e-39, 0.0]:
        got = O.bf16_from_double(v)
        # brute force: neighbours of the truncated bf16 pattern
        f = np.float32(v).view(np.uint32) >> 16
        cands = [np.uint32((int(f) + d) & 0xFFFF) << 16 for d in (-1, 0, 1)]
        vals = [float(np.uint32(cnd).view(np.float32)) for cnd in cands]
        best = min(range(3), key=lambda i: (abs(vals[i] - v), int(cands[i] >> 16) & 1))
        assert got == vals[best] or (v == 0.0 and got == 0.0), (v, got, vals)


def test_e4m3_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got)) and nan.sum() == 2   # 0x7F, 0xFF
    assert np.array_equal(got[~nan], ref[~nan])
    assert O.e4m3_decode(np.uint8(0x7E)) == 448.0


def test_e4m3_encode_matches_torch_in_range_and_saturates():
    g = np.random.default_rng(3)
    x = np.concatenate([g.standard_normal(50000) * 60, g.standard_normal(5000) * 0.01,
                        g.uniform(-448, 448, 5000)]).astype(np.float32)
    x = np.clip(x, -448, 448).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = O.e4m3_encode(x)
    # torch keeps the sign of a zero result; the stored format canonicalises to +0
    zero = O.e4m3_decode(ref) == 0.0
    assert np.array_equal(got[~zero], ref[~zero])
    assert np.all(got[zero] == 0)
    assert list(O.e4m3_encode([449.0, 464.0, 1e6, -1e6])) == [0x7E, 0x7E, 0x7E, 0xFE]
    # every finite code round-trips
    codes = np.array([q for q in range(256) if q not in (0x7F, 0xFF, 0x80)], np.uint8)
    assert np.array_equal(O.e4m3_encode(O.e4m3_decode(codes).astype(np.float32)), codes)


E2M1_GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]   # OCP MX spec, FP4 E2M1 values


def test_e2m1_codes_and_nearest_even():
    for q in range(16):
        assert O.e2m1_decode(np.uint8(q)) == (-1 if q & 8 else 1) * E2M1_GRID[q & 7]
    g = np.random.default_rng(4)
    xs = np.concatenate([g.uniform(-7, 7, 4000), [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -5.0, 6.5, -0.25]])
    for v in xs.astype(np.float32):
        q = int(O.e2m1_encode(np.array([v], np.float32))[0])
        a = min(abs(float(v)), 6.0)
        # brute force nearest grid point, ties to the even code
        best = min(range(8), key=lambda i: (abs(E2M1_GRID[i] - a), i & 1))
        if best == 0:
            assert q == 0
        else:
            assert q == (best | (8 if v < 0 else 0)), (v, q, best)


def test_mx_scale_places_block_max_in_top_binade():
    for amax in [1.0, 0.75, 5.9, 6.0, 7.99, 8.0, 1e-3, 123.0, 3e5]:
        code = O.mx_scale_code(amax)
        scaled = amax / 2.0 ** (code - 127)
        assert 4.0 <= scaled < 8.0, (amax, code)
    assert O.mx_scale_code(0.0) == 127


def test_mxfp4_pack_is_nearest_grid_point_per_block():
    g = np.random.default_rng(5)
    x = (g.standard_normal((6, 128)) * np.array([1, 10, 0.1, 3, 100, 0.5])[:, None]).astype(np.float32)
    codes, scales = O.mxfp4_pack(x)
    deq = O.mxfp4_unpack(codes, scales)
    for i in range(6):
        for b in range(4):
            blk = x[i, 32 * b:32 * b + 32].astype(np.float64)
            s = 2.0 ** (int(scales[i, b]) - 127)
            assert 4.0 <= np.abs(blk).max() / s < 8.0
            for j in range(32):
                a = min(abs(blk[j]) / s, 6.0)
                best = min(range(8), key=lambda k: (abs(E2M1_GRID[k] - a), k & 1))
                assert abs(deq[i, 32 * b + j]) == E2M1_GRID[best] * s
                if best:
                    assert np.sign(deq[i, 32 * b + j]) == np.sign(blk[j])


# ---------------------------------------------------------------------------
# a1: compressor
# ---------------------------------------------------------------------------

def _rand_rows(seed, n, c):
    g = np.random.default_rng(seed)
    return [g.standard_normal((n, c)) for _ in range(4)]


def test_compressor_worked_example():
    d = _gold("compressor_worked.json")
    conv = lambda v: math.log(3) if v == "ln3" else (math.log(2) if v == "ln2" else float(v))
    col = lambda k: np.array([conv(v) for v in d[k]])[:, None]
    E = O.compress(col("Ca"), col("Cb"), col("Za"), col("Zb"), np.zeros((2, 1)), np.zeros((2, 1)), d["m"], True)
    assert np.allclose(E[:, 0], d["expected_entries"], rtol=0, atol=1e-14)


@pytest.mark.parametrize("m,overlap", [(4, True), (3, True), (128, False), (8, False)])
def test_compressor_weights_row_stochastic(m, overlap):
    n, c = 6 * m + (m - 1), 5
    _, _, Za, Zb = _rand_rows(6, n, c)
    g = np.random.default_rng(7)
    Ba, Bb = g.standard_normal((m, c)), g.standard_normal((m, c))
    S = O.compress_weights(Za, Zb, Ba, Bb, m, overlap)
    assert S.shape == (n // m, 2 * m, c)
    assert np.allclose(S.sum(axis=1), 1.0, atol=1e-15, rtol=0)
    assert np.all(S >= 0)
    if overlap:
        assert np.all(S[0, m:] == 0)      # entry 0 has no previous block
        assert np.all(S[1:, m:].sum(axis=1) > 0)
    else:
        assert np.all(S[:, m:] == 0)


def test_compressor_convex_and_constant_rows():
    m, n, c = 4, 40, 6
    Ca, Cb, Za, Zb = _rand_rows(8, n, c)
    g = np.random.default_rng(9)
    Ba, Bb = g.standard_normal((m, c)), g.standard_normal((m, c))
    E = O.compress(Ca, Cb, Za, Zb, Ba, Bb, m, True)
    for i in range(n // m):
        rows = [Ca[m * i:m * i + m]] + ([Cb[m * (i - 1):m * i]] if i else [])
        allr = np.concatenate(rows)
        assert np.all(E[i] <= allr.max(0) + 1e-12) and np.all(E[i] >= allr.min(0) - 1e-12)
    v = g.standard_normal(c)
    const = np.tile(v, (n, 1))
    E2 = O.compress(const, const, Za, Zb, Ba, Bb, m, True)
    assert np.allclose(E2, v, atol=1e-13)


def test_compressor_shift_invariance_per_channel():
    m, n, c = 4, 24, 3
    Ca, Cb, Za, Zb = _rand_rows(10, n, c)
    Ba = np.zeros((m, c)); Bb = np.zeros((m, c))
    shift = np.array([5.0, -7.0, 0.3])
    E1 = O.compress(Ca, Cb, Za, Zb, Ba, Bb, m, True)
    E2 = O.compress(Ca, Cb, Za + shift, Zb + shift, Ba, Bb, m, True)
    assert np.allclose(E1, E2, atol=1e-12)


def test_compressor_zero_logits_give_window_mean_with_exact_indices():
    # C^a_j = j, C^b_j = 1000 + j; with Z = B = 0 entry i is the plain mean of
    # tokens mi..mi+m-1 (a) and 1000 + m(i-1)..m(i-1)+m-1 (b).
    m, n = 4, 23
    Ca = np.arange(n, dtype=np.float64)[:, None]
    Cb = 1000.0 + Ca
    Z = np.zeros((n, 1))
    E = O.compress(Ca, Cb, Z, Z, np.zeros((m, 1)), np.zeros((m, 1)), m, True)
    assert E.shape == (n // m, 1)
    assert E[0, 0] == pytest.approx(np.mean(np.arange(m)), abs=1e-13)
    for i in range(1, n // m):
        a = np.arange(m * i, m * i + m)
        b = 1000.0 + np.arange(m * (i - 1), m * i)
        assert E[i, 0] == pytest.approx((a.sum() + b.sum()) / (2 * m), abs=1e-11)
    # HCA: no overlap, plain mean of each block
    Eh = O.compress(Ca, None, Z, None, np.zeros((m, 1)), None, m, False)
    for i in range(n // m):
        assert Eh[i, 0] == pytest.approx(np.mean(np.arange(m * i, m * i + m)), abs=1e-12)


def test_compressor_bias_rows_pair_with_block_offsets():
    # A huge B^a[r] makes entry i equal C^a of token m*i + r; a huge B^b[r]
    # makes it C^b of token m*(i-1) + r.
    m, n, c = 4, 20, 1
    Ca = np.arange(n, dtype=np.float64)[:, None]
    Cb = -1.0 - Ca
    Z = np.zeros((n, 1))
    for r in range(m):
        Ba = np.zeros((m, 1)); Ba[r] = 200.0
        E = O.compress(Ca, Cb, Z, Z, Ba, np.zeros((m, 1)), m, True)
        assert np.allclose(E[:, 0], m * np.arange(n // m) + r, atol=1e-9)
        Bb = np.zeros((m, 1)); Bb[r] = 200.0
        E = O.compress(Ca, Cb, Z, Z, np.zeros((m, 1)), Bb, m, True)
        assert np.allclose(E[1:, 0], -1.0 - (m * np.arange(n // m - 1) + r), atol=1e-9)


def test_compressor_m1_nonoverlap_is_identity():
    Ca, _, Za, _ = _rand_rows(11, 9, 4)
    E = O.compress(Ca, None, Za, None, np.random.default_rng(1).standard_normal((1, 4)), None, 1, False)
    assert np.allclose(E, Ca, atol=1e-15)


def test_block_accounting_matches_pages():
    k = _gold("constants.json")
    tokens = k["block_raw_tokens"]["value"]
    csa = L.Spec("csa", m=k["csa_m"]["value"], c=512, r=64, n_h=1)
    hca = L.Spec("hca", m=k["hca_m"]["value"], c=512, r=64, n_h=1)
    assert csa.epb == k["csa_entries_per_block"]["value"]
    assert hca.epb == k["hca_entries_per_block"]["value"]
    assert tokens == math.lcm(csa.m, hca.m)
    g = np.random.default_rng(3)
    rows = g.standard_normal((tokens, 2))
    assert O.compress(rows, rows, rows, rows, np.zeros((4, 2)), np.zeros((4, 2)), 4, True).shape[0] == 32
    assert O.compress(rows, None, rows, None, np.zeros((128, 2)), None, 128, False).shape[0] == 1
    assert (2 ** 20) // csa.m == k["csa_entries_at_1M"]["value"]
    assert (2 ** 20) // hca.m == k["hca_entries_at_1M"]["value"]


# ---------------------------------------------------------------------------
# norm and RoPE
# ---------------------------------------------------------------------------

def test_rope_closed_form_and_inverse():
    # r = 2: the single pair rotates by pos * theta^0 = pos radians
    x = np.array([[7.0, 1.0, 0.0]])
    y = O.rope(x, [math.pi / 3], 2, 10000.0)
    assert np.allclose(y, [[7.0, math.cos(math.pi / 3), math.sin(math.pi / 3)]], atol=1e-15)
    # second pair of r = 4 rotates at pos * theta^(-1/2)
    x = np.array([[0.0, 0.0, 1.0, 0.0]])
    y = O.rope(x, [300.0], 4, 100.0)
    assert np.allclose(y[0, 2:], [math.cos(30.0), math.sin(30.0)], atol=1e-14)
    g = np.random.default_rng(12)
    x = g.standard_normal((5, 16))
    pos = g.uniform(0, 1e6, 5)
    back = O.rope(O.rope(x, pos, 8, 10000.0), -pos, 8, 10000.0)
    assert np.allclose(back, x, atol=1e-9)
    assert np.array_equal(O.rope(x, pos, 8, 10000.0)[:, :8], x[:, :8])
    assert np.allclose(np.linalg.norm(O.rope(x, pos, 8, 1e4), axis=1), np.linalg.norm(x, axis=1))


def test_rope_relative_position():
    g = np.random.default_rng(13)
    q, k = g.standard_normal((1, 12)), g.standard_normal((1, 12))
    d1 = (O.rope(q, [1000.0], 8, 1e4) * O.rope(k, [700.0], 8, 1e4)).sum()
    d2 = (O.rope(q, [5300.0], 8, 1e4) * O.rope(k, [5000.0], 8, 1e4)).sum()
    assert d1 == pytest.approx(d2, rel=1e-9)


def test_rmsnorm_properties():
    g = np.random.default_rng(14)
    x = g.standard_normal((4, 64)) * 3
    y = O.rmsnorm(x, np.ones(64), 0.0)
    assert np.allclose((y ** 2).mean(1), 1.0)
    assert np.allclose(O.rmsnorm(5 * x, np.ones(64), 0.0), y)
    gam = g.standard_normal(64)
    assert np.allclose(O.rmsnorm(x, gam, 0.0), y * gam)
    small = np.full((1, 4), 1e-4)
    assert np.allclose(O.rmsnorm(small, np.ones(4), 1e-6), 1e-4 / np.sqrt(1e-8 + 1e-6))


# ---------------------------------------------------------------------------
# a3: indexer
# ---------------------------------------------------------------------------

def test_index_scores_against_matrix_form_and_special_cases():
    g = np.random.default_rng(15)
    T, nh, cI, E = 5, 4, 16, 37
    qI, w, K = g.standard_normal((T, nh, cI)), g.standard_normal((T, nh)), g.standard_normal((E, cI))
    nv = np.array([0, 3, 37, 20, 36], np.int32)
    got = O.index_scores(qI, w, nv, K, 0)
    dots = np.einsum("thc,sc->ths", qI, K)            # matrix form, independent loop order
    ref = (w[:, :, None] * np.maximum(dots, 0)).sum(1).astype(np.float32)
    for t in range(T):
        assert np.allclose(got[t, :nv[t]], ref[t, :nv[t]], rtol=1e-6, atol=1e-6)
        assert np.all(np.isnan(got[t, nv[t]:]))
    # one head, w = 1: ReLU(q.K)
    one = O.index_scores(qI[:, :1], np.ones((T, 1)), np.full(T, E, np.int32), K, 0)
    assert np.allclose(one, np.maximum(dots[:, 0], 0).astype(np.float32), rtol=1e-6, atol=1e-7)
    # linear in w
    two = O.index_scores(qI, 2 * w, np.full(T, E, np.int32), K, 0)
    base = O.index_scores(qI, w, np.full(T, E, np.int32), K, 0)
    assert np.allclose(two, 2 * base, rtol=1e-6, atol=1e-6)
    # all dots negative -> exactly +0
    zero = O.index_scores(-np.abs(qI), w, np.full(T, E, np.int32), np.abs(K), 0)
    assert np.all(zero == 0) and not np.any(np.signbit(zero))
    # bf16 scores are the bf16 rounding of the exact value
    b = O.index_scores(qI, w, np.full(T, E, np.int32), K, 1)
    exact = (w[:, :, None] * np.maximum(dots, 0)).sum(1)
    for t in range(T):
        for s in range(0, E, 5):
            assert b[t, s] == O.bf16_from_double(exact[t, s])


# ---------------------------------------------------------------------------
# a4: top-k
# ---------------------------------------------------------------------------

def test_topk_brute_force_ties_and_padding():
    g = np.random.default_rng(16)
    T, E, k = 7, 300, 40
    sc = np.round(g.standard_normal((T, E)) * 3).astype(np.float32)   # many ties
    nv = np.array([300, 0, 10, 40, 41, 299, 150], np.int32)
    got = O.topk(sc, nv, k)
    for t in range(T):
        V = nv[t]
        order = np.lexsort((np.arange(V), -sc[t, :V].astype(np.float64)))  # score desc, index asc
        want = np.sort(order[:min(k, V)])
        assert np.array_equal(got[t, :len(want)], want)
        assert np.all(got[t, len(want):] == -1)
    storm = O.topk(np.zeros((1, 100), np.float32), [100], 10)
    assert np.array_equal(storm[0], np.arange(10))


# ---------------------------------------------------------------------------
# a5/a6: attention with window and sink
# ---------------------------------------------------------------------------

def test_attention_worked_example():
    d = _gold("attention_worked.json")
    scale = math.log(2) / math.sqrt(2)
    o = O.attend(np.array([d["q_raw"]]), np.ones(2), 0.0, 0.0, 1e4, scale, np.array(d["X"]),
                 np.array([d["sink"]]), 0)
    assert np.allclose(o[0], d["expected_o"], atol=1e-14)


def _dense_sink_attention(q, X, sink, scale):
    """Brute force: softmax over [scale*q X^T, sink] per head, times X."""
    z = scale * q @ X.T                                        # [nh, n]
    zz = np.concatenate([z, sink[:, None]], axis=1)
    zz = zz - zz.max(1, keepdims=True)
    p = np.exp(zz) / np.exp(zz).sum(1, keepdims=True)
    return p[:, :-1] @ X, p[:, -1]


def test_attention_sink_limits():
    g = np.random.default_rng(17)
    nh, c, n = 3, 8, 11
    q, X = g.standard_normal((nh, c)), g.standard_normal((n, c))
    qn = O.rmsnorm(q, np.ones(c), 1e-6)
    # z' = -inf: ordinary softmax
    o = O.attend(q, np.ones(c), 1e-6, 0.0, 1e4, 0.3, X, np.full(nh, -np.inf), 0)
    ref, _ = _dense_sink_attention(qn, X, np.full(nh, -np.inf), 0.3)
    assert np.allclose(o, ref, atol=1e-13)
    # sum p + p_sink = 1: all rows equal v -> o = (1 - p_sink) v
    v = g.standard_normal(c)
    sink = g.standard_normal(nh)
    o = O.attend(q, np.ones(c), 1e-6, 0.0, 1e4, 0.3, np.tile(v, (n, 1)), sink, 0)
    z = 0.3 * qn @ v
    psink = np.exp(sink) / (n * np.exp(z) + np.exp(sink))
    assert np.allclose(o, (1 - psink)[:, None] * v, atol=1e-13)
    # z' -> +inf: output -> 0
    o = O.attend(q, np.ones(c), 1e-6, 0.0, 1e4, 0.3, X, np.full(nh, 800.0), 0)
    assert np.abs(o).max() < 1e-300
    # no rows at all: only the sink, output 0
    assert np.all(O.attend(q, np.ones(c), 1e-6, 0.0, 1e4, 0.3, np.zeros((0, c)), sink, 0) == 0)


def test_attention_relative_position_invariance():
    """Rows rotated at their positions, q at t, output rotated back at -t:
    shifting every position by delta leaves the output unchanged."""
    g = np.random.default_rng(18)
    nh, c, r, n = 2, 16, 8, 9
    q = g.standard_normal((nh, c))
    raw = g.standard_normal((n, c))
    rpos = g.integers(0, 500, n).astype(np.float64)
    t = 600.0
    sink = g.standard_normal(nh)
    outs = []
    for delta in (0.0, 12345.0):
        X = O.rope(O.rmsnorm(raw, np.ones(c), 1e-6), rpos + delta, r, 1e4)
        outs.append(O.attend(q, np.ones(c), 1e-6, t + delta, 1e4, 0.25, X, sink, r))
    assert np.allclose(outs[0], outs[1], atol=1e-9)
    # and a wrong output rotation sign would break it: rotating forward instead differs
    X = O.rope(O.rmsnorm(raw, np.ones(c), 1e-6), rpos, r, 1e4)
    fwd = O.rope(O.rope(outs[0], [t], r, 1e4), [t], r, 1e4)
    assert not np.allclose(fwd, outs[0], atol=1e-3)


def test_layer_reduces_to_dense_causal_mqa():
    """Pin (a): m = 1, no overlap, k = all, no window -> dense causal MQA over
    the normalised, rotated KV rows (brute force with numpy)."""
    g = np.random.default_rng(19)
    n, d, c, r, nh = 12, 8, 8, 4, 3
    spec = L.Spec("csa", m=1, c=c, r=r, n_h=nh, n_hI=2, c_I=4, top_k=n, n_win=1)
    H = g.standard_normal((n, d))
    W = g.standard_normal((d, 2 * c))
    P = H @ W
    Ca = P[:, :c]
    E = O.compress(Ca, None, P[:, c:], None, g.standard_normal((1, c)), None, 1, False)
    assert np.allclose(E, Ca)
    X = O.rope(O.rmsnorm(E, np.ones(c), spec.eps), np.arange(n, dtype=float), r, spec.theta)
    q = g.standard_normal((n, nh, c))
    sink = g.standard_normal(nh)
    sel = np.array([[s if s <= t else -1 for s in range(n)] for t in range(n)], np.int32)
    # window of 1 row = the token itself; drop it by selecting entries < t only
    sel_prev = np.where(sel < np.arange(n)[:, None], sel, -1).astype(np.int32)
    o = O.attend_batch(q, np.ones(c), spec.eps, np.arange(n, dtype=float), spec.theta, spec.scale, X,
                       sel_prev, None, X, 1, sink, r)
    for t in range(n):
        qn = O.rope(O.rmsnorm(q[t], np.ones(c), spec.eps), np.full(nh, float(t)), r, spec.theta)
        ref, _ = _dense_sink_attention(qn, X[:t + 1], sink, spec.scale)
        ref = O.rope(ref, np.full(nh, -float(t)), r, spec.theta)
        assert np.allclose(o[t], ref, atol=1e-12)


def test_dense_hca_uses_visible_entries_and_window():
    g = np.random.default_rng(20)
    spec = L.Spec("hca", m=4, c=8, r=4, n_h=2, n_win=3)
    ent = g.standard_normal((6, 8))
    win = g.standard_normal((25, 8))
    q = g.standard_normal((3, 2, 8))
    pos = np.array([2, 7, 24])
    sink = g.standard_normal(2)
    o = L.attend(spec, q, None, pos, ent, win, sink)
    for i, t in enumerate(pos):
        nv = (t + 1) // 4
        rows = np.concatenate([ent[:nv], win[max(0, t - 2):t + 1]])
        ref = O.attend(q[i], np.ones(8), spec.eps, float(t), spec.theta, spec.scale, rows, sink, 4)
        assert np.allclose(o[i], ref, atol=1e-13)
    assert list(L.visible(spec, pos)) == [0, 2, 6]


# ---------------------------------------------------------------------------
# a2: storage
# ---------------------------------------------------------------------------

def test_fp8_block_fresh_block_matches_torch_scaled_cast():
    spec = L.Spec("csa", m=4, c=64, r=16, n_h=1, kv_fmt="fp8")
    g = np.random.default_rng(21)
    x = g.standard_normal((32, 64)).astype(np.float32)
    blocks, deq = L.store_entries(spec, x, [(0, 32)])
    s = np.float32(np.abs(x[:, :48]).max()) / np.float32(448.0)
    assert blocks[0, :4].view(np.float32)[0] == s
    codes = blocks[0, 64:].reshape(32, 48 + 32)[:, :48]
    ref = torch.from_numpy((x[:, :48] / s).astype(np.float32)).clamp(-448, 448).to(torch.float8_e4m3fn)
    refc = ref.view(torch.uint8).numpy()
    zero = ref.to(torch.float32).numpy() == 0
    assert np.array_equal(codes[~zero], refc[~zero]) and np.all(codes[zero] == 0)
    assert (codes & 0x7F).max() == 0x7E        # the block max hits 448
    rope = blocks[0, 64:].reshape(32, 80)[:, 48:].copy().view(np.uint16)
    assert np.array_equal(rope, torch.from_numpy(x[:, 48:].copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    assert np.allclose(deq[:, :48], x[:, :48], rtol=0.07, atol=s * 2 ** -9)


def test_fp8_block_scale_raise_requantises_earlier_slots():
    spec = L.Spec("csa", m=4, c=64, r=16, n_h=1, kv_fmt="fp8")
    g = np.random.default_rng(22)
    x = g.standard_normal((32, 64)).astype(np.float32)
    x[5:] *= 4.0                                  # later entries are larger
    blocks, deq = L.store_entries(spec, x, [(0, 3), (3, 2), (5, 1), (6, 26)])
    s = blocks[0, :4].view(np.float32)[0]
    assert s == np.float32(np.abs(x[:, :48]).max()) / np.float32(448.0)
    # earlier slots are still within two fp8 rounding steps of their values
    rel = np.abs(deq[:5, :48] - x[:5, :48]) / (np.abs(x[:5, :48]) + s * 2 ** -6)
    assert rel.max() < 2 * 0.0625 + 1e-6
    # no raise when later entries are smaller: earlier codes untouched
    y = g.standard_normal((8, 64)).astype(np.float32)
    y[4:] *= 0.1
    b1, _ = L.store_entries(spec, y[:4], [(0, 4)])
    b2, _ = L.store_entries(spec, y, [(0, 4), (4, 4)])
    assert np.array_equal(b1[0, :64 + 4 * 80], b2[0, :64 + 4 * 80])


# ---------------------------------------------------------------------------
# dense projections around the path
# ---------------------------------------------------------------------------

def test_grouped_output_is_a_block_diagonal_product():
    """The grouped output projection equals one product with the explicit
    block-diagonal matrix of the group projections, then W_O (a different
    formulation: a group index or order mistake, or a transposed block,
    breaks it)."""
    from scipy.linalg import block_diag
    g = np.random.default_rng(5)
    T, n_groups, K, dg, d = 3, 4, 6, 5, 7
    Oh = g.standard_normal((T, n_groups * K))
    W_G = g.standard_normal((n_groups, dg, K))
    W_O = g.standard_normal((d, n_groups * dg))
    want = Oh @ block_diag(*[W_G[j].T for j in range(n_groups)]) @ W_O.T
    got = L.grouped_output(Oh, W_G, W_O, round_mid=False)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_query_path_is_the_low_rank_product():
    """q = (h W_DQ^T) W_UQ^T equals h (W_UQ W_DQ)^T (the low-rank factors
    multiplied first); with c^Q stored in bf16 the difference stays within
    the rounding bound 2^-8 |h W_DQ^T| |W_UQ|^T."""
    g = np.random.default_rng(6)
    T, d, dc, nq, ni, nh = 4, 24, 8, 10, 6, 3
    H = g.standard_normal((T, d))
    W_DQ, W_UQ, W_UQI, W_w = (g.standard_normal(s) for s in [(dc, d), (nq, dc), (ni, dc), (nh, d)])
    q, qI, w = L.query_path(H, W_DQ, W_UQ, W_UQI, W_w, round_mid=False)
    assert np.allclose(q, H @ (W_UQ @ W_DQ).T, rtol=1e-12, atol=1e-12)
    assert np.allclose(qI, H @ (W_UQI @ W_DQ).T, rtol=1e-12, atol=1e-12)
    assert np.allclose(w, np.einsum("td,hd->th", H, W_w), rtol=1e-12, atol=1e-12)
    qr, _, _ = L.query_path(H, W_DQ, W_UQ, W_UQI, W_w, round_mid=True)
    bound = 2.0 ** -8 * np.abs(H @ W_DQ.T) @ np.abs(W_UQ).T
    assert np.all(np.abs(qr - q) <= bound + 1e-15)
    assert np.any(qr != q)                       # the rounding is applied


# ---------------------------------------------------------------------------
# whole-layer composition of the compressor (oracle/layer.py compress_layer)
# and of the query side (csa_queries)
# ---------------------------------------------------------------------------

def _golden_cols(rows):
    return np.array([[math.log(3) if v == "ln3" else math.log(2) if v == "ln2" else float(v) for v in r]
                     for r in rows])


def test_compress_layer_worked_example():
    """Hand-derived composition (tests/golden/compress_layer_worked.json):
    fixes the projection's column order C^a | C^b | Z^a | Z^b, the pairing of
    a- and b-rows, RMSNorm before RoPE, entry i rotated at pos0 + m*i, window
    row j at pos0 + j, and raw (unnormalised, unrotated) indexer keys."""
    d = _gold("compress_layer_worked.json")
    m, c, r, cI = d["m"], d["c"], d["r"], d["c_I"]
    spec = L.Spec("csa", m=m, c=c, r=r, n_h=1, n_hI=1, c_I=cI, top_k=1, eps=0.0, theta=10000.0)
    W = np.concatenate([_golden_cols(d[k]) for k in ("Ca", "Cb", "Za", "Zb")], axis=1)      # [4, 4c]
    W_I = np.concatenate([_golden_cols(d[k]) for k in ("CaI", "CbI", "ZaI", "ZbI")], axis=1)  # [4, 4cI]
    H = np.eye(4)
    z, zI = np.zeros((m, c)), np.zeros((m, cI))
    gam = np.array(d["gamma"])
    E, K, R = L.compress_layer(spec, H, W, z, z, gam, W_I, zI, zI)
    assert np.allclose(E, d["expected_entries"], atol=1e-12)
    assert np.allclose(K, d["expected_keys"], atol=1e-12)
    assert np.allclose(R, d["expected_window"], atol=1e-12)
    E2, K2, R2 = L.compress_layer(spec, H, W, z, z, gam, W_I, zI, zI, pos0=2)
    assert np.allclose(E2, d["pos0_2"]["expected_entries"], atol=1e-12)
    assert np.allclose(K2, d["expected_keys"], atol=1e-12)              # keys carry no position
    assert np.allclose(R2[:2], d["pos0_2"]["expected_window_01"], atol=1e-12)


@pytest.mark.parametrize("kind", ["csa", "hca"])
def test_compress_layer_prefix_and_continuation(kind):
    """Causality: entries, keys and window rows of a prefix do not depend on
    later tokens, and a sequence restarted at pos0 = a (a multiple of m, the
    last 2m rows of history given again, as the decode path does) reproduces
    the full run's later entries, keys and window rows.  For CSA the restart's
    first entry lacks the b-half of the block before it (by design: that
    block's rows are not part of the restarted sequence), so it differs."""
    g = np.random.default_rng(40)
    m = 4 if kind == "csa" else 8
    c, r, cI, dm, n = 16, 4, 8, 24, 72
    spec = L.Spec(kind, m=m, c=c, r=r, n_h=1, n_hI=2, c_I=cI, top_k=4)
    ncol = 4 * c if kind == "csa" else 2 * c
    W = g.standard_normal((dm, ncol)) / math.sqrt(dm)
    W_I = g.standard_normal((dm, 4 * cI)) / math.sqrt(dm) if kind == "csa" else None
    Ba, Bb = g.standard_normal((m, c)), g.standard_normal((m, c)) if kind == "csa" else None
    BaI = g.standard_normal((m, cI)) if kind == "csa" else None
    BbI = g.standard_normal((m, cI)) if kind == "csa" else None
    gam = 1.0 + 0.1 * g.standard_normal(c)
    H = g.standard_normal((n, dm))
    E, K, R = L.compress_layer(spec, H, W, Ba, Bb, gam, W_I, BaI, BbI)
    assert E.shape == (n // m, c) and R.shape == (n, c)
    # prefix: the first n - 8 tokens alone give the same (complete) entries
    Ep, Kp, Rp = L.compress_layer(spec, H[:n - 8], W, Ba, Bb, gam, W_I, BaI, BbI)
    assert np.allclose(Ep, E[:(n - 8) // m], atol=1e-12, rtol=0)
    assert np.allclose(Rp, R[:n - 8], atol=1e-12, rtol=0)
    if kind == "csa":
        assert np.allclose(Kp, K[:(n - 8) // m], atol=1e-12, rtol=0)
    for a in (2 * m, 5 * m):
        Es, Ks, Rs = L.compress_layer(spec, H[a:], W, Ba, Bb, gam, W_I, BaI, BbI, pos0=a)
        first = 1 if kind == "csa" else 0
        assert np.allclose(Es[first:], E[a // m + first:], atol=1e-12, rtol=0)
        assert np.allclose(Rs, R[a:], atol=1e-12, rtol=0)
        if kind == "csa":
            assert np.allclose(Ks[1:], K[a // m + 1:], atol=1e-12, rtol=0)
            assert not np.allclose(Es[0], E[a // m], atol=1e-6)            # b-half missing
            assert not np.allclose(Ks[0], K[a // m], atol=1e-6)
    # a chunked run (prefill n-8, then 8 single tokens, each restarted from the
    # last 2m tokens of history) reproduces every entry and window row
    E_c, R_c = [E[:(n - 8) // m]], [R[:n - 8]]
    for t in range(n - 8, n):
        p0 = (t + 1 - 2 * m) // m * m
        El, _, Rl = L.compress_layer(spec, H[p0:t + 1], W, Ba, Bb, gam, W_I, BaI, BbI, pos0=p0)
        R_c.append(Rl[t - p0:t - p0 + 1])
        if (t + 1) % m == 0:
            E_c.append(El[-1:])
    assert np.allclose(np.concatenate(E_c), E, atol=1e-12, rtol=0)
    assert np.allclose(np.concatenate(R_c), R, atol=1e-12, rtol=0)


def _rot_matrix(c, r, pos, theta):
    """Explicit block-diagonal RoPE matrix: identity on the first c-r channels,
    one 2x2 rotation per pair of the last r channels."""
    M = np.eye(c)
    for j in range(r // 2):
        a = pos * theta ** (-2.0 * j / r)
        i = c - r + 2 * j
        M[i:i + 2, i:i + 2] = [[math.cos(a), -math.sin(a)], [math.sin(a), math.cos(a)]]
    return M


def test_csa_queries_brute_force():
    """The query side of a CSA layer (scores, top-k, attention) against loops
    and explicit matrices: queries with fewer visible entries than k (every
    entry selected, padded with -1) and with more."""
    g = np.random.default_rng(41)
    m, c, r, nh, nhI, cI, k, nwin = 4, 8, 4, 3, 2, 4, 6, 3
    spec = L.Spec("csa", m=m, c=c, r=r, n_h=nh, n_hI=nhI, c_I=cI, top_k=k, n_win=nwin)
    n_tok = 60
    keys = g.standard_normal((n_tok // m, cI))
    ents = g.standard_normal((n_tok // m, c))
    win = g.standard_normal((n_tok, c))
    pos = np.array([2, 9, 22, 23, 45, 59])               # V = 0, 2, 5, 6, 11, 15
    q = g.standard_normal((len(pos), nh, c)).astype(np.float32)
    qI = g.standard_normal((len(pos), nhI, cI)).astype(np.float32)
    w = g.standard_normal((len(pos), nhI)).astype(np.float32)
    sinks = g.standard_normal(nh)
    gq = 1.0 + 0.1 * g.standard_normal(c)
    sc, sel, o = L.csa_queries(spec, q, qI, w, pos, keys, ents, win, sinks, gq)
    for i, t in enumerate(pos):
        V = (t + 1) // m
        ref = np.zeros(V)
        for s in range(V):
            for h in range(nhI):
                ref[s] += float(w[i, h]) * max(0.0, float(np.dot(qI[i, h].astype(np.float64), keys[s])))
        ref32 = ref.astype(np.float32)
        assert np.array_equal(sc[i, :V], ref32) or np.allclose(sc[i, :V], ref32, rtol=2 ** -23, atol=0)
        order = sorted(range(V), key=lambda s: (-float(ref32[s]), s))[:k]
        want = sorted(order) + [-1] * (k - min(k, V))
        assert list(sel[i]) == want
        rows = [ents[s] for s in sorted(order)] + [win[j] for j in range(max(0, t - nwin + 1), t + 1)]
        X = np.array(rows)
        Rt = _rot_matrix(c, r, float(t), spec.theta)
        for h in range(nh):
            qh = q[i, h].astype(np.float64)
            qn = Rt @ (gq * qh / math.sqrt(np.mean(qh * qh) + spec.eps))
            z = X @ qn / math.sqrt(c)
            zmax = max(z.max(), sinks[h])
            p = np.exp(z - zmax) / (np.exp(z - zmax).sum() + math.exp(sinks[h] - zmax))
            oh = Rt.T @ (p @ X)                               # rotated back at -t
            assert np.allclose(o[i, h], oh, atol=1e-12, rtol=0)
