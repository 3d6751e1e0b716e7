"""Pins for the CPU oracle: each check ties an oracle function to something other
than itself -- hand-worked values (tests/golden/, each with its citation), closed
forms, invariants, special cases that reduce to a textbook or library routine,
and brute force on tiny inputs.  Chosen so that a dropped term, a wrong sign or
index, or a transposed operand in oracle.c fails at least one of them."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------- compression
def test_compress_golden_hand_worked():
    g = load("compress_tiny.json")
    out = oracle.compress(np.array(g["A"]), np.array(g["B"]), np.array(g["za"]), np.array(g["zb"]), g["m"])
    np.testing.assert_allclose(out, np.array(g["expected"]), rtol=0, atol=g["tol"])


@pytest.mark.parametrize("m", [1, 2, 4, 7])
def test_compress_uniform_logits_give_window_mean(m):
    rng = np.random.default_rng(1)
    T, c = 6 * m + 3, 5
    A, B = rng.standard_normal((T, c)), rng.standard_normal((T, c))
    z = np.full(T, 0.37)
    out = oracle.compress(A, B, z, z, m)
    assert out.shape == (T // m, c)
    np.testing.assert_allclose(out[0], A[0:m].mean(0), atol=1e-13)  # first block: B half padded
    for j in range(1, T // m):
        want = (A[m * j:m * j + m].sum(0) + B[m * (j - 1):m * j].sum(0)) / (2 * m)
        np.testing.assert_allclose(out[j], want, atol=1e-13)


@pytest.mark.parametrize("stream,r", [("a", 0), ("a", 2), ("b", 1), ("b", 3)])
def test_compress_one_hot_logit_copies_that_row(stream, r):
    """A dominant logit on one slot selects exactly that token of that stream."""
    m, T, c = 4, 24, 3
    rng = np.random.default_rng(2)
    A, B = rng.standard_normal((T, c)), rng.standard_normal((T, c))
    j = 3
    za, zb = np.zeros(T), np.zeros(T)
    tok = m * j + r if stream == "a" else m * (j - 1) + r
    (za if stream == "a" else zb)[tok] = 1e4
    out = oracle.compress(A, B, za, zb, m)
    want = A[tok] if stream == "a" else B[tok]
    np.testing.assert_array_equal(out[j], want)


def test_compress_weights_sum_to_one():
    rng = np.random.default_rng(3)
    m, T, c = 4, 40, 6
    ones = np.ones((T, c))
    out = oracle.compress(ones, ones, rng.standard_normal(T) * 3, rng.standard_normal(T) * 3, m)
    np.testing.assert_allclose(out, 1.0, atol=1e-14)


def test_compress_m1_with_masked_b_is_identity_on_a():
    rng = np.random.default_rng(4)
    T, c = 9, 4
    A, B = rng.standard_normal((T, c)), rng.standard_normal((T, c))
    z = rng.standard_normal(T)
    out = oracle.compress(A, B, z, z, 1, bias_a=np.zeros(1), bias_b=np.array([-np.inf]))
    np.testing.assert_array_equal(out, A)


def test_compress_positional_bias_hand_worked():
    """m=2, c=1, z = 0: bias_a = [0, ln 3], bias_b = [ln 2, 0] -> weights 1:3:2:1 over
    (A[2j], A[2j+1], B[2j-2], B[2j-1])."""
    A = np.array([[1.0], [2.0], [3.0], [4.0]])
    B = np.array([[10.0], [20.0], [30.0], [40.0]])
    z = np.zeros(4)
    out = oracle.compress(A, B, z, z, 2, bias_a=[0.0, math.log(3)], bias_b=[math.log(2), 0.0])
    np.testing.assert_allclose(out[0], [(1 * 1 + 3 * 2) / 4.0], atol=1e-13)
    np.testing.assert_allclose(out[1], [(1 * 3 + 3 * 4 + 2 * 10 + 1 * 20) / 7.0], atol=1e-13)


def test_compress_per_channel_logits():
    """zc == c: each channel has its own softmax; a one-hot on channel 1 only."""
    m, T, c = 2, 8, 3
    rng = np.random.default_rng(5)
    A, B = rng.standard_normal((T, c)), rng.standard_normal((T, c))
    za, zb = np.zeros((T, c)), np.zeros((T, c))
    za[m * 2 + 1, 1] = 1e4
    out = oracle.compress(A, B, za, zb, m)
    assert out[2, 1] == A[m * 2 + 1, 1]
    want0 = (A[4:6, 0].sum() + B[2:4, 0].sum()) / 4
    np.testing.assert_allclose(out[2, 0], want0, atol=1e-13)


def test_compress_token_base_offset_matches_full_rows():
    rng = np.random.default_rng(6)
    m, T, c = 4, 64, 5
    A, B = rng.standard_normal((T, c)), rng.standard_normal((T, c))
    z = rng.standard_normal(T)
    full = oracle.compress(A, B, z, z, m)
    base = 36
    part = oracle.compress(A[base:], B[base:], z[base:], z[base:], m, tok_base=base, entry_begin=10, entry_end=16)
    np.testing.assert_array_equal(part, full[10:16])


# --------------------------------------------------------------------- rmsnorm
def test_rmsnorm_closed_form_and_hand_value():
    x = np.array([[3.0, 4.0]])
    np.testing.assert_allclose(oracle.rmsnorm(x, 0.0), x / math.sqrt(12.5), atol=1e-15)
    rng = np.random.default_rng(7)
    x = rng.standard_normal((5, 64)) * 0.01
    eps = 1e-4
    y = oracle.rmsnorm(x, eps)
    ms = (x ** 2).mean(1)
    np.testing.assert_allclose((y ** 2).mean(1), ms / (ms + eps), rtol=1e-12)


def test_rmsnorm_invariances():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((3, 16))
    np.testing.assert_allclose(oracle.rmsnorm(7.5 * x, 0.0), oracle.rmsnorm(x, 0.0), rtol=1e-13)
    np.testing.assert_allclose(oracle.rmsnorm(-2.0 * x, 0.0), -oracle.rmsnorm(x, 0.0), rtol=1e-13)
    assert np.all(oracle.rmsnorm(np.zeros((2, 8)), 1e-6) == 0.0)
    g = rng.random(16)
    np.testing.assert_allclose(oracle.rmsnorm(x, 1e-6, g), oracle.rmsnorm(x, 1e-6) * g, rtol=1e-13)


def test_visible_count():
    assert oracle.visible(2, 100, 4) == 0      # tokens 0..2: block 0 incomplete
    assert oracle.visible(3, 100, 4) == 1
    assert oracle.visible(2047, 512, 4) == 512
    assert oracle.visible(2047, 100, 4) == 100  # capped by the cache
    assert oracle.visible(1048575, 8192, 128) == 8192


# --------------------------------------------------------------------- indexer
def test_indexer_golden_hand_worked():
    g = load("indexer_tiny.json")
    s = oracle.index_scores(np.array(g["q"]), np.array(g["w"]), np.array(g["K"]))
    np.testing.assert_array_equal(s, np.array(g["expected_scores"]))
    np.testing.assert_array_equal(oracle.topk(s, len(s), g["topk"]), g["expected_topk"])


def test_indexer_single_head_is_relu_dot():
    rng = np.random.default_rng(9)
    q, K = rng.standard_normal((1, 24)), rng.standard_normal((50, 24))
    s = oracle.index_scores(q, [1.0], K)
    np.testing.assert_allclose(s, np.maximum(K @ q[0], 0.0), atol=1e-12)


def test_indexer_zero_weight_removes_head_and_scaling_invariance():
    rng = np.random.default_rng(10)
    q, K = rng.standard_normal((3, 16)), rng.standard_normal((40, 16))
    w = np.array([0.3, 0.0, 0.9])
    s = oracle.index_scores(q, w, K)
    s2 = oracle.index_scores(q[[0, 2]], w[[0, 2]], K)
    np.testing.assert_allclose(s, s2, atol=1e-13)
    s4 = oracle.index_scores(4.0 * q, w, K)         # power of two: exact scaling
    np.testing.assert_array_equal(s4, 4.0 * s)
    np.testing.assert_array_equal(oracle.topk(s4, 40, 7), oracle.topk(s, 40, 7))


# ----------------------------------------------------------------------- top-k
@pytest.mark.parametrize("n,k", [(6, 3), (7, 1), (8, 4), (5, 5)])
def test_topk_brute_force(n, k):
    rng = np.random.default_rng(n * 10 + k)
    s = rng.standard_normal(n)
    got = set(oracle.topk(s, n, k).tolist())
    best = [set(c) for c in itertools.combinations(range(n), k)
            if min(s[list(c)]) > max([s[i] for i in range(n) if i not in c], default=-np.inf)]
    assert len(best) == 1 and got == best[0]


def test_topk_ties_take_lower_index_and_padding():
    s = np.array([1.0, 2.0, 2.0, 2.0, 0.5])
    np.testing.assert_array_equal(oracle.topk(s, 5, 3), [1, 2, 3])
    np.testing.assert_array_equal(oracle.topk(s, 5, 2), [1, 2])
    np.testing.assert_array_equal(oracle.topk(s, 5, 7), [1, 2, 3, 0, 4, -1, -1])
    # only the first V scores are eligible (causal visibility)
    out = oracle.topk(np.array([0.1, 0.2, 9.0, 9.0]), 2, 3)
    np.testing.assert_array_equal(out, [1, 0, -1])


# ------------------------------------------------------------------------- MQA
def test_mqa_golden_hand_worked():
    g = load("mqa_tiny.json")
    out, lse = oracle.sparse_mqa(np.array(g["q"]), np.array(g["kv"]), g["idx"], np.zeros((1, 2)), 0, 0, 0, 1.0, 0.0)
    np.testing.assert_allclose(out, np.array(g["expected_out"]), atol=g["tol"])
    np.testing.assert_allclose(lse, np.array(g["expected_lse"]), atol=g["tol"])


def test_mqa_weights_sum_to_one_identical_rows():
    rng = np.random.default_rng(11)
    row = rng.standard_normal(32)
    kv = np.tile(row, (20, 1))
    kv_raw = np.tile(row, (8, 1))
    q = rng.standard_normal((4, 32)) * 3
    out, _ = oracle.sparse_mqa(q, kv, np.arange(20), kv_raw, 100, 105, 4, 0.3, 1e-6)
    np.testing.assert_allclose(out, np.tile(oracle.rmsnorm(row[None], 1e-6), (4, 1)), atol=1e-13)


def test_mqa_zero_query_gives_mean_of_normalised_rows():
    rng = np.random.default_rng(12)
    kv = rng.standard_normal((30, 16))
    kv_raw = rng.standard_normal((10, 16))
    idx = np.array([3, 7, -1, 12, 29, -1])
    t, raw_base, window = 45, 40, 4   # window tokens 42..45 -> rows 2..5
    out, _ = oracle.sparse_mqa(np.zeros((2, 16)), kv, idx, kv_raw, raw_base, t, window, 0.25, 1e-6)
    rows = np.concatenate([kv[[3, 7, 12, 29]], kv_raw[2:6]])
    want = oracle.rmsnorm(rows, 1e-6).mean(0)
    np.testing.assert_allclose(out, np.tile(want, (2, 1)), atol=1e-13)


def _sdpa(q, kv, scale):
    """torch's scaled_dot_product_attention on CPU in float64, one KV head shared (K = V)."""
    Q = torch.from_numpy(q)[None]          # [1, H, d] -> heads as the query length of one "batch"
    K = torch.from_numpy(kv)[None]
    return torch.nn.functional.scaled_dot_product_attention(Q, K, K, scale=scale)[0].numpy()


def test_m1_reduces_to_plain_mqa():
    """m = 1, B half masked, no window, k >= T: CSA over rmsnorm(A[0..t]) with K = V."""
    rng = np.random.default_rng(13)
    T, d, H, eps, scale = 12, 16, 3, 1e-6, 0.25
    A, B = rng.standard_normal((T, d)), rng.standard_normal((T, d))
    z = rng.standard_normal(T)
    kv = oracle.compress(A, B, z, z, 1, bias_a=[0.0], bias_b=[-np.inf])
    q = rng.standard_normal((H, d))
    t = 9
    V = oracle.visible(t, T, 1)
    idx = oracle.topk(np.arange(V, dtype=float), V, T)       # everything visible
    out, _ = oracle.sparse_mqa(q, kv, idx, np.zeros((1, d)), 0, t, 0, scale, eps)
    want = _sdpa(oracle.rmsnorm(q, eps), oracle.rmsnorm(A[:t + 1], eps), scale)
    np.testing.assert_allclose(out, want, atol=1e-12)


def test_topk_covering_all_entries_equals_dense():
    rng = np.random.default_rng(14)
    N, d, H, m, window = 37, 16, 4, 4, 6
    kv = rng.standard_normal((N, d))
    kv_raw = rng.standard_normal((window, d))
    q = rng.standard_normal((H, d))
    qI, kI, w = rng.standard_normal((2, 8)), rng.standard_normal((N, 8)), rng.random(2)
    t = 4 * 30 + 2                                  # V = 30 < N
    res = oracle.csa_decode_query(q, kv, N, m, qI, w, kI, 64, kv_raw, t - window + 1, t, window, 0.25, 1e-6)
    assert res["visible"] == 30 and np.all(res["idx"][30:] == -1)
    dense, lse_d = oracle.dense_mqa(q, kv, N, m, kv_raw, t - window + 1, t, window, 0.25, 1e-6)
    np.testing.assert_allclose(res["out"], dense, atol=1e-13)
    np.testing.assert_allclose(res["lse"], lse_d, atol=1e-13)


def test_mqa_index_permutation_invariance():
    rng = np.random.default_rng(15)
    kv = rng.standard_normal((50, 32))
    kv_raw = rng.standard_normal((4, 32))
    q = rng.standard_normal((3, 32))
    idx = rng.permutation(50)[:20]
    a, _ = oracle.sparse_mqa(q, kv, idx, kv_raw, 0, 3, 4, 0.2, 1e-6)
    b, _ = oracle.sparse_mqa(q, kv, idx[::-1].copy(), kv_raw, 0, 3, 4, 0.2, 1e-6)
    np.testing.assert_allclose(a, b, atol=1e-13)


def test_window_only_before_first_block_and_short_window():
    """t < m-1: no compressed entry is visible; t < w-1: the window starts at token 0."""
    rng = np.random.default_rng(16)
    d, H = 8, 2
    kv = rng.standard_normal((5, d))
    kv_raw = rng.standard_normal((128, d))
    q = rng.standard_normal((H, d))
    out, _ = oracle.dense_mqa(q, kv, 5, 4, kv_raw, 0, 2, 128, 0.35, 1e-6)
    want = _sdpa(oracle.rmsnorm(q, 1e-6), oracle.rmsnorm(kv_raw[:3], 1e-6), 0.35)
    np.testing.assert_allclose(out, want, atol=1e-12)


def test_sink_joins_the_denominator_only():
    """A sink logit s_h adds exp(s_h) to head h's softmax denominator and nothing to
    its numerator: lse_sink = logaddexp(lse, s); out_sink = out * exp(lse - lse_sink);
    s = -inf changes nothing (techniques map, "Learnable attention sink")."""
    rng = np.random.default_rng(21)
    d, H = 16, 3
    kv = rng.standard_normal((40, d))
    kv_raw = rng.standard_normal((8, d))
    q = rng.standard_normal((H, d))
    idx = np.array([3, 17, -1, 25, 9])
    args = (q, kv, idx, kv_raw, 100, 105, 4, 0.3, 1e-6)
    out, lse = oracle.sparse_mqa(*args)
    sink = np.array([0.5, -2.0, 4.0])
    o_s, l_s = oracle.sparse_mqa(*args, sink=sink)
    np.testing.assert_allclose(l_s, np.logaddexp(lse, sink), rtol=1e-13)
    np.testing.assert_allclose(o_s, out * np.exp(lse - l_s)[:, None], rtol=1e-12, atol=1e-14)
    o_n, l_n = oracle.sparse_mqa(*args, sink=np.full(H, -np.inf))
    np.testing.assert_allclose(o_n, out, rtol=1e-14)
    np.testing.assert_allclose(l_n, lse, rtol=1e-14)
    # dense, and an empty set: out = 0, lse = the sink
    o_d, l_d = oracle.dense_mqa(q, kv, 40, 4, kv_raw, 100, 105, 4, 0.3, 1e-6, sink=sink)
    o_d0, l_d0 = oracle.dense_mqa(q, kv, 40, 4, kv_raw, 100, 105, 4, 0.3, 1e-6)
    np.testing.assert_allclose(l_d, np.logaddexp(l_d0, sink), rtol=1e-13)
    o_e, l_e = oracle.sparse_mqa(q, kv, np.array([-1, -1]), kv_raw, 100, 105, 0, 0.3, 1e-6, sink=sink)
    assert np.all(o_e == 0.0)
    np.testing.assert_allclose(l_e, sink, rtol=1e-15)


def test_window_row_outside_raw_buffer_is_an_error():
    with pytest.raises(ValueError):
        oracle.sparse_mqa(np.ones((1, 4)), np.ones((2, 4)), [0], np.ones((3, 4)), 10, 20, 4, 1.0, 1e-6)


# ----------------------------------------------------------------------- MXFP4
def test_mxfp4_golden_cases():
    g = load("mxfp4_cases.json")
    for case in g["cases"]:
        x = np.zeros(32)
        x[:len(case["x_head"])] = case["x_head"]
        codes, scales = oracle.mxfp4_quantize(x[None])
        assert scales[0, 0] == case["scale_byte"], case["note"]
        deq = oracle.mxfp4_dequantize(codes, scales)[0]
        np.testing.assert_array_equal(deq[:len(case["dequant_head"])], case["dequant_head"], err_msg=case["note"])
        nib = [(codes[0, i // 2] >> (4 * (i % 2))) & 0xF for i in range(len(case["codes_head"]))]
        assert nib == case["codes_head"], case["note"]


def test_mxfp4_grid_values_round_trip():
    rng = np.random.default_rng(17)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    for E in (-5, 0, 3):
        x = rng.choice(grid, size=(8, 32)) * rng.choice([-1, 1], size=(8, 32))
        x[:, 5] = 6.0                                   # pins the block maximum
        x = x * 2.0 ** E
        codes, scales = oracle.mxfp4_quantize(x)
        assert np.all(scales == 127 + E)
        np.testing.assert_array_equal(oracle.mxfp4_dequantize(codes, scales), x)


def test_mxfp4_error_bound_and_monotone():
    rng = np.random.default_rng(18)
    x = rng.standard_normal((64, 128)) * 3
    codes, scales = oracle.mxfp4_quantize(x)
    deq = oracle.mxfp4_dequantize(codes, scales)
    scale = np.repeat(2.0 ** (scales.astype(float) - 127), 32, axis=1)
    err = np.abs(deq - x)
    inside = np.abs(x) <= 6 * scale
    assert np.all(err[inside] <= scale[inside] * 1.0)   # half of the widest grid gap (4..6)
    assert np.all(err[~inside] < scale[~inside] * 2.0)  # saturated: |x| < 8 * 2^E
    assert np.all(np.abs(deq) <= 6 * scale)
    xs = np.sort(x[0, :32])
    xs[-1] = max(xs[-1], 4.0)
    d = oracle.mxfp4_dequantize(*oracle.mxfp4_quantize(xs[None]))[0]
    assert np.all(np.diff(d) >= 0)


# ------------------------------------------------- MXFP4 prefilter + bf16 rescoring
def _rescore_case(seed, V, H=4, d=32):
    rng = np.random.default_rng(seed)
    q, K = rng.standard_normal((H, d)), rng.standard_normal((V, d))
    w = rng.random(H)
    q4 = oracle.mxfp4_dequantize(*oracle.mxfp4_quantize(q))
    k4 = oracle.mxfp4_dequantize(*oracle.mxfp4_quantize(K))
    return q, K, w, q4, k4


def test_rescored_with_every_entry_a_candidate_is_the_plain_selection():
    """cand >= V: every visible entry is rescored, so the result is the plain top-k of
    the rescoring scores."""
    q, K, w, q4, k4 = _rescore_case(31, 50)
    got, cands, _ = oracle.index_topk_rescored(q4, w, k4, q, K, 50, 64, 7)
    np.testing.assert_array_equal(cands, np.arange(50))
    want = np.sort(oracle.topk(oracle.index_scores(q, w, K), 50, 7))
    np.testing.assert_array_equal(got, want)


def test_rescored_with_k_candidates_is_the_prefilter_selection():
    """cand == k: the rescoring only reorders the prefilter's set."""
    q, K, w, q4, k4 = _rescore_case(32, 60)
    got, _, _ = oracle.index_topk_rescored(q4, w, k4, q, K, 60, 9, 9)
    np.testing.assert_array_equal(got, np.sort(oracle.topk(oracle.index_scores(q4, w, k4), 60, 9)))


@pytest.mark.parametrize("V,cand,k", [(40, 12, 5), (30, 8, 8), (6, 12, 9)])
def test_rescored_brute_force(V, cand, k):
    """Explicit sorts by (score desc, index asc) of explicitly summed scores."""
    q, K, w, q4, k4 = _rescore_case(V + cand, V)

    def score(qq, kk):
        return sum(w[h] * max(0.0, float(np.dot(qq[h], kk))) for h in range(len(w)))

    first = sorted(range(V), key=lambda i: (-score(q4, k4[i]), i))[:cand]
    second = sorted(first, key=lambda i: (-score(q, K[i]), i))[:k]
    want = sorted(second) + [-1] * (k - len(second))
    got, cands, s16 = oracle.index_topk_rescored(q4, w, k4, q, K, V, cand, k)
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(cands, sorted(first))
    np.testing.assert_allclose(s16, [score(q, K[i]) for i in sorted(first)], rtol=1e-12)


# ------------------------------------------------------------------------- FP8
def test_fp8_e4m3_hand_values():
    """E4M3 (bias 7, 3 mantissa bits, no infinity, max 448): values worked by hand from
    the format definition, including subnormals, both tie directions, saturation."""
    cases = [(0.0, 0x00), (-0.0, 0x80), (2.0 ** -9, 0x01), (7 * 2.0 ** -9, 0x07), (2.0 ** -6, 0x08),
             (1.0, 0x38), (1.125, 0x39), (1.875, 0x3F), (2.0, 0x40), (240.0, 0x77), (448.0, 0x7E),
             (-3.0, 0xC4),                       # 1.5 * 2^1: e = 8, m = 4
             (1.0625, 0x38),                     # tie between 1.0 (m 0) and 1.125 (m 1): even
             (1.1875, 0x3A),                     # tie between 1.125 (m 1) and 1.25 (m 2): even
             (2.0 ** -10, 0x00),                 # tie between 0 and the smallest subnormal
             (3 * 2.0 ** -10, 0x02),             # tie between codes 1 and 2
             (460.0, 0x7E), (1e6, 0x7E), (-1e6, 0xFE)]   # saturation
    x = np.array([c[0] for c in cases])
    np.testing.assert_array_equal(oracle.fp8_quantize(x), np.array([c[1] for c in cases], dtype=np.uint8))
    np.testing.assert_array_equal(oracle.fp8_dequantize(np.array([0x01, 0x7E, 0xC4, 0x3A], dtype=np.uint8)),
                                  [2.0 ** -9, 448.0, -3.0, 1.25])


def test_fp8_round_trip_and_error_bound():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)   # every finite code
    np.testing.assert_array_equal(oracle.fp8_quantize(oracle.fp8_dequantize(codes)), codes)
    vals = np.sort(oracle.fp8_dequantize(codes[codes < 0x80]))
    assert np.all(np.diff(vals) > 0) and vals[-1] == 448.0
    rng = np.random.default_rng(22)
    x = rng.standard_normal(20000) * np.exp(rng.uniform(-8, 5, 20000))
    q = oracle.fp8_dequantize(oracle.fp8_quantize(x))
    a = np.minimum(np.abs(x), 448.0)
    # half a quantum: 2^(floor(log2 a) - 4) in the normal range, 2^-10 below 2^-6
    half = np.where(a >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 4), 2.0 ** -10)
    assert np.all(np.abs(np.abs(q) - a) <= half * (1 + 1e-12))
    assert np.all(np.sign(q[q != 0]) == np.sign(x[q != 0]))


# --------------------------------------------------------- rope-conjugate output
def _rope_cs(theta):
    """cos and sin per rope dim: each of the 32 pair angles on both dims of its pair."""
    th = np.repeat(theta, 2)
    return np.concatenate([np.cos(th), np.sin(th)])


def _rotate_complex(x, theta):
    """RoPE of the trailing 64 dims written as complex multiplication: the interleaved
    pair (x_{2j}, x_{2j+1}) is x_{2j} + 1j x_{2j+1}, multiplied by exp(1j theta_j)."""
    y = np.array(x, dtype=np.float64)
    z = (y[..., -64::2] + 1j * y[..., -63::2]) * np.exp(1j * theta)
    y[..., -64::2], y[..., -63::2] = z.real, z.imag
    return y


def test_rope_conjugate_undoes_the_rotation():
    rng = np.random.default_rng(41)
    x = rng.standard_normal((3, 512))
    theta = rng.uniform(-40, 40, 32)
    y = oracle.rope_conjugate(_rotate_complex(x, theta), _rope_cs(theta))
    np.testing.assert_allclose(y, x, atol=1e-12)
    # it is the rotation by -theta, and the 448 leading dims pass through unchanged
    np.testing.assert_allclose(oracle.rope_conjugate(x, _rope_cs(theta)), _rotate_complex(x, -theta), atol=1e-12)
    np.testing.assert_array_equal(oracle.rope_conjugate(x, _rope_cs(theta))[:, :448], x[:, :448])


def test_rope_conjugate_quarter_turn_by_hand():
    """theta = pi/2 (cos 0, sin 1): the conjugate turns each interleaved pair (a, b)
    into (b, -a); a perturbation of one rotated dim moves that dim's pair only."""
    x = np.arange(2 * 96, dtype=np.float64).reshape(2, 96) + 1
    cs = np.concatenate([np.zeros(64), np.ones(64)])
    y = oracle.rope_conjugate(x, cs)
    np.testing.assert_array_equal(y[:, :32], x[:, :32])
    np.testing.assert_array_equal(y[:, 32::2], x[:, 33::2])
    np.testing.assert_array_equal(y[:, 33::2], -x[:, 32::2])
    x2 = x.copy()
    x2[:, 32] += 1.0
    moved = np.nonzero(np.any(oracle.rope_conjugate(x2, cs) != y, axis=0))[0]
    np.testing.assert_array_equal(moved, [33])


def test_rope_conjugate_of_attention_over_rotated_inputs():
    """q and every attended row rotated by one common angle (one position): the logits and
    the RMS norms do not change, so the conjugated output is the attention output over
    the unrotated inputs."""
    rng = np.random.default_rng(42)
    H, d, N, k, window = 4, 128, 40, 12, 6
    q = rng.standard_normal((H, d))
    kv = rng.standard_normal((N, d))
    raw = rng.standard_normal((window + 2, d))
    idx = np.sort(rng.choice(N, size=k, replace=False)).astype(np.int32)
    theta = rng.uniform(-3, 3, 32)
    base, t = 100, 100 + window
    o0, l0 = oracle.sparse_mqa(q, kv, idx, raw, base, t, window, 1 / np.sqrt(d), 1e-6)
    o1, l1 = oracle.sparse_mqa(_rotate_complex(q, theta), _rotate_complex(kv, theta), idx,
                               _rotate_complex(raw, theta), base, t, window, 1 / np.sqrt(d), 1e-6)
    np.testing.assert_allclose(l1, l0, atol=1e-12)
    assert np.abs(o1 - o0).max() > 1e-3                     # the rotation is visible in the output
    np.testing.assert_allclose(oracle.rope_conjugate(o1, _rope_cs(theta)), o0, atol=1e-12)
