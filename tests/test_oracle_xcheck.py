"""Cross-checks of the oracle against an independent implementation of DeepSeek-V4's
attention: the PyTorch model code shipped with the installed `transformers` package
(`transformers.models.deepseek_v4`), built here at tiny sizes with random weights and
run on the CPU.  The pages quote lines of that code ("DeepSeek-V4-Pro" techniques map,
"Partial RoPE" and "Gated attention output") without printing all of it; these tests
settle the readings the pages leave open where that code fixes them:

  * the rope-conjugate rotation turns interleaved pairs (2j, 2j+1), one angle a pair;
  * the CSA pooling: per-channel gates (zc = c), the lagging stream over the previous
    block, entry 0 without it, positional biases added to the gates, RMSNorm of the
    pooled entry, RoPE at the position of the entry's first current-block token;
  * the HCA pooling of the module is non-overlapping and single-stream: the oracle's
    two-stream pooling with the lagging half masked (bias_b = -inf);
  * the lightning indexer: sum_h w_h ReLU(q_h . k_s) up to positive constants, the
    causal threshold floor((t+1)/m), top-k with -1 for invalid slots;
  * the core attention with a per-head sink logit in the softmax denominator.

The module computes in float32, so agreement is to float32 rounding.  Nothing here
runs on the GPU and nothing in the library uses this module.
"""
import numpy as np
import pytest
import torch

import oracle

M = pytest.importorskip("transformers.models.deepseek_v4.modeling_deepseek_v4")
Cfg = pytest.importorskip("transformers.models.deepseek_v4.configuration_deepseek_v4").DeepseekV4Config

EPS = 1e-6


def _config(head_dim=16, hidden=64, idx_heads=4, idx_dim=8, m=4, m_hca=8, q_lora=32, topk=4):
    # partial_rotary_factor 0.125: the trailing head_dim / 8 dims are rotated (64 of 512)
    return Cfg(hidden_size=hidden, head_dim=head_dim, num_attention_heads=4, q_lora_rank=q_lora,
               index_n_heads=idx_heads, index_head_dim=idx_dim, index_topk=topk, num_hidden_layers=2,
               compress_rates={"compressed_sparse_attention": m, "heavily_compressed_attention": m_hca},
               o_groups=2, o_lora_rank=8, vocab_size=32, n_routed_experts=4, num_experts_per_tok=2,
               moe_intermediate_size=8, rms_norm_eps=EPS)


def _select(out_features, in_features, start):
    """Weight of a Linear that copies input features start .. start + out_features - 1."""
    w = torch.zeros(out_features, in_features)
    w[torch.arange(out_features), start + torch.arange(out_features)] = 1.0
    return w


@pytest.fixture
def rope_off(monkeypatch):
    """RoPE as the identity inside the module (the pooling and norm alone)."""
    monkeypatch.setattr(M, "apply_rotary_pos_emb", lambda x, cos, sin, unsqueeze_dim=1: x)


# ------------------------------------------------------------------- rope-conjugate
def test_rope_conjugate_matches_v4_rotary():
    """oracle_rope_conjugate == V4's apply_rotary_pos_emb with the sine negated, on cos
    and sin from V4's own rotary embedding at several positions (64 of 512 dims)."""
    cfg = _config(head_dim=512, hidden=512)
    rot = M.DeepseekV4RotaryEmbedding(cfg)
    rng = np.random.default_rng(3)
    H = 6
    x = rng.standard_normal((H, 512)).astype(np.float32)
    for pos in (0, 1, 7, 4093, 1048575):
        cos, sin = rot(torch.zeros(1), torch.tensor([[pos]]), layer_type="compress")   # [1, 1, 32]
        assert cos.shape[-1] == 32
        want = M.apply_rotary_pos_emb(torch.from_numpy(x)[None, None], cos, -sin)[0, 0].double().numpy()
        cs = np.concatenate([np.repeat(cos[0, 0].double().numpy(), 2), np.repeat(sin[0, 0].double().numpy(), 2)])
        got = oracle.rope_conjugate(x, cs)
        np.testing.assert_allclose(got, want, rtol=0, atol=2e-6 * np.abs(x).max())
        np.testing.assert_array_equal(got[:, :448], x[:, :448])


def test_rope_conjugate_pairs_are_interleaved_in_v4():
    """Perturbing rotated dim 448 changes output dims 448 and 449 only, in the module and
    in the oracle."""
    cfg = _config(head_dim=512, hidden=512)
    cos, sin = M.DeepseekV4RotaryEmbedding(cfg)(torch.zeros(1), torch.tensor([[12345]]), layer_type="compress")
    x = np.random.default_rng(4).standard_normal((1, 512)).astype(np.float32)
    x2 = x.copy()
    x2[0, 448] += 1.0
    f = lambda v: M.apply_rotary_pos_emb(torch.from_numpy(v)[None, None], cos, -sin)[0, 0].numpy()
    moved = np.nonzero(f(x2)[0] != f(x)[0])[0]
    np.testing.assert_array_equal(moved, [448, 449])
    cs = np.concatenate([np.repeat(cos[0, 0].double().numpy(), 2), np.repeat(sin[0, 0].double().numpy(), 2)])
    moved_o = np.nonzero(np.abs(oracle.rope_conjugate(x2, cs) - oracle.rope_conjugate(x, cs))[0] > 1e-12)[0]
    np.testing.assert_array_equal(moved_o, [448, 449])


# ------------------------------------------------------------------------ compression
def _csa_compressor_case(c, m, T, seed):
    """A CSA compressor whose projections copy slices of the hidden state:
    hidden = [B rows | A rows | B gates | A gates] (module: Ca = lagging stream,
    Cb = current block)."""
    cfg = _config(head_dim=c, hidden=4 * c, m=m)
    comp = M.DeepseekV4CSACompressor(cfg)
    rng = np.random.default_rng(seed)
    with torch.no_grad():
        comp.kv_proj.weight.copy_(_select(2 * c, 4 * c, 0))
        comp.gate_proj.weight.copy_(_select(2 * c, 4 * c, 2 * c))
        comp.position_bias.copy_(torch.from_numpy(rng.standard_normal((m, 2 * c)).astype(np.float32)))
        comp.kv_norm.weight.fill_(1.0)
    h = rng.standard_normal((T, 4 * c)).astype(np.float32)
    return comp, h


def _module_pool(comp, h, T):
    hs = torch.from_numpy(h)[None]
    pos = torch.arange(T)[None]
    with torch.no_grad():
        ckv, _ = comp(hs, torch.zeros(1, T, 32), pos, None, 0)
    return ckv[0, 0].double().numpy()


def test_compress_matches_v4_csa_compressor(rope_off):
    """oracle_compress with per-channel gates, A = the module's current-block stream (Cb),
    B = its lagging stream (Ca), biases from position_bias, then RMSNorm, equals the
    module's compressed entries (RoPE set aside)."""
    c, m, T = 16, 4, 37   # 9 entries; 1 token left over
    comp, h = _csa_compressor_case(c, m, T, seed=5)
    got = _module_pool(comp, h, T)
    pb = comp.position_bias.detach().double().numpy()
    A, Bv, za, zb = h[:, c:2 * c], h[:, :c], h[:, 3 * c:], h[:, 2 * c:3 * c]
    pooled = oracle.compress(A, Bv, za, zb, m, bias_a=pb[:, c:], bias_b=pb[:, :c])
    assert pooled.shape == got.shape == (T // m, c)
    want = oracle.rmsnorm(pooled, EPS)
    np.testing.assert_allclose(want, got, rtol=0, atol=1e-5)
    # a swapped reading of the two streams is far off
    swapped = oracle.rmsnorm(oracle.compress(Bv, A, zb, za, m, bias_a=pb[:, :c], bias_b=pb[:, c:]), EPS)
    assert np.abs(swapped - got).max() > 0.1


def test_compressed_entry_rope_position_in_v4():
    """With RoPE on, the module's entry j is the pooled, normalised entry rotated (V4's
    interleaved rotation of the trailing dims) at position m*j, the first token of the
    entry's current block; the conjugate rotation at that position recovers it."""
    c, m, T = 64, 4, 40
    comp, h = _csa_compressor_case(c, m, T, seed=6)
    got = _module_pool(comp, h, T)
    pb = comp.position_bias.detach().double().numpy()
    want = oracle.rmsnorm(oracle.compress(h[:, c:2 * c], h[:, :c], h[:, 3 * c:], h[:, 2 * c:3 * c], m,
                                          bias_a=pb[:, c:], bias_b=pb[:, :c]), EPS)
    rot = comp.rotary_emb
    rd = c // 8
    for j in range(T // m):
        cos, sin = rot(torch.zeros(1), torch.tensor([[m * j]]), layer_type="compress")
        assert cos.shape[-1] == rd // 2
        # pad the rotated slice to the 64-dim layout the oracle takes: dims before it untouched
        xx = np.zeros((1, 64))
        xx[0, 64 - c:] = got[j]
        cs = np.concatenate([np.ones(64), np.zeros(64)])
        cs[64 - rd:64] = np.repeat(cos[0, 0].double().numpy(), 2)
        cs[128 - rd:] = np.repeat(sin[0, 0].double().numpy(), 2)
        back = oracle.rope_conjugate(xx, cs)[0, 64 - c:]
        np.testing.assert_allclose(back, want[j], rtol=0, atol=2e-5)
        if j > 0:   # at another position it does not come back
            cos2, sin2 = rot(torch.zeros(1), torch.tensor([[m * j + 1]]), layer_type="compress")
            cs2 = cs.copy()
            cs2[64 - rd:64] = np.repeat(cos2[0, 0].double().numpy(), 2)
            cs2[128 - rd:] = np.repeat(sin2[0, 0].double().numpy(), 2)
            assert np.abs(oracle.rope_conjugate(xx, cs2)[0, 64 - c:] - want[j]).max() > 1e-3


def test_hca_compressor_is_the_masked_single_stream_case(rope_off):
    """V4's HCA compressor pools non-overlapping windows of m' tokens from one stream with
    per-channel gates: oracle_compress with the lagging half masked (bias_b = -inf)."""
    c, mh, T = 16, 8, 50
    cfg = _config(head_dim=c, hidden=2 * c, m_hca=mh)
    comp = M.DeepseekV4HCACompressor(cfg)
    rng = np.random.default_rng(7)
    with torch.no_grad():
        comp.kv_proj.weight.copy_(_select(c, 2 * c, 0))
        comp.gate_proj.weight.copy_(_select(c, 2 * c, c))
        comp.position_bias.copy_(torch.from_numpy(rng.standard_normal((mh, c)).astype(np.float32)))
        comp.kv_norm.weight.fill_(1.0)
    h = rng.standard_normal((T, 2 * c)).astype(np.float32)
    with torch.no_grad():
        ckv, _ = comp(torch.from_numpy(h)[None], torch.zeros(1, T, 32), torch.arange(T)[None], None, 0)
    got = ckv[0, 0].double().numpy()
    pb = comp.position_bias.detach().double().numpy()
    pooled = oracle.compress(h[:, :c], h[:, :c], h[:, c:], h[:, c:], mh, bias_a=pb,
                             bias_b=np.full((mh, c), -np.inf))
    np.testing.assert_allclose(oracle.rmsnorm(pooled, EPS), got, rtol=0, atol=1e-5)


# --------------------------------------------------------------------------- indexer
def test_indexer_scorer_matches_v4_up_to_positive_constants():
    """DeepseekV4IndexerScorer = d^-1/2 * H^-1/2 * oracle_index_scores (weights taken as
    given): the same ranking."""
    H, dI, T = 4, 8, 30
    cfg = _config(hidden=H, idx_heads=H, idx_dim=dI)
    sc = M.DeepseekV4IndexerScorer(cfg)
    with torch.no_grad():
        sc.weights_proj.weight.copy_(torch.eye(H))
    rng = np.random.default_rng(8)
    q = rng.standard_normal((H, dI)).astype(np.float32)
    K = rng.standard_normal((T, dI)).astype(np.float32)
    w = rng.random(H).astype(np.float32)
    with torch.no_grad():
        got = sc(torch.from_numpy(q)[None, None], torch.from_numpy(K)[None], torch.from_numpy(w)[None, None])
    got = got[0, 0].double().numpy()
    want = oracle.index_scores(q, w, K)
    np.testing.assert_allclose(got, want * dI ** -0.5 * H ** -0.5, rtol=1e-5, atol=1e-6)
    np.testing.assert_array_equal(np.argsort(-got, kind="stable"), np.argsort(-want, kind="stable"))


def test_indexer_selection_matches_v4(rope_off):
    """The module's whole lightning indexer over T prefill tokens (index keys compressed
    by its own two-stream pooling and RMS-normalised, causal threshold, top-k, -1 for
    invalid slots) selects the oracle's sets: oracle_compress -> rmsnorm of the keys ->
    oracle_index_scores -> oracle_topk with V(t) = min(N, floor((t+1)/m))."""
    H, dI, m, T, k = 4, 8, 4, 43, 5
    hidden = 4 * dI + H
    cfg = _config(hidden=hidden, idx_heads=H, idx_dim=dI, m=m, q_lora=H * dI, topk=k)
    ix = M.DeepseekV4Indexer(cfg)
    rng = np.random.default_rng(9)
    with torch.no_grad():
        ix.kv_proj.weight.copy_(_select(2 * dI, hidden, 0))
        ix.gate_proj.weight.copy_(_select(2 * dI, hidden, 2 * dI))
        ix.position_bias.copy_(torch.from_numpy(rng.standard_normal((m, 2 * dI)).astype(np.float32)))
        ix.kv_norm.weight.fill_(1.0)
        ix.q_b_proj.weight.copy_(torch.eye(H * dI))
        ix.scorer.weights_proj.weight.copy_(_select(H, hidden, 4 * dI))
    h = rng.standard_normal((T, hidden)).astype(np.float32)
    h[:, 4 * dI:] = rng.random((T, H))          # head weights U[0, 1)
    qres = rng.standard_normal((T, H * dI)).astype(np.float32)
    with torch.no_grad():
        got = ix(torch.from_numpy(h)[None], torch.from_numpy(qres)[None], torch.arange(T)[None], None, 0)
    got = got[0].numpy()
    pb = ix.position_bias.detach().double().numpy()
    keys = oracle.rmsnorm(oracle.compress(h[:, dI:2 * dI], h[:, :dI], h[:, 3 * dI:4 * dI], h[:, 2 * dI:3 * dI], m,
                                          bias_a=pb[:, dI:], bias_b=pb[:, :dI]), EPS)
    N = T // m
    for t in range(T):
        V = oracle.visible(t, N, m)
        assert V == min(N, (t + 1) // m)
        scores = oracle.index_scores(qres[t].reshape(H, dI), h[t, 4 * dI:], keys[:V])
        want = oracle.topk(scores, V, k)
        assert set(int(x) for x in got[t] if x >= 0) == set(int(x) for x in want if x >= 0), t
        assert np.sum(got[t] >= 0) == min(V, k)


# ------------------------------------------------------------------------- attention
class _AttnStub(torch.nn.Module):
    def __init__(self, H, sinks):
        super().__init__()
        self.num_key_value_groups = H
        self.sinks = torch.nn.Parameter(torch.from_numpy(sinks))
        self.training = False


@pytest.mark.parametrize("with_sink", [False, True])
def test_attention_matches_v4_eager(with_sink):
    """oracle_sparse_mqa (RMSNorm of q and of every attended row inside, one softmax over
    the selected entries and the window, optional sink) equals V4's eager attention fed
    with V4's own normalised q and rows over the same set (key = value)."""
    rng = np.random.default_rng(10)
    H, d, N, k, window = 6, 64, 50, 9, 5
    q = rng.standard_normal((H, d)).astype(np.float32)
    kv = rng.standard_normal((N, d)).astype(np.float32)
    raw = rng.standard_normal((window + 3, d)).astype(np.float32)
    idx = np.sort(rng.choice(N, size=k, replace=False)).astype(np.int32)
    idx[-2:] = -1
    base, t = 200, 200 + window + 1
    sinks = (rng.standard_normal(H) if with_sink else np.full(H, -np.inf)).astype(np.float32)
    want, lse = oracle.sparse_mqa(q, kv, idx, raw, base, t, window, d ** -0.5, EPS,
                                  sink=sinks if with_sink else None)
    rows = np.concatenate([kv[idx[idx >= 0]], raw[t - window + 1 - base:t + 1 - base]])
    qn = M.DeepseekV4UnweightedRMSNorm(eps=EPS)(torch.from_numpy(q))
    kn = M.DeepseekV4RMSNorm(d, eps=EPS)(torch.from_numpy(rows))
    with torch.no_grad():
        o, _ = M.eager_attention_forward(_AttnStub(H, sinks), qn[None, :, None], kn[None, None], kn[None, None],
                                         None, d ** -0.5)
    got = o[0, 0].double().numpy()
    np.testing.assert_allclose(got, want, rtol=0, atol=2e-6)
    if with_sink:   # the sink takes weight: the output shrinks against the same set without it
        no_sink, _ = oracle.sparse_mqa(q, kv, idx, raw, base, t, window, d ** -0.5, EPS)
        assert np.all(np.abs(want) <= np.abs(no_sink) + 1e-12) and np.abs(want - no_sink).max() > 1e-3
