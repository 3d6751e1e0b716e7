"""Seeded workload generator: determinism, shapes, and bf16 rounding checked
against torch's own fp32 -> bfloat16 conversion (round to nearest even)."""
import numpy as np
import torch

from long_context_compressed_04_amd import workloads as W


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    x[:4] = [1.00390625, 1.01171875, -3.0, 0.0]     # exact ties and plain values
    ours = W.bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, theirs)
    np.testing.assert_array_equal(W.bf16_to_f64(ours), torch.from_numpy(x).to(torch.bfloat16).double().numpy())


def test_generators_are_deterministic_and_shaped():
    a = W.csa_decode(0, B=2, T=4096, H=16, d=64, HI=8, dI=32, k=32)
    b = W.csa_decode(0, B=2, T=4096, H=16, d=64, HI=8, dI=32, k=32)
    for key in ("kv", "kI", "q", "qI", "w", "kv_raw"):
        np.testing.assert_array_equal(a[key], b[key])
    assert a["kv"].shape == (2, 1024, 64) and a["kv"].dtype == np.uint16
    assert a["kI"].shape == (2, 1024, 32) and a["w"].shape == (2, 8)
    assert np.all((a["w"] >= 0) & (a["w"] < 1))
    c = W.cfg1()
    assert c["A"].shape == (1, 2048, 64) and c["kI"].shape == (1, 512, 32)
    np.testing.assert_array_equal(c["kv_raw"][0], c["A"][0, 1920:2048])
    assert int(c["q_pos"][0]) == 2047 and int(c["raw_base"][0]) == 1920
    p = W.csa_prefill(0, T_prior=256, n_new=32, H=4, d=64, HI=2, dI=32, k=16)
    assert p["A"].shape == (36, 64) and p["tok_base"] == 252 and p["kv_raw"].shape == (32 + 127, 64)
    assert p["q_pos"][0] == 256 and p["q_pos"][-1] == 287 and p["raw_base"] == 256 - 127
