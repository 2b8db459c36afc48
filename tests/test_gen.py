"""The seeded generator: determinism, distributions, host bf16 rounding."""
import numpy as np
import torch

import gen


def test_same_seed_same_bytes():
    a = gen.make_inputs("fwd_bf16_b8_t2048", seed=3, B=2, T=100, with_dO=True)
    b = gen.make_inputs("fwd_bf16_b8_t2048", seed=3, B=2, T=100, with_dO=True)
    c = gen.make_inputs("fwd_bf16_b8_t2048", seed=4, B=2, T=100, with_dO=True)
    for key in ("q", "k", "v", "g", "dO"):
        assert a[key].tobytes() == b[key].tobytes()
        assert a[key].tobytes() != c[key].tobytes()


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100_000).astype(np.float32) * 3
    x[:4] = [1.00390625, 1.01171875, -2.5e-39, 65504.0]     # ties and a denormal
    ours = gen.bf16_round(x)
    ref = torch.tensor(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(gen.bf16_bits(x),
                                  torch.tensor(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def test_distributions():
    d = gen.make_inputs("fwd_f32_b1_t2048", seed=0)
    assert d["q"].dtype == np.float32 and d["q"].shape == (1, 2048, 16, 96)
    assert abs(d["q"].std() * np.sqrt(96) - 1) < 0.02
    assert abs(d["v"].mean()) < 0.01
    gam = np.exp(d["g"].astype(np.float64))
    assert 0.97 < gam.mean() < 0.99 and np.all(d["g"] <= 0)
    assert d["S0"] is None
    h = gen.make_inputs("fwd_bf16_b1_t65536", seed=0, T=256)
    # one log-decay per head, held over tokens, within logsigmoid([2, 8])
    assert np.all(h["g"] == h["g"][:, :1, :])
    assert np.all(h["g"] >= gen.logsigmoid(2.0) - 1e-7) and np.all(h["g"] <= gen.logsigmoid(8.0) + 1e-7)
    assert abs(h["S0"].std() - 0.1) < 0.002
    assert np.array_equal(gen.bf16_round(h["q"]), h["q"])
    z = gen.make_inputs("fwd_bf16_b8_t2048", B=1, T=10, g="zero")
    assert np.all(np.isneginf(z["g"]))
    o = gen.make_inputs("fwd_bf16_b8_t2048", B=1, T=10, g="one")
    assert np.all(o["g"] == 0)


def test_decode_inputs():
    s = gen.make_decode_step(64, step=5)
    assert s["q"].shape == (64, 16, 96) and s["v"].shape == (64, 16, 192) and s["g"].shape == (64, 16)
    s2 = gen.make_decode_step(64, step=6)
    assert not np.array_equal(s["q"], s2["q"])
    st = gen.make_decode_state(8)
    assert st.shape == (8, 16, 96, 192) and abs(st.std() - 0.1) < 0.002
