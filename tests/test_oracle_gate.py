"""Pins of the oracle's output gate (gate_silu, forward_gated) that do not
reuse its formula: a hand-worked fixture, torch's silu, the limits of the
SiLU, and planted mistakes that the fixture catches."""
import numpy as np
import pytest
import torch

import gen
import oracle
from conftest import read_golden


def test_hand_worked_values():
    d = read_golden("gate_five_values.txt")
    y = oracle.gate_silu(d["o"], d["gate"])
    np.testing.assert_allclose(y, d["gated"], rtol=1e-15, atol=1e-16)
    # the SiLU factor alone: the gated value of o = 1
    np.testing.assert_allclose(oracle.gate_silu(np.ones(5), d["gate"]), d["silu_gate"], rtol=1e-15, atol=1e-16)


def test_against_torch_silu():
    r = np.random.default_rng(3)
    o = r.standard_normal((2, 7, 3, 192))
    gate = 3.0 * r.standard_normal((2, 7, 3, 192))
    ref = (torch.from_numpy(o) * torch.nn.functional.silu(torch.from_numpy(gate))).numpy()
    np.testing.assert_allclose(oracle.gate_silu(o, gate), ref, rtol=1e-14, atol=1e-300)


def test_limits():
    o = np.array([1.5, -2.0, 0.25])
    # SiLU(a) -> a for large a, -> 0 for very negative a, SiLU(0) = 0
    np.testing.assert_allclose(oracle.gate_silu(o, np.full(3, 60.0)), o * 60.0, rtol=1e-15)
    assert np.all(np.abs(oracle.gate_silu(o, np.full(3, -800.0))) == 0.0)
    assert np.all(oracle.gate_silu(o, np.zeros(3)) == 0.0)


def test_forward_gated_is_gated_forward():
    d = gen.make_inputs("fwd_bf16_b8_t2048", seed=7, B=1, T=9, H=2, S0="normal0.1")
    gate = np.random.default_rng(8).standard_normal(d["v"].shape)
    y, S = oracle.forward_gated(d["q"], d["k"], d["v"], d["g"], gate, d["S0"])
    o, S2 = oracle.forward(d["q"], d["k"], d["v"], d["g"], d["S0"])
    assert np.array_equal(S, S2)
    # token by token against the hand-worked SiLU factor: y / o = SiLU(gate)
    sig = 1.0 / (1.0 + np.exp(-gate))
    np.testing.assert_allclose(y, o * gate * sig, rtol=1e-14)


@pytest.mark.parametrize("mistake", ["sigmoid_only", "roles_swapped", "no_gate", "gate_before_sum"])
def test_planted_mistakes_are_caught(mistake):
    d = read_golden("gate_five_values.txt")
    o, gate = d["o"], d["gate"]
    silu = lambda a: a / (1.0 + np.exp(-a))
    wrong = {"sigmoid_only": lambda: o / (1.0 + np.exp(-gate)),
             "roles_swapped": lambda: silu(o) * gate,
             "no_gate": lambda: o,
             "gate_before_sum": lambda: silu(o * gate)}[mistake]()
    assert not np.allclose(wrong, d["gated"], rtol=1e-6, atol=1e-9)
