"""Pins of the oracle's causal depth-wise convolution with SiLU
(oracle.conv1d_silu) against a hand-worked example, torch's own conv1d and
silu, and the chaining of a sequence split in pieces.  Broken copies of the
oracle (kernel reversed, SiLU missing, history ignored, short sequences not
shifting the history) must fail them."""
import numpy as np
import pytest
import torch

import oracle
from conftest import read_golden


def torch_ref(x, w, bias, hist):
    """Library reference on one sequence: pad with the window's last three rows
    on the left, depth-wise conv1d, silu.  x [L, D], w [D, 4], hist [4, D]."""
    xt = torch.from_numpy(np.concatenate([hist[1:], x], 0).T[None].copy())    # [1, D, L+3]
    a = torch.nn.functional.conv1d(xt, torch.from_numpy(w[:, None, :].copy()),
                                   torch.from_numpy(bias.copy()), groups=w.shape[0])
    return torch.nn.functional.silu(a)[0].T.numpy()                             # [L, D]


def _seqs(seed, lengths, D=6, n_slots=5):
    r = np.random.default_rng(seed)
    N = int(sum(lengths))
    x = r.standard_normal((N, D))
    w = r.standard_normal((D, 4))
    bias = r.standard_normal(D)
    state = r.standard_normal((n_slots, 4, D))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    slots = r.permutation(n_slots)[:len(lengths)].astype(np.int32)
    return x, w, bias, state, cu, slots


def pin_golden(conv):
    d = read_golden("conv_five_tokens.txt")
    y, st = conv(d["x"], d["w"], d["bias"], [0, 5], d["history"][None], None, True)
    want = torch.nn.functional.silu(torch.from_numpy(d["a"])).numpy()
    np.testing.assert_allclose(y, want, rtol=1e-14, atol=1e-14)
    np.testing.assert_array_equal(st[0], d["new_history"])


def pin_torch_conv(conv):
    x, w, bias, state, cu, slots = _seqs(1, [9, 1, 0, 4])
    for init in (False, True):
        y, st = conv(x, w, bias, cu, state, slots, init)
        for b in range(4):
            t0, t1 = cu[b], cu[b + 1]
            hist = state[slots[b]] if init else np.zeros((4, x.shape[1]))
            if t1 > t0:
                np.testing.assert_allclose(y[t0:t1], torch_ref(x[t0:t1], w, bias, hist), rtol=1e-12, atol=1e-12)
            np.testing.assert_array_equal(st[slots[b]], np.concatenate([hist, x[t0:t1]], 0)[-4:])


def pin_chaining(conv):
    x, w, bias, state, cu, slots = _seqs(2, [11])
    y, st = conv(x, w, bias, cu, state, slots, True)
    cur = state
    ys = []
    for a, b in ((0, 1), (1, 3), (3, 3), (3, 8), (8, 11)):       # pieces of 1, 2, 0, 5, 3 tokens
        yp, cur = conv(x[a:b], w, bias, [0, b - a], cur, slots, True)
        ys.append(yp)
    np.testing.assert_allclose(np.concatenate(ys, 0), y, rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(cur, st)


def pin_untouched(conv):
    x, w, bias, state, cu, slots = _seqs(3, [2, 5], n_slots=6)
    s0 = state.copy()
    _, st = conv(x, w, bias, cu, state, slots, True)
    np.testing.assert_array_equal(state, s0)
    for s in set(range(6)) - set(int(v) for v in slots):
        np.testing.assert_array_equal(st[s], state[s])


PINS = [pin_golden, pin_torch_conv, pin_chaining, pin_untouched]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_conv_pins(pin):
    pin(oracle.conv1d_silu)


def test_no_state_means_zero_history():
    x, w, bias, state, cu, slots = _seqs(4, [7, 3])
    y0, st0 = oracle.conv1d_silu(x, w, bias, cu)
    y1, _ = oracle.conv1d_silu(x, w, bias, cu, state, slots, False)
    assert st0 is None
    np.testing.assert_array_equal(y0, y1)


def _mutant(kind):
    def conv(x, w, bias, cu_seqlens, state=None, slot_idx=None, init_from_state=False):
        x, w = np.asarray(x, np.float64), np.asarray(w, np.float64)
        D = x.shape[1]
        bias = np.zeros(D) if bias is None else np.asarray(bias, np.float64)
        if kind == "kernel_reversed":
            w = w[:, ::-1]
        cu = [int(c) for c in cu_seqlens]
        slots = list(range(len(cu) - 1)) if slot_idx is None else [int(s) for s in slot_idx]
        state = None if state is None else np.asarray(state, np.float64)
        y = np.zeros_like(x)
        new = None if state is None else state.copy()
        for b in range(len(cu) - 1):
            t0, t1 = cu[b], cu[b + 1]
            use = state is not None and init_from_state and kind != "history_ignored"
            hist = state[slots[b]] if use else np.zeros((4, D))
            z = np.concatenate([hist, x[t0:t1]], 0)
            off = 0 if kind == "oldest_row_read" else 1
            for t in range(t1 - t0):
                a = bias + sum(w[:, j] * z[t + off + j] for j in range(4))
                y[t0 + t] = a if kind == "no_silu" else a / (1 + np.exp(-a))
            if new is not None:
                if kind == "short_not_shifted" and t1 - t0 < 4:
                    new[slots[b]] = np.concatenate([x[t0:t1], hist], 0)[:4]
                else:
                    new[slots[b]] = z[-4:]
        return y, new
    return conv


@pytest.mark.parametrize("kind", ["kernel_reversed", "no_silu", "history_ignored", "short_not_shifted",
                                  "oldest_row_read"])
def test_pins_catch_planted_conv_mistakes(kind):
    failures = 0
    for pin in PINS:
        try:
            pin(_mutant(kind))
        except AssertionError:
            failures += 1
    assert failures > 0, f"no conv pin rejects the '{kind}' mutant"
