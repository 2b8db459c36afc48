"""Pins of the oracle's packed-sequence prefill (oracle.forward_packed).

Each sequence of a packed batch must equal the brute-force closed form of the
recurrence started from its slot's state; slots of no sequence must keep
their state; a prompt split in two and continued from the pool must equal
the whole prompt.  Broken copies of forward_packed (state carried from one
sequence into the next, slot index ignored, rows shifted) must fail them.
"""
import numpy as np
import pytest

import gen
import oracle
from test_oracle import closed_form


def _packed(seed, lengths, n_slots=7, H=2, dk=4, dv=5):
    r = np.random.default_rng(seed)
    N = int(sum(lengths))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    q = r.standard_normal((N, H, dk))
    k = r.standard_normal((N, H, dk))
    v = r.standard_normal((N, H, dv))
    g = gen.logsigmoid(r.standard_normal((N, H)) + 1.0)
    pool = r.standard_normal((n_slots, H, dk, dv))
    slots = r.permutation(n_slots)[:len(lengths)].astype(np.int32)
    return q, k, v, g, cu, pool, slots


def pin_closed_form(fp):
    lengths = [5, 0, 9, 1, 6]
    q, k, v, g, cu, pool, slots = _packed(1, lengths)
    for init in (False, True):
        o, new = fp(q, k, v, g, cu, pool, slots, init)
        for b in range(len(lengths)):
            t0, t1 = cu[b], cu[b + 1]
            S0 = pool[slots[b]][None] if init else None
            if t1 == t0:
                want = pool[slots[b]] if init else np.zeros_like(pool[0])
                np.testing.assert_array_equal(new[slots[b]], want)
                continue
            o_ref, S_ref = closed_form(q[None, t0:t1], k[None, t0:t1], v[None, t0:t1], g[None, t0:t1], S0)
            np.testing.assert_allclose(o[t0:t1], o_ref[0], rtol=1e-11, atol=1e-11)
            np.testing.assert_allclose(new[slots[b]], S_ref[0], rtol=1e-11, atol=1e-11)


def pin_untouched_slots(fp):
    q, k, v, g, cu, pool, slots = _packed(2, [4, 3], n_slots=6)
    pool0 = pool.copy()
    _, new = fp(q, k, v, g, cu, pool, slots, True)
    np.testing.assert_array_equal(pool, pool0)                  # input not modified
    for s in set(range(6)) - set(int(x) for x in slots):
        np.testing.assert_array_equal(new[s], pool[s])


def pin_continuation(fp):
    lengths = [7, 12, 3]
    cut = [3, 12, 0]
    q, k, v, g, cu, pool, slots = _packed(3, lengths)
    o_all, p_all = fp(q, k, v, g, cu, pool, slots, True)
    first = np.concatenate([np.arange(cu[b], cu[b] + cut[b]) for b in range(3)])
    second = np.concatenate([np.arange(cu[b] + cut[b], cu[b + 1]) for b in range(3)])
    cu1 = np.concatenate([[0], np.cumsum(cut)]).astype(np.int32)
    cu2 = np.concatenate([[0], np.cumsum(np.subtract(lengths, cut))]).astype(np.int32)
    o1, p1 = fp(q[first], k[first], v[first], g[first], cu1, pool, slots, True)
    o2, p2 = fp(q[second], k[second], v[second], g[second], cu2, p1, slots, True)
    np.testing.assert_allclose(o1, o_all[first], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(o2, o_all[second], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(p2, p_all, rtol=1e-12, atol=1e-12)


PINS = [pin_closed_form, pin_untouched_slots, pin_continuation]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_packed_pins(pin):
    pin(oracle.forward_packed)


def test_equal_lengths_match_batched_forward():
    q, k, v, g, S0 = (np.random.default_rng(4).standard_normal(s) for s in
                      ((3, 10, 2, 4), (3, 10, 2, 4), (3, 10, 2, 5), (3, 10, 2), (3, 2, 4, 5)))
    g = gen.logsigmoid(g)
    o, S = oracle.forward(q, k, v, g, S0)
    cu = np.arange(0, 31, 10, dtype=np.int32)
    fl = lambda x: x.reshape((30,) + x.shape[2:])
    op, pool = oracle.forward_packed(fl(q), fl(k), fl(v), fl(g), cu, S0, None, True)
    np.testing.assert_array_equal(op, fl(o))
    np.testing.assert_array_equal(pool, S)


def _mutant(kind):
    def fp(q, k, v, g, cu_seqlens, pool, slot_idx=None, init_from_pool=False):
        q, k, v, g, pool = (np.asarray(x, np.float64) for x in (q, k, v, g, pool))
        cu = [int(c) for c in cu_seqlens]
        n = len(cu) - 1
        slots = list(range(n)) if slot_idx is None else [int(s) for s in slot_idx]
        if kind == "slot_ignored":
            slots = list(range(n))
        o = np.zeros(q.shape[:2] + (v.shape[-1],))
        new = pool.copy()
        carry = None
        for b in range(n):
            t0, t1 = cu[b], cu[b + 1]
            S0 = pool[slots[b]][None] if init_from_pool else None
            if kind == "state_carried" and carry is not None:
                S0 = carry
            if kind == "rows_shifted":
                t0, t1 = min(t0 + 1, cu[-1]), min(t1 + 1, cu[-1])
            if t1 <= t0:
                new[slots[b]] = pool[slots[b]] if init_from_pool else 0.0
                continue
            ob, S = oracle.forward(q[None, t0:t1], k[None, t0:t1], v[None, t0:t1], g[None, t0:t1], S0)
            o[t0:t1] = ob[0]
            new[slots[b]] = S[0]
            carry = S
        return o, new
    return fp


@pytest.mark.parametrize("kind", ["state_carried", "slot_ignored", "rows_shifted"])
def test_pins_catch_planted_packed_mistakes(kind):
    failures = 0
    for pin in PINS:
        try:
            pin(_mutant(kind))
        except AssertionError:
            failures += 1
    assert failures > 0, f"no packed pin rejects the '{kind}' mutant"
