"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each pin is a function of the forward/backward callables so that the same
checks can be replayed against deliberately broken copies of the oracle
(test_pins_catch_planted_mistakes): a pin that cannot tell a wrong oracle
from the right one pins nothing.
"""
import math

import numpy as np
import pytest
import torch

import gen
import oracle
from conftest import read_golden


def _rand(seed, B=2, T=37, H=3, dk=5, dv=7, s0=True, g="logsig_n4"):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, T, H, dk))
    k = r.standard_normal((B, T, H, dk))
    v = r.standard_normal((B, T, H, dv))
    if g == "logsig_n4":
        gg = gen.logsigmoid(r.standard_normal((B, T, H)) + 1.0)
    elif g == "one":
        gg = np.zeros((B, T, H))
    elif g == "zero":
        gg = np.full((B, T, H), -np.inf)
    S0 = r.standard_normal((B, H, dk, dv)) if s0 else None
    return q, k, v, gg, S0


# --------------------------------------------------------------------------
# forward pins
# --------------------------------------------------------------------------

def pin_golden_scalar(fwd, bwd):
    d = read_golden("scalar_three_tokens.txt")
    sh = lambda x: np.asarray(x, np.float64).reshape(1, -1, 1, 1)
    g = np.log(d["gamma"]).reshape(1, -1, 1)
    o, S = fwd(sh(d["q"]), sh(d["k"]), sh(d["v"]), g,
               np.array(d["S0"]).reshape(1, 1, 1, 1))
    np.testing.assert_allclose(o.ravel(), d["o"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(S.ravel(), np.ravel(d["S_T"]), rtol=0, atol=1e-12)
    if bwd is not None:
        dq, dk, dv, dg, dS0 = bwd(sh(d["q"]), sh(d["k"]), sh(d["v"]), g,
                                  sh(d["dO"]), np.array(d["S0"]).reshape(1, 1, 1, 1))
        for name, got in (("dq", dq), ("dk", dk), ("dv", dv), ("dg", dg)):
            np.testing.assert_allclose(got.ravel(), d[name], rtol=0, atol=1e-12,
                                       err_msg=name)
        np.testing.assert_allclose(dS0.ravel(), np.ravel(d["dS0"]), rtol=0, atol=1e-12)


def pin_golden_matrix(fwd, bwd=None):
    d = read_golden("matrix_two_tokens.txt")
    q = d["q"].reshape(1, 2, 1, 2)
    k = d["k"].reshape(1, 2, 1, 2)
    v = d["v"].reshape(1, 2, 1, 3)
    g = np.log(d["gamma"]).reshape(1, 2, 1)
    o, S = fwd(q, k, v, g, None)
    np.testing.assert_allclose(o.reshape(2, 3), d["o"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(S.reshape(2, 3), d["S_T"], rtol=0, atol=1e-12)


def closed_form(q, k, v, g, S0):
    """Brute force: o_t = sum_{s<=t} (prod_{r=s+1..t} gamma_r)(q_t.k_s) v_s
    + (prod_{r<=t} gamma_r) q_t S0, and the matching final state."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    gam = np.exp(g)
    o = np.zeros((B, T, H, dv))
    S_T = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            for t in range(T):
                acc = np.zeros(dv)
                for s in range(t + 1):
                    w = np.prod(gam[b, s + 1:t + 1, h])
                    acc += w * np.dot(q[b, t, h], k[b, s, h]) * v[b, s, h]
                if S0 is not None:
                    acc += np.prod(gam[b, :t + 1, h]) * (q[b, t, h] @ S0[b, h])
                o[b, t, h] = acc
            for s in range(T):
                w = np.prod(gam[b, s + 1:, h])
                S_T[b, h] += w * np.outer(k[b, s, h], v[b, s, h])
            if S0 is not None:
                S_T[b, h] += np.prod(gam[b, :, h]) * S0[b, h]
    return o, S_T


def pin_closed_form(fwd, bwd=None):
    for T, s0, seed in ((1, True, 0), (2, False, 1), (5, True, 2), (13, True, 3)):
        q, k, v, g, S0 = _rand(seed, B=2, T=T, H=2, dk=3, dv=4, s0=s0)
        o, S = fwd(q, k, v, g, S0)
        o_ref, S_ref = closed_form(q, k, v, g, S0)
        np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(S, S_ref, rtol=1e-12, atol=1e-12)


def pin_gamma_one(fwd, bwd=None):
    # No decay: plain causal linear attention, tril(Q K^T) V + Q S0.
    q, k, v, g, S0 = _rand(4, B=1, T=40, H=2, dk=6, dv=5, g="one")
    o, S = fwd(q, k, v, g, S0)
    for h in range(2):
        Q, K, V = q[0, :, h], k[0, :, h], v[0, :, h]
        ref = np.tril(Q @ K.T) @ V + Q @ S0[0, h]
        np.testing.assert_allclose(o[0, :, h], ref, rtol=1e-12, atol=1e-11)
        np.testing.assert_allclose(S[0, h], S0[0, h] + K.T @ V, rtol=1e-12, atol=1e-11)


def pin_gamma_zero(fwd, bwd=None):
    # Full forgetting: o_t = (q_t . k_t) v_t and S_T = k_{T-1}^T v_{T-1}; S0 drops out.
    q, k, v, g, S0 = _rand(5, B=2, T=9, H=2, dk=4, dv=3, g="zero")
    o, S = fwd(q, k, v, g, S0)
    ref = np.einsum("bthd,bthd->bth", q, k)[..., None] * v
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, np.einsum("bhd,bhc->bhdc", k[:, -1], v[:, -1]),
                               rtol=1e-12, atol=1e-12)


def pin_constant_gamma(fwd, bwd=None):
    # Constant gamma per head: weights gamma^(t-s) (geometric closed form).
    B, T, H, dk, dv = 1, 30, 3, 4, 6
    r = np.random.default_rng(6)
    q, k = r.standard_normal((B, T, H, dk)), r.standard_normal((B, T, H, dk))
    v, S0 = r.standard_normal((B, T, H, dv)), r.standard_normal((B, H, dk, dv))
    gh = np.array([0.9, 0.5, 0.999])
    g = np.broadcast_to(np.log(gh), (B, T, H)).copy()
    o, S = fwd(q, k, v, g, S0)
    t = np.arange(T)
    for h in range(H):
        W = np.where(t[:, None] >= t[None, :],
                     gh[h] ** (t[:, None] - t[None, :]).clip(min=0), 0.0)
        Q, K, V = q[0, :, h], k[0, :, h], v[0, :, h]
        ref = (W * (Q @ K.T)) @ V + (gh[h] ** (t + 1))[:, None] * (Q @ S0[0, h])
        np.testing.assert_allclose(o[0, :, h], ref, rtol=1e-11, atol=1e-11)
        Sref = (gh[h] ** (T - 1 - t))[:, None, None] * np.einsum("td,tc->tdc", K, V)
        np.testing.assert_allclose(S[0, h], Sref.sum(0) + gh[h] ** T * S0[0, h],
                                   rtol=1e-11, atol=1e-11)


FWD_PINS = [pin_golden_scalar, pin_golden_matrix, pin_closed_form, pin_gamma_one,
            pin_gamma_zero, pin_constant_gamma]


@pytest.mark.parametrize("pin", FWD_PINS, ids=lambda p: p.__name__)
def test_forward_pins(pin):
    pin(oracle.forward, oracle.backward)


def test_chaining_padding_linearity():
    q, k, v, g, S0 = _rand(7, B=2, T=50, H=2, dk=4, dv=5)
    o, S = oracle.forward(q, k, v, g, S0)
    # chaining: the state is the whole summary of the prefix
    o1, S1 = oracle.forward(q[:, :23], k[:, :23], v[:, :23], g[:, :23], S0)
    o2, S2 = oracle.forward(q[:, 23:], k[:, 23:], v[:, 23:], g[:, 23:], S1)
    np.testing.assert_allclose(np.concatenate([o1, o2], 1), o, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(S2, S, rtol=1e-13, atol=1e-13)
    # padding with k = v = 0, g = 0 is an identity step
    pad = lambda x, n: np.concatenate([x, np.zeros((x.shape[0], n) + x.shape[2:])], 1)
    op, Sp = oracle.forward(pad(q, 9), pad(k, 9), pad(v, 9), pad(g, 9), S0)
    np.testing.assert_allclose(op[:, :50], o, rtol=0, atol=0)
    np.testing.assert_allclose(Sp, S, rtol=0, atol=0)
    # o is linear in (v, S0) jointly
    v2, S02 = np.random.default_rng(8).standard_normal(v.shape), np.random.default_rng(9).standard_normal(S0.shape)
    oa, Sa = oracle.forward(q, k, v2, g, S02)
    ob, Sb = oracle.forward(q, k, 2 * v - 3 * v2, g, 2 * S0 - 3 * S02)
    np.testing.assert_allclose(ob, 2 * o - 3 * oa, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(Sb, 2 * S - 3 * Sa, rtol=1e-11, atol=1e-11)


def test_step_matches_forward():
    q, k, v, g, S0 = _rand(10, B=3, T=11, H=2, dk=4, dv=5)
    o, S = oracle.forward(q, k, v, g, S0)
    St = S0
    for t in range(11):
        ot, St = oracle.step(St, q[:, t], k[:, t], v[:, t], g[:, t])
        np.testing.assert_allclose(ot, o[:, t], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(St, S, rtol=1e-13, atol=1e-13)


def test_page_sizes():
    d = read_golden("page_sizes.txt")
    H, dk, dv = int(d["H"]), int(d["dk"]), int(d["dv"])
    assert H * (2 * dk + 2 * dv) == d["qkvg_rows"]
    assert d["chunks"] * d["chunk_tokens"] == 2048
    assert gen.WORKLOADS["fwd_bf16_b8_t2048"]["T"] == 2048
    per_layer = oracle.state_bytes(H, dk, dv)
    assert per_layer == 1_179_648
    # fp32 mixer states of all layers plus an fp32 conv window (width-1 past
    # inputs are the minimum; the pages' figure fits width x D per layer)
    total = d["layers"] * (per_layer + d["conv_width"] * d["D"] * 4)
    assert abs(total / 1e6 - d["state_mb_per_sequence"]) < 0.05
    # a bf16 state would not reach the printed size
    assert d["layers"] * oracle.state_bytes(H, dk, dv, 2) / 1e6 < 20



# --------------------------------------------------------------------------
# backward pins
# --------------------------------------------------------------------------

def _loss(fwd, q, k, v, g, S0, dO, dST):
    o, S = fwd(q, k, v, g, S0)
    return float(np.sum(dO * o) + np.sum(dST * S))


def pin_finite_differences(fwd, bwd):
    q, k, v, g, S0 = _rand(11, B=1, T=19, H=2, dk=3, dv=4)
    r = np.random.default_rng(12)
    dO, dST = r.standard_normal((1, 19, 2, 4)), r.standard_normal((1, 2, 3, 4))
    grads = bwd(q, k, v, g, dO, S0, dST)
    args = [q, k, v, g, S0]
    eps = 1e-6
    for i in range(5):
        for trial in range(2):
            d = r.standard_normal(args[i].shape)
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[i] = args[i] + eps * d
            minus[i] = args[i] - eps * d
            fd = (_loss(fwd, *plus, dO, dST) - _loss(fwd, *minus, dO, dST)) / (2 * eps)
            an = float(np.sum(grads[i] * d))
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (i, fd, an)


def pin_elementwise_fd(fwd, bwd):
    q, k, v, g, S0 = _rand(13, B=1, T=4, H=1, dk=2, dv=3)
    r = np.random.default_rng(14)
    dO, dST = r.standard_normal((1, 4, 1, 3)), r.standard_normal((1, 1, 2, 3))
    grads = bwd(q, k, v, g, dO, S0, dST)
    args = [q, k, v, g, S0]
    eps = 1e-6
    for i in range(5):
        it = np.nditer(args[i], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[i][idx] += eps
            minus[i][idx] -= eps
            fd = (_loss(fwd, *plus, dO, dST) - _loss(fwd, *minus, dO, dST)) / (2 * eps)
            assert abs(fd - grads[i][idx]) <= 1e-7 * max(1.0, abs(fd)), (i, idx)


def _torch_closed_form(q, k, v, g, S0):
    """Differentiable closed form in torch fp64 via cumulative log-decay."""
    T = q.shape[1]
    beta = torch.cumsum(g, dim=1)                       # [B,T,H]
    bt = beta.permute(0, 2, 1)                          # [B,H,T]
    diff = bt[:, :, :, None] - bt[:, :, None, :]        # beta_t - beta_s
    mask = torch.tril(torch.ones(T, T, dtype=torch.bool))
    W = torch.where(mask, torch.exp(torch.where(mask, diff, torch.zeros_like(diff))),
                    torch.zeros_like(diff))
    Q, K, V = (x.permute(0, 2, 1, 3) for x in (q, k, v))
    A = torch.matmul(Q, K.transpose(-1, -2).contiguous()) * W
    o = torch.matmul(A, V) + torch.exp(bt)[..., None] * torch.matmul(Q, S0)
    wT = torch.exp(bt[:, :, -1:] - bt)                  # prod_{r>s} gamma_r
    S = torch.matmul((K * wT[..., None]).transpose(-1, -2).contiguous(), V)
    S = S + torch.exp(bt[:, :, -1])[..., None, None] * S0
    return o.permute(0, 2, 1, 3), S


def pin_torch_autograd(fwd, bwd):
    q, k, v, g, S0 = _rand(15, B=2, T=23, H=2, dk=3, dv=5)
    r = np.random.default_rng(16)
    dO, dST = r.standard_normal((2, 23, 2, 5)), r.standard_normal((2, 2, 3, 5))
    ts = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, g, S0)]
    o, S = _torch_closed_form(*ts)
    np.testing.assert_allclose(fwd(q, k, v, g, S0)[0], o.detach().numpy(), rtol=1e-10, atol=1e-10)
    L = (o * torch.tensor(dO)).sum() + (S * torch.tensor(dST)).sum()
    L.backward()
    grads = bwd(q, k, v, g, dO, S0, dST)
    for i, name in enumerate(("dq", "dk", "dv", "dg", "dS0")):
        np.testing.assert_allclose(grads[i], ts[i].grad.numpy(), rtol=1e-9, atol=1e-9,
                                   err_msg=name)


def pin_gamma_one_grads(fwd, bwd):
    # No decay: textbook gradients of tril(QK^T)V + Q S0 and S_T = S0 + K^T V.
    q, k, v, g, S0 = _rand(17, B=1, T=25, H=1, dk=4, dv=6, g="one")
    r = np.random.default_rng(18)
    dO, dST = r.standard_normal((1, 25, 1, 6)), r.standard_normal((1, 1, 4, 6))
    dq, dk, dv, dg, dS0 = bwd(q, k, v, g, dO, S0, dST)
    Q, K, V, G, Sd = q[0, :, 0], k[0, :, 0], v[0, :, 0], dO[0, :, 0], dST[0, 0]
    M = np.tril(G @ V.T)
    np.testing.assert_allclose(dq[0, :, 0], M @ K + G @ S0[0, 0].T, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dk[0, :, 0], M.T @ Q + V @ Sd.T, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dv[0, :, 0], np.tril(Q @ K.T).T @ G + K @ Sd, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dS0[0, 0], Sd + Q.T @ G, rtol=1e-11, atol=1e-11)


def pin_dg_identity(fwd, bwd):
    # d-log-decay equals the reverse cumulative sum of q.dq - k.dk plus <dS_T, S_T>
    # (derivative through the cumulative log-decay), an identity independent of
    # the direct formula the oracle uses.
    q, k, v, g, S0 = _rand(19, B=2, T=31, H=2, dk=3, dv=4)
    r = np.random.default_rng(20)
    dO, dST = r.standard_normal((2, 31, 2, 4)), r.standard_normal((2, 2, 3, 4))
    dq, dk, dv, dg, _ = bwd(q, k, v, g, dO, S0, dST)
    _, S_T = fwd(q, k, v, g, S0)
    rr = np.einsum("bthd,bthd->bth", q, dq) - np.einsum("bthd,bthd->bth", k, dk)
    suffix = np.flip(np.cumsum(np.flip(rr, 1), 1), 1)
    const = np.einsum("bhdc,bhdc->bh", dST, S_T)[:, None, :]
    np.testing.assert_allclose(dg, suffix + const, rtol=1e-10, atol=1e-10)


def pin_gamma_zero_grads(fwd, bwd):
    # Full forgetting: o_t = (q_t . k_t) v_t, so each token's gradients only
    # involve itself, and the log-decay gets no gradient.
    q, k, v, g, S0 = _rand(21, B=1, T=8, H=2, dk=3, dv=4, g="zero")
    dO = np.random.default_rng(22).standard_normal((1, 8, 2, 4))
    dq, dk, dv, dg, dS0 = bwd(q, k, v, g, dO, S0, None)
    assert np.all(dg == 0.0)
    assert np.all(dS0 == 0.0)
    dov = np.einsum("bthc,bthc->bth", dO, v)[..., None]
    np.testing.assert_allclose(dq, k * dov, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dk, q * dov, rtol=1e-12, atol=1e-12)
    qk = np.einsum("bthd,bthd->bth", q, k)[..., None]
    np.testing.assert_allclose(dv, qk * dO, rtol=1e-12, atol=1e-12)


BWD_PINS = [pin_finite_differences, pin_elementwise_fd, pin_torch_autograd,
            pin_gamma_one_grads, pin_dg_identity, pin_gamma_zero_grads]


@pytest.mark.parametrize("pin", BWD_PINS, ids=lambda p: p.__name__)
def test_backward_pins(pin):
    pin(oracle.forward, oracle.backward)


def test_backward_checkpoint_interval_irrelevant():
    q, k, v, g, S0 = _rand(23, B=1, T=45, H=2, dk=3, dv=4)
    dO = np.random.default_rng(24).standard_normal((1, 45, 2, 4))
    a = oracle.backward(q, k, v, g, dO, S0, None, ckpt=16)
    b = oracle.backward(q, k, v, g, dO, S0, None, ckpt=7)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


# --------------------------------------------------------------------------
# the pins must reject plausible mistakes (planted in copies of the oracle)
# --------------------------------------------------------------------------

def _fwd_variant(kind):
    def fwd(q, k, v, g, S0=None):
        q, k, v, g = (np.asarray(x, np.float64) for x in (q, k, v, g))
        B, T, H, dk = q.shape
        dv = v.shape[-1]
        S = np.zeros((B, H, dk, dv)) if S0 is None else np.array(S0, np.float64)
        o = np.empty((B, T, H, dv))
        for t in range(T):
            gam = np.exp(g[:, t])[:, :, None, None]
            kv = k[:, t, :, :, None] * v[:, t, :, None, :]
            if kind == "read_before_update":
                o[:, t] = np.matmul(q[:, t, :, None, :], S)[:, :, 0, :]
            if kind == "decay_after_add":
                S = gam * (S + kv)
            elif kind == "decay_not_applied_to_S0" and t == 0:
                S = S + kv
            elif kind == "gamma_squared":
                S = gam * gam * S + kv
            else:
                S = gam * S + kv
            if kind != "read_before_update":
                o[:, t] = np.matmul(q[:, t, :, None, :], S)[:, :, 0, :]
            if kind == "drop_last_token_state" and t == T - 1:
                S = S - kv
        return o, S
    return fwd


def _bwd_variant(kind):
    def bwd(q, k, v, g, dO, S0=None, dS_T=None):
        dq, dk, dv, dg, dS0 = oracle.backward(q, k, v, g, dO, S0, dS_T)
        if kind == "dg_sign":
            dg = -dg
        elif kind == "dg_missing_gamma":
            dg = dg / np.exp(np.asarray(g, np.float64))
        elif kind == "dk_without_own_readout":
            dov = np.einsum("bthc,bthc->bth", dO, v)[..., None]
            dk = dk - np.asarray(q, np.float64) * dov
        elif kind == "dv_without_own_readout":
            qk = np.einsum("bthd,bthd->bth", q, k)[..., None]
            dv = dv - qk * np.asarray(dO, np.float64)
        elif kind == "dS0_undecayed":
            dS0 = dS0 / np.exp(np.asarray(g, np.float64)[:, 0, :, None, None])
        elif kind == "dq_shifted":
            dq = np.roll(dq, 1, axis=1)
        return dq, dk, dv, dg, dS0
    return bwd


@pytest.mark.parametrize("kind", ["read_before_update", "decay_after_add",
                                  "decay_not_applied_to_S0", "gamma_squared",
                                  "drop_last_token_state"])
def test_pins_catch_planted_forward_mistakes(kind):
    bad = _fwd_variant(kind)
    failures = 0
    for pin in FWD_PINS:
        try:
            pin(bad, None)
        except AssertionError:
            failures += 1
    assert failures > 0, f"no forward pin rejects the '{kind}' mutant"


@pytest.mark.parametrize("kind", ["dg_sign", "dg_missing_gamma", "dk_without_own_readout",
                                  "dv_without_own_readout",
                                  "dS0_undecayed", "dq_shifted"])
def test_pins_catch_planted_backward_mistakes(kind):
    bad = _bwd_variant(kind)
    failures = 0
    np.seterr(divide="ignore", invalid="ignore")
    for pin in BWD_PINS:
        try:
            pin(oracle.forward, bad)
        except AssertionError:
            failures += 1
    assert failures > 0, f"no backward pin rejects the '{kind}' mutant"


def test_transposed_read_caught():
    # o = S q instead of q S only type-checks when dk == dv; the golden matrix
    # example has dk != dv, so check the square case against the closed form.
    def bad(q, k, v, g, S0=None):
        q, k, v, g = (np.asarray(x, np.float64) for x in (q, k, v, g))
        B, T, H, d = q.shape
        S = np.zeros((B, H, d, d)) if S0 is None else np.array(S0, np.float64)
        o = np.empty((B, T, H, d))
        for t in range(T):
            S = np.exp(g[:, t])[:, :, None, None] * S + k[:, t, :, :, None] * v[:, t, :, None, :]
            o[:, t] = np.matmul(S, q[:, t, :, :, None])[..., 0]
        return o, S
    q, k, v, g, S0 = _rand(25, B=1, T=6, H=1, dk=4, dv=4)
    o_ref, _ = closed_form(q, k, v, g, S0)
    assert not np.allclose(bad(q, k, v, g, S0)[0], o_ref)
    np.testing.assert_allclose(oracle.forward(q, k, v, g, S0)[0], o_ref, rtol=1e-12, atol=1e-12)
