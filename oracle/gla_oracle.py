"""Plain fp64 CPU oracle for the Simple GLA mixer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
run this module: only the test suite, the package smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP path.

What it computes
----------------
The pages describe the mixer only in words ("Cómo i14 llevó Laplace 3B a AWS
Trainium2", sections "Por qué atención lineal importa" and "Diseño esencial
de Laplace 3B"; "AWS serve Laplace 3B di i14 con uno stato fisso di 29,5 MB",
section "GLA sostituisce i token conservati con uno stato ricorrente"): every
layer keeps a matrix state of fixed size, updates it once per token, lets it
decay, and reads it by content with the query.  The plainest reading of that,
with a scalar ("Simple") decay per head and token, is

    S_t = gamma_t * S_{t-1} + k_t^T v_t          (S is dk x dv)
    o_t = q_t S_t                                 (reads the updated state)
    gamma_t = exp(g_t),  g_t <= 0 the log-decay

with S_{-1} = S0 (zero when absent).  The pages give no scale on q, so there
is none.  The chunk size (16 chunks of 128 tokens in the Trainium2 rewrite,
section "Adaptaciones para AWS Trainium2", item 1) does not change the result
and does not appear here: the oracle walks token by token.

Two more functions follow the same recurrence or sit next to it:
forward_packed runs `forward` on each sequence of a packed batch from its
pool slot's state ("AWS serve Laplace 3B di i14 con uno stato fisso di 29,5
MB", sections "Lo stato di Laplace 3B resta fisso durante l'inferenza" and
"I risultati dichiarati hanno limiti precisi"), and conv1d_silu is the causal
depth-wise convolution of width 4 with SiLU that precedes the mixer ("Diseño
esencial de Laplace 3B"), and gate_silu (with forward_gated) is the output
gate of the fused projection applied to the mixer's output (same section; the
formula is a reading, see its docstring).  q16_encode, q16_decode and step_q16 hold the
decode state in 16 bits (an int16 mantissa per element, one power-of-two
exponent per state column), after the INT16 storage of the HEAL summary
(section "A. Mitigando o Truncamento de Atenção via Quantização INT16").
Every function is pinned by tests that do not reuse its formula:
tests/test_oracle.py, tests/test_oracle_packed.py, tests/test_oracle_conv.py,
tests/test_oracle_q16.py and tests/test_oracle_gate.py with the fixtures
under tests/golden/.

Everything is float64.  Inputs may be any float dtype; callers pass the exact
values the device sees (bf16 inputs already rounded to bf16).

Layouts: q, k [B, T, H, dk]; v, o, dO [B, T, H, dv]; g [B, T, H];
S0, S_T, dS_T, dS0 [B, H, dk, dv]; packed sequences: [N, H, ...] rows split
by sequence offsets, states in a pool [n_slots, H, dk, dv].
"""
from __future__ import annotations

import numpy as np

__all__ = ["forward", "forward_packed", "step", "backward", "conv1d_silu", "state_bytes", "gate_silu", "forward_gated",
           "q16_encode", "q16_decode", "step_q16", "Q16_MAX", "Q16_NAN"]


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def forward(q, k, v, g, S0=None):
    """Token-by-token recurrence.  Returns (o, S_T) in float64.

    For each token t: gamma = exp(g_t) (exp(-inf) = 0 exactly), the state
    decays, the outer product k_t^T v_t is added, and the query reads the
    updated state.
    """
    q, k, v, g, S0 = _f64(q), _f64(k), _f64(v), _f64(g), _f64(S0)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if S0 is None else S0.copy()
    o = np.empty((B, T, H, dv))
    for t in range(T):
        gamma = np.exp(g[:, t, :])                       # [B, H]
        S *= gamma[:, :, None, None]
        S += k[:, t, :, :, None] * v[:, t, :, None, :]
        o[:, t] = np.matmul(q[:, t, :, None, :], S)[:, :, 0, :]
    return o, S


def step(S, q, k, v, g):
    """One decode step for a batch of sequences.

    S [N, H, dk, dv]; q, k [N, H, dk]; v [N, H, dv]; g [N, H].
    Returns (o [N, H, dv], S_new), both float64; S is not modified.
    """
    S = _f64(S).copy()
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(g)
    S *= np.exp(g)[:, :, None, None]
    S += k[:, :, :, None] * v[:, :, None, :]
    o = np.matmul(q[:, :, None, :], S)[:, :, 0, :]
    return o, S


def backward(q, k, v, g, dO, S0=None, dS_T=None, ckpt=16):
    """Reverse-mode gradient of L = <dO, o> + <dS_T, S_T> for `forward`.

    Returns (dq, dk, dv, dg, dS0) in float64.  The pages state only that the
    backward is sequential over the chunk steps ("Adaptaciones para AWS
    Trainium2", item 3; "Trainium2 ha richiesto modifiche ai kernel e alla
    comunicazione"); the steps below are the chain rule of the recurrence.

    Let U_t be the gradient with respect to S_t through every later use.
    Walking t from T-1 down to 0, with U starting at dS_T:
        U   <- U + q_t^T dO_t          (the read-out of token t)
        dq_t = S_t dO_t^T ; dk_t = U v_t^T ; dv_t = k_t U
        dg_t = gamma_t * <U, S_{t-1}>  (d gamma / d g = gamma)
        U   <- gamma_t U               (gradient reaching S_{t-1})
    and dS0 = U at the end.  S_t is recomputed in float64 from checkpoints
    taken every `ckpt` tokens, which reproduces the forward bit for bit.
    """
    q, k, v, g, dO = _f64(q), _f64(k), _f64(v), _f64(g), _f64(dO)
    S0, dS_T = _f64(S0), _f64(dS_T)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if S0 is None else S0.copy()
    gam = np.exp(g)                                       # [B, T, H]

    # Forward pass keeping the state entering every block of `ckpt` tokens.
    n_blk = (T + ckpt - 1) // ckpt
    ck = np.empty((n_blk, B, H, dk, dv))
    for t in range(T):
        if t % ckpt == 0:
            ck[t // ckpt] = S
        S *= gam[:, t, :, None, None]
        S += k[:, t, :, :, None] * v[:, t, :, None, :]

    dq = np.empty_like(q)
    dkk = np.empty_like(k)
    dvv = np.empty_like(v)
    dg = np.empty((B, T, H))
    U = np.zeros((B, H, dk, dv)) if dS_T is None else dS_T.copy()
    for blk in range(n_blk - 1, -1, -1):
        t0, t1 = blk * ckpt, min(T, (blk + 1) * ckpt)
        # states[i] = S_{t0 + i - 1}, i.e. states[0] is the state before t0.
        states = np.empty((t1 - t0 + 1, B, H, dk, dv))
        states[0] = ck[blk]
        for t in range(t0, t1):
            Sn = states[t - t0] * gam[:, t, :, None, None]
            Sn += k[:, t, :, :, None] * v[:, t, :, None, :]
            states[t - t0 + 1] = Sn
        for t in range(t1 - 1, t0 - 1, -1):
            S_t, S_prev = states[t - t0 + 1], states[t - t0]
            U += q[:, t, :, :, None] * dO[:, t, :, None, :]
            dq[:, t] = np.matmul(S_t, dO[:, t, :, :, None])[..., 0]
            dkk[:, t] = np.matmul(U, v[:, t, :, :, None])[..., 0]
            dvv[:, t] = np.matmul(k[:, t, :, None, :], U)[:, :, 0, :]
            dg[:, t] = gam[:, t] * np.einsum("bhij,bhij->bh", U, S_prev)
            U *= gam[:, t, :, None, None]
    return dq, dkk, dvv, dg, U


def forward_packed(q, k, v, g, cu_seqlens, pool, slot_idx=None, init_from_pool=False):
    """Prefill of sequences of different lengths packed along one token axis,
    each with its state in a slot of a pool.

    The pages serve many concurrent sequences with each one's recurrent state
    held in a memory pool, and prompts of different lengths ("AWS serve
    Laplace 3B di i14 con uno stato fisso di 29,5 MB", sections "Lo stato di
    Laplace 3B resta fisso durante l'inferenza" and "I risultati dichiarati
    hanno limiti precisi").  Sequence b is rows cu_seqlens[b] to
    cu_seqlens[b+1] of q, k [N, H, dk], v [N, H, dv], g [N, H]; it runs the
    recurrence of `forward` on its own, from its slot's state when
    init_from_pool is set (else from zero), and its final state replaces
    that slot.  slot_idx[b] is sequence b's slot (None: slot b).

    Returns (o [N, H, dv], new pool [n_slots, H, dk, dv]) in float64; the
    pool passed in is not modified and slots of no sequence keep their state.
    """
    q, k, v, g, pool = _f64(q), _f64(k), _f64(v), _f64(g), _f64(pool)
    cu = [int(c) for c in cu_seqlens]
    n_seq = len(cu) - 1
    slots = list(range(n_seq)) if slot_idx is None else [int(s) for s in slot_idx]
    o = np.zeros((q.shape[0], q.shape[1], v.shape[-1]))
    new_pool = pool.copy()
    for b in range(n_seq):
        t0, t1 = cu[b], cu[b + 1]
        S0 = pool[slots[b]][None] if init_from_pool else None
        if t1 == t0:
            new_pool[slots[b]] = pool[slots[b]] if init_from_pool else 0.0
            continue
        ob, S = forward(q[None, t0:t1], k[None, t0:t1], v[None, t0:t1], g[None, t0:t1], S0)
        o[t0:t1] = ob[0]
        new_pool[slots[b]] = S[0]
    return o, new_pool


def conv1d_silu(x, w, bias, cu_seqlens, state=None, slot_idx=None, init_from_state=False):
    """Causal depth-wise convolution of width 4 followed by SiLU, per sequence.

    The pages put it ahead of the mixer: every residual vector goes through a
    causal depth-wise Conv1d of width 4 with SiLU, a 4-gram summary of the
    recent tokens ("Cómo i14 llevó Laplace 3B a AWS Trainium2", section
    "Diseño esencial de Laplace 3B").  For channel c of sequence token t,

        a_t[c] = bias[c] + sum_{j=0..3} w[c, j] * x_{t-3+j}[c]
        y_t[c] = a_t[c] / (1 + exp(-a_t[c]))           (SiLU)

    so w[c, 3] weights the current token.  Tokens before the sequence's first
    come from its slot of `state` when init_from_state is set, else are zero.
    A slot is the convolution's window of the last four inputs,
    [n_slots, 4, D] with row m holding x_{m-4}: the width of the filter, the
    form in which the per-sequence state reaches the 29.5 MB the pages print
    (24 layers of a float32 mixer state and a float32 window of 4 x 3,072;
    "Lo stato di Laplace 3B resta fisso durante l'inferenza").  Row 0, the
    oldest, is not read by the next token; it is kept so that the window is
    the filter's full width.  x is [N, D] with sequence b at rows
    cu_seqlens[b] to cu_seqlens[b+1]; w is [D, 4]; bias [D] or None.

    Returns (y [N, D], new state or None) in float64: with a state, each
    sequence's slot receives the last four rows of its window followed by its
    tokens (the window of zeros when init_from_state is not set); other slots
    keep theirs; the state passed in is not modified.
    """
    x, w = _f64(x), _f64(w)
    N, D = x.shape
    bias = np.zeros(D) if bias is None else _f64(bias)
    cu = [int(c) for c in cu_seqlens]
    n_seq = len(cu) - 1
    slots = list(range(n_seq)) if slot_idx is None else [int(s) for s in slot_idx]
    state = _f64(state)
    y = np.zeros((N, D))
    new_state = None if state is None else state.copy()
    for b in range(n_seq):
        t0, t1 = cu[b], cu[b + 1]
        hist = state[slots[b]] if (state is not None and init_from_state) else np.zeros((4, D))
        z = np.concatenate([hist, x[t0:t1]], 0)        # z[m] = x_{m-4}
        for t in range(t1 - t0):
            a = bias.copy()
            for j in range(4):
                a += w[:, j] * z[t + 1 + j]             # x_{t-3+j}
            y[t0 + t] = a / (1.0 + np.exp(-a))
        if new_state is not None:
            new_state[slots[b]] = z[-4:]
    return y, new_state


# ---------------------------------------------------------------------------
# 16-bit state ("Q16").  The HEAL summary ("Resumo Técnico: Desmistificando a
# Instabilidade Numérica na Inferência de LLMs com HEAL", section "A.
# Mitigando o Truncamento de Atenção via Quantização INT16") keeps tensors in
# 16-bit integers to hold memory at 16 bits per element with less truncation
# than a 16-bit float, and rescales rare outlier channels to stay in range.
# Here the decode state is stored that way: every element of column d (a
# value channel) is an int16 mantissa m with one shared power-of-two
# exponent e[d], value m * 2^e[d].  e[d] is set from the column's largest
# magnitude M so that M / 2^e lies in [2^14, 2^15) (one step higher when M
# would round up to 2^15): the largest entry keeps 15 bits and the rounding
# error is at most half a quantum 2^e <= 2^-14 M.  Arithmetic stays fp64 here
# (fp32 on the device); only the stored state is 16-bit.

Q16_MAX = 32767       # largest mantissa magnitude
Q16_NAN = -32768      # reserved mantissa: the column held a non-finite value


def q16_encode(S):
    """Encode states S [..., dk, dv] as (m int16 [..., dk, dv], e int32 [..., dv]).

    Per column: M = max |S[:, d]|; with M = f 2^x, f in [1/2, 1) (frexp),
    e = x - 15, so M / 2^e = f 2^15 in [2^14, 2^15), and e = x - 14 when
    M / 2^(x-15) >= 32767.5 (it would round to 2^15); M = 0 gives e = -15.
    m = round-half-even(S / 2^e), within +-32767.  A column with a
    non-finite entry is stored as Q16_NAN throughout with e = 0.
    """
    S = _f64(S)
    finite = np.isfinite(S).all(axis=-2)                       # [..., dv]
    M = np.where(finite, np.abs(np.where(np.isfinite(S), S, 0.0)).max(axis=-2), 0.0)
    _, x = np.frexp(M)
    e = x - 15
    e = e + (np.ldexp(M, -e) >= Q16_MAX + 0.5)
    e = np.where(finite, e, 0).astype(np.int32)
    scaled = np.ldexp(np.where(np.isfinite(S), S, 0.0), -e[..., None, :])
    m = np.rint(scaled)
    assert np.all(np.abs(m) <= Q16_MAX)
    m = np.where(finite[..., None, :], m, Q16_NAN)
    return m.astype(np.int16), e


def q16_decode(m, e):
    """Values m * 2^e[d] in float64 (NaN where m is Q16_NAN)."""
    m = np.asarray(m)
    v = np.ldexp(m.astype(np.float64), np.asarray(e, np.int64)[..., None, :])
    return np.where(m == Q16_NAN, np.nan, v)


def step_q16(m, e, q, k, v, g):
    """One decode step on 16-bit states.

    m [N, H, dk, dv] int16, e [N, H, dv] int32; q, k [N, H, dk]; v [N, H, dv];
    g [N, H].  The stored state is decoded, updated as in `step` in float64,
    the query reads the updated state before it is rounded, and the new state
    is encoded.  Returns (o [N, H, dv] float64, m_new, e_new).
    """
    o, S = step(q16_decode(m, e), q, k, v, g)
    m_new, e_new = q16_encode(S)
    return o, m_new, e_new


def gate_silu(o, gate):
    """The output gate applied to the mixer's output: o_t * SiLU(gate_t).

    The fused projection of "Diseño esencial de Laplace 3B" ("Cómo i14 llevó
    Laplace 3B a AWS Trainium2") splits into q, k, v and a gate g_t, dv values
    per head (9,216 = H(2dk + 2dv)); the pages do not print how the gate meets
    the mixer's output.  The plainest reading: elementwise, through the one
    activation that section names (SiLU, after the convolution),

        y_t[h, c] = o_t[h, c] * gate_t[h, c] / (1 + exp(-gate_t[h, c]))

    o and gate have the same shape ([..., dv]); returns y in float64.
    """
    o, gate = _f64(o), _f64(gate)
    with np.errstate(over="ignore"):
        return o * (gate / (1.0 + np.exp(-gate)))


def forward_gated(q, k, v, g, gate, S0=None):
    """`forward` followed by `gate_silu` on its output: (y, S_T)."""
    o, S = forward(q, k, v, g, S0)
    return gate_silu(o, gate), S


def state_bytes(H, dk, dv, itemsize=4):
    """Bytes of one layer's recurrent state for one sequence (fp32 state)."""
    return H * dk * dv * itemsize
