"""Seeded sweeps over the shapes and options of every entry point, against the
fp64 oracle: batch, length (ragged tails included), heads, input and output
dtypes, initial states, decay recipes and forced segment counts for the
prefill and the backward; random packed lengths (empty sequences included)
and slot maps; decode on float32 and 16-bit pools; the convolution with and
without history.  The cases are drawn once from fixed seeds, so every run
checks the same ones; each is small enough for the oracle to finish in
milliseconds.  Tolerances are those of the dedicated tests.
"""
import os

import numpy as np
import pytest
import torch

import gen
import oracle
from gpu_util import assert_close, assert_close_bf16_out, dev, to_dev, to_np

pytestmark = pytest.mark.gpu

TDT = {"bf16": torch.bfloat16, "f32": torch.float32}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import linear_attention_sequence_simple_amd as gla
    gla.lib()
    return gla


def _check_out(got, ref, in_dt, out_dt, name):
    tol = 1e-2 if in_dt == "bf16" else 1e-4
    if out_dt == "bf16":
        assert_close_bf16_out(got, ref, tol, name)
    else:
        assert_close(got, ref, tol, name)


def _fwd_cases():
    r = np.random.default_rng(2024)
    cases = []
    for i in range(32):
        T = int(r.choice([1, 2, 127, 128, 129, int(r.integers(3, 800)), int(r.integers(257, 900)),
                          int(r.integers(257, 900))]))
        n_chunks = (T + 127) // 128
        cases.append(dict(i=i, B=int(r.integers(1, 4)), T=T, H=int(r.integers(1, 6)),
                          in_dt=str(r.choice(["bf16", "f32"])), out_dt=str(r.choice(["bf16", "f32"])),
                          S0=str(r.choice(["zero", "normal0.1"])),
                          g=str(r.choice(["logsig_n4", "logsig_u28_head", "one"])),
                          seg=None if r.random() < 0.4 else int(r.integers(1, n_chunks + 1))))
    return cases


@pytest.mark.parametrize("c", _fwd_cases(), ids=lambda c: f"fwd{c['i']}")
def test_prefill_sweep(c):
    import linear_attention_sequence_simple_amd as gla
    print(f"case prefill {c}", flush=True)
    wl = "fwd_bf16_b8_t2048" if c["in_dt"] == "bf16" else "fwd_f32_b1_t2048"
    d = gen.make_inputs(wl, seed=100 + c["i"], B=c["B"], T=c["T"], H=c["H"], S0=c["S0"], g=c["g"])
    o, S = gla.gla_chunk_fwd(to_dev(d["q"], TDT[c["in_dt"]]), to_dev(d["k"], TDT[c["in_dt"]]),
                             to_dev(d["v"], TDT[c["in_dt"]]), to_dev(d["g"], torch.float32),
                             to_dev(d["S0"], torch.float32), out_dtype=TDT[c["out_dt"]], segments=c["seg"])
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.forward(d["q"], d["k"], d["v"], d["g"], d["S0"])
    _check_out(to_np(o), o_ref, c["in_dt"], c["out_dt"], "o")
    assert_close(to_np(S), S_ref, 1e-2 if c["in_dt"] == "bf16" else 1e-4, "S_T")


def _bwd_cases():
    r = np.random.default_rng(2025)
    cases = []
    for i in range(16):
        T = int(r.choice([1, 128, 129, int(r.integers(2, 600)), int(r.integers(257, 700))]))
        n_chunks = (T + 127) // 128
        cases.append(dict(i=i, B=int(r.integers(1, 3)), T=T, H=int(r.integers(1, 4)),
                          S0=bool(r.random() < 0.5), dS_T=bool(r.random() < 0.5),
                          out_dt=str(r.choice(["bf16", "f32"])),
                          seg=None if r.random() < 0.4 else int(r.integers(1, n_chunks + 1))))
    return cases


@pytest.mark.parametrize("c", _bwd_cases(), ids=lambda c: f"bwd{c['i']}")
def test_backward_sweep(c):
    import linear_attention_sequence_simple_amd as gla
    print(f"case backward {c}", flush=True)
    d = gen.make_inputs("bwd_bf16_b4_t4096", seed=200 + c["i"], B=c["B"], T=c["T"], H=c["H"], S0="normal0.1",
                        with_dO=True, with_dS_T=True)
    S0 = d["S0"] if c["S0"] else None
    dS_T = d["dS_T"] if c["dS_T"] else None
    got = gla.gla_chunk_bwd(to_dev(d["q"], torch.bfloat16), to_dev(d["k"], torch.bfloat16),
                            to_dev(d["v"], torch.bfloat16), to_dev(d["g"], torch.float32),
                            to_dev(d["dO"], torch.bfloat16), S0=to_dev(S0, torch.float32),
                            dS_T=to_dev(dS_T, torch.float32), out_dtype=TDT[c["out_dt"]], want_dS0=True,
                            segments=c["seg"])
    torch.cuda.synchronize()
    ref = oracle.backward(d["q"], d["k"], d["v"], d["g"], d["dO"], S0, dS_T)
    for name, x, y in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
        _check_out(to_np(x), y, "bf16", c["out_dt"], name)
    assert_close(to_np(got[3]), ref[3], 1e-2, "dg")
    if c["S0"] or c["dS_T"]:
        assert_close(to_np(got[4]), ref[4], 1e-2, "dS0")


def _packed_cases():
    r = np.random.default_rng(2026)
    cases = []
    for i in range(16):
        n = int(r.integers(1, 7))
        lengths = [int(x) if r.random() > 0.2 else 0 for x in r.integers(1, 400, size=n)]
        top = max(max(lengths), 1)
        cases.append(dict(i=i, lengths=lengths, H=int(r.integers(1, 4)), init=bool(r.random() < 0.5),
                          in_dt=str(r.choice(["bf16", "f32"])), out_dt=str(r.choice(["bf16", "f32"])),
                          seg=None if r.random() < 0.5 else int(r.integers(1, (top + 127) // 128 + 1))))
    return cases


@pytest.mark.parametrize("c", _packed_cases(), ids=lambda c: f"packed{c['i']}")
def test_packed_sweep(c):
    import linear_attention_sequence_simple_amd as gla
    print(f"case packed {c}", flush=True)
    n_slots = len(c["lengths"]) + 3
    d = gen.make_packed_inputs(seed=300 + c["i"], lengths=c["lengths"], n_slots=n_slots, H=c["H"],
                               dtype=c["in_dt"])
    pool = gla.gla_state_alloc(n_slots, H=c["H"])
    pool.view().copy_(to_dev(d["pool"], torch.float32))
    N = d["q"].shape[0]
    o = gla.gla_chunk_fwd_varlen(to_dev(d["q"], TDT[c["in_dt"]]), to_dev(d["k"], TDT[c["in_dt"]]),
                                 to_dev(d["v"], TDT[c["in_dt"]]), to_dev(d["g"], torch.float32),
                                 torch.from_numpy(d["cu_seqlens"]).to(dev()), max(1, max(c["lengths"])),
                                 pool, torch.from_numpy(d["slot_idx"]).to(dev()), init_from_pool=c["init"],
                                 out_dtype=TDT[c["out_dt"]], segments=c["seg"])
    torch.cuda.synchronize()
    o_ref, pool_ref = oracle.forward_packed(d["q"], d["k"], d["v"], d["g"], d["cu_seqlens"], d["pool"],
                                            d["slot_idx"], c["init"])
    if N:
        _check_out(to_np(o), o_ref, c["in_dt"], c["out_dt"], "o")
    got = to_np(pool.view())
    used = sorted(int(s) for s in d["slot_idx"])
    assert_close(got[used], pool_ref[used], 1e-2 if c["in_dt"] == "bf16" else 1e-4, "slots")
    rest = sorted(set(range(n_slots)) - set(used))
    np.testing.assert_array_equal(got[rest], d["pool"][rest].astype(np.float64))
    pool.free()


def _decode_cases():
    r = np.random.default_rng(2027)
    return [dict(i=i, n_slots=int(r.integers(1, 40)), q16=bool(i % 2), in_dt=str(r.choice(["bf16", "f32"])),
                 out_dt=str(r.choice(["bf16", "f32"])), idx=bool(r.random() < 0.6)) for i in range(12)]


@pytest.mark.parametrize("c", _decode_cases(), ids=lambda c: f"decode{c['i']}")
def test_decode_sweep(c):
    import linear_attention_sequence_simple_amd as gla
    print(f"case decode {c}", flush=True)
    r = np.random.default_rng(400 + c["i"])
    n = c["n_slots"]
    B = int(r.integers(1, n + 1)) if c["idx"] else n
    slots = r.permutation(n)[:B].astype(np.int32) if c["idx"] else np.arange(n, dtype=np.int32)
    S = gen.make_decode_state(n, seed=400 + c["i"])
    pool = gla.gla_state_alloc_q16(n) if c["q16"] else gla.gla_state_alloc(n)
    gla.gla_state_write(pool, torch.from_numpy(S).to(dev()))
    for step in range(3):
        x = gen.make_decode_step(B, step, seed=400 + c["i"], dtype=c["in_dt"])
        before = gla.gla_state_read(pool).cpu().numpy().astype(np.float64)
        if c["q16"]:
            m0, e0 = (t.cpu().numpy() for t in pool.q16_views())
        o = gla.gla_recurrent_step(pool, to_dev(x["q"], TDT[c["in_dt"]]), to_dev(x["k"], TDT[c["in_dt"]]),
                                   to_dev(x["v"], TDT[c["in_dt"]]), to_dev(x["g"], torch.float32),
                                   slot_idx=torch.from_numpy(slots).to(dev()) if c["idx"] else None,
                                   out_dtype=TDT[c["out_dt"]])
        torch.cuda.synchronize()
        if c["q16"]:
            o_ref, _, _ = oracle.step_q16(m0[slots], e0[slots], x["q"], x["k"], x["v"], x["g"])
        else:
            o_ref, _ = oracle.step(before[slots], x["q"], x["k"], x["v"], x["g"])
        _check_out(to_np(o), o_ref, "f32", c["out_dt"], f"o step {step}")
        after = gla.gla_state_read(pool).cpu().numpy().astype(np.float64)
        _, S_ref = oracle.step(before[slots], x["q"], x["k"], x["v"], x["g"])
        if c["q16"]:
            quantum = np.exp2(pool.q16_views()[1].cpu().numpy()[slots].astype(np.float64))[..., None, :]
            assert np.all(np.abs(after[slots] - S_ref) <= quantum), "16-bit state beyond one quantum"
        else:
            assert_close(after[slots], S_ref, 1e-4, "state")
        rest = np.setdiff1d(np.arange(n), slots)
        np.testing.assert_array_equal(after[rest], before[rest])
    pool.free()


def _conv_cases():
    r = np.random.default_rng(2028)
    return [dict(i=i, B=int(r.integers(1, 4)), T=int(r.choice([1, 2, 3, 31, 32, 33, int(r.integers(4, 300))])),
                 D=8 * int(r.integers(1, 40)), hist=bool(r.random() < 0.6), packed=bool(r.random() < 0.4),
                 in_dt=str(r.choice(["bf16", "f32"])), out_dt=str(r.choice(["bf16", "f32"]))) for i in range(12)]


@pytest.mark.parametrize("c", _conv_cases(), ids=lambda c: f"conv{c['i']}")
def test_conv_sweep(c):
    import linear_attention_sequence_simple_amd as gla
    print(f"case conv {c}", flush=True)
    r = np.random.default_rng(500 + c["i"])
    B, T, D = c["B"], c["T"], c["D"]
    lengths = [int(x) for x in r.integers(0, T + 1, size=B)] if c["packed"] else [T] * B
    if sum(lengths) == 0:
        lengths[0] = T
    N = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    x = r.standard_normal((N, D)).astype(np.float32)
    w = (r.standard_normal((D, 4)) * 0.5).astype(np.float32)
    bias = (r.standard_normal(D) * 0.1).astype(np.float32)
    state = r.standard_normal((B + 2, 4, D)).astype(np.float32) if c["hist"] else None
    if c["in_dt"] == "bf16":
        x = gen.bf16_round(x)
    slots = r.permutation(B + 2)[:B].astype(np.int32) if c["hist"] else None
    st = to_dev(state, torch.float32) if c["hist"] else None
    xin = to_dev(x, TDT[c["in_dt"]]) if c["packed"] else to_dev(x.reshape(B, T, D), TDT[c["in_dt"]])
    y = gla.gla_conv1d_silu(xin, to_dev(w, torch.float32), to_dev(bias, torch.float32), conv_state=st,
                            slot_idx=torch.from_numpy(slots).to(dev()) if c["hist"] else None,
                            init_from_state=c["hist"],
                            cu_seqlens=torch.from_numpy(cu).to(dev()) if c["packed"] else None,
                            max_seqlen=T if c["packed"] else None, out_dtype=TDT[c["out_dt"]])
    torch.cuda.synchronize()
    y_ref, st_ref = oracle.conv1d_silu(x, w, bias, cu, state, slots, c["hist"])
    if N:
        got = to_np(y).reshape(N, D)
        if c["out_dt"] == "bf16":
            rms = np.sqrt(np.mean(y_ref * y_ref))
            assert np.all(np.abs(got - y_ref) <= 1e-5 * rms + 2.0 ** -8 * np.abs(y_ref)), "y (bf16)"
        else:
            assert_close(got, y_ref, 1e-5, "y")
    if c["hist"]:
        np.testing.assert_array_equal(to_np(st), st_ref)
