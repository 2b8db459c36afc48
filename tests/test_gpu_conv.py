"""Parity of the causal depth-wise convolution with SiLU (gla_conv1d_silu) on
the GPU against the fp64 oracle (oracle.conv1d_silu).

Tolerance: the kernel forms each output from four fp32 products, the bias and
one fp32 exponential, so fp32 outputs stay within 1e-5 of rms(ref) (measured
near 1e-6); bf16 outputs add their own rounding, 2^-8 |ref| per element.  The
window (the last four inputs, float32) is a copy of inputs and is compared bit
for bit.
"""
import numpy as np
import pytest
import torch

import gen
import oracle
from gpu_util import assert_close, check_q16_state, dev, to_dev, to_np

pytestmark = pytest.mark.gpu

TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import linear_attention_sequence_simple_amd as gla
    gla.lib()
    return gla


def _inputs(seed, N, D, dtype, n_slots=0):
    r = np.random.default_rng(seed)
    x = r.standard_normal((N, D)).astype(np.float32)
    w = (r.standard_normal((D, 4)) * 0.5).astype(np.float32)
    bias = (r.standard_normal(D) * 0.1).astype(np.float32)
    state = r.standard_normal((n_slots, 4, D)).astype(np.float32) if n_slots else None
    if dtype == "bf16":
        x = gen.bf16_round(x)
    return x, w, bias, state


def _assert_bf16_out(got, ref, name):
    rms = np.sqrt(np.mean(ref * ref))
    bad = np.abs(got - ref) > TOL * rms + 2.0 ** -8 * np.abs(ref)
    assert not bad.any(), f"{name}: {bad.sum()} elements outside the bf16-output bound"


TDT = {"bf16": torch.bfloat16, "f32": torch.float32}


@pytest.mark.parametrize("in_dt,out_dt", [("bf16", "f32"), ("f32", "f32"), ("bf16", "bf16"), ("f32", "bf16")])
def test_conv_batch(in_dt, out_dt):
    import linear_attention_sequence_simple_amd as gla
    B, T, D = 3, 77, 64
    x, w, bias, _ = _inputs(1, B * T, D, in_dt)
    print(f"case conv batch in={in_dt} out={out_dt}", flush=True)
    y = gla.gla_conv1d_silu(to_dev(x.reshape(B, T, D), TDT[in_dt]), to_dev(w, torch.float32),
                            to_dev(bias, torch.float32), out_dtype=TDT[out_dt])
    torch.cuda.synchronize()
    y_ref, _ = oracle.conv1d_silu(x, w, bias, np.arange(B + 1) * T)
    got = to_np(y).reshape(B * T, D)
    if out_dt == "bf16":
        _assert_bf16_out(got, y_ref, "y")
    else:
        assert_close(got, y_ref, TOL, "y")


@pytest.mark.parametrize("init", [False, True])
@pytest.mark.parametrize("in_dt", ["bf16", "f32"])
def test_conv_packed_with_history(init, in_dt):
    import linear_attention_sequence_simple_amd as gla
    lengths = [0, 1, 2, 3, 31, 32, 33, 100, 65]
    D, n_slots = 136, 12
    N = sum(lengths)
    x, w, bias, state = _inputs(2, N, D, in_dt, n_slots)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    slots = np.random.default_rng(3).permutation(n_slots)[:len(lengths)].astype(np.int32)
    print(f"case conv packed in={in_dt} init={init}", flush=True)
    st = to_dev(state, torch.float32)
    y = gla.gla_conv1d_silu(to_dev(x, TDT[in_dt]), to_dev(w, torch.float32), to_dev(bias, torch.float32),
                            conv_state=st, slot_idx=torch.from_numpy(slots).to(dev()), init_from_state=init,
                            cu_seqlens=torch.from_numpy(cu).to(dev()), max_seqlen=max(lengths),
                            out_dtype=torch.float32)
    torch.cuda.synchronize()
    y_ref, st_ref = oracle.conv1d_silu(x, w, bias, cu, state, slots, init)
    assert_close(to_np(y), y_ref, TOL, "y")
    np.testing.assert_array_equal(to_np(st), st_ref)


def test_conv_decode_steps_equal_one_call():
    """T single-token calls carrying the history equal one call over T tokens, bit for bit."""
    import linear_attention_sequence_simple_amd as gla
    B, T, D = 4, 20, 256
    x, w, bias, state = _inputs(4, B * T, D, "bf16", n_slots=B)
    xd = to_dev(x.reshape(B, T, D), torch.bfloat16)
    wd, bd = to_dev(w, torch.float32), to_dev(bias, torch.float32)
    st_full = to_dev(state, torch.float32)
    y_full = gla.gla_conv1d_silu(xd, wd, bd, conv_state=st_full, init_from_state=True, out_dtype=torch.float32)
    st_step = to_dev(state, torch.float32)
    ys = [gla.gla_conv1d_silu(xd[:, t:t + 1].contiguous(), wd, bd, conv_state=st_step, init_from_state=True,
                              out_dtype=torch.float32) for t in range(T)]
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(ys, 1), y_full)
    assert torch.equal(st_step, st_full)


def test_conv_full_size_sampled():
    """B=8, T=2048, D=3,072 (the pages' residual width), bf16 in and out, with a
    history per sequence, in the launch configuration the benchmark times;
    sequences 0 and 7 against the oracle, the whole window bit for bit."""
    import linear_attention_sequence_simple_amd as gla
    B, T, D = 8, 2048, 3072
    x, w, bias, state = _inputs(5, B * T, D, "bf16", n_slots=B)
    print("case conv full size", flush=True)
    st = to_dev(state, torch.float32)
    y = gla.gla_conv1d_silu(to_dev(x.reshape(B, T, D), torch.bfloat16), to_dev(w, torch.float32),
                            to_dev(bias, torch.float32), conv_state=st, init_from_state=True,
                            out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    got = to_np(y).reshape(B * T, D)
    got_st = to_np(st)
    for b in (0, 7):
        rows = slice(b * T, (b + 1) * T)
        y_ref, st_ref = oracle.conv1d_silu(x[rows], w, bias, [0, T], state[b:b + 1], None, True)
        _assert_bf16_out(got[rows], y_ref, f"y seq {b}")
        np.testing.assert_array_equal(got_st[b], st_ref[0])
    # every other sequence's window is its own last four tokens (T >= 4)
    np.testing.assert_array_equal(got_st, x.reshape(B, T, D)[:, -4:].astype(np.float64))


def test_conv_window_in_the_pool_with_the_mixer_state():
    """A serving layer's slots hold both parts of a sequence's state: the
    convolution's window and the mixer's state.  A packed prompt pass (the
    convolution, then the packed prefill on other inputs) and decode steps
    (the convolution with T = 1, then the mixer step) through the same slot
    indices: every window and state against the oracle, slots of no sequence
    unchanged, and neither call touching the other's part of a slot."""
    import linear_attention_sequence_simple_amd as gla
    D, n_slots, H = 3072, 7, 16
    lengths = [37, 0, 130, 5]
    n_seq = len(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    slots = np.array([5, 0, 2, 6], np.int32)
    x, w, bias, win0 = _inputs(8, int(cu[-1]), D, "bf16", n_slots)
    pk = gen.make_packed_inputs(seed=9, lengths=lengths, n_slots=n_slots, H=H)
    pool = gla.gla_state_alloc_conv(n_slots, D)
    assert pool.conv_D == D and pool.seq_bytes == 16 * 96 * 192 * 4 + 4 * D * 4
    pool.conv_view().copy_(to_dev(win0, torch.float32))
    pool.view().copy_(to_dev(pk["pool"], torch.float32))
    sl = torch.from_numpy(slots).to(dev())
    cud = torch.from_numpy(cu).to(dev())
    wd, bd = to_dev(w, torch.float32), to_dev(bias, torch.float32)
    print("case conv window in the pool: prompts", flush=True)
    y = gla.gla_conv1d_silu_pool(to_dev(x, torch.bfloat16), wd, pool, bias=bd, slot_idx=sl, init_from_pool=True,
                                 cu_seqlens=cud, max_seqlen=max(lengths), out_dtype=torch.float32)
    o = gla.gla_chunk_fwd_varlen(to_dev(pk["q"], torch.bfloat16), to_dev(pk["k"], torch.bfloat16),
                                 to_dev(pk["v"], torch.bfloat16), to_dev(pk["g"], torch.float32),
                                 torch.from_numpy(pk["cu_seqlens"]).to(dev()), max(lengths), pool,
                                 torch.from_numpy(pk["slot_idx"]).to(dev()), init_from_pool=True,
                                 out_dtype=torch.float32)
    torch.cuda.synchronize()
    y_ref, win_ref = oracle.conv1d_silu(x, w, bias, cu, win0, slots, True)
    o_ref, S_ref = oracle.forward_packed(pk["q"], pk["k"], pk["v"], pk["g"], pk["cu_seqlens"], pk["pool"],
                                         pk["slot_idx"], True)
    assert_close(to_np(y), y_ref, TOL, "y")
    np.testing.assert_array_equal(to_np(pool.conv_view()), win_ref)
    assert_close(to_np(o), o_ref, 1e-2, "o")
    used = sorted(int(s) for s in pk["slot_idx"])
    assert_close(to_np(pool.view())[used], S_ref[used], 1e-2, "mixer states")
    S_cur = to_np(pool.view())
    for step in range(3):
        print(f"case conv window in the pool: decode step {step}", flush=True)
        xs = gen.bf16_round(np.random.default_rng(100 + step).standard_normal((n_seq, D)).astype(np.float32))
        ys = gla.gla_conv1d_silu_pool(to_dev(xs[:, None], torch.bfloat16), wd, pool, bias=bd, slot_idx=sl,
                                      init_from_pool=True, out_dtype=torch.float32)
        xd = gen.make_decode_step(n_seq, step, seed=10)
        od = gla.gla_recurrent_step(pool, *(to_dev(xd[c], torch.bfloat16) for c in ("q", "k", "v")),
                                    to_dev(xd["g"], torch.float32), slot_idx=sl, out_dtype=torch.float32)
        torch.cuda.synchronize()
        ys_ref, win_ref = oracle.conv1d_silu(xs, w, bias, np.arange(n_seq + 1), win_ref, slots, True)
        od_ref, S_new = oracle.step(S_cur[slots], xd["q"], xd["k"], xd["v"], xd["g"])
        S_cur[slots] = S_new
        assert_close(to_np(ys).reshape(n_seq, D), ys_ref, TOL, "y step")
        np.testing.assert_array_equal(to_np(pool.conv_view()), win_ref)
        assert_close(to_np(od), od_ref, 1e-4, "o step")
        assert_close(to_np(pool.view()), S_cur, 1e-4, "mixer states after the step")
    pool.free()


def test_conv_window_in_a_16bit_pool():
    """A 16-bit pool with convolution windows: the windows (float32) and the
    16-bit mixer states live side by side in the slots; a convolution call and
    a decode step through the same slot indices leave each other's part
    untouched, and both match the oracle."""
    import linear_attention_sequence_simple_amd as gla
    D, n_slots, n = 256, 5, 3
    slots = np.array([4, 1, 2], np.int32)
    x, w, bias, win0 = _inputs(11, n, D, "bf16", n_slots)
    pool = gla.gla_state_alloc_conv(n_slots, D, fmt=gla.GLA_STATE_Q16)
    assert pool.fmt == gla.GLA_STATE_Q16 and pool.conv_D == D
    assert pool.seq_bytes == 16 * (96 * 192 * 2 + 192 * 4) + 4 * D * 4
    S0 = gen.make_decode_state(n_slots, seed=12)
    gla.gla_state_write(pool, torch.from_numpy(S0).to(dev()))
    pool.conv_view().copy_(to_dev(win0, torch.float32))
    m0, e0 = (t.cpu().numpy() for t in pool.q16_views())
    sl = torch.from_numpy(slots).to(dev())
    print("case conv window in a 16-bit pool", flush=True)
    y = gla.gla_conv1d_silu_pool(to_dev(x[:, None], torch.bfloat16), to_dev(w, torch.float32), pool,
                                 bias=to_dev(bias, torch.float32), slot_idx=sl, init_from_pool=True,
                                 out_dtype=torch.float32)
    xd = gen.make_decode_step(n, 0, seed=13)
    o = gla.gla_recurrent_step(pool, *(to_dev(xd[c], torch.bfloat16) for c in ("q", "k", "v")),
                               to_dev(xd["g"], torch.float32), slot_idx=sl, out_dtype=torch.float32)
    torch.cuda.synchronize()
    y_ref, win_ref = oracle.conv1d_silu(x, w, bias, np.arange(n + 1), win0, slots, True)
    assert_close(to_np(y).reshape(n, D), y_ref, TOL, "y")
    np.testing.assert_array_equal(to_np(pool.conv_view()), win_ref)
    o_ref, m_ref, e_ref = oracle.step_q16(m0[slots], e0[slots], xd["q"], xd["k"], xd["v"], xd["g"])
    assert_close(to_np(o), o_ref, 1e-4, "o")
    m1, e1 = (t.cpu().numpy() for t in pool.q16_views())
    rest = np.setdiff1d(np.arange(n_slots), slots)
    assert np.array_equal(m1[rest], m0[rest]) and np.array_equal(e1[rest], e0[rest])
    # the stored states of the stepped slots: within one quantum of the oracle's
    _, S_ref = oracle.step(oracle.q16_decode(m0[slots], e0[slots]), xd["q"], xd["k"], xd["v"], xd["g"])
    check_q16_state(m1[slots], e1[slots], m_ref, e_ref, S_ref, "state")
    pool.free()
