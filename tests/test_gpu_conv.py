"""Parity of the causal depth-wise convolution with SiLU (gla_conv1d_silu) on
the GPU against the fp64 oracle (oracle.conv1d_silu).

Tolerance: the kernel forms each output from four fp32 products, the bias and
one fp32 exponential, so fp32 outputs stay within 1e-5 of rms(ref) (measured
near 1e-6); bf16 outputs add their own rounding, 2^-8 |ref| per element.  The
history is a copy of inputs and is compared bit for bit.
"""
import numpy as np
import pytest
import torch

import gen
import oracle
from gpu_util import assert_close, dev, to_dev, to_np

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
    state = r.standard_normal((n_slots, 3, D)).astype(np.float32) if n_slots else None
    if dtype == "bf16":
        x = gen.bf16_round(x)
        state = None if state is None else gen.bf16_round(state)
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
    st = to_dev(state, TDT[in_dt])
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
    st_full = to_dev(state, torch.bfloat16)
    y_full = gla.gla_conv1d_silu(xd, wd, bd, conv_state=st_full, init_from_state=True, out_dtype=torch.float32)
    st_step = to_dev(state, torch.bfloat16)
    ys = [gla.gla_conv1d_silu(xd[:, t:t + 1].contiguous(), wd, bd, conv_state=st_step, init_from_state=True,
                              out_dtype=torch.float32) for t in range(T)]
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(ys, 1), y_full)
    assert torch.equal(st_step, st_full)


def test_conv_full_size_sampled():
    """B=8, T=2048, D=3,072 (the pages' residual width), bf16 in and out, with a
    history per sequence, in the launch configuration the benchmark times;
    sequences 0 and 7 against the oracle, the whole history bit for bit."""
    import linear_attention_sequence_simple_amd as gla
    B, T, D = 8, 2048, 3072
    x, w, bias, state = _inputs(5, B * T, D, "bf16", n_slots=B)
    print("case conv full size", flush=True)
    st = to_dev(state, torch.bfloat16)
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
    # every other sequence's history is its own last three tokens (T >= 3)
    np.testing.assert_array_equal(got_st, x.reshape(B, T, D)[:, -3:].astype(np.float64))
