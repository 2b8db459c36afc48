"""Decode parity: gla_recurrent_step on the GPU against the fp64 oracle."""
import numpy as np
import pytest
import torch

import gen
import oracle
from gpu_util import assert_close, assert_close_bf16_out, dev, to_dev, to_np

pytestmark = pytest.mark.gpu

TOL = 1e-4   # the decode step keeps everything in fp32; bf16 only rounds the inputs


def _pool(n, S0):
    import linear_attention_sequence_simple_amd as gla
    pool = gla.gla_state_alloc(n)
    view = pool.view()
    assert view.shape == (n, 16, 96, 192) and view.data_ptr() == pool.ptr(0)
    if S0 is not None:
        view.copy_(torch.from_numpy(S0).to(dev()))
    torch.cuda.synchronize()
    return pool, view


@pytest.mark.parametrize("in_dtype,out_dtype", [(torch.bfloat16, torch.float32),
                                                (torch.float32, torch.float32),
                                                (torch.bfloat16, torch.bfloat16)])
def test_steps_reduced(in_dtype, out_dtype):
    import linear_attention_sequence_simple_amd as gla
    n = 37
    S = gen.make_decode_state(n, seed=1)
    pool, view = _pool(n, S)
    Sref = S.astype(np.float64)
    for step in range(5):
        x = gen.make_decode_step(n, step, seed=1, dtype="bf16" if in_dtype == torch.bfloat16 else "f32")
        o = gla.gla_recurrent_step(pool, to_dev(x["q"], in_dtype), to_dev(x["k"], in_dtype),
                                   to_dev(x["v"], in_dtype), to_dev(x["g"], torch.float32),
                                   out_dtype=out_dtype)
        o_ref, Sref = oracle.step(Sref, x["q"], x["k"], x["v"], x["g"])
        torch.cuda.synchronize()
        if out_dtype == torch.bfloat16:
            # elementwise: the fp32 step's tolerance plus bf16's half ulp
            assert_close_bf16_out(to_np(o), o_ref, TOL, "o(bf16)")
        else:
            assert_close(to_np(o), o_ref, TOL, "o")
    assert_close(to_np(view), Sref, TOL, "state")
    pool.free()


def test_slot_indices_and_special_decays():
    import linear_attention_sequence_simple_amd as gla
    n, m = 20, 12
    S = gen.make_decode_state(n, seed=2)
    pool, view = _pool(n, S)
    slots = np.random.default_rng(0).permutation(n)[:m].astype(np.int32)
    x = gen.make_decode_step(m, 0, seed=2)
    x["g"][0] = 0.0            # gamma == 1
    x["g"][1] = -np.inf        # gamma == 0
    o = gla.gla_recurrent_step(pool, to_dev(x["q"], torch.bfloat16), to_dev(x["k"], torch.bfloat16),
                               to_dev(x["v"], torch.bfloat16), to_dev(x["g"], torch.float32),
                               slot_idx=torch.from_numpy(slots).to(dev()), out_dtype=torch.float32)
    o_ref, S_new = oracle.step(S[slots], x["q"], x["k"], x["v"], x["g"])
    torch.cuda.synchronize()
    assert_close(to_np(o), o_ref, TOL, "o")
    after = to_np(view)
    assert_close(after[slots], S_new, TOL, "updated slots")
    untouched = np.setdiff1d(np.arange(n), slots)
    assert np.array_equal(after[untouched], S[untouched].astype(np.float64))
    pool.free()


def test_fwd_equals_decode_steps():
    # S_T of the chunked prefill equals T successive decode steps from the same S0.
    import linear_attention_sequence_simple_amd as gla
    B, T, H = 3, 150, 16
    d = gen.make_inputs("fwd_bf16_b8_t2048", seed=3, B=B, T=T, H=H, S0="normal0.1")
    o, S_T = gla.gla_chunk_fwd(to_dev(d["q"], torch.bfloat16), to_dev(d["k"], torch.bfloat16),
                               to_dev(d["v"], torch.bfloat16), to_dev(d["g"], torch.float32),
                               to_dev(d["S0"], torch.float32), out_dtype=torch.float32)
    pool, view = _pool(B, d["S0"])
    outs = []
    for t in range(T):
        outs.append(gla.gla_recurrent_step(pool, to_dev(d["q"][:, t], torch.bfloat16),
                                           to_dev(d["k"][:, t], torch.bfloat16),
                                           to_dev(d["v"][:, t], torch.bfloat16),
                                           to_dev(d["g"][:, t], torch.float32), out_dtype=torch.float32))
    torch.cuda.synchronize()
    steps_o = np.stack([to_np(x) for x in outs], 1)
    assert_close(to_np(view), to_np(S_T), 1e-2, "state: decode vs prefill")
    assert_close(steps_o, to_np(o), 1e-2, "o: decode vs prefill")
    o_ref, S_ref = oracle.forward(d["q"], d["k"], d["v"], d["g"], d["S0"])
    assert_close(steps_o, o_ref, TOL, "decode o vs oracle")
    pool.free()


def test_decode_workload_sampled():
    # 1,280 sequences x 16 heads, one layer's pool, 64 steps; the oracle
    # follows 64 sampled sequences through all steps.
    import linear_attention_sequence_simple_amd as gla
    n, steps = 1280, 64
    S = gen.make_decode_state(n, seed=0)
    pool, view = _pool(n, S)
    sample = np.arange(0, n, n // 64)
    Sref = S[sample].astype(np.float64)
    last = None
    for step in range(steps):
        x = gen.make_decode_step(n, step, seed=0)
        o = gla.gla_recurrent_step(pool, to_dev(x["q"], torch.bfloat16), to_dev(x["k"], torch.bfloat16),
                                   to_dev(x["v"], torch.bfloat16), to_dev(x["g"], torch.float32),
                                   out_dtype=torch.float32)
        o_ref, Sref = oracle.step(Sref, x["q"][sample], x["k"][sample], x["v"][sample], x["g"][sample])
        last = (o, o_ref)
    torch.cuda.synchronize()
    assert_close(to_np(last[0])[sample], last[1], TOL, "o at the last step")
    assert_close(to_np(view)[sample], Sref, TOL, "sampled states after 64 steps")
    pool.free()
