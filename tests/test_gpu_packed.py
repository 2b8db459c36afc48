"""Packed-sequence prefill parity: gla_chunk_fwd_varlen on the GPU against the
fp64 oracle (oracle.forward_packed), with the states in pool slots."""
import os

import numpy as np
import pytest
import torch

import gen
import oracle
from gpu_util import assert_close, assert_close_bf16_out, dev, to_dev, to_np

pytestmark = pytest.mark.gpu

TOL_BF16 = 1e-2
TOL_F32 = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import linear_attention_sequence_simple_amd as gla
    gla.lib()
    return gla


def run_packed(d, in_dtype, out_dtype, init, max_seqlen=None, segments=None, n_slots=None, cu=None):
    """Pool filled with d["pool"]; returns (o, pool after the call) as float64."""
    import linear_attention_sequence_simple_amd as gla
    n_slots = d["pool"].shape[0] if n_slots is None else n_slots
    pool = gla.gla_state_alloc(n_slots, H=d["q"].shape[1])
    pool.view().copy_(to_dev(d["pool"], torch.float32))
    cu = d["cu_seqlens"] if cu is None else cu
    lengths = np.diff(cu)
    max_seqlen = int(max(1, lengths.max())) if max_seqlen is None else max_seqlen
    try:
        N, H = d["q"].shape[:2]
        o = torch.full((N, H, 192), 7.0, dtype=out_dtype, device=dev())   # rows of no sequence keep 7
        gla.gla_chunk_fwd_varlen(to_dev(d["q"], in_dtype), to_dev(d["k"], in_dtype), to_dev(d["v"], in_dtype),
                                 to_dev(d["g"], torch.float32),
                                 torch.from_numpy(np.asarray(cu, np.int32)).to(dev()), max_seqlen, pool,
                                 torch.from_numpy(d["slot_idx"]).to(dev()), init_from_pool=init,
                                 out_dtype=out_dtype, o=o, segments=segments)
        torch.cuda.synchronize()
        out = to_np(o), to_np(pool.view())
    finally:
        pool.free()
    return out


def check_pool(got, ref, slots, tol, name):
    used = sorted(int(s) for s in slots)
    assert_close(got[used], ref[used], tol, name)
    rest = sorted(set(range(ref.shape[0])) - set(used))
    np.testing.assert_array_equal(got[rest], np.asarray(ref[rest], np.float32).astype(np.float64))


LENGTHS = [0, 1, 77, 128, 129, 300, 513, 0, 256]


@pytest.mark.parametrize("init", [False, True])
@pytest.mark.parametrize("in_dt,out_dt", [("bf16", "f32"), ("f32", "f32"), ("f32", "bf16")])
def test_packed_ragged(init, in_dt, out_dt):
    d = gen.make_packed_inputs(seed=11, lengths=LENGTHS, n_slots=12, H=2, dtype=in_dt)
    print(f"case packed ragged in={in_dt} out={out_dt} init={init}", flush=True)
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}
    o, pool = run_packed(d, tdt[in_dt], tdt[out_dt], init)
    o_ref, pool_ref = oracle.forward_packed(d["q"], d["k"], d["v"], d["g"], d["cu_seqlens"], d["pool"],
                                            d["slot_idx"], init)
    tol = TOL_BF16 if in_dt == "bf16" else TOL_F32
    if out_dt == "bf16":
        assert_close_bf16_out(o, o_ref, tol, "o(bf16)")
    else:
        assert_close(o, o_ref, tol, "o")
    check_pool(pool, pool_ref, d["slot_idx"], tol, "slots")


def test_packed_bf16_output():
    d = gen.make_packed_inputs(seed=12, lengths=[200, 0, 333, 64], n_slots=6, H=2)
    o, pool = run_packed(d, torch.bfloat16, torch.bfloat16, True)
    o_ref, pool_ref = oracle.forward_packed(d["q"], d["k"], d["v"], d["g"], d["cu_seqlens"], d["pool"],
                                            d["slot_idx"], True)
    assert_close_bf16_out(o, o_ref, TOL_BF16, "o(bf16)")
    check_pool(pool, pool_ref, d["slot_idx"], TOL_BF16, "slots")


@pytest.mark.parametrize("lengths,segments", [([1024, 0, 300, 1000], 4), ([640, 129, 1], 5)])
def test_packed_segments(lengths, segments):
    """Segment plan: the segments past a shorter sequence's end are empty."""
    d = gen.make_packed_inputs(seed=13, lengths=lengths, n_slots=9, H=2)
    print(f"case packed segments {lengths} nseg={segments}", flush=True)
    o, pool = run_packed(d, torch.bfloat16, torch.float32, True, segments=segments)
    o_ref, pool_ref = oracle.forward_packed(d["q"], d["k"], d["v"], d["g"], d["cu_seqlens"], d["pool"],
                                            d["slot_idx"], True)
    assert_close(o, o_ref, TOL_BF16, "o")
    check_pool(pool, pool_ref, d["slot_idx"], TOL_BF16, "slots")


@pytest.mark.parametrize("segments", [None, 3])
def test_packed_equals_batched(segments):
    """Equal lengths: the packed call gives the batched call's results bit for bit."""
    import linear_attention_sequence_simple_amd as gla
    B, T, H = 3, 300, 4
    d = gen.make_packed_inputs(seed=14, lengths=[T] * B, n_slots=B, H=H)
    d["slot_idx"] = np.arange(B, dtype=np.int32)
    o, pool = run_packed(d, torch.bfloat16, torch.bfloat16, True, segments=segments)
    bt = lambda x, dt: to_dev(x.reshape((B, T) + x.shape[1:]), dt)
    ob, Sb = gla.gla_chunk_fwd(bt(d["q"], torch.bfloat16), bt(d["k"], torch.bfloat16),
                               bt(d["v"], torch.bfloat16), bt(d["g"], torch.float32),
                               to_dev(d["pool"], torch.float32), out_dtype=torch.bfloat16, segments=segments)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(o, to_np(ob).reshape(o.shape))
    np.testing.assert_array_equal(pool, to_np(Sb))


def test_packed_continuation():
    """A prompt prefilled in two calls (the second from the pool) equals one call."""
    lengths, cut = [700, 131, 256], [300, 131, 0]
    d = gen.make_packed_inputs(seed=15, lengths=lengths, n_slots=5, H=2)
    cu = d["cu_seqlens"]
    first = np.concatenate([np.arange(cu[b], cu[b] + cut[b]) for b in range(3)])
    second = np.concatenate([np.arange(cu[b] + cut[b], cu[b + 1]) for b in range(3)])
    part = lambda idx, c: dict(q=d["q"][idx], k=d["k"][idx], v=d["v"][idx], g=d["g"][idx],
                               cu_seqlens=np.concatenate([[0], np.cumsum(c)]).astype(np.int32),
                               slot_idx=d["slot_idx"], pool=d["pool"])
    d1 = part(first, cut)
    o1, pool1 = run_packed(d1, torch.bfloat16, torch.float32, False)
    d2 = part(second, np.subtract(lengths, cut))
    d2["pool"] = pool1.astype(np.float32)
    o2, pool2 = run_packed(d2, torch.bfloat16, torch.float32, True)
    o_ref, pool_ref = oracle.forward_packed(d["q"], d["k"], d["v"], d["g"], cu, d["pool"], d["slot_idx"], False)
    assert_close(o1, o_ref[first], TOL_BF16, "o first part")
    assert_close(o2, o_ref[second], TOL_BF16, "o second part")
    check_pool(pool2, pool_ref, d["slot_idx"], TOL_BF16, "slots")


def test_packed_length_clamped_to_max_seqlen():
    """A sequence longer than max_seqlen is cut there: later rows are not written."""
    d = gen.make_packed_inputs(seed=16, lengths=[300], n_slots=2, H=2)
    o, pool = run_packed(d, torch.bfloat16, torch.float32, False, max_seqlen=200)
    cut = dict(d, q=d["q"][:200], k=d["k"][:200], v=d["v"][:200], g=d["g"][:200])
    o_ref, pool_ref = oracle.forward_packed(cut["q"], cut["k"], cut["v"], cut["g"], np.array([0, 200], np.int32),
                                            d["pool"], d["slot_idx"], False)
    assert_close(o[:200], o_ref, TOL_BF16, "o")
    assert np.all(o[200:] == 7.0)
    check_pool(pool, pool_ref, d["slot_idx"], TOL_BF16, "slots")


def test_serving_prefill_full_size_sampled():
    """The serving workload at full size (16 prompts of 2,048-8,192 tokens into a
    1,280-slot pool, bf16 in and out), in the launch configuration the
    benchmark times; sampled sequences and heads against the oracle."""
    import linear_attention_sequence_simple_amd as gla
    d = gen.make_packed_inputs(seed=0, with_pool=False)
    w = d["meta"]
    cu = d["cu_seqlens"]
    N, H = d["q"].shape[:2]
    print(f"case serving prefill N={N}", flush=True)
    pool = gla.gla_state_alloc(w["n_slots"])
    try:
        o = gla.gla_chunk_fwd_varlen(to_dev(d["q"], torch.bfloat16), to_dev(d["k"], torch.bfloat16),
                                     to_dev(d["v"], torch.bfloat16), to_dev(d["g"], torch.float32),
                                     torch.from_numpy(cu).to(dev()), w["len_hi"], pool,
                                     torch.from_numpy(d["slot_idx"]).to(dev()), init_from_pool=False,
                                     out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        for b, h in ((0, 0), (3, 15), (int(np.argmax(np.diff(cu))), 7)):
            t0, t1 = int(cu[b]), int(cu[b + 1])
            sl = int(d["slot_idx"][b])
            o_ref, S_ref = oracle.forward(d["q"][None, t0:t1, h:h + 1], d["k"][None, t0:t1, h:h + 1],
                                          d["v"][None, t0:t1, h:h + 1], d["g"][None, t0:t1, h:h + 1])
            assert_close_bf16_out(to_np(o[t0:t1, h]), o_ref[0, :, 0], TOL_BF16, f"o seq {b} head {h}")
            assert_close(to_np(pool.view()[sl, h]), S_ref[0, 0], TOL_BF16, f"slot {sl} head {h}")
    finally:
        pool.free()


@pytest.mark.parametrize("init", [False, True])
def test_packed_all_sequences_empty(init):
    """A batch whose sequences are all empty (no tokens at all): the slots of
    the batch get their initial state (zero, or the slot's own), nothing else
    changes."""
    import linear_attention_sequence_simple_amd as gla
    H = 2
    pool = gla.gla_state_alloc(4, H=H)
    st0 = torch.from_numpy(np.random.default_rng(17).standard_normal((4, H, 96, 192)).astype(np.float32)).to(dev())
    pool.view().copy_(st0)
    empty = lambda c: torch.empty((0, H, c), dtype=torch.bfloat16, device=dev())
    o = gla.gla_chunk_fwd_varlen(empty(96), empty(96), empty(192), torch.empty((0, H), device=dev()),
                                 torch.zeros(3, dtype=torch.int32, device=dev()), 128, pool,
                                 torch.tensor([3, 1], dtype=torch.int32, device=dev()), init_from_pool=init)
    torch.cuda.synchronize()
    got = pool.view().clone()
    pool.free()
    assert o.shape == (0, H, 192)
    want = st0.clone()
    if not init:
        want[[3, 1]] = 0
    assert torch.equal(got, want)


def test_packed_segments_f32():
    """fp32 inputs (three dv-slices, the fp32 state walk in pass 1) on the segment plan."""
    d = gen.make_packed_inputs(seed=18, lengths=[700, 0, 300, 1], n_slots=6, H=2, dtype="f32")
    o, pool = run_packed(d, torch.float32, torch.float32, True, segments=3)
    o_ref, pool_ref = oracle.forward_packed(d["q"], d["k"], d["v"], d["g"], d["cu_seqlens"], d["pool"],
                                            d["slot_idx"], True)
    assert_close(o, o_ref, TOL_F32, "o")
    check_pool(pool, pool_ref, d["slot_idx"], TOL_F32, "slots")
