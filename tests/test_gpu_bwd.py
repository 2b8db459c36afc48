"""Backward parity: gla_chunk_bwd on the GPU against the fp64 oracle backward."""
import os

import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close, assert_close_bf16_out, inputs, rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu

TOL = 1e-2


def run_bwd(d, S0=True, dS_T=True, out_dtype=torch.float32, segments=None):
    import linear_attention_sequence_simple_amd as gla
    r = gla.gla_chunk_bwd(to_dev(d["q"], torch.bfloat16), to_dev(d["k"], torch.bfloat16),
                          to_dev(d["v"], torch.bfloat16), to_dev(d["g"], torch.float32),
                          to_dev(d["dO"], torch.bfloat16),
                          S0=to_dev(d["S0"], torch.float32) if S0 else None,
                          dS_T=to_dev(d.get("dS_T"), torch.float32) if dS_T else None,
                          out_dtype=out_dtype, want_dS0=True, segments=segments)
    torch.cuda.synchronize()
    return [to_np(x) for x in r]


def check(d, got, S0=True, dS_T=True):
    ref = oracle.backward(d["q"], d["k"], d["v"], d["g"], d["dO"], d["S0"] if S0 else None,
                          d.get("dS_T") if dS_T else None)
    for name, x, y in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
        assert_close(x, y, TOL, name)
    dg, dg_ref = got[3], ref[3]
    if np.all(dg_ref == 0):
        # no decay gradient at all (gamma == 0): compare with the scale of the
        # terms that cancel, q.dq
        scale = np.sqrt(np.mean(np.einsum("bthd,bthd->bth", d["q"], ref[0]) ** 2))
        assert np.max(np.abs(dg)) <= TOL * scale
    else:
        assert_close(dg, dg_ref, TOL, "dg")
    if S0 or dS_T:
        assert_close(got[4], ref[4], TOL, "dS0")


@pytest.mark.parametrize("T", [1, 77, 128, 200, 300, 513])
@pytest.mark.parametrize("s0,dst", [(True, True), (False, False)])
def test_reduced(T, s0, dst):
    d = inputs("bwd_bf16_b4_t4096", seed=T, B=2, T=T, H=2, S0="normal0.1", with_dO=True, with_dS_T=True)
    print(f"case bwd T={T} S0={s0} dS_T={dst}", flush=True)
    got = run_bwd(d, s0, dst)
    check(d, got, s0, dst)


@pytest.mark.parametrize("B,T,H", [(128, 3, 16), (64, 130, 2)])
def test_wide_batches(B, T, H):
    """Many short sequences (2,048 (b, h) pairs for B=128, H=16): every
    gradient against the oracle."""
    d = inputs("bwd_bf16_b4_t4096", seed=5, B=B, T=T, H=H, S0="normal0.1", with_dO=True, with_dS_T=True)
    print(f"case bwd wide batch B={B} T={T} H={H}", flush=True)
    check(d, run_bwd(d))


@pytest.mark.parametrize("g", ["one", "zero"])
def test_special_decays(g):
    d = inputs("bwd_bf16_b4_t4096", seed=4, B=1, T=260, H=2, g=g, S0="normal0.1", with_dO=True,
               with_dS_T=True)
    got = run_bwd(d)
    check(d, got)


@pytest.mark.parametrize("T,segments", [(1024, 4), (1100, 3)])
def test_segments(T, segments):
    d = inputs("bwd_bf16_b4_t4096", seed=6, B=1, T=T, H=2, S0="normal0.1", with_dO=True, with_dS_T=True)
    got = run_bwd(d, segments=segments)
    check(d, got)


@pytest.mark.parametrize("T,s0,dst,out", [(1100, True, True, "f32"), (1100, False, False, "bf16"),
                                          (260, True, False, "f32"), (385, False, True, "bf16"),
                                          (2048, True, True, "bf16")])
def test_two_segments(T, s0, dst, out):
    """Two segments: the walks' second segments start from the states their
    first segments left one launch earlier (no state pass); segment 1 holds
    one chunk at T = 260 and 385."""
    d = inputs("bwd_bf16_b4_t4096", seed=40 + T, B=1, T=T, H=2, S0="normal0.1", with_dO=True, with_dS_T=True)
    print(f"case bwd two segments T={T} S0={s0} dS_T={dst} out={out}", flush=True)
    out_dtype = torch.bfloat16 if out == "bf16" else torch.float32
    got = run_bwd(d, s0, dst, out_dtype=out_dtype, segments=2)
    if out == "f32":
        check(d, got, s0, dst)
        return
    ref = oracle.backward(d["q"], d["k"], d["v"], d["g"], d["dO"], d["S0"] if s0 else None,
                          d["dS_T"] if dst else None)
    for name, x, y in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
        assert_close_bf16_out(x, y, TOL, name + "(bf16)")
    assert_close(got[3], ref[3], TOL, "dg")
    if s0 or dst:
        assert_close(got[4], ref[4], TOL, "dS0")


def test_bf16_gradients():
    # gradients written in bf16: elementwise bound of the rounding on top of
    # the tolerance; dg stays fp32
    d = inputs("bwd_bf16_b4_t4096", seed=9, B=2, T=333, H=2, S0="normal0.1", with_dO=True, with_dS_T=True)
    got = run_bwd(d, out_dtype=torch.bfloat16)
    ref = oracle.backward(d["q"], d["k"], d["v"], d["g"], d["dO"], d["S0"], d["dS_T"])
    for name, x, y in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
        assert_close_bf16_out(x, y, TOL, name + "(bf16)")
    assert_close(got[3], ref[3], TOL, "dg")
    assert_close(got[4], ref[4], TOL, "dS0")


def test_backward_workload_sampled():
    # B=4, H=16, T=4096, S0 = 0, dS_T = 0; the oracle checks sampled (b, h).
    d = inputs("bwd_bf16_b4_t4096", seed=0, with_dO=True)
    got = run_bwd(d, S0=False, dS_T=False)
    bs, hs = [0, 3], [2, 13]
    sub = lambda x: x[np.ix_(bs, range(x.shape[1]), hs)]
    ref = oracle.backward(sub(d["q"]), sub(d["k"]), sub(d["v"]), sub(d["g"]), sub(d["dO"]))
    for name, x, y in zip(("dq", "dk", "dv", "dg"), got[:4], ref[:4]):
        assert_close(sub(x), y, TOL, name)
    for x in got[:4]:
        assert np.isfinite(x).all()


def test_backward_workload_bf16_sampled():
    """The timed backward: B=4, H=16, T=4096, bf16 gradients (two segments,
    staggered launches); every gradient of sampled (b, h) against the oracle
    with the elementwise bf16-output bound."""
    d = inputs("bwd_bf16_b4_t4096", seed=1, with_dO=True)
    got = run_bwd(d, S0=False, dS_T=False, out_dtype=torch.bfloat16)
    bs, hs = [1, 2], [0, 15]
    sub = lambda x: x[np.ix_(bs, range(x.shape[1]), hs)]
    ref = oracle.backward(sub(d["q"]), sub(d["k"]), sub(d["v"]), sub(d["g"]), sub(d["dO"]))
    for name, x, y in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
        assert_close_bf16_out(sub(x), y, TOL, name + "(bf16)")
    assert_close(sub(got[3]), ref[3], TOL, "dg")


def test_longest_supported_sequence():
    """T = 131,072, the backward's limit of 1,024 chunks, on one head (the
    segment plan with every kernel at its largest chunk count)."""
    d = inputs("bwd_bf16_b4_t4096", seed=12, B=1, T=131_072, H=1, S0="normal0.1", with_dO=True,
               with_dS_T=True)
    print("case bwd T=131072", flush=True)
    got = run_bwd(d)
    ref = oracle.backward(d["q"], d["k"], d["v"], d["g"], d["dO"], d["S0"], d["dS_T"], ckpt=1024)
    for name, x, y in zip(("dq", "dk", "dv", "dg", "dS0"), got, ref):
        assert_close(x, y, TOL, name)


# ---------------------------------------------------------------------------
# fp32 inputs: the same gradients on the fp32 matrix cores, bound 1e-4

TOL_F32 = 1e-4


def run_bwd_f32(d, S0=True, dS_T=True, out_dtype=torch.float32, segments=None):
    import linear_attention_sequence_simple_amd as gla
    r = gla.gla_chunk_bwd(to_dev(d["q"], torch.float32), to_dev(d["k"], torch.float32),
                          to_dev(d["v"], torch.float32), to_dev(d["g"], torch.float32),
                          to_dev(d["dO"], torch.float32),
                          S0=to_dev(d["S0"], torch.float32) if S0 else None,
                          dS_T=to_dev(d.get("dS_T"), torch.float32) if dS_T else None,
                          out_dtype=out_dtype, want_dS0=True, segments=segments)
    torch.cuda.synchronize()
    return [to_np(x) for x in r]


def check_f32(d, got, S0=True, dS_T=True, tol=TOL_F32):
    ref = oracle.backward(d["q"], d["k"], d["v"], d["g"], d["dO"], d["S0"] if S0 else None,
                          d.get("dS_T") if dS_T else None)
    for name, x, y in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
        assert_close(x, y, tol, name)
    dg, dg_ref = got[3], ref[3]
    if np.all(dg_ref == 0):
        scale = np.sqrt(np.mean(np.einsum("bthd,bthd->bth", d["q"], ref[0]) ** 2))
        assert np.max(np.abs(dg)) <= tol * scale
    else:
        assert_close(dg, dg_ref, tol, "dg")
    if S0 or dS_T:
        assert_close(got[4], ref[4], tol, "dS0")


@pytest.mark.parametrize("T", [1, 77, 128, 300, 513])
@pytest.mark.parametrize("s0,dst", [(True, True), (False, False), (False, True)])
def test_f32_reduced(T, s0, dst):
    d = inputs("fwd_f32_b1_t2048", seed=60 + T, B=2, T=T, H=2, S0="normal0.1", with_dO=True, with_dS_T=True)
    print(f"case bwd fp32 T={T} S0={s0} dS_T={dst}", flush=True)
    check_f32(d, run_bwd_f32(d, s0, dst), s0, dst)


@pytest.mark.parametrize("g", ["one", "zero"])
def test_f32_special_decays(g):
    d = inputs("fwd_f32_b1_t2048", seed=70, B=1, T=260, H=2, g=g, S0="normal0.1", with_dO=True, with_dS_T=True)
    print(f"case bwd fp32 g={g}", flush=True)
    check_f32(d, run_bwd_f32(d))


@pytest.mark.parametrize("T,segments,s0,dst", [(1024, 4, True, True), (1000, 3, False, True), (640, 5, True, False),
                                               (300, 1, True, True)])
def test_f32_segments(T, segments, s0, dst):
    """The fp32 backward's segment plan: state-only walks of both recurrences
    and a scan give every segment's entering state; one segment is the whole
    sequence."""
    d = inputs("fwd_f32_b1_t2048", seed=80 + segments, B=1, T=T, H=2, S0="normal0.1", with_dO=True, with_dS_T=True)
    print(f"case bwd fp32 T={T} segments={segments} S0={s0} dS_T={dst}", flush=True)
    check_f32(d, run_bwd_f32(d, s0, dst, segments=segments), s0, dst)


def test_f32_training_shape():
    """B=1, H=16, T=2048 (the fp32 workload's shape), every gradient of every
    head against the oracle."""
    d = inputs("fwd_f32_b1_t2048", seed=71, with_dO=True, with_dS_T=True, S0="normal0.1")
    print("case bwd fp32 B=1 T=2048 H=16", flush=True)
    check_f32(d, run_bwd_f32(d))


def test_f32_bf16_gradients():
    d = inputs("fwd_f32_b1_t2048", seed=72, B=2, T=333, H=2, S0="normal0.1", with_dO=True, with_dS_T=True)
    print("case bwd fp32 in, bf16 out", flush=True)
    got = run_bwd_f32(d, out_dtype=torch.bfloat16)
    ref = oracle.backward(d["q"], d["k"], d["v"], d["g"], d["dO"], d["S0"], d["dS_T"])
    for name, x, y in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
        assert_close_bf16_out(x, y, TOL_F32, name + "(bf16)")
    assert_close(got[3], ref[3], TOL_F32, "dg")
    assert_close(got[4], ref[4], TOL_F32, "dS0")


@pytest.mark.parametrize("eq,ek,ev,edo", [(15, -15, 10, -10), (-10, -10, 20, 20)])
def test_input_magnitudes(eq, ek, ev, edo):
    """bf16 q, k, v and dO scaled by powers of two far from unit scale: the
    gradients keep the unit-scale error relative to their rms."""
    d = inputs("bwd_bf16_b4_t4096", seed=12, B=1, T=300, H=2, with_dO=True, with_dS_T=True,
               S0="normal0.1")
    d["q"] = d["q"] * 2.0 ** eq
    d["k"] = d["k"] * 2.0 ** ek
    d["v"] = d["v"] * 2.0 ** ev
    d["dO"] = d["dO"] * 2.0 ** edo
    d["S0"] = d["S0"] * 2.0 ** (ek + ev)
    d["dS_T"] = d["dS_T"] * 2.0 ** (eq + edo)
    print(f"case bwd magnitudes 2^{eq}, 2^{ek}, 2^{ev}, 2^{edo}", flush=True)
    check(d, run_bwd(d))
