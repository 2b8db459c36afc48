"""Prefill over strided views (gla_chunk_fwd_strided): q, k, v read in place
from a fused projection output of 9,216 columns per token, g from a wider
buffer, o written into a wider buffer.  The results must equal the dense call
on contiguous copies bit for bit (the same kernels walk the same values), and
the oracle within the bf16 / fp32 bounds."""
import os

import numpy as np
import pytest
import torch

import gen
import oracle
from gpu_util import assert_close, dev, to_dev, to_np

pytestmark = pytest.mark.gpu

H, DK, DV = 16, 96, 192
FUSED = H * (2 * DK + 2 * DV)          # 9,216


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import linear_attention_sequence_simple_amd as gla
    gla.lib()
    return gla


def fused_views(q, k, v, layout, gate=None):
    """Place q, k, v (and the gate) into one [B, T, 9216] buffer and return
    views of it.  blocked: all heads' q, then k, v, gate; per_head: per head
    q, k, v, gate."""
    B, T = q.shape[:2]
    buf = torch.full((B, T, FUSED), float("nan"), dtype=q.dtype, device=q.device)
    if layout == "blocked":
        qv = buf[..., :H * DK].unflatten(-1, (H, DK))
        kv = buf[..., H * DK:2 * H * DK].unflatten(-1, (H, DK))
        vv = buf[..., 2 * H * DK:2 * H * DK + H * DV].unflatten(-1, (H, DV))
        gtv = buf[..., 2 * H * DK + H * DV:].unflatten(-1, (H, DV))
    else:
        per = buf.unflatten(-1, (H, 2 * DK + 2 * DV))
        qv, kv, vv = per[..., :DK], per[..., DK:2 * DK], per[..., 2 * DK:2 * DK + DV]
        gtv = per[..., 2 * DK + DV:]
    qv.copy_(q)
    kv.copy_(k)
    vv.copy_(v)
    if gate is None:
        return buf, qv, kv, vv
    gtv.copy_(gate)
    return buf, qv, kv, vv, gtv


@pytest.mark.parametrize("layout", ["blocked", "per_head"])
@pytest.mark.parametrize("dtype,segments", [("bf16", None), ("bf16", 3), ("f32", None), ("f32", 3)])
def test_fused_layout(layout, dtype, segments):
    import linear_attention_sequence_simple_amd as gla
    B, T = 2, 300
    wl = "fwd_bf16_b8_t2048" if dtype == "bf16" else "fwd_f32_b1_t2048"
    d = gen.make_inputs(wl, seed=21, B=B, T=T, H=H, S0="normal0.1")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    print(f"case strided {layout} {dtype} segments={segments}", flush=True)
    q, k, v = (to_dev(d[n], tdt) for n in ("q", "k", "v"))
    g = to_dev(d["g"], torch.float32)
    S0 = to_dev(d["S0"], torch.float32)
    _, qv, kv, vv = fused_views(q, k, v, layout)
    gbuf = torch.full((B, T, H + 5), float("nan"), device=dev())
    gv = gbuf[..., 2:2 + H]
    gv.copy_(g)
    obuf = torch.full((B, T, H * DV + 64), 7.0, dtype=torch.float32, device=dev())
    ov = obuf[..., 32:32 + H * DV].unflatten(-1, (H, DV))
    o_s, S_s = gla.gla_chunk_fwd_strided(qv, kv, vv, gv, S0, out_dtype=torch.float32, o=ov, segments=segments)
    o_d, S_d = gla.gla_chunk_fwd(q, k, v, g, S0, out_dtype=torch.float32, segments=segments)
    torch.cuda.synchronize()
    assert torch.equal(o_s, o_d) and torch.equal(S_s, S_d)
    assert torch.all(obuf[..., :32] == 7.0) and torch.all(obuf[..., 32 + H * DV:] == 7.0)
    o_ref, S_ref = oracle.forward(d["q"], d["k"], d["v"], d["g"], d["S0"])
    tol = 1e-2 if dtype == "bf16" else 1e-4
    assert_close(to_np(o_s), o_ref, tol, "o")
    assert_close(to_np(S_s), S_ref, tol, "S_T")


def test_fused_layout_bf16_output_training_shape():
    """B=8, T=2048 read from the fused [8, 2048, 9216] buffer, bf16 out, in the
    launch configuration the benchmark times: equal to the dense call."""
    import linear_attention_sequence_simple_amd as gla
    d = gen.make_inputs("fwd_bf16_b8_t2048", seed=0)
    q, k, v = (to_dev(d[n], torch.bfloat16) for n in ("q", "k", "v"))
    g = to_dev(d["g"], torch.float32)
    _, qv, kv, vv = fused_views(q, k, v, "blocked")
    o_s, S_s = gla.gla_chunk_fwd_strided(qv, kv, vv, g, None, out_dtype=torch.bfloat16)
    o_d, S_d = gla.gla_chunk_fwd(q, k, v, g, None, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o_s, o_d) and torch.equal(S_s, S_d)


@pytest.mark.parametrize("layout", ["blocked", "per_head"])
@pytest.mark.parametrize("dtype,out,segments,T", [("bf16", "f32", None, 300), ("bf16", "bf16", None, 517),
                                                  ("bf16", "f32", 3, 640), ("f32", "f32", None, 300),
                                                  ("f32", "f32", 3, 400), ("bf16", "f32", None, 1)])
def test_fused_gate(layout, dtype, out, segments, T):
    """The output gate read in place from the fused buffer's fourth part:
    o * SiLU(gate) against the oracle's gated forward; S_T is not gated and
    equals the ungated call's bit for bit."""
    import linear_attention_sequence_simple_amd as gla
    from gpu_util import assert_close_bf16_out
    B = 2
    wl = "fwd_bf16_b8_t2048" if dtype == "bf16" else "fwd_f32_b1_t2048"
    d = gen.make_inputs(wl, seed=31 + T, B=B, T=T, H=H, S0="normal0.1", with_gate=True)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    odt = torch.bfloat16 if out == "bf16" else torch.float32
    print(f"case gate {layout} {dtype}->{out} segments={segments} T={T}", flush=True)
    q, k, v, gate = (to_dev(d[n], tdt) for n in ("q", "k", "v", "gate"))
    g = to_dev(d["g"], torch.float32)
    S0 = to_dev(d["S0"], torch.float32)
    _, qv, kv, vv, gtv = fused_views(q, k, v, layout, gate)
    y, S_g = gla.gla_chunk_fwd_strided(qv, kv, vv, g, S0, out_dtype=odt, segments=segments, gate=gtv)
    _, S_u = gla.gla_chunk_fwd_strided(qv, kv, vv, g, S0, out_dtype=odt, segments=segments)
    torch.cuda.synchronize()
    assert torch.equal(S_g, S_u)
    y_ref, S_ref = oracle.forward_gated(d["q"], d["k"], d["v"], d["g"], d["gate"], d["S0"])
    tol = 1e-2 if dtype == "bf16" else 1e-4
    if out == "bf16":
        assert_close_bf16_out(to_np(y), y_ref, tol, "y(bf16)")
    else:
        assert_close(to_np(y), y_ref, tol, "y")
    assert_close(to_np(S_g), S_ref, tol, "S_T")


def test_fused_gate_training_shape():
    """B=8, T=2048, bf16 in and out, q, k, v and the gate read in place from
    the [8, 2048, 9216] buffer (the benchmark's gated launch), sampled (b, h)
    pairs against the oracle's gated forward."""
    import linear_attention_sequence_simple_amd as gla
    from gpu_util import assert_close_bf16_out
    d = gen.make_inputs("fwd_bf16_b8_t2048", seed=0, with_gate=True)
    q, k, v, gate = (to_dev(d[n], torch.bfloat16) for n in ("q", "k", "v", "gate"))
    g = to_dev(d["g"], torch.float32)
    _, qv, kv, vv, gtv = fused_views(q, k, v, "blocked", gate)
    print("case gate training shape", flush=True)
    y, S = gla.gla_chunk_fwd_strided(qv, kv, vv, g, None, out_dtype=torch.bfloat16, gate=gtv)
    torch.cuda.synchronize()
    bs, hs = [0, 7], [0, 8, 15]
    T = d["q"].shape[1]
    sub = lambda x: x[np.ix_(bs, range(T), hs)]
    y_ref, S_ref = oracle.forward_gated(sub(d["q"]), sub(d["k"]), sub(d["v"]), sub(d["g"]), sub(d["gate"]))
    assert_close_bf16_out(to_np(y)[np.ix_(bs, range(T), hs)], y_ref, 1e-2, "y(bf16)")
    assert_close(to_np(S)[np.ix_(bs, hs)], S_ref, 1e-2, "S_T")
