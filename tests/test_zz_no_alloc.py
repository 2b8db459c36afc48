"""gla_chunk_fwd_noalloc through the C ABI against gla_chunk_fwd with a
workspace: two calls in a row, the second on a smaller input, each equal to
the workspace call bit for bit (the same kernels and plan), and both within
the bf16 tolerance of the oracle on sampled heads."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close, inputs, to_dev, to_np

pytestmark = pytest.mark.gpu


def _noalloc(gla, q, k, v, g, S0, o, S_T):
    B, T, H, _ = q.shape
    dims = gla.GlaDims(B, T, H, 96, 192, 128, gla.GLA_BF16, gla._dtype_code(o.dtype))
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    st = gla.lib().gla_chunk_fwd_noalloc(ctypes.byref(dims), p(q), p(k), p(v), p(g), p(S0), p(o), p(S_T),
                                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, gla.lib().gla_last_error().decode()


@pytest.mark.parametrize("shape", [[(1, 16384, 16), (1, 3000, 4)]])
def test_noalloc_equals_workspace_call(shape):
    import linear_attention_sequence_simple_amd as gla
    for i, (B, T, H) in enumerate(shape):
        d = inputs("fwd_bf16_b1_t65536", seed=40 + i, B=B, T=T, H=H)
        dims = gla.GlaDims(B, T, H, 96, 192, 128, gla.GLA_BF16, gla.GLA_F32)
        need = gla.gla_workspace_size(gla.GLA_OP_FWD, dims)
        assert 0 < need <= 32 << 20                      # a segmented plan that uses the scratch
        print(f"case noalloc call {i}: B={B} T={T} H={H}, scratch {need} B", flush=True)
        q, k, v = (to_dev(d[c], torch.bfloat16) for c in ("q", "k", "v"))
        g, S0 = to_dev(d["g"], torch.float32), to_dev(d["S0"], torch.float32)
        o_ref, S_ref = gla.gla_chunk_fwd(q, k, v, g, S0, out_dtype=torch.float32)
        o = torch.full_like(o_ref, 7.0)
        S_T = torch.full_like(S_ref, 7.0)
        _noalloc(gla, q, k, v, g, S0, o, S_T)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(S_T, S_ref)
        hs = [0, H - 1]
        sl = lambda x: x[:, :, hs]
        o64, S64 = oracle.forward(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["g"]), d["S0"][:, hs])
        assert_close(to_np(o)[:, :, hs], o64, 1e-2, "o")
        assert_close(to_np(S_T)[:, hs], S64, 1e-2, "S_T")
