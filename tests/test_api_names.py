"""The binding's short names (chunk_fwd, recurrent_step, chunk_bwd,
StatePool) map onto the gla_-prefixed calls; checked here without a GPU by
replacing the call underneath."""
import inspect

import linear_attention_sequence_simple_amd as gla


def test_short_names_exist():
    assert gla.chunk_fwd is gla.gla_chunk_fwd
    assert gla.recurrent_step is gla.gla_recurrent_step
    assert list(inspect.signature(gla.chunk_fwd).parameters)[:6] == ["q", "k", "v", "g", "S0", "out_dtype"]
    assert list(inspect.signature(gla.recurrent_step).parameters)[:7] == [
        "pool", "q", "k", "v", "g", "slot_idx", "out_dtype"]
    assert list(inspect.signature(gla.StatePool).parameters)[:4] == ["n_slots", "H", "dk", "dv"]
    for name in ("chunk_fwd", "recurrent_step", "chunk_bwd", "StatePool"):
        assert name in gla.__all__


def test_chunk_bwd_returns_dS0_only_with_an_initial_state(monkeypatch):
    calls = []

    def fake(q, k, v, g, dO, S0=None, dS_T=None, out_dtype=None, want_dS0=False, workspace=None):
        calls.append((S0, dS_T, want_dS0))
        return ("dq", "dk", "dv", "dg", "dS0" if want_dS0 else None)

    monkeypatch.setattr(gla, "gla_chunk_bwd", fake)
    assert gla.chunk_bwd(1, 2, 3, 4, 5) == ("dq", "dk", "dv", "dg")
    assert gla.chunk_bwd(1, 2, 3, 4, 5, S0="S0") == ("dq", "dk", "dv", "dg", "dS0")
    assert gla.chunk_bwd(1, 2, 3, 4, 5, dS_T="dST", want_dS0=True) == ("dq", "dk", "dv", "dg", "dS0")
    assert gla.chunk_bwd(1, 2, 3, 4, 5, S0="S0", want_dS0=False) == ("dq", "dk", "dv", "dg")
    assert calls == [(None, None, False), ("S0", None, True), (None, "dST", True), ("S0", None, False)]
