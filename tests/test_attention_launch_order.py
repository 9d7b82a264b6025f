"""The attention backward reports its launches in the order backward_launches
lists them (CPU only: the library's execute calls are replaced by stubs, so
only the sequencing in attention.py runs; plans are host-only)."""
import pytest
import torch

from tensor_relational_algebra_amd import attention


@pytest.mark.parametrize("fuse", [False, True])
def test_on_step_names_follow_backward_launches(fuse, monkeypatch):
    calls = []
    monkeypatch.setattr(attention, "tra_execute", lambda p, x, y, z, ws, s: calls.append("execute"))
    monkeypatch.setattr(attention, "tra_execute_chain", lambda *a: calls.append("chain"))
    monkeypatch.setattr(attention, "tra_execute_contract_chain", lambda *a: calls.append("contract_chain"))
    # large enough that the dAttn product runs unsplit on the matrix cores (the
    # condition for the product chain)
    layer = attention.AttentionLayer(2048, 1024, 8, 128, fuse_product_chain=fuse)
    assert layer.fuse_product_chain == fuse
    env = {}
    for name, spec, ins, *_ in attention.FORWARD + attention.BACKWARD:
        for t in ins:
            env.setdefault(t, torch.zeros(1))
    seen = []
    layer.backward(env, torch.zeros(1), on_step=seen.append)
    assert seen == list(layer.backward_launches)
    assert len(seen) == len(calls) == len(set(seen))
    if fuse:
        assert calls[seen.index("dScores")] == "contract_chain" and "dAttn" not in seen
    else:
        assert calls[seen.index("dScores")] == "chain" and seen.index("dAttn") < seen.index("dScores")
