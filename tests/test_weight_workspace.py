"""WeightWorkspace caching rules (host logic; the quantizer is a stand-in that counts calls)."""
import torch

from mxfp4_block_scaled_cast_amd.quant import MXFP4Quantizer, WeightWorkspace


class CountingQuantizer(MXFP4Quantizer):
    calls = 0

    def quantize(self, x):
        CountingQuantizer.calls += 1
        return ("quantized", x.data_ptr(), x._version)


def fresh():
    CountingQuantizer.calls = 0
    return CountingQuantizer("weight"), WeightWorkspace()


def test_same_weight_is_cached():
    q, ws = fresh()
    w = torch.zeros(64, 32, dtype=torch.bfloat16)
    a = ws.get_or_quantize(w, q, cache_name="mlp_gate")
    b = ws.get_or_quantize(w, q, cache_name="mlp_gate")
    assert a is b and CountingQuantizer.calls == 1 and ws.hits == 1 and ws.misses == 1
    assert "mlp_gate" in ws and len(ws) == 1


def test_in_place_update_requantizes():
    q, ws = fresh()
    w = torch.zeros(64, 32, dtype=torch.bfloat16)
    ws.get_or_quantize(w, q, cache_name="w")
    w.add_(1)  # e.g. an optimizer step: bumps the version counter
    ws.get_or_quantize(w, q, cache_name="w")
    assert CountingQuantizer.calls == 2


def test_other_tensor_or_view_requantizes():
    q, ws = fresh()
    w = torch.zeros(64, 32, dtype=torch.bfloat16)
    ws.get_or_quantize(w, q, cache_name="w")
    ws.get_or_quantize(torch.zeros(64, 32, dtype=torch.bfloat16), q, cache_name="w")
    assert CountingQuantizer.calls == 2
    ws.get_or_quantize(w[:32], q, cache_name="w")  # same storage, other view
    assert CountingQuantizer.calls == 3


def test_other_tensor_object_requantizes():
    # a view with the same storage, shape, strides and version counter is another tensor
    # object: it may not reuse the entry (the allocator can also hand a new tensor a freed
    # weight's address with the same version)
    q, ws = fresh()
    w = torch.zeros(64, 32, dtype=torch.bfloat16)
    ws.get_or_quantize(w, q, cache_name="w")
    alias = w.view(64, 32)
    assert alias.data_ptr() == w.data_ptr() and alias._version == w._version
    ws.get_or_quantize(alias, q, cache_name="w")
    assert CountingQuantizer.calls == 2


def test_dead_weight_entry_never_matches():
    q, ws = fresh()
    w = torch.zeros(64, 32, dtype=torch.bfloat16)
    ws.get_or_quantize(w, q, cache_name="w")
    del w
    w2 = torch.zeros(64, 32, dtype=torch.bfloat16)
    ws.get_or_quantize(w2, q, cache_name="w")
    assert CountingQuantizer.calls == 2


def test_data_updates_need_invalidate():
    # w.data has its own version counter: the documented case for invalidate()
    q, ws = fresh()
    w = torch.zeros(64, 32, dtype=torch.bfloat16)
    ws.get_or_quantize(w, q, cache_name="w")
    w.data.add_(1)
    ws.get_or_quantize(w, q, cache_name="w")
    assert CountingQuantizer.calls == 1
    ws.invalidate("w")
    ws.get_or_quantize(w, q, cache_name="w")
    assert CountingQuantizer.calls == 2


def test_names_and_roles_are_separate_entries():
    q, ws = fresh()
    w = torch.zeros(64, 32, dtype=torch.bfloat16)
    ws.get_or_quantize(w, q, cache_name="a")
    ws.get_or_quantize(w, q, cache_name="b")
    ws.get_or_quantize(w, CountingQuantizer("weight", True, False), cache_name="a")  # row copy only
    assert CountingQuantizer.calls == 3 and len(ws) == 2


def test_invalidate():
    q, ws = fresh()
    w = torch.zeros(64, 32, dtype=torch.bfloat16)
    ws.get_or_quantize(w, q, cache_name="a")
    ws.get_or_quantize(w, q, cache_name="b")
    ws.invalidate("a")
    assert "a" not in ws and "b" in ws
    ws.get_or_quantize(w, q, cache_name="a")
    assert CountingQuantizer.calls == 3
    ws.invalidate()
    assert len(ws) == 0


def test_role_constructors():
    assert MXFP4Quantizer.for_weight() == MXFP4Quantizer("weight", True, True)
    assert MXFP4Quantizer.for_activation(columnwise=False).columnwise is False
    assert MXFP4Quantizer.for_grad().role == "grad"
