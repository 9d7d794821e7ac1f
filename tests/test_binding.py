"""Host-side checks of the Python binding (no GPU needed)."""
import types

import pytest
import torch

import rope_fp8_quant_amd as rq


def test_stream_on_another_device_is_refused():
    # the library launches on the current HIP device: a stream of another
    # device would pair foreign pointers with it, so the binding refuses
    other = types.SimpleNamespace(device=torch.device("cuda", 1), cuda_stream=0)
    with pytest.raises(ValueError, match="stream is on cuda:1"):
        rq._launch("inv_rope_fp8_quant", None, 0, other, ())


def test_cpu_tensors_are_refused_before_any_launch():
    o = torch.zeros((2, 8, 512), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        rq.inv_rope_fp8_quant(o, torch.zeros(2, dtype=torch.int64),
                              torch.zeros((16, 64)), 8, None, None)


def test_unknown_scale_format_is_refused():
    with pytest.raises(ValueError, match="scale_fmt"):
        rq.empty_inv_rope_fp8_quant_outputs(4, 8, 8, "cpu", "fp8")


def test_prepare_propagates_a_refusal_and_leaves_no_capture_behind():
    o = torch.zeros((2, 8, 512), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        rq.prepare(rq.inv_rope_fp8_quant, o, torch.zeros(2, dtype=torch.int64),
                   torch.zeros((16, 64)), 8, None, None)
    assert rq._capture.slot is None


def test_prepare_captures_one_launch_without_launching(monkeypatch):
    # a stand-in op that marshals like the real ones: prepare() must take its
    # single _call, launch nothing, and hand back the marshalled arguments
    launched = []
    monkeypatch.setattr(rq, "_launch", lambda *a: launched.append(a))
    monkeypatch.setattr(rq, "functions", lambda: {"qnorm_rope": "fn"})

    def op(x):
        rq._call("qnorm_rope", 0, None, x, 7)
    call = rq.prepare(op, 3)
    assert launched == [] and call.name == "qnorm_rope" and call._args == (3, 7)
    call()
    assert launched == [("qnorm_rope", "fn", 0, None, (3, 7))]
