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
        rq._call("inv_rope_fp8_quant", torch.device("cuda", 0), other)


def test_cpu_tensors_are_refused_before_any_launch():
    o = torch.zeros((2, 8, 512), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        rq.inv_rope_fp8_quant(o, torch.zeros(2, dtype=torch.int64),
                              torch.zeros((16, 64)), 8, None, None)


def test_unknown_scale_format_is_refused():
    with pytest.raises(ValueError, match="scale_fmt"):
        rq.empty_inv_rope_fp8_quant_outputs(4, 8, 8, "cpu", "fp8")
