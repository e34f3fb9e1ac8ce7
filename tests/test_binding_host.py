"""The Python binding refuses host tensors before anything reaches the library:
a host pointer handed to a kernel would be read and written on the GPU."""
import pytest
import torch

import quant_row_workgroup_amd as qrw


def _calls():
    x = torch.zeros((4, 256), dtype=torch.bfloat16)
    w = torch.zeros(256, dtype=torch.bfloat16)
    c = torch.zeros((4, 64), dtype=torch.bfloat16)
    qkv = torch.zeros((4, 3 * 128), dtype=torch.bfloat16)
    hw = torch.zeros(128, dtype=torch.bfloat16)
    kc = torch.zeros((8, 128), dtype=torch.uint8)
    ks = torch.zeros((8, 1), dtype=torch.float32)
    flat = torch.zeros(100, dtype=torch.float16)
    return {
        "rmsnorm_fwd": lambda: qrw.rmsnorm_fwd(x, w),
        "layernorm_fwd": lambda: qrw.layernorm_fwd(x, w, w),
        "rope_apply_interleaved": lambda: qrw.rope_apply_interleaved(x, c, c, 2, 128),
        "rope_apply_neox": lambda: qrw.rope_apply_neox(x, c, c, 2, 128),
        "rmsnorm_rope_fp8_fwd": lambda: qrw.rmsnorm_rope_fp8_fwd(x, w, c, c, 2, 128),
        "rmsnorm_rope_fp8_rounded_fwd": lambda: qrw.rmsnorm_rope_fp8_rounded_fwd(x, w, c, c, 2,
                                                                                 128),
        "act_quant_fp8_fwd": lambda: qrw.act_quant_fp8_fwd(x, 128),
        "qk_norm_rope_fwd": lambda: qrw.qk_norm_rope_fwd(qkv, hw, hw, c, c, 1, 1, 128),
        "qk_norm_rope_fp8_kv_fwd": lambda: qrw.qk_norm_rope_fp8_kv_fwd(qkv, hw, hw, c, c, kc, kc,
                                                                       ks, ks, 1, 1, 128),
        "ew_add_fwd": lambda: qrw.ew_add_fwd(flat, flat),
        "ew_scale_cast_fwd": lambda: qrw.ew_scale_cast_fwd(flat, 2.0),
        "ew_scale_add_fwd": lambda: qrw.ew_scale_add_fwd(flat, flat, 2.0),
    }


@pytest.mark.parametrize("name", sorted(_calls()))
def test_host_tensors_are_refused(name):
    with pytest.raises(ValueError, match="ROCm device"):
        _calls()[name]()


def test_every_entry_point_is_covered():
    assert set(_calls()) == set(qrw._binding.EXPORTS) - {"qrw_status_string"}
