"""The Python binding's buffer checks, on the CPU: wrong dtype, layout, size
or device raises ValueError before the library is called (the C ABI sees only
raw pointers and cannot check buffer sizes)."""
import dataclasses

import pytest
import torch


@pytest.fixture(scope="module")
def coat():
    from test_abi_exports import _ensure_built
    _ensure_built()
    from adamw_coat_fp8_amd import coat
    return coat


def test_quantize_act_checks(coat):
    x = torch.zeros(4, 128, dtype=torch.bfloat16)
    codes = torch.zeros(4, 128, dtype=torch.uint8)
    scales = torch.zeros(4, 1, dtype=torch.float32)
    with pytest.raises(ValueError, match="device"):
        coat.quantize_act(x, codes, scales, group_size=128)          # CPU tensors
    with pytest.raises(ValueError, match="needs at least"):
        coat.quantize_act(x, codes[:3], scales, group_size=128)       # short codes
    with pytest.raises(ValueError, match="needs at least"):
        coat.quantize_act(x, codes, scales, group_size=16)            # 8 scales needed
    with pytest.raises(ValueError, match="dtype"):
        coat.quantize_act(x.float(), codes, scales, group_size=128)
    with pytest.raises(ValueError, match="contiguous"):
        coat.quantize_act(x, codes.t().contiguous().t(), scales, group_size=128)
    with pytest.raises(ValueError, match="needs at least"):
        coat.quantize_act(x, codes, scales, torch.zeros(10, dtype=torch.uint8), group_size=128)


def test_gemm_checks(coat):
    a = torch.zeros(8, 128, dtype=torch.uint8)
    b = torch.zeros(128, 128, dtype=torch.uint8)
    codes = torch.zeros(8, 128, dtype=torch.uint8)
    scales = torch.zeros(8, 1, dtype=torch.float32)
    with pytest.raises(ValueError, match="device"):
        coat.gemm_group_quant(a, b, 1.0, 1.0, codes, scales, group_size=128)
    with pytest.raises(ValueError, match="needs at least"):
        coat.gemm_group_quant(a, b, 1.0, 1.0, codes[:4], scales, group_size=128)
    with pytest.raises(ValueError, match="needs at least"):
        coat.gemm_group_quant(a, b, 1.0, 1.0, codes, scales, group_size=16)
    with pytest.raises(ValueError, match="disagree"):
        coat.gemm_group_quant(a, b[:, :64], 1.0, 1.0, codes, scales)
    with pytest.raises(ValueError, match="needs at least"):
        coat.gemm_bf16(a, b, 1.0, 1.0, torch.zeros(8, 64, dtype=torch.int16))


def test_step_and_codec_checks(coat):
    n, G = 1000, 128
    slot = coat.ParamSlot(torch.zeros(n), torch.zeros(n, dtype=torch.bfloat16),
                          coat.QuantState.zeros(n, G, "cpu"), coat.QuantState.zeros(n, G, "cpu"))
    with pytest.raises(ValueError, match="device"):
        coat.adamw_fp8_step([slot], lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8,
                            weight_decay=0.1, step=1, group_size=G)
    m64 = coat.QuantState.zeros(n, 64, "cpu")
    short = coat.ParamSlot(torch.zeros(n), torch.zeros(n, dtype=torch.bfloat16),
                           dataclasses.replace(m64, scale=m64.scale[:5]),
                           coat.QuantState.zeros(n, G, "cpu"))
    with pytest.raises(dataclasses.FrozenInstanceError):
        short.m.scale = m64.scale                  # a built slot cannot change its buffers
    with pytest.raises(ValueError, match="tensors\\[0\\].m.scale"):
        coat.adamw_fp8_step([short], lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8,
                            weight_decay=0.1, step=1, group_size=G)
    with pytest.raises(ValueError, match="needs at least"):
        coat.e4m3_encode(torch.zeros(16), torch.zeros(8, dtype=torch.uint8))
    with pytest.raises(ValueError, match="needs at least"):
        coat.dequantize_expand(coat.QuantState.zeros(n, G, "cpu"), torch.zeros(10), group_size=G)
