"""Host logic of the fp8 widening route (no GPU): the 256-entry level table
the widening pass looks codes up in, and the choice of route."""

import pytest
import torch

from block_sparse_attention_tile_amd import api


def test_fp8_levels_decode_every_code():
    """Level l holds the value of code byte l ^ 0x80 (level = code + 128 for
    the int8 view of the byte), exactly as torch decodes e4m3fn; every
    finite value is exact in bf16, so widening loses nothing."""
    lv = api._fp8_levels("cpu")
    assert lv.dtype == torch.float32 and lv.numel() == 256
    for level in range(256):
        byte = level ^ 0x80
        want = torch.tensor([byte], dtype=torch.uint8).view(torch.float8_e4m3fn).float()
        got = lv[level:level + 1]
        if torch.isnan(want).item():
            assert torch.isnan(got).item()
        else:
            assert got.item() == want.item(), (level, byte)
            assert got.to(torch.bfloat16).float().item() == want.item()
    # the int8 view of a byte is its code: code + 128 is the level
    for code in (-128, -1, 0, 1, 127):
        byte = code & 0xFF
        assert (code + 128) == (byte ^ 0x80)


def test_fp8_levels_spot_values():
    lv = api._fp8_levels("cpu")
    assert lv[0x80 ^ 0x00].item() == 0.0          # byte 0x00: +0
    assert lv[0x80 ^ 0x38].item() == 1.0          # byte 0x38: 1.0
    assert lv[0x80 ^ 0x7E].item() == 448.0        # largest finite
    assert lv[0x80 ^ 0xFE].item() == -448.0
    assert lv[0x80 ^ 0x01].item() == 2.0 ** -9    # smallest subnormal
    assert torch.isnan(lv[0x80 ^ 0x7F]).item()    # e4m3fn NaN


def test_fp8_route_choice():
    over = api.ORDER_MIN_UNITS + 1
    assert api._widen_fp8(1, 1, over, "auto")
    assert not api._widen_fp8(1, 1, api.ORDER_MIN_UNITS, "auto")
    assert api._widen_fp8(1, 1, 1, "widen")
    assert not api._widen_fp8(1, 1, over, "kernel")
    with pytest.raises(ValueError):
        api._widen_fp8(1, 1, 1, "fast")
