"""Pins for the oracle's E4M3 encoder: the format definition's landmark
values, torch's own float8_e4m3fn cast (bit for bit, in range), saturation and
the per-block scale rule."""
import numpy as np
import torch

from oracle import fp8


def test_landmark_values():
    assert fp8.e4m3_value(0x38) == 1.0
    assert fp8.e4m3_value(0x7E) == 448.0
    assert fp8.e4m3_value(0xFE) == -448.0
    assert fp8.e4m3_value(0x01) == 2.0 ** -9
    assert fp8.e4m3_value(0x08) == 2.0 ** -6
    assert fp8.e4m3_value(0x07) == 7 * 2.0 ** -9
    assert np.isnan(fp8.e4m3_value(0x7F)) and np.isnan(fp8.e4m3_value(0xFF))
    assert fp8.e4m3_value(0x80) == 0.0


def test_matches_torch_cast_in_range():
    g = torch.Generator().manual_seed(0)
    x = torch.randn(200000, generator=g) * torch.exp(torch.randn(200000, generator=g) * 3)
    x = x.clamp(-448, 448)
    # exact ties between neighbouring codes and subnormal midpoints
    vals = torch.tensor([fp8.e4m3_value(c) for c in range(127)], dtype=torch.float64)
    mids = ((vals[1:] + vals[:-1]) / 2).to(torch.float32)
    x = torch.cat([x, mids, -mids, torch.tensor([0.0, -0.0, 2.0 ** -10, 3 * 2.0 ** -11])])
    ours = fp8.encode_e4m3(x.numpy())
    ref = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (ours == ref).all(), np.nonzero(ours != ref)[0][:10]


def test_saturation_and_nan():
    codes = fp8.encode_e4m3(np.array([1000.0, -1e9, 464.0, np.nan], np.float32))
    assert list(codes[:3]) == [0x7E, 0xFE, 0x7E]
    assert codes[3] == 0x7F


def test_block_scales_and_roundtrip():
    g = torch.Generator().manual_seed(1)
    x = torch.randn(2, 300, 3, 16, generator=g).numpy()
    x[1, 128:256, 2] = 0.0
    sc = fp8.block_scales(x, 128)
    assert sc.shape == (2, 3, 3)
    assert sc[1, 2, 1] == 1.0
    amax = np.abs(x[0, 256:300, 1]).max()
    assert sc[0, 1, 2] == np.float32(np.float32(amax) / np.float32(448.0))
    codes, sc2 = fp8.quantize_blocks(x, 128)
    assert (sc2 == sc).all()
    xd = fp8.dequantize_blocks(codes, sc, 128)
    # relative rounding error of E4M3 normals is at most 2^-4 (3 mantissa bits)
    scale_tok = np.repeat(sc, 128, axis=2)[:, :, :300].transpose(0, 2, 1)[..., None]
    err = np.abs(xd - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, scale_tok * 2.0 ** -10)
    assert (err <= bound + 1e-12).all()
    # every block's largest element maps to +-448 exactly
    assert np.abs(codes[0, :128, 0].astype(np.int32) & 0x7F).max() == 0x7E
