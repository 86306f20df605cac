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


# ---- MX (microscaling) FP8 pins ----------------------------------------------

def mx_case(seed, shape):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(*shape, generator=g) * torch.exp(torch.randn(*shape, generator=g) * 2)
    return x.numpy().astype(np.float32)


def smallest_fitting_exponent(amax):
    """The least e with amax <= 448 * 2^e, by search (exact in float64)."""
    if amax == 0:
        return 0
    e = int(np.floor(np.log2(amax))) - 10
    while amax > 448.0 * 2.0 ** e:
        e += 1
    return max(-127, min(127, e))


def test_mx_exponent_closed_form():
    amax = np.array([1.0, 1.5, 0.75, 448.0, 449.0, 512.0, 1.76, 2.0 ** -100, 3.0e38, 0.0])
    e = fp8.mx_exponent(amax)
    assert list(e) == [-8, -8, -9, 0, 1, 1, -7, -108, 120, 0]
    assert list(e) == [smallest_fitting_exponent(a) for a in amax]
    # the block maximum lands in (224, 448] * 2^e: no clipping, top two binades
    nz = amax > 0
    r = amax[nz] / np.exp2(e[nz].astype(np.float64))
    assert ((r > 224) & (r <= 448)).all()
    assert fp8.mx_exponent(np.array([2.0 ** -130]))[0] == -127   # clamped


def test_mx_codes_match_torch_cast():
    # codes are torch's own e4m3fn cast of x / 2^e (clamped to the finite range)
    x = mx_case(2, (2, 40, 3, 64))
    codes, sc = fp8.quantize_mx(x, "d")
    assert sc.shape == (2, 40, 3, 2) and sc.dtype == np.uint8
    e = np.repeat(sc.astype(np.int64) - 127, 32, axis=3)
    y = torch.from_numpy((x / np.exp2(e).astype(np.float32)).astype(np.float32)).clamp(-448, 448)
    ref = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (codes == ref).all()
    amax = np.abs(x).reshape(2, 40, 3, 2, 32).max(axis=4)
    want = np.vectorize(smallest_fitting_exponent)(amax.astype(np.float64)) + 127
    assert (sc == want.astype(np.uint8)).all()


def test_mx_token_blocks_and_roundtrip():
    # V: blocks of 32 tokens per (batch, head, d), a partial last block, a zero block
    x = mx_case(3, (1, 70, 2, 64))
    x[0, 32:64, 1, 5] = 0.0
    codes, sc = fp8.quantize_mx(x, "s")
    assert sc.shape == (1, 2, 3, 64)
    assert sc[0, 1, 1, 5] == 127 and (codes[0, 32:64, 1, 5] & 0x7F == 0).all()
    amax_tail = np.abs(x[0, 64:70, 0, 7]).max()
    assert sc[0, 0, 2, 7] == smallest_fitting_exponent(float(amax_tail)) + 127
    xd = fp8.dequantize_mx(codes, sc, "s")
    e_el = np.repeat(sc.astype(np.int64) - 127, 32, axis=2)[:, :, :70].transpose(0, 2, 1, 3)
    step = np.exp2(e_el.astype(np.float64))
    # nothing saturates: the rounding error is at most half a step of 3
    # mantissa bits (2^-4 relative) or half the subnormal spacing 2^-10
    err = np.abs(xd - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, step * 2.0 ** -10)
    assert (np.abs(x) / step <= 448).all()
    assert (err <= bound + 1e-300).all()
    # every nonzero block's largest element decodes into E4M3's top two binades
    top = np.abs(codes[0, :32, 0, 0].astype(np.int32) & 0x7F).max()
    assert (top >> 3) >= 14


# ---- per-tensor quantisation and the MX decoder along d ----------------------

def test_quantize_tensor_pins():
    """Per-tensor quantisation, pinned independently of the oracle's code:
    the scale is the tensor's amax / 448 in fp32 (computed here with torch),
    the largest magnitude encodes to 0x7E (448), every code is torch's own
    e4m3fn cast of the fp32 quotient x / scale, and a zero tensor gets
    scale 1 with all-zero codes."""
    g = torch.Generator().manual_seed(11)
    xt = torch.randn(2, 70, 3, 32, generator=g) * torch.exp(torch.randn(2, 70, 3, 32, generator=g))
    xt[1, 5, 2, 7] = -37.5                       # a unique largest magnitude, negative
    xt = xt.clamp(-30.0, 30.0)
    xt[1, 5, 2, 7] = -37.5
    codes, s = fp8.quantize_tensor(xt.numpy())
    s_want = (xt.abs().max() / torch.tensor(448.0)).item()
    assert np.float32(s) == np.float32(s_want)
    assert codes[1, 5, 2, 7] == 0xFE             # -448
    assert ((codes & 0x7F) <= 0x7E).all()
    # only the largest element (up to ties) reaches the top code
    assert int(((codes & 0x7F) == 0x7E).sum()) == 1
    y = (xt / torch.tensor(np.float32(s))).to(torch.float32)
    ref = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (codes == ref).all()
    # the decoded tensor is within E4M3's rounding of x
    xd = fp8.decode_e4m3(codes) * np.float64(s)
    x = xt.numpy().astype(np.float64)
    assert (np.abs(xd - x) <= np.maximum(np.abs(x) * 2.0 ** -4, float(s) * 2.0 ** -10) + 1e-12).all()
    z_codes, z_s = fp8.quantize_tensor(np.zeros((1, 3, 2, 16), np.float32))
    assert np.float32(z_s) == 1.0 and (z_codes == 0).all()


def test_quantize_blocks_codes_match_torch_cast():
    """Per-block codes are torch's e4m3fn cast of x / (its block's scale)."""
    g = torch.Generator().manual_seed(12)
    x = (torch.randn(1, 260, 2, 64, generator=g) * 3).numpy()
    codes, sc = fp8.quantize_blocks(x, 128)
    tok = np.repeat(sc, 128, axis=2)[:, :, :260].transpose(0, 2, 1)[..., None]
    y = torch.from_numpy((x / tok.astype(np.float32)).astype(np.float32))
    ref = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (codes == ref).all()


def test_mx_d_roundtrip():
    """dequantize_mx along d inverts quantize_mx within E4M3's rounding, with
    each 32-element block's step taken from the shared exponent computed here
    by exact search; a zero block decodes to zeros."""
    x = mx_case(4, (2, 9, 3, 96))
    x[1, 4, 2, 32:64] = 0.0
    codes, sc = fp8.quantize_mx(x, "d")
    xd = fp8.dequantize_mx(codes, sc, "d")
    assert xd.shape == x.shape and xd.dtype == np.float64
    amax = np.abs(x).reshape(2, 9, 3, 3, 32).max(axis=4).astype(np.float64)
    e = np.vectorize(smallest_fitting_exponent)(amax)
    step = np.exp2(np.repeat(e, 32, axis=3).astype(np.float64))
    err = np.abs(xd - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, step * 2.0 ** -10)
    assert (err <= bound + 1e-300).all()
    assert (xd[1, 4, 2, 32:64] == 0.0).all()
    # decoding with a scale byte one higher doubles every value of that block
    sc2 = sc.copy()
    sc2[0, 0, 0, 1] += 1
    xd2 = fp8.dequantize_mx(codes, sc2, "d")
    assert np.array_equal(xd2[0, 0, 0, 32:64], 2.0 * xd[0, 0, 0, 32:64])
    assert np.array_equal(xd2[0, 0, 0, :32], xd[0, 0, 0, :32])
