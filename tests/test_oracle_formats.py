"""Pins of the oracle's number formats against the OCP MX definitions and library casts."""
import numpy as np
import pytest
import torch

from oracle import formats as F


def test_e4m3_table_special_points():
    # OCP E4M3FN: max normal 448 (0x7E), min normal 2^-6 (0x08), min subnormal 2^-9 (0x01),
    # 1.0 = 0x38, NaN at 0x7F / 0xFF, no infinities, sign-magnitude.
    t = F.E4M3_TABLE
    assert t[0x7E] == 448.0 and t[0x08] == 2.0 ** -6 and t[0x01] == 2.0 ** -9 and t[0x38] == 1.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert t[0x00] == 0.0 and np.signbit(t[0x80])
    assert np.array_equal(t[0x80:0xFF], -t[0x00:0x7F])
    assert np.all(np.diff(t[:0x7F]) > 0)


def test_e4m3_table_vs_torch_cast():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = F.E4M3_TABLE
    same = (ref == ours) | (np.isnan(ref) & np.isnan(ours))
    assert same.all()


def test_e2m1_table_ocp_values():
    # OCP MX v1.0 E2M1 magnitudes; the walk-through page's "[0.5, 7.5] with NaN" is garbled.
    assert list(F.E2M1_TABLE[:8]) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert np.array_equal(F.E2M1_TABLE[8:], -F.E2M1_TABLE[:8])


def test_e8m0_vs_torch_cast():
    codes = torch.arange(255, dtype=torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(F.decode_e8m0(np.arange(255)), ref)
    assert np.isnan(F.decode_e8m0(np.array([255]))[0])


def test_fp4_nibble_order():
    packed = np.array([[0x21, 0x7F]], np.uint8)   # low nibble first
    assert list(F.unpack_fp4(packed)[0]) == [1, 2, 0xF, 0x7]
    assert list(F.decode_e2m1_packed(packed)[0]) == [0.5, 1.0, -6.0, 6.0]


def _e4m3_test_values(rng):
    pos = F.E4M3_TABLE[:0x7F]
    mids = (pos[1:] + pos[:-1]) / 2                                   # exact ties
    f32 = lambda a: np.asarray(a, np.float32)
    near = np.concatenate([np.nextafter(f32(mids), np.float32(0)), np.nextafter(f32(mids), np.float32(1e9))])
    rnd = rng.uniform(-448, 448, 200_000).astype(np.float32)
    small = (rng.uniform(-1, 1, 50_000) * 2.0 ** -5).astype(np.float32)
    tiny = (rng.uniform(-1, 1, 20_000) * 2.0 ** -11).astype(np.float32)
    v = np.concatenate([pos, -pos, mids, -mids, near, -near, rnd, small, tiny, [0.0, -0.0]]).astype(np.float32)
    return v[np.abs(v) <= 448]


def test_encode_e4m3_rne_vs_torch_cast():
    v = _e4m3_test_values(np.random.default_rng(0))
    ours = F.encode_e4m3_rne(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_encode_e4m3_rejects_out_of_range():
    with pytest.raises(ValueError):
        F.encode_e4m3_rne(np.array([449.0]))


def test_bf16_rne_vs_torch_cast():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 32, 1_000_000, dtype=np.uint64).astype(np.uint32)
    # force a share of exact ties and near-ties in the dropped half
    bits[:200_000] = (bits[:200_000] & 0xFFFF0000) | 0x8000
    bits[200_000:300_000] = (bits[200_000:300_000] & 0xFFFF0000) | 0x7FFF
    bits[300_000:400_000] = (bits[300_000:400_000] & 0xFFFF0000) | 0x8001
    v = bits.view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) < 3.0e38)]
    ours = F.bf16_rne(v)
    ref = torch.from_numpy(v.copy()).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


def _scale_code_brute(amax):
    """Smallest code c in [0, 254] with amax * 2**(127 - c) <= 448, by exhaustive search."""
    out = []
    for a in amax:
        for c in range(255):
            if float(a) * 2.0 ** (127 - c) <= 448.0:
                out.append(c)
                break
        else:
            out.append(254)
    return np.array(out, np.uint8)


def test_requant_scale_code_brute_force():
    rng = np.random.default_rng(2)
    a = np.abs(rng.standard_normal(3000) * np.exp(rng.uniform(-30, 30, 3000))).astype(np.float32)
    edges = []
    for s in range(-20, 30):
        b = np.float32(448.0 * 2.0 ** s)
        edges += [b, np.nextafter(b, np.float32(0)), np.nextafter(b, np.float32(1e30)),
                  np.float32(2.0 ** s), np.float32(1.75 * 2.0 ** s)]
    a = np.concatenate([a, np.array(edges, np.float32), np.array([0.0, 1e-40, 1.4e-45, 3e38], np.float32)])
    assert np.array_equal(F.requant_scale_code(a), _scale_code_brute(a))


def test_requant_scale_code_keeps_fp8_range():
    rng = np.random.default_rng(3)
    a = np.abs(rng.standard_normal(10000) * 30).astype(np.float32) + 1e-6
    c = F.requant_scale_code(a).astype(np.int64)
    assert np.all(a * 2.0 ** (127 - c) <= 448)
    assert np.all(a * 2.0 ** (127 - (c - 1)) > 448)
