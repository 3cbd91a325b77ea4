"""CPU checks of the parity gate helpers used by the GPU tests."""
import numpy as np

from oracle import formats as F
from parity import (assert_fp8_gate, assert_y_gate, e4m3_step_distance, fp8_flip_bound, fp8_ulp_distance,
                    fp8_values, y_errors)


def test_fp8_values_match_oracle_decode():
    q = np.arange(256, dtype=np.uint8).reshape(8, 32)
    q[q == 0x7F] = 0x7E
    q[q == 0xFF] = 0xFE
    sf = np.array([[120], [121], [127], [130], [0], [254], [100], [127]], np.uint8)
    want = F.decode_e4m3(q) * np.repeat(F.decode_e8m0(sf), 32, axis=1)
    assert np.array_equal(fp8_values(q, sf), want)


def test_ulp_distance_same_scale_is_code_distance():
    rng = np.random.default_rng(0)
    q = rng.integers(0, 0x7E, size=(4, 32)).astype(np.uint8)
    q2 = np.clip(q.astype(int) + rng.integers(-1, 2, size=q.shape), 0, 0x7E).astype(np.uint8)
    sf = np.full((4, 1), 120, np.uint8)
    d = fp8_ulp_distance(q2, sf, q, sf)
    steps = e4m3_step_distance(q2, q)
    same_binade = np.maximum(q >> 3, 1) == np.maximum(q2 >> 3, 1)
    assert np.all(d <= steps) and np.array_equal(d[same_binade], steps[same_binade])


def test_ulp_distance_across_scales():
    # the same value held at two adjacent scales is 0 apart; 1.125*2^k vs 2.0*2^(k-1)... one coarse ulp
    q_a = np.full((1, 32), 0x40, np.uint8)          # 2.0 at scale 2^-7
    q_b = np.full((1, 32), 0x38, np.uint8)          # 1.0 at scale 2^-6
    assert np.all(fp8_ulp_distance(q_a, np.array([[120]], np.uint8), q_b, np.array([[121]], np.uint8)) == 0)
    q_c = np.full((1, 32), 0x39, np.uint8)          # 1.125 at scale 2^-6 -> differs from 2.0*2^-7 by 1 ulp
    assert np.all(fp8_ulp_distance(q_a, np.array([[120]], np.uint8), q_c, np.array([[121]], np.uint8)) == 1)


def test_fp8_gate_counts_and_exemption():
    q = np.zeros((10, 32 * 10), np.uint8) + 0x38
    sf = np.full((10, 10), 120, np.uint8)
    q2 = q.copy()
    q2[0, 0] = 0x3A                                  # 2 ulps off
    cancel = np.zeros(q.shape, bool)
    try:
        assert_fp8_gate(q2, sf, q, sf, cancel)
        raise RuntimeError("expected failure")
    except AssertionError:
        pass
    cancel[0, 0] = True
    assert_fp8_gate(q2, sf, q, sf, cancel)            # exempt from the ulp clause, 1 of 3200 < 0.1%
    q3 = q.copy()
    q3[:, :4] = 0x39                                  # 40 of 3200 elements off by one ulp: 1.25% > 0.1%
    try:
        assert_fp8_gate(q3, sf, q, sf, cancel)
        raise RuntimeError("expected failure")
    except AssertionError:
        pass


def test_y_errors():
    ref = np.array([1.0, -2.0, 4.0], np.float32)
    assert y_errors(ref, ref) == (0.0, 0.0)
    mx, mean = y_errors(ref + np.array([0.04, 0, 0], np.float32), ref)
    assert abs(mx - 0.01) < 1e-7 and abs(mean - 0.04 / 7) < 1e-7


def test_flip_bound_covers_every_admitted_difference():
    # brute force: every finite E4M3 code of the oracle at scale 2^0, every device code at the same scale or
    # one step coarser or finer; wherever the 1-ulp clause admits the pair, the difference is within the bound
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    qr, qg = np.meshgrid(codes, codes, indexing="ij")
    qr = np.repeat(qr.reshape(-1, 1), 32, axis=1)
    qg = np.repeat(qg.reshape(-1, 1), 32, axis=1)
    sr = np.full((qr.shape[0], 1), 127, np.uint8)
    checked = 0
    for dsf in (-1, 0, 1):
        sg = (sr.astype(int) + dsf).astype(np.uint8)
        ok = fp8_ulp_distance(qg, sg, qr, sr) <= 1.0
        diff = np.abs(fp8_values(qg, sg) - fp8_values(qr, sr))
        assert np.all(diff[ok] <= fp8_flip_bound(qr, sr)[ok])
        checked += int(ok.sum())
    assert checked > 0


def test_y_gate_allowance_admits_only_the_propagated_amount():
    ref = np.full((10, 100), 100.0)
    y = ref.copy()
    y[3, 7] += 3.0                                  # 3% of max |ref| at one element; mean error stays tiny
    allow_here = np.zeros_like(ref)
    allow_here[3, 7] = 2.5                          # leaves 0.5% of max |ref|
    allow_elsewhere = np.full_like(ref, 5.0)
    allow_elsewhere[3, 7] = 0.0
    for allowance, passes in ((None, False), (allow_here, True), (allow_elsewhere, False)):
        try:
            assert_y_gate(y, ref, "case", allowance=allowance)
            ok = True
        except AssertionError:
            ok = False
        assert ok == passes


def test_cancellation_at_matches_rowwise():
    """The element-wise Linear1 cancellation mask agrees with the row-wise one at every element."""
    from parity import linear1_cancellation, linear1_cancellation_at
    rng = np.random.default_rng(5)
    H, I = 256, 64
    a = rng.standard_normal((6, H))
    w1 = rng.standard_normal((2 * I, H))
    # make some exact sums cancel: copy a row of W1 with a sign flip half way
    w1[3, H // 2:] = -w1[3, :H // 2] * (a[2, :H // 2] / a[2, H // 2:])
    full = linear1_cancellation(a, w1)
    assert full.any() and not full.all()
    r, c = np.nonzero(np.ones_like(full))
    got = linear1_cancellation_at(a[r], lambda rows: w1[rows], c)
    assert np.array_equal(got, full[r, c])
