"""Comparison helpers for GPU-vs-oracle parity tests (correctness gates).

Gates (one reading of the stated bars):
* routing tables: bit-exact over their defined ranges;
* FP8 intermediates: on at most 0.1% of the elements of valid rows may the
  (code, scale) pair differ from the oracle's; a differing scale code counts
  all 32 elements of its group.  Where they differ, the represented values
  (code times scale) are at most 1 E4M3 ulp apart, the ulp taken at the
  coarser of the two scales.  Elements whose exact Linear1 gate or up
  accumulator is within 2**-14 of its sum of |products| from zero are
  exempt from the 1-ulp clause (they still count toward the 0.1%): there the
  BF16 input of the epilogue is not determined by the accumulation at all,
  since gfx950's scaled MFMA carries a dot-product error up to about
  2**-19 of the sum of |products| (measured), 32x below that threshold;
* y (BF16): max |y - ref| <= 1e-2 * max |ref| and
  sum |y - ref| / sum |ref| <= 5e-3, as stated, for every fixed case.
  Only the seeded shape fuzz may widen the max clause, and only for a case
  that fails it as stated: by a (per element of y), how far the FP8
  differences admitted above can move it (Linear2 is linear in h, so an
  admitted difference of at most fp8_flip_bound in h[r, c] moves slot row r
  by at most that times |W2[:, c]|, and the combine adds a token's slot
  rows; one admitted flip of an element that dominates its row moves that
  token's y by a few percent of max |ref|).  The fuzz reports how many
  cases needed it.
"""
import numpy as np

PLAN_FIELDS = ("counts", "offsets", "slot", "row_token", "row_topk", "block_expert", "slack", "pull_order")


def gpu_plan_to_numpy(v: dict, T: int, k: int) -> dict:
    out = {f: v[f].cpu().numpy() for f in PLAN_FIELDS}
    out["slot"] = out["slot"].reshape(T, k)
    out["scalars"] = v["scalars"].cpu().numpy()
    return out


def assert_plan_equal(g: dict, p) -> None:
    r_pad, n_pull, n_valid, n_blocks = (int(x) for x in g["scalars"][:4])
    assert (r_pad, n_pull, n_valid, n_blocks) == (p.r_pad, p.n_pull, p.num_valid, p.n_blocks)
    assert np.array_equal(g["counts"], p.counts)
    assert np.array_equal(g["offsets"], p.offsets)
    assert np.array_equal(g["slot"], p.slot)
    assert np.array_equal(g["row_token"][:r_pad], p.row_token)
    assert np.array_equal(g["row_topk"][:r_pad], p.row_topk)
    assert np.array_equal(g["block_expert"][:n_blocks], p.block_expert)
    assert np.array_equal(g["slack"][:n_blocks], p.slack)
    assert np.array_equal(g["pull_order"][:n_pull], p.pull_order)


def e4m3_step_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Number of E4M3 grid steps between two code arrays (+0 and -0 are equal)."""
    a = a.astype(np.int64)
    b = b.astype(np.int64)
    sa = np.where((a & 0x7F) == 0, 0, np.where(a & 0x80, -1, 1)) * (a & 0x7F)
    sb = np.where((b & 0x7F) == 0, 0, np.where(b & 0x80, -1, 1)) * (b & 0x7F)
    return np.abs(sa - sb)


_E4M3_MAG = np.array([(m * 2.0 ** -9) if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
                      for e in range(16) for m in range(8)])   # magnitudes of codes 0x00..0x7F


def fp8_values(q, sf):
    """Represented values of (E4M3 code, UE8M0 per-32 scale) pairs, float64."""
    q = np.asarray(q)
    mag = _E4M3_MAG[q & 0x7F]
    sign = np.where(q & 0x80, -1.0, 1.0)
    scale = np.repeat(np.ldexp(1.0, np.asarray(sf, np.int64) - 127), 32, axis=-1)
    return sign * mag * scale


def fp8_ulp_distance(q_gpu, sf_gpu, q_ref, sf_ref):
    """|value difference| in E4M3 ulps at the coarser scale and the larger magnitude."""
    vg, vr = fp8_values(q_gpu, sf_gpu), fp8_values(q_ref, sf_ref)
    scale = np.repeat(np.ldexp(1.0, np.maximum(np.asarray(sf_gpu, np.int64), np.asarray(sf_ref, np.int64)) - 127),
                      32, axis=-1)
    m = np.maximum(np.abs(vg), np.abs(vr)) / scale                 # magnitude on the E4M3 grid
    _, e = np.frexp(np.maximum(m, 1e-300))
    ulp = np.ldexp(1.0, np.maximum(e - 1, -6) - 3)                 # 2**-9 in the subnormal range
    return np.abs(vg - vr) / (ulp * scale)


def assert_fp8_gate(q_gpu, sf_gpu, q_ref, sf_ref, cancel=None, what="", rate=True):
    """The FP8 gate above; `cancel` marks elements with near-total cancellation in Linear1.  Returns
    (elements whose code or scale differs, elements compared).  rate=False checks only the 1-ulp clause,
    for callers that apply the 0.1% to elements pooled over several small cases (on a few thousand
    elements one mismatch more or less moves the fraction by several hundredths of a percent)."""
    if q_ref.size == 0:
        return 0, 0
    code_bad = (e4m3_step_distance(q_gpu, q_ref) > 0) | np.repeat(sf_gpu != sf_ref, 32, axis=1)
    frac = float(code_bad.mean())
    dist = fp8_ulp_distance(q_gpu, sf_gpu, q_ref, sf_ref)
    judged = dist if cancel is None else dist[~cancel]
    worst = float(judged.max()) if judged.size else 0.0
    assert (frac <= 1e-3 or not rate) and worst <= 1.0, (
        f"{what}: FP8 mismatch on {frac:.4%} of elements, worst {worst:.2f} ulp outside cancellation "
        f"(scale mismatches {int((sf_gpu != sf_ref).sum())})")
    return int(code_bad.sum()), int(code_bad.size)


def linear1_cancellation(a_rows, w1_rows_deq):
    """Mask [n, I] of elements whose exact gate or up sum is within 2**-14 * sum|products| of zero."""
    from oracle.forward import deinterleave_gate_up
    z = a_rows @ w1_rows_deq.T
    s = np.abs(a_rows) @ np.abs(w1_rows_deq).T
    zg, zu = deinterleave_gate_up(z)
    sg, su = deinterleave_gate_up(s)
    return (np.abs(zg) < 2.0 ** -14 * sg) | (np.abs(zu) < 2.0 ** -14 * su)


def linear1_cancellation_at(a_rows, w1_rows_of, chans):
    """For elements i (activation row a_rows[i] of one expert, SwiGLU channel chans[i]): whether the exact
    gate or up sum is within 2**-14 * sum|products| of zero.  w1_rows_of(rows) returns the expert's
    dequantized W1 rows (interleaved order); the channel -> row map is the oracle's de-interleave."""
    from oracle.forward import deinterleave_gate_up
    out = np.zeros(len(chans), bool)
    if len(chans) == 0:
        return out
    n2 = 2 * (int(chans.max()) // 8 + 1) * 8
    gate_row, up_row = deinterleave_gate_up(np.arange(n2))
    for i0 in range(0, len(chans), 4096):
        a = a_rows[i0:i0 + 4096]
        ch = chans[i0:i0 + 4096]
        for rows in (gate_row[ch], up_row[ch]):
            w = w1_rows_of(rows)
            z = np.einsum("ij,ij->i", a, w)
            s = np.einsum("ij,ij->i", np.abs(a), np.abs(w))
            out[i0:i0 + 4096] |= np.abs(z) < 2.0 ** -14 * s
    return out


def bf16_to_f32(bits_i16: np.ndarray) -> np.ndarray:
    return (bits_i16.astype(np.uint16).astype(np.uint32) << 16).view(np.float32)


def y_errors(y, ref):
    err = np.abs(y.astype(np.float64) - ref.astype(np.float64))
    mx = float(np.abs(ref).max()) if ref.size else 0.0
    rel_max = float(err.max()) / mx if mx > 0 else float(err.max())
    den = float(np.abs(ref).sum())
    rel_mean = float(err.sum()) / den if den > 0 else float(err.sum())
    return rel_max, rel_mean


def fp8_flip_bound(q_ref, sf_ref):
    """Per element, an upper bound on the value difference the FP8 gate's 1-ulp clause admits, from the
    oracle's (code, scale) alone: one ulp at up to twice the scale (a scale one step coarser) and up to the
    next binade (the larger of the two magnitudes), i.e. 4 ulp of the oracle's value at its own scale."""
    s = np.repeat(np.ldexp(1.0, np.asarray(sf_ref, np.int64) - 127), 32, axis=-1)
    m = np.abs(fp8_values(q_ref, sf_ref)) / s
    _, e = np.frexp(np.maximum(m, 1e-300))
    return 4.0 * np.ldexp(1.0, np.maximum(e - 1, -6) - 3) * s


def y_gate_ok(y, ref, allowance=None):
    """(passes, max clause value, mean clause value) of the y gate; `allowance` is the fuzz's a."""
    rel_max, rel_mean = y_errors(y, ref)
    if allowance is not None:
        m = float(np.abs(ref).max()) if ref.size else 0.0
        over = np.abs(np.asarray(y, np.float64) - ref) - allowance
        rel_max = float(max(over.max(), 0.0)) / m if m > 0 else float(max(over.max(), 0.0))
    return rel_max <= 1e-2 and rel_mean <= 5e-3, rel_max, rel_mean


def assert_y_gate(y, ref, what="", allowance=None):
    """The y gate above (as stated when allowance is None)."""
    ok, rel_max, rel_mean = y_gate_ok(y, ref, allowance)
    assert np.all(np.isfinite(y)), f"{what}: y holds non-finite values"
    assert ok, f"{what}: y max err {rel_max:.3e}, mean rel err {rel_mean:.3e}"
    return rel_max, rel_mean


def tile_columns(which):
    """Weight row (within a 256-row block) stored at each tile column of the tiled weight layout, as
    documented for moe_prepare_weights in include/moe.h (which = 1: W1, 2: W2)."""
    c = np.arange(256)
    if which == 1:
        G, b, j = c >> 6, (c >> 4) & 3, c & 15
        ch = 32 * G + 2 * j + (b & 1)                  # SwiGLU channel; gate rows for b < 2, up rows for b >= 2
        return (ch // 8) * 16 + (ch % 8) + 8 * (b >= 2)
    S, b, j = c >> 7, (c >> 4) & 7, c & 15
    return 128 * S + 8 * j + b
