"""Pins for the oracle's MXFP4 (e2m1 + e8m0 per 32) quantisation.

The reading pinned here: shared exponent s = floor(log2(amax)) - 2 clamped to
[-127, 127]; each element goes to the nearest e2m1 magnitude of |v| / 2^s,
ties to the even code, saturating at 6; element 2i in the low nibble.
"""
import numpy as np
import pytest

MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
MIDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
# A tie at a midpoint whose lower neighbour has an odd code rounds up.
TIE_UP = np.array([False, True, False, True, False, True, False])


def _threshold_codes(q: np.ndarray) -> np.ndarray:
    """Independent rule: count the midpoints below |q| (at a midpoint, round
    towards the even code)."""
    a = np.abs(q)[..., None]
    c = (a > MIDS).sum(-1) + ((a == MIDS) & TIE_UP).sum(-1)
    return (c | np.where(np.signbit(q), 8, 0)).astype(np.uint8)


def _all_finite_bf16():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = (b.astype(np.uint32) << 16).view(np.float32)
    keep = np.isfinite(v)
    return b[keep], v[keep].astype(np.float64)


@pytest.mark.parametrize("s", [-3, -1, 0, 2, 3])
def test_exhaustive_bf16_against_threshold_rule(orc, s):
    b, v = _all_finite_bf16()
    n = b.size
    anchor = np.float32(2.0 ** (s + 2))
    anchor_bits = np.array([anchor], dtype=np.float32).view(np.uint32)[0] >> 16
    rows = np.zeros((n, 32), dtype=np.uint16)
    rows[:, 0] = anchor_bits
    rows[:, 1] = b
    codes, scales = orc.mxfp4_quant(rows)
    amax = np.maximum(float(anchor), np.abs(v))
    s_eff = np.clip(np.floor(np.log2(amax)) - 2, -127, 127)
    assert (scales[:, 0].astype(np.int64) == s_eff.astype(np.int64) + 127).all()
    q = v / np.exp2(s_eff)
    want = _threshold_codes(q)
    got = codes[:, 0] >> 4                              # element 1 is the high nibble
    assert (got == want).all()
    assert ((codes[:, 0] & 15) == _threshold_codes(float(anchor) / np.exp2(s_eff))).all()


def test_grid_values_round_trip(orc):
    for s in (-5, 0, 4):
        vals = np.concatenate([MAGS, -MAGS[1:], MAGS[:8], -MAGS[1:7], [6.0, -6.0, 4.0]])[:32]
        x = (vals * 2.0 ** s).astype(np.float32)
        # largest magnitude is 6 * 2^s -> floor(log2) = s + 2 -> shared exponent s
        c, sc = orc.mxfp4_quant_f32(x)
        assert sc[0] == s + 127
        assert (orc.mxfp4_dequant(c[None], sc[None])[0] == x.astype(np.float64)).all()


def test_dequant_error_within_half_step(orc):
    rng = np.random.default_rng(0)
    x = rng.standard_normal(32 * 4096).astype(np.float32) * 3.0
    c, sc = orc.mxfp4_quant_f32(x)
    d = orc.mxfp4_dequant(c, sc)
    scale = np.repeat(np.exp2(sc.astype(np.float64) - 127), 32)
    q = np.abs(x.astype(np.float64)) / scale
    step = np.where(q < 2, 0.5, np.where(q < 4, 1.0, 2.0))
    err = np.abs(d - x) / scale
    sat = q > 6
    assert (err[~sat] <= step[~sat] / 2 + 1e-12).all()
    assert (np.abs(d[sat]) == 6 * scale[sat]).all()
    # the scale rule puts amax / 2^s in [4, 8)
    amax = np.abs(x.reshape(-1, 32)).max(1)
    r = amax / np.exp2(sc.astype(np.float64) - 127)
    assert ((r >= 4) & (r < 8)).all()


def test_sign_and_nibble_order(orc):
    x = np.zeros(32, dtype=np.float32)
    x[0], x[1], x[2], x[3] = 4.0, -1.0, 0.5, -0.0
    c, sc = orc.mxfp4_quant_f32(x)
    assert sc[0] == 127                       # amax 4 -> floor(log2) 2 -> s 0
    assert c[0] == (0x6 | (0xA << 4))          # 4.0 -> 6 (low), -1.0 -> 8|2 (high)
    assert c[1] == (0x1 | (0x8 << 4))          # 0.5 -> 1, -0.0 -> sign only


def test_zero_and_tiny_groups(orc):
    c, sc = orc.mxfp4_quant_f32(np.zeros(32, dtype=np.float32))
    assert sc[0] == 0 and (c == 0).all()
    tiny = np.full(32, 2.0 ** -130, dtype=np.float32)   # subnormal fp32
    c, sc = orc.mxfp4_quant_f32(tiny)
    assert sc[0] == 0                                    # clamped at -127
    # 2^-130 / 2^-127 = 0.125 -> rounds to 0
    assert (c == 0).all()
