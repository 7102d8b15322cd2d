"""fp32 inputs that isolate the fp32 -> bf16 round-to-nearest-even step of
the weightless RMS rescale (test data only: bit patterns and an exact
power-of-two scaling, no arithmetic of the method)."""
import numpy as np

H = 64  # one anchor + 63 test values per row


def rounding_patterns() -> np.ndarray:
    """fp32 bit patterns (uint32) that exercise every branch of
    round-to-nearest-even to bf16: the dropped 16 bits below, at and above
    one half (0x7FFF, 0x8000, 0x8001) with an even and an odd kept bit,
    exact values, a carry out of the kept mantissa into the exponent,
    subnormals (a tie among them, and the round-up into the smallest
    normal), both signs.  Every magnitude is below 2^-12."""
    pats = []
    for exp_field in (0, 1, 2, 40, 100, 114):  # 114: |t| < 2^-12
        for hi in (0x00, 0x01, 0x02, 0x3F, 0x40, 0x7E, 0x7F):  # the 7 kept mantissa bits
            for lo in (0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x1234, 0xC000):
                u = (exp_field << 23) | (hi << 16) | lo
                pats += [u, u | 0x80000000]
    pats += [0x007FFFFF, 0x007F8000, 0x00008000, 0x00018000, 0x00000001]  # subnormal edges
    return np.array(sorted(set(p for p in pats if p & 0x7FFFFFFF)), np.uint32)


def anchored_rows():
    """Rows y[R][64] = [2^20, t_1 * 2^17, ..., t_63 * 2^17] and the patterns
    t[R][63] they carry.  |t * 2^17| < 32, so the 63 squares sum to less
    than 2^16, half an ulp of 2^40, in any order: the sum of squares of a
    row is exactly 2^40 however it is summed, the mean 2^34, and the RMS
    factor exactly 2^-17, so y * factor reproduces t exactly."""
    t = rounding_patterns().view(np.float32)
    rows = -(-t.size // (H - 1))
    tt = np.zeros(rows * (H - 1), np.float32)
    tt[:t.size] = t
    tt = tt.reshape(rows, H - 1)
    y = np.empty((rows, H), np.float32)
    y[:, 0] = np.float32(2.0 ** 20)
    y[:, 1:] = tt * np.float32(2.0 ** 17)
    assert np.array_equal(y[:, 1:] * np.float32(2.0 ** -17), tt)  # the scaling is exact
    assert np.all(np.abs(y[:, 1:]) < 32.0)
    assert float(np.sum(y[:, 1:].astype(np.float64) ** 2, axis=1).max()) < 2.0 ** 16
    return y, tt


def anchored_row_7168():
    """One row of 7168 fp32 values: seven anchors 2^20 (at multiples of
    1024) and the rounding patterns t scaled by 2^15 elsewhere (zeros past
    them).  The squares of the non-anchor values sum to less than 2^16, half
    an ulp of 2^40, so in any summation order the sum of squares is exactly
    7 * 2^40, the mean 2^30 and the RMS factor exactly 2^-15: the rescaled
    row is the anchors' 32.0 and exactly the patterns t.  Returns (y[7168],
    t-row[7168], anchor mask)."""
    t = rounding_patterns().view(np.float32)
    n = 7168
    anchor = np.zeros(n, bool)
    anchor[::1024] = True
    free = np.nonzero(~anchor)[0]
    assert t.size <= free.size
    trow = np.zeros(n, np.float32)
    trow[free[:t.size]] = t
    y = trow * np.float32(2.0 ** 15)
    y[anchor] = np.float32(2.0 ** 20)
    trow[anchor] = np.float32(32.0)
    assert np.array_equal(y[~anchor] * np.float32(2.0 ** -15), trow[~anchor])
    assert float(np.sum(y[~anchor].astype(np.float64) ** 2)) < 2.0 ** 16
    return y, trow, anchor
