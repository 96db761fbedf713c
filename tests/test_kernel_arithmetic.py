"""CPU replays of float64 shortcuts the HIP kernels take, each checked against
the plain definition it stands in for.  numpy's float64 operations are IEEE
correctly rounded, as are the kernel's v_mul_f64 and its double division, so
the replay takes the same decisions as the kernel."""
import numpy as np


def codes_by_division(x, delta):
    """The definition: rint of the rounded quotient, clamped to [-127, 127]."""
    return np.clip(np.rint(x / delta), -127.0, 127.0)


def codes_by_product(x, delta):
    """The quantisation kernel's route: x * (1 / delta), with the division
    itself inside a 2^-40 band around half-integers."""
    y = x * (1.0 / delta)
    q = np.rint(y)
    near = np.abs(np.abs(y - np.trunc(y)) - 0.5) < 2.0 ** -40
    q[near] = np.rint(x[near] / delta)
    return np.clip(q, -127.0, 127.0), int(near.sum())


def to_bf16(a):
    """Round float32 values to bfloat16 (ties to even) and widen back."""
    u = np.asarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def test_product_codes_equal_division_codes_on_blocks():
    rng = np.random.default_rng(20261203)
    for trial in range(200):
        scale = 10.0 ** rng.uniform(-6, 4)
        x = to_bf16(rng.standard_normal(128 * 128) * scale)
        if trial % 2:                       # K blocks: minus a float64 channel mean
            x = x - to_bf16(rng.standard_normal(128) * scale).repeat(128)
        m = np.max(np.abs(x))
        delta = m / 127.0 if m > 0 else 1.0
        q, _ = codes_by_product(x, delta)
        assert np.array_equal(q, codes_by_division(x, delta))


def test_product_codes_equal_division_codes_at_near_ties():
    """x placed on and a few ulps around (k + 1/2) delta for every k, where
    the product and the quotient can fall on different sides of the tie."""
    rng = np.random.default_rng(7)
    fallbacks = 0
    for _ in range(50):
        m = 10.0 ** rng.uniform(-5, 5) * rng.uniform(1, 2)
        delta = m / 127.0
        ties = (np.arange(-127, 127) + 0.5) * delta
        xs = [ties]
        for steps in range(1, 6):
            up, dn = ties.copy(), ties.copy()
            for _ in range(steps):
                up = np.nextafter(up, np.inf)
                dn = np.nextafter(dn, -np.inf)
            xs += [up, dn]
        x = np.clip(np.concatenate(xs), -m, m)
        q, n = codes_by_product(x, delta)
        fallbacks += n
        assert np.array_equal(q, codes_by_division(x, delta))
    # the band is where the division is needed, and it was exercised
    assert fallbacks > 0


def test_guard_band_is_wide_enough():
    """|x * (1/delta) - fl(x / delta)| stays far inside the 2^-40 band for
    |x / delta| <= 127."""
    rng = np.random.default_rng(11)
    delta = 10.0 ** rng.uniform(-8, 8, 20000)
    x = rng.uniform(-127, 127, 20000) * delta
    gap = np.abs(x * (1.0 / delta) - x / delta)
    assert gap.max() < 2.0 ** -44


def dpp_source(ctrl):
    """Source lane of each of 64 lanes for the DPP controls the pooling
    kernel uses (the moves stay inside 16-lane rows)."""
    lanes = np.arange(64)
    base, i = lanes & ~15, lanes & 15
    if ctrl == "quad_1032":
        return base + (i & ~3) + np.array([1, 0, 3, 2])[i & 3]
    if ctrl == "quad_2301":
        return base + (i & ~3) + np.array([2, 3, 0, 1])[i & 3]
    if ctrl == "half_mirror":
        return base + (i & ~7) + (7 - (i & 7))
    if ctrl == "mirror":
        return base + (15 - i)
    raise ValueError(ctrl)


def test_dpp_group_sums_equal_xor_butterfly():
    """The pooling kernel sums each token's squares over groups of 8 or 16
    lanes with DPP moves (quad permutations, then mirrors) where an xor
    butterfly used to run; both add the same operands in the same order, so
    the float64 sums are identical bit for bit."""
    rng = np.random.default_rng(3)
    steps = {8: ["quad_1032", "quad_2301", "half_mirror"], 16: ["quad_1032", "quad_2301", "half_mirror", "mirror"]}
    for width, ctrls in steps.items():
        for _ in range(200):
            x = rng.standard_normal(64) * 10.0 ** rng.uniform(-8, 8, 64)
            dpp = x.copy()
            for c in ctrls:
                dpp = dpp + dpp[dpp_source(c)]
            xor = x.copy()
            off = 1
            while off < width:
                xor = xor + xor[np.arange(64) ^ off]
                off <<= 1
            assert np.array_equal(dpp, xor)
            # every lane of a group holds that group's total
            groups = dpp.reshape(-1, width)
            assert np.all(groups == groups[:, :1])


def test_half_wave_swap_sum_equals_xor_32():
    """x[l % 32] + x[32 + l % 32] (the two results of v_permlane32_swap) is
    x[l] + x[l ^ 32] in every lane."""
    rng = np.random.default_rng(4)
    for _ in range(100):
        x = rng.standard_normal(64) * 10.0 ** rng.uniform(-8, 8, 64)
        lanes = np.arange(64)
        swap = x[lanes % 32] + x[32 + lanes % 32]
        assert np.array_equal(swap, x + x[lanes ^ 32])


def test_block_sum_tree_equals_halving_loop():
    """mask_rows sums 256 doubles as (v[t] + v[t+128]) + (v[t+64] + v[t+192])
    for t < 64, then an xor butterfly over those 64 lanes, and takes lane 0.
    That is the tree of the LDS loop x[t] += x[t + off], off = 128 .. 1, so
    the softmax denominator is the same number bit for bit."""
    rng = np.random.default_rng(6)
    for _ in range(300):
        v = rng.standard_normal(256) * 10.0 ** rng.uniform(-10, 10, 256)
        x = v.copy()
        off = 128
        while off:
            x[:off] = x[:off] + x[off:2 * off]
            off >>= 1
        y = (v[:64] + v[128:192]) + (v[64:128] + v[192:256])
        off = 32
        while off:
            y = y + y[np.arange(64) ^ off]
            off >>= 1
        assert y[0] == x[0]
