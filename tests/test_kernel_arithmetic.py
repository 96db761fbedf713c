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


# ---------------------------------------------------------------------------
# mask_rows' TopCdf: a radix select over the probabilities' bit patterns with
# exact 2^-62 fixed-point sums, replayed in Python integers
# ---------------------------------------------------------------------------

def topcdf_threshold(F, tau):
    """The kernel's fixed-point threshold TF = ceil(tau * F), from tau's
    integer mantissa m and exponent (tau = m * 2^-s) and the exact product
    m * F, as mask_rows computes it in 128-bit integers."""
    bits = int(np.array([tau], dtype=np.float64).view(np.uint64)[0])
    ex = (bits >> 52) & 0x7FF
    m = bits & ((1 << 52) - 1)
    s = 1074
    if ex:
        m |= 1 << 52
        s = 1075 - ex
    if m == 0 or F == 0:
        return 0
    if s >= 117:
        return 1
    prod = m * F
    assert prod < 1 << 128
    return (prod + (1 << s) - 1) >> s


def topcdf_radix_select(pr, tau):
    """mask_rows' selection for one row of probabilities ``pr`` (float64, in
    ascending column order): returns the kept mask.  Raises if no histogram
    bin crosses the threshold (the kernel would then read its boundary
    digit uninitialised)."""
    key = pr.view(np.uint64).astype(object)
    fx = [int(x) for x in np.floor(pr * 2.0 ** 62)]   # (uint64)(pr * 2^62): a truncation
    F = sum(fx)
    TF = topcdf_threshold(F, tau)
    prefix, above = 0, 0
    for pas in range(8):
        shift = 56 - 8 * pas
        cnt = [0] * 256
        sums = [0] * 256
        for k, f in zip(key, fx):
            if (k >> shift) >> 8 == prefix:
                cnt[(k >> shift) & 255] += 1
                sums[(k >> shift) & 255] += f
        cum, digit = above, None
        for dgt in range(255, -1, -1):
            if cum < TF <= cum + sums[dgt]:
                digit, new_above = dgt, cum
            cum += sums[dgt]
        if digit is None:
            raise AssertionError("no bin crosses the threshold")
        prefix = (prefix << 8) | digit
        above = new_above
        if pas < 7 and cnt[digit] == 1:
            prefix = next(k for k in key if (k >> shift) == prefix)
            break
    v = prefix
    fv = int(np.floor(np.array([v], dtype=np.uint64).view(np.float64)[0] * 2.0 ** 62))
    n_ties = sum(1 for k in key if k == v)
    tie_keep = n_ties if fv == 0 else min(n_ties, (TF - above + fv - 1) // fv)
    keep = np.zeros(len(pr), dtype=bool)
    rank = 0
    for x, k in enumerate(key):
        if k > v:
            keep[x] = True
        elif k == v:
            keep[x] = rank < tie_keep
            rank += 1
    return keep, F, TF


def topcdf_fixed_point_definition(pr, TF):
    """Eq. 8 on the fixed-point values: in the order (p descending, column
    ascending), entry r is kept iff its exclusive prefix is below TF."""
    fx = [int(x) for x in np.floor(pr * 2.0 ** 62)]
    order = sorted(range(len(pr)), key=lambda x: (-pr[x], x))
    keep = np.zeros(len(pr), dtype=bool)
    excl = 0
    for x in order:
        keep[x] = excl < TF
        excl += fx[x]
    return keep


def _rows(rng, n_rows):
    for r in range(n_rows):
        n = int(rng.integers(1, 300))
        z = rng.standard_normal(n) * rng.choice([0.1, 1.0, 5.0, 40.0])
        if r % 4 == 0:                       # exact ties
            z = np.round(z * 4) / 4
        e = np.exp(z - z.max())
        yield e / e.sum()


def test_radix_select_equals_the_sorted_prefix_rule():
    rng = np.random.default_rng(8)
    for tau in (0.05, 0.5, 0.9, 0.95, np.nextafter(1.0, 0.0), 1.0):
        for pr in _rows(rng, 60):
            keep, F, TF = topcdf_radix_select(pr, tau)
            assert TF <= F
            assert np.array_equal(keep, topcdf_fixed_point_definition(pr, TF))
            assert keep.any()


def test_tau_one_keeps_every_entry_with_a_nonzero_fixed_point_value():
    rng = np.random.default_rng(9)
    for pr in _rows(rng, 120):
        keep, _, _ = topcdf_radix_select(pr, 1.0)
        assert np.array_equal(keep, np.floor(pr * 2.0 ** 62) > 0)


def test_threshold_is_the_exact_ceiling():
    """TF = ceil(tau * F) for every tau in (0, 1] (normal, subnormal, 1 and
    the double below it) and F up to 2^64, against exact rational arithmetic;
    so 1 <= TF <= F and an integer prefix c < tau * F iff c < TF.  A float64
    product tau * (double)F would not do: near 2^62, (double)F is F rounded
    to a multiple of 2^9, on either side of F."""
    import math
    from fractions import Fraction
    rng = np.random.default_rng(13)
    taus = [1.0, np.nextafter(1.0, 0.0), 0.5, 0.9, 0.95, 1e-300, 5e-324, 2.0 ** -60]
    taus += list(rng.uniform(0, 1, 200))
    Fs = [1, 2, 3, (1 << 62) - 1, 1 << 62, (1 << 62) + 12345, (1 << 64) - 1]
    Fs += [int(x) for x in rng.integers(1, 1 << 62, 50, dtype=np.int64)]
    overshoot = 0
    for tau in taus:
        for F in Fs:
            TF = topcdf_threshold(F, float(tau))
            assert TF == math.ceil(Fraction(float(tau)) * F)
            assert 1 <= TF <= F
            overshoot += int(float(tau) * float(F)) > F
    assert overshoot > 0        # the float64 route does overshoot


def test_radix_select_agrees_with_the_float64_oracle_outside_its_window():
    """Against the oracle's float64 rule (sorted cumulative sum, exclusive
    prefix < tau * sum): the two may differ only where the oracle's
    exclusive prefix lies within 1e-4 of tau * sum, the window the GPU
    parity tests exclude."""
    from oracle import sparge_oracle as O
    rng = np.random.default_rng(12)
    for tau in (0.5, 0.9, 0.95, 1.0):
        for pr in _rows(rng, 60):
            keep, _, _ = topcdf_radix_select(pr, tau)
            ref, info = O.topcdf(pr, tau)
            near = np.abs(info["excl"] - info["thresh"]) <= 1e-4
            assert np.array_equal(keep & ~near, ref & ~near)


# ---------------------------------------------------------------------------
# the pilot that chooses the stage-2 path, replayed on the oracle's scores
# ---------------------------------------------------------------------------

def pilot_estimate(Q, K, mg, lam, causal, blocks_cap=256, tiles=4):
    """attn_pilot's weighted vote rate: sampled block g * stride + stride / 2,
    its first listed tile seeding the running max, then one tile from the
    middle of each of up to tiles - 1 strata of the rest of the list, voted
    per 32-row wavefront against the running max of the sample; samples
    weighted by the listed tiles they stand for.  Returns the rate and the
    sampled blocks' mean listed tiles."""
    import math
    from oracle import sparge_oracle as O
    B, H, N, d = Q.shape
    Hkv = K.shape[1]
    Tm = O.num_blocks(N, 128)
    total = B * H * Tm
    stride = -(-total // blocks_cap)
    live = O.tile_live(N, 128, 64, causal)
    votes = pairs = 0
    listed = sampled = 0
    for s in range(-(-total // stride)):
        g = s * stride + stride // 2
        g = g if g < total else s * stride
        i, bh = g % Tm, g // Tm
        b, h = divmod(bh, H)
        hk = h // (H // Hkv)
        lst = [j for j in range(mg.shape[3]) if mg[b, h, i, j] and live[i, j]]
        UC = len(lst)
        listed += UC
        sampled += 1
        if UC == 0:
            continue
        S = min(tiles - 1, UC - 1) if UC > 1 else 0
        rows = O.block_rows(N, 128, i)
        mk = []
        for e in [0] + [1 + (2 * k - 1) * (UC - 1) // (2 * S) for k in range(1, S + 1)]:
            keys = O.block_rows(N, 64, lst[e])
            Sc = Q[b, h, rows.start:rows.stop] @ K[b, hk, keys.start:keys.stop].T / math.sqrt(d)
            if causal:
                Sc = np.where(np.arange(keys.start, keys.stop)[None, :] > np.arange(rows.start, rows.stop)[:, None],
                              -np.inf, Sc)
            mk.append(Sc.max(axis=1))
        for w in range(0, len(rows), 32):
            m = [x[w:w + 32] for x in mk]
            first = 1 if np.isfinite(m[0]).any() else 0
            run, v, p = m[0], 0, 0
            for x in m[1:]:
                new = np.maximum(run, x)
                fin = np.isfinite(x)
                if fin.any():
                    p += 1
                    v += 1 if np.any(fin & ~(x - new < lam)) else 0
                run = new
            ws = (UC - 1) * (840 // S) if S > 0 else 0
            votes += v * ws + first * 840
            pairs += p * ws + first * 840
    return votes / pairs, listed / sampled


FUSED_MEAN_TILES = 224    # kFusedMeanTiles of csrc/common.hpp
FUSED_MEAN_TILES_I8 = 112  # kFusedMeanTilesI8 (int8 Q/K)
FUSED_MEAN_TILES_F8 = 448  # kFusedMeanTilesF8 (16-bit Q/K, fp8 P~V)
FUSED_MEAN_TILES_I8F8 = 64  # kFusedMeanTilesI8F8 (int8 Q/K, fp8 P~V)


def test_pilot_estimate_separates_the_recipes():
    """The pilot overstates the vote rate (a short sample sets new maxima more
    often than the whole row): it stays under its nine-tenths bar on the LLM
    recipe, where a quarter of the pairs vote, and reaches 1 on the image and
    video recipes, where all do.  The automatic path takes the fused pass on
    the rate, or on short rows (the LLM recipe at N 8192 lists some 40 tiles
    per block), and two passes on the LLM recipe's long rows at N 65536."""
    from oracle import sparge_oracle as O
    from free_block_sparse_mask_amd import inputs as I
    cases = [(2, dict(N=8192, H=4, H_kv=2), False, True),
             (3, dict(N=4 * 16 * 12, H=2, H_kv=1, grid=(4, 16, 12)), True, True),
             (1, dict(N=64 + 24 * 24, H=2, H_kv=2, grid=(24, 24), text_tokens=64), True, True),
             (2, dict(N=65536, H=2, H_kv=1), False, False)]
    for wid, over, by_rate, fused in cases:
        w = I.workload(wid, **over)
        q, k, v = I.make_qkv(w)
        Q, K, V = (O.widen(x, w.dtype) for x in (q, k, v))
        mg = O.predict_mask(Q, K, w.tau, w.theta, w.causal)["mg"]
        est, mean_listed = pilot_estimate(Q, K, mg, w.lam, w.causal)
        if w.N <= 8192:
            _, c, _ = O.sparse_attention(Q, K, V, mg, w.lam, w.causal)
            true = c["pv_exec"] / (c["pv_exec"] + c["pv_skip"])
            assert est >= true - 1e-12, (w.name, est, true)
        assert (est >= 0.9) == by_rate, (w.name, est)
        assert (est >= 0.9 or mean_listed <= FUSED_MEAN_TILES) == fused, (w.name, est, mean_listed)


def test_int8_tile_bound_separates_16k_from_32k():
    """With int8 Q/K the automatic path takes the fused pass on the LLM
    recipe's rows at N 16384 (where it measured faster) and two passes at
    32768 (where it measured slower): the pilot's mean listed tiles fall on
    either side of the int8 bound, and both under the 16-bit one."""
    from oracle import sparge_oracle as O
    from free_block_sparse_mask_amd import inputs as I
    means = {}
    for N in (16384, 32768):
        w = I.workload(2, N=N, H=1, H_kv=1)
        q, k, _ = I.make_qkv(w)
        Q, K = (O.widen(x, w.dtype) for x in (q, k))
        mg = O.predict_mask(Q, K, w.tau, w.theta, w.causal)["mg"]
        est, means[N] = pilot_estimate(Q, K, mg, w.lam, w.causal)
        assert est < 0.9, (N, est)
    assert means[16384] <= FUSED_MEAN_TILES_I8 < means[32768] <= FUSED_MEAN_TILES, means


def test_fp8_tile_bound_takes_the_fused_pass_at_64k():
    """With fp8 P~V the fused pass measured faster on the LLM recipe up to N
    65536 and slower at 131072 (the 128K GQA workload lists 622 tiles per
    block on average): the pilot's mean at 65536 falls under the fp8 bound
    and over the 16-bit one."""
    from oracle import sparge_oracle as O
    from free_block_sparse_mask_amd import inputs as I
    w = I.workload(2, N=65536, H=1, H_kv=1)
    q, k, _ = I.make_qkv(w)
    Q, K = (O.widen(x, w.dtype) for x in (q, k))
    mg = O.predict_mask(Q, K, w.tau, w.theta, w.causal)["mg"]
    est, mean = pilot_estimate(Q, K, mg, w.lam, w.causal)
    assert est < 0.9 and FUSED_MEAN_TILES < mean <= FUSED_MEAN_TILES_F8 < 622, (est, mean)


# ---------------------------------------------------------------------------
# Attention tile bookkeeping: the first tile with dead scores, vote codes
# ---------------------------------------------------------------------------
def has_dead_scores(N, j, q0, causal, bq_rows=32, bk=64):
    """The definition, score by score: some (row, key) of the tile is dead
    (key at or beyond N, row at or beyond N, or, causal, key after the row)."""
    rows = np.arange(q0, q0 + bq_rows)[:, None]
    keys = np.arange(j * bk, j * bk + bk)[None, :]
    dead = (keys >= N) | (rows >= N)
    if causal:
        dead |= keys > rows
    return bool(dead.any())


def first_masked_tile(N, q0, causal):
    """The kernels' route: every tile from this index on has dead scores."""
    if q0 + 32 > N:
        return 0
    jn = N // 64
    return min(jn, (q0 + 1) // 64) if causal else jn


def test_first_masked_tile_equals_the_dead_score_test():
    for N in list(range(1, 300, 7)) + [4096, 4097, 46080, 131072 + 5]:
        tn = (N + 63) // 64
        for q0 in range(0, N + 32, 32):
            if q0 > 600 and q0 + 700 < N:
                continue                       # the middle of long rows adds nothing new
            for causal in (False, True):
                jm = first_masked_tile(N, q0, causal)
                for j in range(tn):
                    assert has_dead_scores(N, j, q0, causal) == (j >= jm), (N, q0, causal, j, jm)


def test_vote_codes_counted_from_the_packed_words():
    """Codes 1 (P~V), 2 (skipped) and 3 (no finite score), two bits per entry,
    sixteen entries a word, counted by the bit masks the first pass uses."""
    rng = np.random.default_rng(7)
    for n in (0, 1, 15, 16, 17, 100, 2048):
        codes = rng.integers(1, 4, size=n)
        words = np.zeros((n + 15) // 16, dtype=np.uint64)
        for e, c in enumerate(codes):
            words[e >> 4] |= np.uint64(int(c) << (2 * (e & 15)))
        n1 = n2 = n3 = 0
        for w in words.tolist():
            lo = w & 0x55555555
            hi = (w >> 1) & 0x55555555
            n1 += bin(lo & ~hi & 0xFFFFFFFF).count("1")
            n2 += bin(hi & ~lo & 0xFFFFFFFF).count("1")
            n3 += bin(lo & hi).count("1")
        assert (n1, n2, n3) == (int((codes == 1).sum()), int((codes == 2).sum()), int((codes == 3).sum()))
    # the code itself: 3 - any_finite - exec, with exec implying a finite score
    for fin in (0, 1):
        for ex in (0, 1):
            if ex and not fin:
                continue
            want = 1 if ex else (2 if fin else 3)
            assert 3 - fin - ex == want


def test_int8_fp8_tile_bound_separates_8k_from_16k():
    """With int8 Q/K and fp8 P~V the fused pass measured faster on the LLM
    recipe at N 8192 and slower at 16384: the pilot's mean listed tiles fall
    on either side of that pair's bound, and both under the int8 one."""
    from oracle import sparge_oracle as O
    from free_block_sparse_mask_amd import inputs as I
    means = {}
    for N in (8192, 16384):
        w = I.workload(2, N=N, H=1, H_kv=1)
        q, k, _ = I.make_qkv(w)
        Q, K = (O.widen(x, w.dtype) for x in (q, k))
        mg = O.predict_mask(Q, K, w.tau, w.theta, w.causal)["mg"]
        est, means[N] = pilot_estimate(Q, K, mg, w.lam, w.causal)
        assert est < 0.9, (N, est)
    assert means[8192] <= FUSED_MEAN_TILES_I8F8 < means[16384] <= FUSED_MEAN_TILES_I8, means
