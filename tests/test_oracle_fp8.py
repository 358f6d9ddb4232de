"""Pins for the oracle's OCP e4m3fn codec and its Hadamard rotation.

The FP8 indexer of the DeepSeek-V3.2 model documentation page ("DeepSeek Sparse
Attention (DSA)", lightning indexer) rotates q and k by an orthogonal Hadamard
transform before FP8, which leaves q.k unchanged.  The codec is checked against
torch's own float8_e4m3fn conversion (a library routine) and against the
format's definition; the rotation against orthogonality and an independent
butterfly transform written here.
"""
import numpy as np
import pytest
import torch


def test_decode_all_codes_match_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    ours = orc.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def test_encode_roundtrips_every_finite_code(orc):
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = orc.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(orc.e4m3_encode(vals), codes)


def _neighbour_probes(orc):
    pos = orc.e4m3_decode(np.arange(0x7F, dtype=np.uint8))  # 0 .. 448, increasing
    assert np.all(np.diff(pos) > 0)
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)      # exact in fp32
    probes = [pos.astype(np.float32), mids,
              np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(-np.inf))]
    rng = np.random.default_rng(0)
    lo = pos[:-1]
    hi = pos[1:]
    for _ in range(40):
        probes.append((lo + (hi - lo) * rng.random(lo.shape)).astype(np.float32))
    y = np.concatenate(probes)
    y = y[np.abs(y) <= 448.0]
    return np.concatenate([y, -y])


def test_encode_matches_torch_rne_on_grid_midpoints_and_between(orc):
    y = _neighbour_probes(orc)
    ours = orc.e4m3_encode(y)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_encode_matches_torch_on_random_sweep(orc):
    rng = np.random.default_rng(1)
    y = (rng.standard_normal(2_000_000) * np.exp(rng.uniform(-12, 6, 2_000_000))).astype(np.float32)
    y = y[np.abs(y) <= 448.0]
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(orc.e4m3_encode(y), ref)


def test_encode_ties_to_even_and_saturates(orc):
    # 1.0625 lies halfway between 1.0 (mantissa 0, even) and 1.125 (mantissa 1).
    assert orc.e4m3_encode(np.float32([1.0625]))[0] == 0x38
    # 1.1875 lies halfway between 1.125 (odd) and 1.25 (even).
    assert orc.e4m3_encode(np.float32([1.1875]))[0] == 0x3A
    # half the smallest subnormal rounds to zero (even); just above it rounds up
    tiny = np.float32(2.0 ** -10)
    assert orc.e4m3_encode(np.float32([tiny]))[0] == 0x00
    assert orc.e4m3_encode(np.float32([np.nextafter(tiny, np.float32(1))]))[0] == 0x01
    big = orc.e4m3_encode(np.float32([449.0, 1e6, -1e30]))
    assert list(big) == [0x7E, 0x7E, 0xFE]
    assert orc.e4m3_encode(np.float32([-0.0]))[0] == 0x80


@pytest.mark.parametrize("D", [2, 16, 32, 128, 256])
def test_hadamard_is_orthonormal_and_symmetric(orc, D):
    H = orc.hadamard(D)
    assert np.allclose(H @ H.T, np.eye(D), atol=1e-12)
    assert np.array_equal(H, H.T)
    assert np.allclose(np.abs(H), D ** -0.5, atol=0)
    e0 = np.zeros(D)
    e0[0] = 1
    assert np.allclose(H @ e0, np.full(D, D ** -0.5), atol=1e-15)


def _fwht(x):
    """Iterative butterfly (natural order), then the 1/sqrt(D) normalisation."""
    x = np.array(x, dtype=np.float64)
    D = x.shape[-1]
    h = 1
    while h < D:
        y = x.reshape(*x.shape[:-1], D // (2 * h), 2, h)
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        x = y.reshape(*x.shape[:-1], D)
        h *= 2
    return x / np.sqrt(D)


def test_rotation_equals_butterfly_transform(orc):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((300, 128)).astype(np.float32)
    ours = orc.rotate(x)
    ref = _fwht(x.astype(np.float64)).astype(np.float32)
    assert np.allclose(ours, ref, rtol=2.5e-7, atol=1e-12)
    assert np.mean(ours == ref) > 0.999


def test_rotation_leaves_index_scores_unchanged(orc):
    # Hq . Hk = q . k  (orthogonality): scores on rotated operands equal the plain ones.
    rng = np.random.default_rng(3)
    B, T, H, D, L = 1, 16, 8, 128, 64
    q = (rng.standard_normal((B, T, H, D)) / np.sqrt(D)).astype(np.float32)
    k = (rng.standard_normal((B, L, D)) / np.sqrt(D)).astype(np.float32)
    w = (rng.standard_normal((B, T, H)) / np.sqrt(H)).astype(np.float32)
    kl = np.array([L], dtype=np.int32)
    plain = orc.index_scores(q, w, k, kl)
    rot = orc.index_scores(orc.rotate(q), w, orc.rotate(k), kl)
    fin = np.isfinite(plain)
    assert np.array_equal(fin, np.isfinite(rot))
    rel = np.abs(plain[fin] - rot[fin]).max() / np.abs(plain[fin]).max()
    assert rel < 1e-5


def test_rotate_quant_properties(orc):
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((200, 128)) * np.exp(rng.standard_normal((200, 1)))).astype(np.float32)
    x[7] = 0.0
    codes, scales = orc.rotate_quant(x)
    assert codes.dtype == np.uint8 and scales.shape == (200,)
    assert np.all(codes[7] == 0) and scales[7] == 1.0
    dec = orc.e4m3_decode(codes)
    live = np.arange(200) != 7
    # the largest rotated magnitude lands on +-448
    assert np.all(np.abs(dec[live]).max(axis=1) == 448.0)
    xr = orc.rotate(x).astype(np.float64)
    amax = np.abs(xr).max(axis=1)
    assert np.array_equal(scales[live], (amax[live] / 448.0).astype(np.float32))
    # dequantised values are within half an e4m3 step of the rotated ones
    deq = orc.dequant(codes, scales)
    err = np.abs(deq - xr)[live]
    assert np.all(err <= np.maximum(np.abs(xr[live]) * 2.0 ** -4, 2.0 ** -10 * amax[live, None] / 448 * 1.01))


# ------------------------------------------------------------ cache append
def test_cache_built_by_appends_equals_one_shot_quantisation(orc):
    """Appending keys in chunks (kv_len growing with each chunk) must place every
    row where quantising the whole key sequence at once puts it."""
    rng = np.random.default_rng(5)
    B, L, D = 3, 40, 64
    k = rng.standard_normal((B, L, D)).astype(np.float32)
    whole_codes, whole_scales = orc.rotate_quant(k)
    codes = np.zeros((B, L, D), np.uint8)
    scales = np.zeros((B, L), np.float32)
    for start, t_new in [(0, 8), (8, 1), (9, 16), (25, 15)]:
        kv_len = np.full(B, start + t_new, np.int32)
        codes, scales = orc.index_cache_append(k[:, start:start + t_new], kv_len, codes, scales)
    assert np.array_equal(codes, whole_codes)
    assert np.array_equal(scales, whole_scales)


def test_cache_append_touches_only_the_new_rows(orc):
    rng = np.random.default_rng(6)
    B, max_kv, D, t_new = 3, 20, 32, 4
    codes0 = rng.integers(0, 256, (B, max_kv, D), dtype=np.uint8)
    scales0 = rng.random((B, max_kv)).astype(np.float32)
    k_new = rng.standard_normal((B, t_new, D)).astype(np.float32)
    # sequence 0 ends at row 12; sequence 1 holds only 2 keys (the two oldest new keys
    # fall before row 0 and are skipped); sequence 2 fills the cache to its last row
    kv_len = np.array([13, 2, 20], np.int32)
    codes, scales = orc.index_cache_append(k_new, kv_len, codes0, scales0)
    nc, ns = orc.rotate_quant(k_new)
    expect_rows = {0: {9: 0, 10: 1, 11: 2, 12: 3}, 1: {0: 2, 1: 3}, 2: {16: 0, 17: 1, 18: 2, 19: 3}}
    for b in range(B):
        for p in range(max_kv):
            if p in expect_rows[b]:
                t = expect_rows[b][p]
                assert np.array_equal(codes[b, p], nc[b, t]) and scales[b, p] == ns[b, t]
            else:
                assert np.array_equal(codes[b, p], codes0[b, p]) and scales[b, p] == scales0[b, p]


# ------------------------------------------------- exact rounding of the rotation
# The rotated value of element i is (S x)_i / sqrt(D) with S the +-1 Sylvester
# matrix.  The pins below compute it with exact integer / rational arithmetic and
# round it to fp32 themselves (nearest, ties to even), so they fix the rounding of
# every rotated element, not only its closeness.  S is built here by the Kronecker
# recursion S_2D = [[S, S], [S, -S]] (the oracle uses the popcount formula).
from fractions import Fraction
import math


def _sylvester_int(D):
    S = np.array([[1]], dtype=object)
    while S.shape[0] < D:
        S = np.block([[S, S], [S, -S]])
    return S


def _exact_ints(row):
    """row (fp32) -> (python ints n_j, e) with row[j] == n_j * 2**e exactly."""
    parts = [math.frexp(float(v)) for v in row]
    exps = [e - 24 for m, e in parts if m != 0.0]
    e0 = min(exps) if exps else 0
    return [int(m * (1 << 24)) << (e - 24 - e0) if m != 0.0 else 0 for m, e in parts], e0


def _nearest_f32(cmp, approx):
    """The fp32 value nearest to an exact value v known only through cmp(m) = sign(v - m)
    for rational m; ties go to the even significand."""
    c = np.float32(approx)
    for _ in range(64):
        up = np.nextafter(c, np.float32(np.inf))
        dn = np.nextafter(c, np.float32(-np.inf))
        hi = (Fraction(float(c)) + Fraction(float(up))) / 2
        lo = (Fraction(float(dn)) + Fraction(float(c))) / 2
        ch, cl = cmp(hi), cmp(lo)
        if ch > 0:
            c = up
        elif cl < 0:
            c = dn
        elif ch == 0:
            return c if int(c.view(np.uint32)) % 2 == 0 else up
        elif cl == 0:
            return c if int(c.view(np.uint32)) % 2 == 0 else dn
        else:
            return c
    raise AssertionError("no convergence")


def _sign(x):
    return (x > 0) - (x < 0)


def _exact_rotation(x):
    """Correctly rounded fp32(S x / sqrt(D)) for every row of x, by exact arithmetic:
    rationals when sqrt(D) is an integer, else v = A sqrt(2) with A rational, compared
    with a rational m through the signs and squares of both sides."""
    D = x.shape[-1]
    S = _sylvester_int(D)
    r = math.isqrt(D)
    rational = r * r == D
    c2 = math.isqrt(D // 2)  # D = 2 c2^2 otherwise: 1/sqrt(D) = sqrt(2) / (2 c2)
    out = np.empty(x.shape, dtype=np.float32)
    for i, row in enumerate(x):
        n, e = _exact_ints(row)
        sn = S.dot(np.array(n, dtype=object))
        scale = Fraction(2) ** e
        for k in range(D):
            if rational:
                v = Fraction(int(sn[k])) * scale / r
                out[i, k] = _nearest_f32(lambda m, v=v: _sign(v - m), float(v))
            else:
                A = Fraction(int(sn[k])) * scale / (2 * c2)  # v = A sqrt(2)

                def cmp(m, A=A):
                    if A >= 0 and m <= 0:
                        return 0 if (A == 0 and m == 0) else 1
                    if A <= 0 and m >= 0:
                        return -1
                    d = 2 * A * A - m * m  # |v|^2 - |m|^2, same signs
                    return _sign(d) if A > 0 else -_sign(d)

                out[i, k] = _nearest_f32(cmp, float(A) * math.sqrt(2.0))
    return out


@pytest.mark.parametrize("D,rows", [(16, 100), (32, 100), (64, 64), (128, 48), (256, 24)])
def test_rotation_is_correctly_rounded_fp32_of_the_exact_product(orc, D, rows):
    """Every rotated element equals the correctly rounded fp32 of the exact H x (about
    20K elements over the five widths): Gaussian rows, rows under lognormal scales, and
    rows whose exact products land on fp32 midpoints (ties to even) where sqrt(D) is an
    integer."""
    rng = np.random.default_rng(40 + D)
    x = rng.standard_normal((rows, D)) * np.exp(rng.normal(0.0, 2.0, (rows, 1)))
    x = x.astype(np.float32)
    if D in (16, 64, 256):
        # 2^24 + small odd integers: (S x)_i / sqrt(D) falls halfway between fp32 values
        x[0] = 0.0
        x[0, 0], x[0, 1] = 2.0 ** 24, 1.0
        x[1] = 0.0
        x[1, 0], x[1, 1], x[1, 2] = 2.0 ** 24, 3.0, -2.0
        x[2] = 0.0
        x[2, 0], x[2, 3] = -(2.0 ** 25), 3.0
    ref = _exact_rotation(x)
    got = orc.rotate(x)
    bad = np.nonzero(got.view(np.uint32) != ref.view(np.uint32))
    assert bad[0].size == 0, f"{bad[0].size} elements differ, first at {bad[0][0]}, {bad[1][0]}"


def test_rotate_quant_scale_and_codes_from_exact_arithmetic(orc):
    """The quantiser's arithmetic (reading of the FP8 indexer): amax of the rotated row,
    r = fp32(448 / amax), y = fp32(x' r), code = e4m3 round-to-nearest-even of y
    (saturating), scale = fp32(amax / 448).  Recomputed here with exact rationals for
    every rounding and torch's float8_e4m3fn cast (a library routine) for the codes."""
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((64, 128)) * np.exp(rng.normal(0.0, 1.5, (64, 1)))).astype(np.float32)
    codes, scales = orc.rotate_quant(x)
    xr = orc.rotate(x)  # pinned exactly above
    for i in range(x.shape[0]):
        amax = Fraction(float(np.abs(xr[i]).max()))
        sc = _nearest_f32(lambda m: _sign(amax / 448 - m), float(amax) / 448.0)
        assert scales[i] == sc, i
        r = _nearest_f32(lambda m: _sign(448 / amax - m), 448.0 / float(amax))
        y = np.array([_nearest_f32(lambda m, v=Fraction(float(v)) * Fraction(float(r)): _sign(v - m),
                                   float(v) * float(r)) for v in xr[i]], dtype=np.float32)
        y = np.clip(y, -448.0, 448.0)
        ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(codes[i], ref), i
