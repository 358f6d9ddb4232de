"""Pins for the oracle's fp8 sparse MLA (MLA over e4m3 codes of the latent cache and queries).

The pages run the lightning indexer in FP8 behind a Hadamard rotation and call FP8 a
precision optimisation (DeepSeek-V3.2 model documentation, "DeepSeek Sparse Attention
(DSA)", lightning indexer).  The fp8 MLA applies the same per-row e4m3 codec to the
latent rows and queries, without the rotation (the first v_dim columns of a latent row
are the values).  The codec without rotation is pinned against the rotating one, the
attention against the bf16/fp32 oracle on inputs the codec represents exactly.
"""
import numpy as np


def test_quant_of_rotated_rows_equals_rotate_quant(orc):
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((64, 128)) * np.exp(rng.standard_normal((64, 1)))).astype(np.float32)
    x[3] = 0.0
    c1, s1 = orc.rotate_quant(x)
    c2, s2 = orc.quant(orc.rotate(x))
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_quant_keeps_exact_rows_and_zero_rows(orc):
    rng = np.random.default_rng(12)
    codes = rng.integers(0, 0x7E, size=(40, 576), dtype=np.uint8) | (rng.integers(0, 2, (40, 576), dtype=np.uint8) << 7)
    codes[:, 5] = 0x7E  # +448 in every row: the row scale is exactly 1
    x = orc.e4m3_decode(codes).astype(np.float32)
    x[9] = 0.0
    c, s = orc.quant(x)
    assert s[9] == 1.0 and np.all(c[9] == 0)
    live = np.arange(40) != 9
    assert np.all(s[live] == 1.0)
    assert np.array_equal(orc.dequant(c, s)[live], x[live].astype(np.float64))


def test_quant_of_a_row_scaled_by_a_power_of_two(orc):
    rng = np.random.default_rng(13)
    x = rng.standard_normal((8, 576)).astype(np.float32)
    c1, s1 = orc.quant(x)
    c2, s2 = orc.quant(x * np.float32(2.0 ** -7))
    assert np.array_equal(c1, c2)
    assert np.array_equal(s2, (s1.astype(np.float64) * 2.0 ** -7).astype(np.float32))


def test_kv_row_layout(orc):
    rng = np.random.default_rng(14)
    x = rng.standard_normal((3, 5, 576)).astype(np.float32)
    rows = orc.kv_rows_fp8(x)
    c, s = orc.quant(x)
    assert rows.shape == (3, 5, 592) and rows.dtype == np.uint8
    assert np.array_equal(rows[..., :576], c)
    assert np.array_equal(rows[..., 576:580].copy().view("<f4")[..., 0], s)
    assert np.all(rows[..., 580:] == 0)


def test_fp8_attention_on_exact_codes_equals_plain_attention(orc):
    """Queries and latent rows whose values the codec represents exactly (codes over
    64, with one 448 / 64 per row, so every scale is 1 / 64) give the plain oracle's
    attention."""
    rng = np.random.default_rng(15)
    B, T, H, L, K, D, Dv = 2, 3, 4, 50, 16, 576, 512

    def exact(shape):
        c = rng.integers(0, 0x60, size=shape + (D,), dtype=np.uint8) | (rng.integers(0, 2, shape + (D,), dtype=np.uint8) << 7)
        c[..., 7] = 0x7E
        return orc.e4m3_decode(c).astype(np.float32)

    q = exact((B, T, H)) / np.float32(64.0)   # a power-of-two step keeps the values exact
    kv = exact((B, L)) / np.float32(64.0)
    idx = np.stack([np.sort(rng.choice(L, K, replace=False)) for _ in range(B * T)]).astype(np.int32)
    idx[1, 3] = -1
    sm = 1.0 / np.sqrt(192.0)
    qc, qs = orc.quant(q)
    kc, ks = orc.quant(kv)
    o8, l8 = orc.sparse_mla_fp8(qc, qs, kc, ks, idx, sm, v_dim=Dv)
    o, l = orc.sparse_mla(q, kv, idx, sm, v_dim=Dv)
    assert np.array_equal(o8, o) and np.array_equal(l8, l)
