"""Pins for the oracle's lightning-indexer scores and its top-k.

Method: DeepSeek-V3.2 model documentation page, section "DeepSeek Sparse
Attention (DSA)": each query is scored against all previous keys of a
single-head index-key cache (item 1) and keeps its top index_topk tokens
(item 2).  Score form read as sum_h w_h * relu(q_h . k); a query may see its
own position.
"""
import numpy as np
import pytest

from workloads import make_scores


def _int_case(rng, B, T, H, D, Lmax, lens):
    q = rng.integers(-3, 4, (B, T, H, D)).astype(np.float32)
    k = rng.integers(-3, 4, (B, Lmax, D)).astype(np.float32)
    w = rng.integers(-4, 5, (B, T, H)).astype(np.float32)
    return q, w, k, np.array(lens, dtype=np.int32)


def _brute_int(q, w, k, kv_len):
    """Python-int arithmetic: exact by construction."""
    B, T, H, D = q.shape
    Lmax = k.shape[1]
    out = np.full((B * T, Lmax), -np.inf)
    qi, wi, ki = q.astype(np.int64), w.astype(np.int64), k.astype(np.int64)
    for b in range(B):
        for t in range(T):
            p = int(kv_len[b]) - T + t
            for s in range(p + 1):
                tot = 0
                for h in range(H):
                    dot = int((qi[b, t, h] * ki[b, s]).sum())
                    tot += int(wi[b, t, h]) * max(dot, 0)
                out[b * T + t, s] = tot
    return out


def test_integer_inputs_are_exact(orc):
    rng = np.random.default_rng(0)
    q, w, k, kl = _int_case(rng, 2, 5, 4, 16, 40, [40, 23])
    ours = orc.index_scores(q, w, k, kl)
    assert np.array_equal(ours, _brute_int(q, w, k, kl).astype(np.float32))


def test_closed_form_recency(orc):
    # k_s = (s+1) e0, q_h = e0, w = +1  ->  I[t, s] = H (s + 1)  (most recent wins)
    B, T, H, D, L = 1, 4, 3, 8, 20
    q = np.zeros((B, T, H, D), np.float32)
    q[..., 0] = 1
    k = np.zeros((B, L, D), np.float32)
    k[0, :, 0] = np.arange(1, L + 1)
    kl = np.array([L], np.int32)
    for sign in (1, -1):
        w = np.full((B, T, H), float(sign), np.float32)
        s = orc.index_scores(q, w, k, kl)
        for t in range(T):
            p = L - T + t
            assert np.array_equal(s[t, :p + 1], sign * H * np.arange(1, p + 2, dtype=np.float32))
            assert np.all(np.isneginf(s[t, p + 1:]))
        idx = orc.topk(s, kl, T, 5)
        for t in range(T):
            p = L - T + t
            want = list(range(p, p - 5, -1)) if sign > 0 else list(range(5))
            assert list(idx[t]) == want


def test_relu_zero_and_masked_tail(orc):
    # q . k < 0 on every head -> the score is exactly 0 (whatever w is)
    B, T, H, D, L, Lmax = 1, 2, 4, 8, 6, 9
    q = np.zeros((B, T, H, D), np.float32)
    q[..., 1] = 1
    k = np.zeros((B, Lmax, D), np.float32)
    k[..., 1] = -1
    w = np.random.default_rng(1).standard_normal((B, T, H)).astype(np.float32)
    s = orc.index_scores(q, w, k, np.array([L], np.int32))
    assert np.all(s[0, :L - 1] == 0) and np.all(np.isneginf(s[0, L - 1:]))
    assert np.all(s[1, :L] == 0) and np.all(np.isneginf(s[1, L:]))


def test_ragged_lengths_and_row_subsets(orc):
    rng = np.random.default_rng(2)
    B, T, H, D, Lmax = 3, 4, 4, 16, 50
    lens = [50, 4, 31]
    q = rng.standard_normal((B, T, H, D)).astype(np.float32)
    k = rng.standard_normal((B, Lmax, D)).astype(np.float32)
    w = rng.standard_normal((B, T, H)).astype(np.float32)
    kl = np.array(lens, np.int32)
    full = orc.index_scores(q, w, k, kl)
    for r in range(B * T):
        b, t = divmod(r, T)
        p = lens[b] - T + t
        assert np.all(np.isfinite(full[r, :p + 1])) and np.all(np.isneginf(full[r, p + 1:]))
    rows = [7, 0, 11, 5]
    assert np.array_equal(orc.index_scores(q, w, k, kl, rows=rows), full[rows])


def test_fp8_scores_equal_plain_scores_on_exact_dequantised_values(orc):
    # Codes of small integers with power-of-two scales dequantise exactly, so the
    # fp8 score path must reproduce the plain path bit for bit.
    rng = np.random.default_rng(3)
    B, T, H, D, L = 2, 3, 4, 32, 24
    qv = rng.integers(-6, 7, (B, T, H, D)).astype(np.float32)
    kv = rng.integers(-6, 7, (B, L, D)).astype(np.float32)
    w = rng.standard_normal((B, T, H)).astype(np.float32)
    qs = (2.0 ** rng.integers(-3, 3, (B, T, H))).astype(np.float32)
    ks = (2.0 ** rng.integers(-3, 3, (B, L))).astype(np.float32)
    qc = orc.e4m3_encode(qv)
    kc = orc.e4m3_encode(kv)
    kl = np.array([L, L - 5], np.int32)
    s8 = orc.index_scores_fp8(qc, qs, w, kc, ks, kl)
    sp = orc.index_scores(qv * qs[..., None], w, kv * ks[..., None], kl)
    assert np.array_equal(s8, sp)


# ------------------------------------------------------------------- top-k
def _brute_topk(row, p, K):
    order = sorted(range(p + 1), key=lambda s: (-float(row[s]), s))
    keff = min(K, p + 1)
    return order[:keff] + [-1] * (K - keff)


@pytest.mark.parametrize("kind", ["gauss", "ties", "int", "const", "signed_zero"])
def test_topk_matches_brute_force(orc, kind):
    B, T, Lmax, K = 2, 6, 70, 16
    sc = make_scores(B * T, Lmax, seed=3, kind=kind).numpy()
    kl = np.array([70, 9], np.int32)
    # entries past each row's last visible key never matter
    for r in range(B * T):
        b, t = divmod(r, T)
        sc[r, kl[b] - T + t + 1:] = -np.inf
    idx = orc.topk(sc, kl, T, K)
    for r in range(B * T):
        b, t = divmod(r, T)
        assert list(idx[r]) == _brute_topk(sc[r], int(kl[b]) - T + t, K)


def test_topk_short_rows_keep_everything(orc):
    T, L, K = 8, 8, 32
    sc = make_scores(T, L, seed=5).numpy()
    idx = orc.topk(sc, np.array([L], np.int32), T, K)
    for t in range(T):
        assert sorted(idx[t][idx[t] >= 0].tolist()) == list(range(t + 1))
        assert np.all(idx[t][t + 1:] == -1)


def test_topk_queries_before_the_cache_have_no_candidates(orc):
    # kv_len < T: query t sits at p = kv_len - T + t < 0 for the first T - kv_len
    # queries, which have no candidates at all (all -1), however negative p is
    T, L, K = 9, 12, 2048
    kl = np.array([5], np.int32)
    sc = make_scores(T, L, seed=7).numpy()
    idx = orc.topk(sc, kl, T, K)
    for t in range(T):
        p = 5 - T + t
        assert sorted(idx[t][idx[t] >= 0].tolist()) == list(range(max(p + 1, 0)))
        assert np.all(idx[t][max(p + 1, 0):] == -1)


def test_topk_invariant_under_positive_weight_scaling(orc):
    rng = np.random.default_rng(6)
    B, T, H, D, L, K = 1, 8, 8, 32, 200, 20
    q = rng.standard_normal((B, T, H, D)).astype(np.float32)
    k = rng.standard_normal((B, L, D)).astype(np.float32)
    w = rng.standard_normal((B, T, H)).astype(np.float32)
    kl = np.array([L], np.int32)
    base = orc.topk(orc.index_scores(q, w, k, kl), kl, T, K)
    for c in (2.0, 0.125):  # exact scalings keep every comparison
        assert np.array_equal(orc.topk(orc.index_scores(q, w * c, k, kl), kl, T, K), base)
    # an inexact factor on integer inputs is still exact
    qi = rng.integers(-3, 4, (B, T, H, D)).astype(np.float32)
    ki = rng.integers(-3, 4, (B, L, D)).astype(np.float32)
    wi = rng.integers(-3, 4, (B, T, H)).astype(np.float32)
    b2 = orc.topk(orc.index_scores(qi, wi, ki, kl), kl, T, K)
    assert np.array_equal(orc.topk(orc.index_scores(qi, wi * 3, ki, kl), kl, T, K), b2)


def test_lengths_past_the_cache_are_clamped_to_it(orc):
    """A kv_len larger than the cache capacity reads as the capacity (reading R19: a
    sequence cannot have keys past its cache rows): scores, top-k and the masked-dense
    attention equal those of kv_len = Lmax, and no query sees a position >= Lmax."""
    rng = np.random.default_rng(11)
    B, T, H, D, L, K = 2, 3, 4, 16, 10, 6
    q = rng.standard_normal((B, T, H, D)).astype(np.float32)
    k = rng.standard_normal((B, L, D)).astype(np.float32)
    w = rng.standard_normal((B, T, H)).astype(np.float32)
    long_ = np.array([L + 7, L], np.int32)
    exact = np.array([L, L], np.int32)
    s1, s2 = orc.index_scores(q, w, k, long_), orc.index_scores(q, w, k, exact)
    assert np.array_equal(s1, s2)
    i1, i2 = orc.topk(s1, long_, T, K), orc.topk(s2, exact, T, K)
    assert np.array_equal(i1, i2) and i1.max() < L
    qm = rng.standard_normal((B, T, 2, 24)).astype(np.float32)
    kv = rng.standard_normal((B, L, 24)).astype(np.float32)
    o1, l1 = orc.masked_dense_mla(qm, kv, long_, i1, 0.3, v_dim=16)
    o2, l2 = orc.masked_dense_mla(qm, kv, exact, i2, 0.3, v_dim=16)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
