"""Pins for the oracle's sparse absorbed-latent MLA.

Method: DeepSeek-V3.2 model documentation page, section "DeepSeek Sparse
Attention (DSA)", item 2: main MLA attention runs only over the selected tokens
(an additive mask in Transformers; a gather at O(index_topk) per query with a
sparse kernel).  Absorbed reading: one shared latent row is the key, its first
v_dim columns the value.
"""
import numpy as np
import torch
import torch.nn.functional as F


def _rand(rng, *shape, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float32)


def _sdpa_reference(q, kv, kv_len, sm_scale, Dv):
    """Dense causal attention through torch's scaled_dot_product_attention (fp64, CPU)."""
    B, T, H, Dqk = q.shape
    outs, lses = [], []
    for b in range(B):
        L = int(kv_len[b])
        qt = torch.from_numpy(q[b]).double().permute(1, 0, 2)            # [H, T, Dqk]
        kt = torch.from_numpy(kv[b, :L]).double()[None].expand(H, L, Dqk)
        vt = torch.from_numpy(kv[b, :L, :Dv]).double()[None].expand(H, L, Dv)
        pos = torch.arange(T)[:, None] + (L - T)
        mask = torch.arange(L)[None, :] <= pos                             # [T, L]
        o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=sm_scale)
        logits = (qt @ kt.transpose(-1, -2)) * sm_scale
        lse = torch.logsumexp(logits.masked_fill(~mask, float("-inf")), dim=-1)
        outs.append(o.permute(1, 0, 2).numpy())
        lses.append(lse.permute(1, 0).numpy())
    return np.concatenate(outs), np.concatenate(lses)


def test_sparse_equals_dense_causal_when_topk_covers_context(orc):
    # With index_topk >= L every previous token is selected, so sparse attention
    # is dense causal attention.
    rng = np.random.default_rng(0)
    B, T, H, Dqk, Dv, Lmax, K = 2, 12, 4, 80, 64, 40, 64
    lens = [40, 17]
    q = _rand(rng, B, T, H, Dqk, scale=Dqk ** -0.5)
    kv = _rand(rng, B, Lmax, Dqk)
    kl = np.array(lens, np.int32)
    qi = _rand(rng, B, T, 4, 32)
    ki = _rand(rng, B, Lmax, 32)
    wi = _rand(rng, B, T, 4)
    idx = orc.topk(orc.index_scores(qi, wi, ki, kl), kl, T, K)
    sm = Dqk ** -0.5
    out, lse = orc.sparse_mla(q, kv, idx, sm, v_dim=Dv)
    ref_o, ref_l = _sdpa_reference(q, kv, kl, sm, Dv)
    assert np.abs(out - ref_o).max() < 1e-12 * max(1.0, np.abs(ref_o).max())
    assert np.abs(lse - ref_l).max() < 1e-12 * max(1.0, np.abs(ref_l).max())


def test_additive_mask_form_equals_gather_form(orc):
    rng = np.random.default_rng(1)
    B, T, H, Dqk, Dv, Lmax, K = 2, 6, 5, 48, 32, 90, 24
    lens = [90, 30]
    q = _rand(rng, B, T, H, Dqk)
    kv = _rand(rng, B, Lmax, Dqk)
    kl = np.array(lens, np.int32)
    sc = _rand(rng, B * T, Lmax)
    idx = orc.topk(sc, kl, T, K)
    sm = 0.2
    o1, l1 = orc.sparse_mla(q, kv, idx, sm, v_dim=Dv)
    o2, l2 = orc.masked_dense_mla(q, kv, kl, idx, sm, v_dim=Dv)
    assert np.abs(o1 - o2).max() < 1e-12
    assert np.abs(l1 - l2).max() < 1e-12


def test_zero_query_averages_selected_values(orc):
    rng = np.random.default_rng(2)
    B, T, H, Dqk, Dv, Lmax, K = 1, 3, 2, 32, 16, 50, 10
    q = np.zeros((B, T, H, Dqk), np.float32)
    kv = _rand(rng, B, Lmax, Dqk)
    idx = np.array([[3, 9, 1, 44, 20, -1, -1, -1, -1, -1],
                    list(range(10)),
                    [49, -1, -1, -1, -1, -1, -1, -1, -1, 0]], np.int32)
    out, lse = orc.sparse_mla(q, kv, idx, 0.3, v_dim=Dv)
    for r in range(T):
        sel = idx[r][idx[r] >= 0]
        want = kv[0, sel, :Dv].astype(np.float64).mean(axis=0)
        assert np.allclose(out[r], want[None], atol=1e-14)
        assert np.allclose(lse[r], np.log(len(sel)), atol=1e-14)


def test_first_query_sees_only_itself(orc):
    rng = np.random.default_rng(3)
    B, T, H, Dqk, Dv, L, K = 1, 4, 3, 64, 48, 4, 8
    q = _rand(rng, B, T, H, Dqk)
    kv = _rand(rng, B, L, Dqk)
    kl = np.array([L], np.int32)
    sc = _rand(rng, T, L)
    idx = orc.topk(sc, kl, T, K)
    assert list(idx[0]) == [0] + [-1] * (K - 1)
    out, lse = orc.sparse_mla(q, kv, idx, 0.125, v_dim=Dv)
    assert np.allclose(out[0], np.broadcast_to(kv[0, 0, :Dv], (H, Dv)), atol=1e-15)
    want = 0.125 * (q[0, 0].astype(np.float64) @ kv[0, 0].astype(np.float64))
    assert np.allclose(lse[0], want, atol=1e-14)


def test_two_keys_closed_form(orc):
    rng = np.random.default_rng(4)
    H, Dqk, Dv = 2, 16, 8
    q = _rand(rng, 1, 1, H, Dqk)
    kv = _rand(rng, 1, 6, Dqk)
    idx = np.array([[5, -1, 2]], np.int32)
    sm = 0.7
    out, lse = orc.sparse_mla(q, kv, idx, sm, v_dim=Dv)
    for h in range(H):
        za = sm * float(q[0, 0, h].astype(np.float64) @ kv[0, 5].astype(np.float64))
        zb = sm * float(q[0, 0, h].astype(np.float64) @ kv[0, 2].astype(np.float64))
        pa = 1.0 / (1.0 + np.exp(zb - za))
        want = pa * kv[0, 5, :Dv] + (1 - pa) * kv[0, 2, :Dv]
        assert np.allclose(out[0, h], want, atol=1e-14)
        assert np.isclose(lse[0, h], np.logaddexp(za, zb), atol=1e-14)


def test_permutation_invariance_and_empty_rows(orc):
    rng = np.random.default_rng(5)
    B, T, H, Dqk, Dv, Lmax, K = 1, 4, 3, 40, 24, 64, 12
    q = _rand(rng, B, T, H, Dqk)
    kv = _rand(rng, B, Lmax, Dqk)
    idx = np.stack([rng.permutation(Lmax)[:K] for _ in range(T)]).astype(np.int32)
    idx[1, 5:] = -1
    idx[3, :] = -1
    o1, l1 = orc.sparse_mla(q, kv, idx, 0.15, v_dim=Dv)
    perm = np.stack([rng.permutation(K) for _ in range(T)])
    o2, l2 = orc.sparse_mla(q, kv, np.take_along_axis(idx, perm, 1), 0.15, v_dim=Dv)
    assert np.allclose(o1, o2, atol=1e-14) and np.allclose(l1[:3], l2[:3], atol=1e-14)
    assert np.all(o1[3] == 0) and np.all(np.isneginf(l1[3]))
