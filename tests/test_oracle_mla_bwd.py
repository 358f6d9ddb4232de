"""Pins for the oracle's sparse MLA backward (gradients of sum(dO * O)).

DeepSeek-V3.2 model documentation, model description: DSA is trainable.  The
oracle's gradients are pinned against central finite differences of the forward
oracle (inputs on a 2^-8 grid, steps of 2^-12, so every perturbed input is exact
in fp32), against torch autograd in float64 through the dense additive-mask
formulation (a different computation of the same function), and on the
structural cases: rows nobody selects get no gradient, an empty list gives zero
gradients, and a row listed twice equals that row listed once with its logit
raised by ln 2.
"""
import numpy as np
import torch


def _grid(rng, shape, scale=1.0):
    return (np.round(rng.standard_normal(shape) * scale * 256) / 256).astype(np.float32)


def _loss(orc, q, kv, dout, idx, sm, Dv):
    o, _ = orc.sparse_mla(q, kv, idx, sm, v_dim=Dv)
    return float((o * dout.reshape(o.shape).astype(np.float64)).sum())


def test_backward_matches_finite_differences(orc):
    rng = np.random.default_rng(41)
    B, T, H, L, K, D, Dv = 2, 2, 3, 7, 5, 8, 6
    q = _grid(rng, (B, T, H, D))
    kv = _grid(rng, (B, L, D))
    dout = _grid(rng, (B, T, H, Dv))
    idx = np.array([[0, 3, 3, -1, 6], [1, 2, 4, 5, 0], [6, 5, -1, 1, 2], [2, 2, 2, 0, -1]], dtype=np.int32)
    sm = 0.37
    dq, dkv = orc.sparse_mla_bwd(q, kv, dout, idx, sm, v_dim=Dv)
    eps = np.float32(2.0 ** -12)
    for pos in [(0, 0, 0, 0), (0, 1, 2, 7), (1, 0, 1, 3), (1, 1, 0, 5)]:
        qp, qm = q.copy(), q.copy()
        qp[pos] += eps
        qm[pos] -= eps
        fd = (_loss(orc, qp, kv, dout, idx, sm, Dv) - _loss(orc, qm, kv, dout, idx, sm, Dv)) / (2 * float(eps))
        b, t, h, d = pos
        assert abs(fd - dq[b * T + t, h, d]) < 1e-6 * max(1.0, abs(fd)), (pos, fd, dq[b * T + t, h, d])
    for pos in [(0, 0, 0), (0, 3, 5), (0, 6, 7), (1, 2, 1), (1, 5, 4), (1, 0, 6)]:
        kp, km = kv.copy(), kv.copy()
        kp[pos] += eps
        km[pos] -= eps
        fd = (_loss(orc, q, kp, dout, idx, sm, Dv) - _loss(orc, q, km, dout, idx, sm, Dv)) / (2 * float(eps))
        assert abs(fd - dkv[pos]) < 1e-6 * max(1.0, abs(fd)), (pos, fd, dkv[pos])


def test_backward_matches_dense_masked_autograd(orc):
    """torch float64 autograd through dense logits + a 0/-inf mask (not the gather form)."""
    rng = np.random.default_rng(42)
    B, T, H, L, K, D, Dv = 2, 3, 4, 60, 16, 576, 512
    q = rng.standard_normal((B, T, H, D)).astype(np.float32)
    kv = (rng.standard_normal((B, L, D)) * 0.5).astype(np.float32)
    dout = rng.standard_normal((B, T, H, Dv)).astype(np.float32)
    idx = np.stack([rng.choice(L, K, replace=False) for _ in range(B * T)]).astype(np.int32)
    idx[4, 3] = -1
    sm = 1.0 / np.sqrt(192.0)
    dq, dkv = orc.sparse_mla_bwd(q, kv, dout, idx, sm, v_dim=Dv)
    qt = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    kt = torch.tensor(kv, dtype=torch.float64, requires_grad=True)
    mask = torch.full((B, T, L), float("-inf"), dtype=torch.float64)
    for r in range(B * T):
        for s in idx[r]:
            if s >= 0:
                mask[r // T, r % T, s] = 0.0
    logits = sm * torch.einsum("bthd,bld->bthl", qt, kt) + mask[:, :, None, :]
    p = torch.softmax(logits, dim=-1)
    o = torch.einsum("bthl,ble->bthe", p, kt[..., :Dv])
    (o * torch.tensor(dout, dtype=torch.float64)).sum().backward()
    assert np.allclose(dq.reshape(B, T, H, D), qt.grad.numpy(), rtol=1e-9, atol=1e-9)
    assert np.allclose(dkv, kt.grad.numpy(), rtol=1e-9, atol=1e-9)


def test_backward_unselected_rows_and_empty_lists(orc):
    rng = np.random.default_rng(43)
    B, T, H, L, K, D, Dv = 1, 2, 2, 9, 3, 8, 4
    q = _grid(rng, (B, T, H, D))
    kv = _grid(rng, (B, L, D))
    dout = _grid(rng, (B, T, H, Dv))
    idx = np.array([[1, 4, 7], [-1, -1, -1]], dtype=np.int32)
    dq, dkv = orc.sparse_mla_bwd(q, kv, dout, idx, 0.5, v_dim=Dv)
    assert np.all(dq[1] == 0)
    untouched = [s for s in range(L) if s not in (1, 4, 7)]
    assert np.all(dkv[0, untouched] == 0)
    assert np.any(dkv[0, [1, 4, 7]] != 0)


def test_backward_duplicate_entry_equals_doubled_weight(orc):
    """Listing row a twice is the attention with row a's weight doubled: the gradient
    with respect to q equals that of a list holding a once whose key, for the logit
    only, is shifted so that its logit rises by ln 2 (q along e_0, so shifting
    component 0 of k_a by ln 2 / (sm q_0) does it)."""
    rng = np.random.default_rng(44)
    D, Dv, sm = 8, 4, 0.5
    q = np.zeros((1, 1, 1, D), dtype=np.float32)
    q[..., 0] = 2.0
    kv = _grid(rng, (1, 5, D))
    dout = _grid(rng, (1, 1, 1, Dv))
    two = np.array([[0, 2, 2, 4]], dtype=np.int32)
    o2, _ = orc.sparse_mla(q, kv, two, sm, v_dim=Dv)
    kv1 = kv.astype(np.float64).copy()
    kv1[0, 2, 0] += np.log(2.0) / (sm * 2.0)
    # the same output with row 2 listed once and its logit raised by ln 2
    logits = sm * (kv1[0, [0, 2, 4]] @ q[0, 0, 0].astype(np.float64))
    p = np.exp(logits - logits.max())
    p /= p.sum()
    o1 = p @ kv.astype(np.float64)[0, [0, 2, 4], :Dv]
    assert np.allclose(o2[0, 0], o1, rtol=1e-12, atol=1e-12)
    # value gradients: q is zero outside component 0, so on value columns 1.. the
    # gradient of a row is its total softmax weight times dO; row 2 collects the
    # weights of both of its entries, which equal p[1] of the single-entry form
    _, dkv = orc.sparse_mla_bwd(q, kv, dout, two, sm, v_dim=Dv)
    d = dout[0, 0, 0].astype(np.float64)
    for row, w in ((0, p[0]), (2, p[1]), (4, p[2])):
        assert np.allclose(dkv[0, row, 1:Dv], w * d[1:], rtol=1e-12, atol=1e-15)
