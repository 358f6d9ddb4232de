"""GPU parity of each entry point against the CPU oracle (same seeded inputs).

Entry points: dsa_rotate_quant_fp8, dsa_index_scores, dsa_topk,
dsa_sparse_mla_fwd (bf16, f32 and fp8), dsa_mla_kv_quant_fp8, all called
through the C ABI.  Integer-valued inputs make
the indexer exact on both sides (bit-for-bit comparison); Gaussian inputs are
compared at the dtype tolerance; top-k is compared exactly on shared score rows.
"""
import numpy as np
import pytest
import torch

from helpers import TOL, announce, rel_rowmax
from workloads import get, make_inputs, make_scores

pytestmark = pytest.mark.gpu
DEV = "cuda"


def shape_of(dsa, **kw):
    base = dict(batch=1, n_q=1, max_kv=64, idx_heads=64, idx_dim=128, topk=64, heads=128, qk_dim=576, v_dim=512,
                sm_scale=1 / 192 ** 0.5, idx_dtype="bf16", mla_dtype="bf16")
    base.update(kw)
    return dsa.DsaShape(**base)


# ------------------------------------------------------------ rotate + quantise
@pytest.mark.parametrize("dim", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("xdt", [torch.bfloat16, torch.float32])
def test_rotate_quant_codes_and_scales_exact(dsa, orc, dim, xdt):
    g = torch.Generator().manual_seed(dim)
    x = torch.randn(2000, dim, generator=g) * torch.exp(0.5 * torch.randn(2000, 1, generator=g))
    x[3] = 0
    x[7] = 0
    x[7, 5] = -3e-3
    x[11] *= 1e-6
    x = x.to(xdt)
    codes, scales = dsa.rotate_quant_fp8(x.to(DEV))
    torch.cuda.synchronize()
    oc, os_ = orc.rotate_quant(x)
    gc = codes.cpu().numpy()
    bad = int((gc != oc).sum())
    assert bad == 0, f"{bad} codes differ"
    assert np.array_equal(scales.cpu().numpy(), os_)


# ------------------------------------------------------ index-key cache append
@pytest.mark.parametrize("dim,t_new,xdt", [(128, 1, torch.bfloat16), (128, 5, torch.float32), (64, 3, torch.bfloat16),
                                           (256, 2, torch.float32)])
def test_cache_append_matches_oracle(dsa, orc, dim, t_new, xdt):
    g = torch.Generator().manual_seed(dim + t_new)
    B, max_kv = 5, 50
    codes0 = torch.randint(0, 256, (B, max_kv, dim), generator=g, dtype=torch.uint8)
    scales0 = torch.rand(B, max_kv, generator=g)
    k_new = (torch.randn(B, t_new, dim, generator=g) * torch.exp(torch.randn(B, t_new, 1, generator=g))).to(xdt)
    k_new[0, 0] = 0  # all-zero row: codes 0, scale 1
    # full cache, mid cache, only part of the new keys inside the cache, exactly t_new, one key
    kv_len = torch.tensor([max_kv, 17, max(1, t_new - 1), t_new, 1], dtype=torch.int32)
    codes, scales = codes0.clone().to(DEV), scales0.clone().to(DEV)
    dsa.index_cache_append_fp8(k_new.to(DEV), kv_len.to(DEV), codes, scales)
    torch.cuda.synchronize()
    oc, os_ = orc.index_cache_append(k_new, kv_len.numpy(), codes0.numpy(), scales0.numpy())
    assert np.array_equal(codes.cpu().numpy(), oc)
    assert np.array_equal(scales.cpu().numpy(), os_)


def test_cache_built_by_appends_equals_rotate_quant(dsa, orc):
    """A cache built one decode step at a time holds the codes of the whole key sequence."""
    g = torch.Generator().manual_seed(3)
    B, L, D = 4, 24, 128
    k = torch.randn(B, L, D, generator=g).bfloat16()
    codes = torch.zeros(B, L, D, dtype=torch.uint8, device=DEV)
    scales = torch.zeros(B, L, device=DEV)
    kd = k.to(DEV)
    for p in range(L):
        kl = torch.full((B,), p + 1, dtype=torch.int32, device=DEV)
        dsa.index_cache_append_fp8(kd[:, p:p + 1].contiguous(), kl, codes, scales)
    torch.cuda.synchronize()
    oc, os_ = orc.rotate_quant(k)
    assert np.array_equal(codes.cpu().numpy(), oc)
    assert np.array_equal(scales.cpu().numpy(), os_)


# ------------------------------------------------------------------- indexer
def _int_inputs(B, T, H, D, Lmax, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randint(-3, 4, (B, T, H, D), generator=g).float()
    k = torch.randint(-3, 4, (B, Lmax, D), generator=g).float()
    w = torch.randint(-4, 5, (B, T, H), generator=g).float()
    return q, w, k


@pytest.mark.parametrize("dt,D,H", [("f32", 32, 4), ("f32", 64, 64), ("f32", 128, 20), ("bf16", 128, 64),
                                    ("bf16", 128, 16), ("bf16", 128, 7)])
@pytest.mark.parametrize("T", [1, 2, 5, 37])
def test_indexer_integer_inputs_bit_exact(dsa, orc, dt, D, H, T):
    B, Lmax = 2, 300
    lens = [300, 150]
    q, w, k = _int_inputs(B, T, H, D, Lmax, seed=T * 100 + H)
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    kl = torch.tensor(lens, dtype=torch.int32)
    s = shape_of(dsa, batch=B, n_q=T, max_kv=Lmax, idx_heads=H, idx_dim=D, idx_dtype=dt)
    got = dsa.index_scores(s, q.to(tdt).to(DEV), w.to(DEV), k.to(tdt).to(DEV), kl.to(DEV))
    ref = orc.index_scores(q, w, k, kl).reshape(B, T, Lmax)
    assert np.array_equal(got.cpu().numpy(), ref)


@pytest.mark.parametrize("T", [1, 2, 9])
def test_indexer_fp8_exact_codes(dsa, orc, T):
    # small-integer codes with power-of-two scales: every partial sum is exact
    B, H, D, Lmax = 2, 64, 128, 200
    g = torch.Generator().manual_seed(T)
    qv = torch.randint(-4, 5, (B, T, H, D), generator=g).float()
    kv = torch.randint(-4, 5, (B, Lmax, D), generator=g).float()
    w = torch.randint(-3, 4, (B, T, H), generator=g).float()
    qs = 2.0 ** torch.randint(-2, 3, (B, T, H), generator=g).float()
    ks = 2.0 ** torch.randint(-2, 3, (B, Lmax), generator=g).float()
    qc = torch.from_numpy(orc.e4m3_encode(qv.numpy()))
    kc = torch.from_numpy(orc.e4m3_encode(kv.numpy()))
    kl = torch.tensor([200, 77], dtype=torch.int32)
    s = shape_of(dsa, batch=B, n_q=T, max_kv=Lmax, idx_dtype="fp8")
    got = dsa.index_scores(s, qc.to(DEV), w.to(DEV), kc.to(DEV), kl.to(DEV), q_scale=qs.to(DEV),
                           k_scale=ks.to(DEV))
    ref = orc.index_scores_fp8(qc, qs, w, kc, ks, kl).reshape(B, T, Lmax)
    assert np.array_equal(got.cpu().numpy(), ref)


@pytest.mark.parametrize("dt", ["bf16", "fp8"])
@pytest.mark.parametrize("H", [20, 40, 64])
def test_indexer_prefill_edge_lengths_bit_exact(dsa, orc, dt, H):
    """Prefill score rows (T = 37: ragged against the 8-row blocks) with a sequence
    shorter than T, an empty one and one whose length passes the cache (clamped to
    it), at head counts that fill one 32-head tile, part of a second, and two.
    Small-integer operands (and power-of-two fp8 scales) make every sum exact, so
    the rows must equal the oracle's bit for bit, -inf past each query's position."""
    B, T, D, Lmax = 4, 37, 128, 300
    lens = [300, 20, 0, 350]
    g = torch.Generator().manual_seed(H * 7 + (dt == "fp8"))
    qv = torch.randint(-3, 4, (B, T, H, D), generator=g).float()
    kv = torch.randint(-3, 4, (B, Lmax, D), generator=g).float()
    w = torch.randint(-4, 5, (B, T, H), generator=g).float()
    kl = torch.tensor(lens, dtype=torch.int32)
    s = shape_of(dsa, batch=B, n_q=T, max_kv=Lmax, idx_heads=H, idx_dim=D, idx_dtype=dt)
    announce(f"indexer prefill edge lengths {dt} H={H}")
    if dt == "bf16":
        got = dsa.index_scores(s, qv.to(torch.bfloat16).to(DEV), w.to(DEV), kv.to(torch.bfloat16).to(DEV), kl.to(DEV))
        ref = orc.index_scores(qv, w, kv, kl).reshape(B, T, Lmax)
    else:
        qs = 2.0 ** torch.randint(-2, 3, (B, T, H), generator=g).float()
        ks = 2.0 ** torch.randint(-2, 3, (B, Lmax), generator=g).float()
        qc = torch.from_numpy(orc.e4m3_encode(qv.numpy()))
        kc = torch.from_numpy(orc.e4m3_encode(kv.numpy()))
        got = dsa.index_scores(s, qc.to(DEV), w.to(DEV), kc.to(DEV), kl.to(DEV), q_scale=qs.to(DEV),
                               k_scale=ks.to(DEV))
        ref = orc.index_scores_fp8(qc, qs, w, kc, ks, kl).reshape(B, T, Lmax)
    assert np.array_equal(got.cpu().numpy(), ref)


@pytest.mark.parametrize("name,seqs,rows", [("tiny_f32", None, None), ("prefill_4k", None, [0, 1, 7, 8, 2047, 2048,
                                                                                             3001, 4095]),
                                            ("decode_32k", [0, 33, 63], None)])
def test_indexer_gaussian_within_tolerance(dsa, orc, name, seqs, rows):
    wl = get(name)
    inp = make_inputs(wl, device=DEV, with_mla=False)
    s = dsa.DsaShape.of(wl)
    got = dsa.index_scores(s, inp["q_idx"], inp["w"], inp["k_idx"], inp["kv_len"]).cpu()
    T = wl.n_q
    if seqs is not None:
        sub = {k: v[seqs].cpu() for k, v in inp.items()}
        ref = orc.index_scores(sub["q_idx"], sub["w"], sub["k_idx"], sub["kv_len"])
        g = got[seqs].reshape(len(seqs) * T, -1).numpy()
    else:
        r = list(range(wl.rows)) if rows is None else rows
        cpu = {k: v.cpu() for k, v in inp.items()}
        ref = orc.index_scores(cpu["q_idx"], cpu["w"], cpu["k_idx"], cpu["kv_len"], rows=r)
        g = got.reshape(wl.rows, -1)[r].numpy()
    err = rel_rowmax(g, ref)
    assert err.max() < TOL[wl.idx_dtype] / 10, err.max()


def test_indexer_fp8_on_oracle_codes_long_context(dsa, orc):
    # 2 sequences of the 131072-token fp8 workload; codes made by the oracle feed both sides
    wl = get("decode_128k_fp8").replace(batch=2)
    inp = make_inputs(wl, with_mla=False)
    qc, qs = orc.rotate_quant(inp["q_idx"])
    kc, ks = orc.rotate_quant(inp["k_idx"])
    s = dsa.DsaShape.of(wl)
    t = lambda a: torch.from_numpy(a).to(DEV)
    got = dsa.index_scores(s, t(qc), inp["w"].to(DEV), t(kc), inp["kv_len"].to(DEV), q_scale=t(qs),
                           k_scale=t(ks)).cpu().reshape(2, -1).numpy()
    ref = orc.index_scores_fp8(qc, qs, inp["w"], kc, ks, inp["kv_len"])
    assert rel_rowmax(got, ref).max() < 1e-4
    # the method's own precision loss: fp8 scores against unquantised ones
    plain = orc.index_scores(inp["q_idx"], inp["w"], inp["k_idx"], inp["kv_len"])
    assert rel_rowmax(got, plain).max() < TOL["fp8"]


# --------------------------------------------------------------------- top-k
TOPK_CASES = [
    # (B, T, Lmax, lens, K)
    (2, 3, 5000, [5000, 2100], 2048),
    (1, 300, 300, [300], 64),
    (2, 1, 40000, [40000, 33000], 2048),  # rows longer than the LDS-resident limit
    (3, 4, 900, [900, 10, 3], 1),
    (1, 8, 100, [100], 4096),             # every row shorter than K
    (2, 2, 2049, [2049, 2048], 2048),     # one candidate over / exactly K
    # few long rows: each row split over 4096-entry chunks
    (4, 2, 12000, [12000, 9000, 8193, 5000], 2048),
    (3, 1, 20000, [20000, 2048, 1], 2048),
    (2, 1, 9000, [9000, 8500], 1000),     # K not a power of two
    (1, 1, 131072, [131072], 2048),
    (2, 1, 70000, [70000, 5000], 4096),   # the largest K
    (5, 4, 9000, [9000, 8200, 4000, 100, 8999], 512),  # 20 rows: three ticket groups, ragged
    (1, 1, 140000, [140000], 2048),       # over 32 chunks: the three-launch split path
    # many long rows: one workgroup per row, 16 and 32 staged keys per thread
    (1, 260, 12000, [12000], 1000),
    (2, 150, 20000, [20000, 19000], 2048),
]


@pytest.mark.parametrize("kind", ["gauss", "ties", "int", "const", "signed_zero", "narrow"])
@pytest.mark.parametrize("case", TOPK_CASES)
def test_topk_exact_against_oracle(dsa, orc, kind, case):
    B, T, Lmax, lens, K = case
    sc = make_scores(B * T, Lmax, seed=len(kind) + Lmax, kind=kind).reshape(B, T, Lmax).clone()
    # entries past each row's last visible position must never be read
    for b in range(B):
        for t in range(T):
            p = lens[b] - T + t
            sc[b, t, max(p + 1, 0):] = 1e30
    kl = torch.tensor(lens, dtype=torch.int32)
    s = shape_of(dsa, batch=B, n_q=T, max_kv=Lmax, topk=K)
    got = dsa.topk(s, sc.to(DEV), kl.to(DEV)).cpu().numpy().reshape(B * T, K)
    ref = orc.topk(sc.reshape(B * T, Lmax), kl, T, K)
    for r in range(B * T):
        want = sorted(x for x in ref[r] if x >= 0)
        want = want + [-1] * (K - len(want))
        assert list(got[r]) == want, f"row {r}"


# ---------------------------------------------------------------- sparse MLA
def _mla_case(B, T, H, Dqk, Dv, Lmax, lens, K, dt, seed, kind="topk"):
    g = torch.Generator().manual_seed(seed)
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    q = (torch.randn(B, T, H, Dqk, generator=g) * 3).to(tdt)  # logits ~ N(0, 9): a peaked softmax
    kv = (torch.randn(B, Lmax, Dqk, generator=g)).to(tdt)
    idx = torch.full((B, T, K), -1, dtype=torch.int32)
    for b in range(B):
        for t in range(T):
            p = lens[b] - T + t
            n = max(0, min(K, p + 1))
            perm = torch.randperm(max(p + 1, 1), generator=g)[:n]
            idx[b, t, :n] = (perm.sort().values if kind.startswith("sorted") else perm).int()
            if kind == "sorted_dup" and n >= 4:
                idx[b, t, 2] = idx[b, t, 1]          # adjacent duplicate in an ascending list
            if kind == "sorted_gap" and n >= 4:
                idx[b, t, 2] = -1                    # a skipped entry before valid ones
            if kind in ("messy", "poison") and K >= 8:
                idx[b, t, 0] = idx[b, t, 1]          # a duplicate
                idx[b, t, 2] = lens[b] + 5           # out of range -> skipped
                idx[b, t, 3] = -7                    # negative -> skipped
    return q, kv, idx, torch.tensor(lens, dtype=torch.int32)


MLA_CASES = [
    # B, T, H, Dqk, Dv, Lmax, lens, K, dt, kind
    (1, 256, 4, 80, 64, 256, [256], 64, "f32", "topk"),
    (2, 3, 9, 80, 64, 100, [100, 40], 64, "f32", "messy"),
    (4, 1, 128, 576, 512, 4096, [4096, 3000, 2048, 700], 2048, "bf16", "topk"),
    (1, 40, 128, 576, 512, 1000, [1000], 256, "bf16", "messy"),
    (2, 5, 20, 192, 128, 600, [600, 300], 128, "bf16", "topk"),
    (3, 2, 128, 576, 512, 64, [64, 2, 1], 32, "bf16", "topk"),
    # rows past kv_len hold NaN (one sequence is empty): they must never be read
    (3, 2, 128, 576, 512, 80, [80, 0, 1], 32, "bf16", "poison"),
    # lists of eight or more tiles per split take the one-wave-per-SIMD kernel:
    # two splits + combine; one split with lse; a partial second head block;
    # duplicates and skipped entries
    (1, 128, 128, 576, 512, 1024, [1024], 512, "bf16", "topk"),
    (1, 300, 128, 576, 512, 2048, [2048], 384, "bf16", "topk"),
    (1, 256, 200, 576, 512, 600, [600], 320, "bf16", "topk"),
    (1, 256, 128, 576, 512, 900, [900], 288, "bf16", "messy"),
    (2, 64, 128, 576, 512, 700, [700, 0], 512, "bf16", "poison"),
]


def _poison_rows(kv, lens, value):
    for b, L in enumerate(lens):
        kv[b, L:] = value


@pytest.mark.parametrize("case", MLA_CASES)
def test_sparse_mla_against_oracle(dsa, orc, case):
    B, T, H, Dqk, Dv, Lmax, lens, K, dt, kind = case
    q, kv, idx, kl = _mla_case(B, T, H, Dqk, Dv, Lmax, lens, K, dt, seed=B * 1000 + T + H, kind=kind)
    if kind == "poison":
        _poison_rows(kv, lens, float("nan"))
    announce(f"sparse_mla {case}")
    sm = Dqk ** -0.5
    s = shape_of(dsa, batch=B, n_q=T, max_kv=Lmax, heads=H, qk_dim=Dqk, v_dim=Dv, topk=K, sm_scale=sm,
                 mla_dtype=dt)
    out, lse = dsa.sparse_mla_fwd(s, q.to(DEV), kv.to(DEV), idx.to(DEV), kl.to(DEV))
    out = out.float().cpu().numpy().reshape(B * T, H, Dv)
    lse = lse.cpu().numpy().reshape(B * T, H)
    # the oracle skips out-of-range entries the same way the header defines
    ix = idx.clone().reshape(B * T, K)
    for r in range(B * T):
        L = lens[r // T]
        bad = (ix[r] >= L) | (ix[r] < 0)
        ix[r][bad] = -1
    ro, rl = orc.sparse_mla(q, kv, ix, sm, v_dim=Dv)
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(lse), empty)
    assert np.all(out[empty] == 0)
    live = ~empty
    err = rel_rowmax(out[live], ro[live])
    assert err.max() < TOL[dt], err.max()
    assert np.abs(lse[live] - rl[live]).max() < TOL[dt] * max(1.0, np.abs(rl[live]).max())


# ------------------------------------------------ fp8 latent cache and fp8 MLA
@pytest.mark.parametrize("dim,xdt", [(576, torch.bfloat16), (576, torch.float32), (16, torch.bfloat16),
                                     (512, torch.bfloat16), (1024, torch.float32)])
def test_mla_kv_quant_rows_exact(dsa, orc, dim, xdt):
    """fp8 latent-cache rows: codes, scale and zero pad bit-identical to the oracle's."""
    g = torch.Generator().manual_seed(dim + 7)
    x = torch.randn(3, 37, dim, generator=g) * torch.exp(2 * torch.randn(3, 37, 1, generator=g))
    x[0, 5] = 0.0                  # zero row: codes 0, scale 1
    x[1, 2, 3] = 1e4               # one dominant entry
    x[2, 9] = torch.randint(-3, 4, (dim,), generator=g).float() * 64  # few distinct values
    x = x.to(xdt)
    announce(f"mla_kv_quant dim={dim} {xdt}")
    got = dsa.mla_kv_quant_fp8(x.to(DEV)).cpu().numpy()
    assert np.array_equal(got, orc.kv_rows_fp8(x))


def test_mla_kv_quant_appends_into_a_cache(dsa, orc):
    """Pointing kv_rows at row p of a cache writes rows p.. only."""
    g = torch.Generator().manual_seed(5)
    cache = torch.full((2, 50, 592), 0xCD, dtype=torch.uint8, device=DEV)
    x = torch.randn(3, 576, generator=g).to(torch.bfloat16)
    announce("mla_kv_quant append")
    dsa.mla_kv_quant_fp8(x.to(DEV), kv_rows=cache[1, 10:13])
    c = cache.cpu().numpy()
    assert np.array_equal(c[1, 10:13], orc.kv_rows_fp8(x))
    keep = np.ones((2, 50), dtype=bool)
    keep[1, 10:13] = False
    assert np.all(c[keep] == 0xCD)


MLA_FP8_CASES = [
    # B, T, H, Lmax, lens, K, kind
    (4, 1, 128, 4096, [4096, 3000, 2048, 700], 2048, "topk"),   # decode: the list is split, then combined
    (1, 40, 128, 1000, [1000], 256, "messy"),
    (3, 2, 128, 64, [64, 2, 1], 32, "topk"),
    (2, 3, 20, 300, [300, 150], 96, "topk"),                     # a partial head block
    (1, 2, 200, 128, [128], 64, "topk"),                         # two head blocks
    (3, 2, 128, 80, [80, 0, 1], 32, "poison"),                   # rows past kv_len are NaN bytes
    # eight or more tiles per split: the one-wave-per-SIMD fp8 kernel
    (1, 128, 128, 1024, [1024], 512, "topk"),                    # two splits + combine
    (1, 256, 200, 600, [600], 320, "messy"),                     # one split, partial head block
    (2, 64, 128, 700, [700, 0], 512, "poison"),
]


@pytest.mark.parametrize("case", MLA_FP8_CASES)
def test_sparse_mla_fp8_against_oracle(dsa, orc, case):
    """fp8 MLA on cache rows from dsa_mla_kv_quant_fp8 (bit-checked above) against the
    oracle on its own codes of the same inputs.  Both sides attend over the same
    dequantised values, so the tolerance is the bf16 path's (bf16 weights and output)."""
    B, T, H, Lmax, lens, K, kind = case
    q, kv, idx, kl = _mla_case(B, T, H, 576, 512, Lmax, lens, K, "bf16", seed=B * 977 + T + H, kind=kind)
    sm = 192 ** -0.5
    s = shape_of(dsa, batch=B, n_q=T, max_kv=Lmax, heads=H, topk=K, sm_scale=sm, mla_dtype="fp8")
    announce(f"sparse_mla fp8 {case}")
    rows = dsa.mla_kv_quant_fp8(kv.to(DEV))
    if kind == "poison":
        _poison_rows(rows, lens, 0xFF)  # e4m3 NaN codes and a NaN scale
    out, lse = dsa.sparse_mla_fwd(s, q.to(DEV), rows, idx.to(DEV), kl.to(DEV))
    assert out.dtype == torch.bfloat16
    out = out.float().cpu().numpy().reshape(B * T, H, 512)
    lse = lse.cpu().numpy().reshape(B * T, H)
    ix = idx.clone().reshape(B * T, K)
    for r in range(B * T):
        L = lens[r // T]
        ix[r][(ix[r] >= L) | (ix[r] < 0)] = -1
    qc, qs = orc.quant(q)
    kc, ks = orc.quant(kv)
    ro, rl = orc.sparse_mla_fp8(qc, qs, kc, ks, ix, sm, v_dim=512)
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(lse), empty)
    assert np.all(out[empty] == 0)
    live = ~empty
    err = rel_rowmax(out[live], ro[live])
    assert err.max() < TOL["bf16"], err.max()
    assert np.abs(lse[live] - rl[live]).max() < TOL["bf16"] * max(1.0, np.abs(rl[live]).max())


@pytest.mark.parametrize("T", [1, 256])
@pytest.mark.parametrize("dt", ["bf16", "fp8"])
def test_sparse_mla_large_logit_jumps(dsa, orc, dt, T):
    """Later tiles whose logits exceed every earlier one by far more than the
    kernels' softmax reference slack (2^64 and 2^8 in log2 units): the result must
    still be the oracle's.  Queries are all ones; the listed rows are small random
    values except three rows, in tiles 2, 5 and 9 of the first query's list, whose
    logits are about 100, 200 and 300 (natural log units) above the rest.  T = 1
    splits each list in three (short-list kernels), T = 256 keeps whole 12-tile
    lists (one-wave-per-SIMD kernels, whose restart path this takes)."""
    g = torch.Generator().manual_seed(31)
    B, H, L, K, D, Dv = 2, 128, 512, 384, 576, 512
    q = torch.ones(B, T, H, D)
    q[:, :, 1::2] *= 0.5                       # two groups of heads with different logit scales
    kv = torch.randn(B, L, D, generator=g) * 0.05
    idx = torch.stack([torch.randperm(L, generator=g)[:K] for _ in range(B * T)]).int().reshape(B, T, K)
    sm = 1.0 / 24.0
    for b in range(B):
        for tile, c in ((2, 100.0), (5, 200.0), (9, 300.0)):
            r = int(idx[b, 0, 32 * tile + 7])
            kv[b, r] = c / (sm * D) + 0.02 * torch.randn(D, generator=g)
    q, kv = q.to(torch.bfloat16), kv.to(torch.bfloat16)
    kl = torch.full((B,), L, dtype=torch.int32)
    s = shape_of(dsa, batch=B, n_q=T, max_kv=L, heads=H, topk=K, sm_scale=sm, mla_dtype=dt)
    announce(f"sparse_mla large logit jumps {dt}")
    if dt == "fp8":
        out, lse = dsa.sparse_mla_fwd(s, q.to(DEV), dsa.mla_kv_quant_fp8(kv.to(DEV)), idx.to(DEV), kl.to(DEV))
        qc, qs = orc.quant(q)
        kc, ks = orc.quant(kv)
        ro, rl = orc.sparse_mla_fp8(qc, qs, kc, ks, idx.reshape(B * T, K), sm, v_dim=Dv)
    else:
        out, lse = dsa.sparse_mla_fwd(s, q.to(DEV), kv.to(DEV), idx.to(DEV), kl.to(DEV))
        ro, rl = orc.sparse_mla(q, kv, idx.reshape(B * T, K), sm, v_dim=Dv)
    out = out.float().cpu().numpy().reshape(B * T, H, Dv)
    lse = lse.cpu().numpy().reshape(B * T, H)
    err = rel_rowmax(out, ro)
    assert err.max() < TOL["bf16"], err.max()
    assert np.abs(lse - rl).max() < TOL["bf16"] * np.abs(rl).max()


# ------------------------------------------------------------ sparse MLA backward
MLA_BWD_CASES = [
    # B, T, H, Dqk, Dv, Lmax, lens, K, kind
    (2, 3, 128, 576, 512, 300, [300, 120], 64, "topk"),          # one split: dq stored
    (4, 1, 128, 576, 512, 4096, [4096, 3000, 2048, 700], 2048, "topk"),  # split decode: dq atomics
    (1, 40, 128, 576, 512, 1000, [1000], 256, "messy"),          # duplicates and skipped entries
    (2, 5, 20, 192, 128, 600, [600, 300], 128, "topk"),          # padded heads, the 192/128 shape
    (3, 2, 128, 576, 512, 80, [80, 0, 1], 32, "poison"),         # an empty sequence, NaN rows past kv_len
    (2, 3, 128, 576, 512, 500, [500, 2], 100, "messy"),          # K not a multiple of 32; a query before the cache
    (1, 70, 96, 576, 512, 4096, [4096], 1000, "topk"),           # two list splits of a long list, 96 heads
    # one query per sequence, ascending lists (top-k's layout): rows updated with plain stores
    (4, 1, 128, 576, 512, 4096, [4096, 3000, 2048, 700], 2048, "sorted"),
    (3, 1, 20, 192, 128, 600, [600, 1, 0], 128, "sorted"),
    # one query per sequence whose list repeats or skips rows mid-list: atomics again
    (3, 1, 128, 576, 512, 2000, [2000, 1500, 40], 512, "messy"),
    (2, 1, 128, 576, 512, 3000, [3000, 2000], 1024, "sorted_dup"),
    (2, 1, 128, 576, 512, 3000, [3000, 2000], 1024, "sorted_gap"),
]


def _bwd_run(dsa, case, seed, ws_bytes=None, accumulate=False, dkv=None):
    B, T, H, Dqk, Dv, Lmax, lens, K, kind = case
    q, kv, idx, kl = _mla_case(B, T, H, Dqk, Dv, Lmax, lens, K, "bf16", seed=seed, kind=kind)
    if kind == "poison":
        _poison_rows(kv, lens, float("nan"))
    g = torch.Generator().manual_seed(seed + 1)
    dout = torch.randn(B, T, H, Dv, generator=g).to(torch.bfloat16)
    sm = Dqk ** -0.5
    s = shape_of(dsa, batch=B, n_q=T, max_kv=Lmax, heads=H, qk_dim=Dqk, v_dim=Dv, topk=K, sm_scale=sm)
    dev = [x.to(DEV) for x in (q, kv, idx, kl, dout)]
    _, lse = dsa.sparse_mla_fwd(s, dev[0], dev[1], dev[2], dev[3])
    ws = None if ws_bytes is None else torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    dq, dkv = dsa.sparse_mla_bwd(s, dev[0], dev[1], dev[2], dev[3], lse, dev[4], dkv=dkv,
                                 accumulate_dkv=accumulate, workspace=ws)
    torch.cuda.synchronize()
    return (q, kv, idx, kl, dout, sm), dq, dkv, s


def _bwd_ref(orc, case, inputs):
    B, T, H, Dqk, Dv, Lmax, lens, K, kind = case
    q, kv, idx, kl, dout, sm = inputs
    ix = idx.clone().reshape(B * T, K)
    for r in range(B * T):
        L = lens[r // T]
        ix[r][(ix[r] >= L) | (ix[r] < 0)] = -1
    return orc.sparse_mla_bwd(q, kv, dout, ix, sm, v_dim=Dv), ix


@pytest.mark.parametrize("case", MLA_BWD_CASES)
def test_sparse_mla_bwd_against_oracle(dsa, orc, case):
    """dq and dkv against the fp64 oracle at the bf16 tolerance (per-row max norm:
    p and dz enter the MFMAs in bf16).  Cache rows nobody selects and queries with
    no valid entry stay exactly zero."""
    B, T, H, Dqk, Dv, Lmax, lens, K, kind = case
    announce(f"sparse_mla_bwd {case}")
    inputs, dq, dkv, _ = _bwd_run(dsa, case, seed=B * 131 + T + H)
    (rq, rkv), ix = _bwd_ref(orc, case, inputs)
    dq = dq.cpu().numpy().reshape(B * T, H, Dqk)
    dkv = dkv.cpu().numpy()
    # queries with no valid entry get exactly zero; a list whose entries all hold
    # one row has a vanishing exact dq (dz = p (dP - D) cancels), compared in
    # absolute terms against the largest gradient; every other row per row
    empty = (ix.numpy() < 0).all(axis=1)
    assert np.all(dq[empty] == 0)
    big = np.abs(rq).max()
    live = np.abs(rq).max(axis=-1) > 1e-3 * big
    assert np.abs(dq[~live] - rq[~live]).max(initial=0.0) < TOL["bf16"] * big
    err = rel_rowmax(dq[live], rq[live])
    assert err.max() < TOL["bf16"], err.max()
    touched = np.abs(rkv).max(axis=-1) > 0
    assert np.all(dkv[~touched] == 0)
    err = rel_rowmax(dkv[touched], rkv[touched])
    assert err.max() < TOL["bf16"], err.max()


def test_sparse_mla_bwd_chunked_and_accumulated(dsa, orc):
    """The smallest workspace (one query at a time) gives the one-pass gradients;
    accumulate_dkv adds to what dkv holds."""
    case = (1, 40, 128, 576, 512, 1000, [1000], 256, "messy")
    announce("sparse_mla_bwd chunked")
    inputs, dq1, dkv1, s = _bwd_run(dsa, case, seed=77)
    small = dsa.sparse_mla_bwd_min_workspace_size(s)
    _, dq2, dkv2, _ = _bwd_run(dsa, case, seed=77, ws_bytes=small)
    assert torch.allclose(dq1, dq2, rtol=1e-4, atol=1e-6 * dq1.abs().max().item())
    assert torch.allclose(dkv1, dkv2, rtol=1e-4, atol=1e-6 * dkv1.abs().max().item())
    _, _, dkv3, _ = _bwd_run(dsa, case, seed=77, accumulate=True, dkv=dkv1.clone())
    assert torch.allclose(dkv3, 2 * dkv1, rtol=1e-4, atol=1e-6 * dkv1.abs().max().item())
    # the same with one query per sequence and ascending lists
    case = (4, 1, 128, 576, 512, 3000, [3000, 2500, 900, 64], 512, "sorted")
    _, _, dkv1, _ = _bwd_run(dsa, case, seed=78)
    _, _, dkv3, _ = _bwd_run(dsa, case, seed=78, accumulate=True, dkv=dkv1.clone())
    assert torch.allclose(dkv3, 2 * dkv1, rtol=1e-4, atol=1e-6 * dkv1.abs().max().item())
