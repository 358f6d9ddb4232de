"""Streaming indexer -> top-k (dsa_index_topk) against the oracle.

Integer-valued inputs make every score exact on both sides, so the selection must
equal the oracle's top-k (score descending, position ascending) entry for entry,
ties included; candidate lists much shorter than the rows force repeated cuts.
Gaussian inputs at the prefill_4k shape are held to the top-k tie band on sampled
rows against the oracle, and, for every dtype and for prefill and decode shapes, must
select exactly what dsa_index_scores followed by dsa_topk select (the header's
bit-for-bit promise).  The entry point is called through the C ABI.
"""
import numpy as np
import pytest
import torch

from helpers import announce, topk_valid
from workloads import get, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def shape_of(dsa, **kw):
    base = dict(batch=1, n_q=1, max_kv=64, idx_heads=64, idx_dim=128, topk=64, heads=128, qk_dim=576, v_dim=512,
                sm_scale=1 / 192 ** 0.5, idx_dtype="bf16", mla_dtype="bf16")
    base.update(kw)
    return dsa.DsaShape(**base)


def _expected(orc, scores, kl, T, K):
    """Oracle top-k rows as the entry point writes them: ascending positions, -1 padded."""
    ref = orc.topk(scores, kl, T, K)
    out = np.full((ref.shape[0], K), -1, dtype=np.int64)
    for r in range(ref.shape[0]):
        sel = sorted(int(x) for x in ref[r] if x >= 0)
        out[r, :len(sel)] = sel
    return out


INT_CASES = [
    # dt, D, H, B, T, Lmax, lens, K, value range
    ("bf16", 128, 64, 2, 37, 300, [300, 150], 16, 3),      # many ties, cuts every few tiles
    ("bf16", 128, 16, 1, 64, 4096, [4096], 64, 3),         # long rows: about fifteen cuts each
    ("f32", 32, 4, 1, 256, 256, [256], 64, 2),              # the tiny shape
    ("bf16", 128, 7, 3, 9, 2000, [2000, 1500, 5], 2048, 3),  # rows shorter than K; a 5-token sequence
    ("f32", 64, 64, 2, 20, 5000, [5000, 4000], 1000, 8),    # one cut late in the row
    ("bf16", 128, 64, 1, 3, 600, [600], 1, 3),              # K = 1
    ("bf16", 128, 64, 4, 1, 3000, [3000, 2000, 1, 0], 256, 3),  # one query per sequence; an empty one
    # lists longer than the final select's LDS stage: rows of the 10000-key sequence never fill
    # their 12032-entry lists, so they end with 9993..10000 entries
    ("bf16", 128, 16, 2, 8, 20000, [20000, 10000], 3000, 3),
]


@pytest.mark.parametrize("case", INT_CASES)
def test_index_topk_integer_inputs_exact(dsa, orc, case):
    dt, D, H, B, T, Lmax, lens, K, vr = case
    announce(f"index_topk integer {case}")
    g = torch.Generator().manual_seed(B * 1000 + T + K)
    q = torch.randint(-vr, vr + 1, (B, T, H, D), generator=g).float()
    k = torch.randint(-vr, vr + 1, (B, Lmax, D), generator=g).float()
    w = torch.randint(-4, 5, (B, T, H), generator=g).float()
    kl = torch.tensor(lens, dtype=torch.int32)
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    s = shape_of(dsa, batch=B, n_q=T, max_kv=Lmax, idx_heads=H, idx_dim=D, idx_dtype=dt, topk=K)
    got = dsa.index_topk(s, q.to(tdt).to(DEV), w.to(DEV), k.to(tdt).to(DEV), kl.to(DEV)).cpu().numpy()
    scores = orc.index_scores(q, w, k, kl).reshape(B * T, Lmax)
    want = _expected(orc, scores, kl, T, K)
    assert np.array_equal(got.reshape(B * T, K), want)


def test_index_topk_fp8_exact_codes(dsa, orc):
    # small-integer e4m3 codes with power-of-two scales: every score is exact
    B, T, H, D, Lmax, K = 2, 9, 64, 128, 700, 32
    g = torch.Generator().manual_seed(5)
    qv = torch.randint(-4, 5, (B, T, H, D), generator=g).float()
    kv = torch.randint(-4, 5, (B, Lmax, D), generator=g).float()
    w = torch.randint(-3, 4, (B, T, H), generator=g).float()
    qs = 2.0 ** torch.randint(-2, 3, (B, T, H), generator=g).float()
    ks = 2.0 ** torch.randint(-2, 3, (B, Lmax), generator=g).float()
    qc = torch.from_numpy(orc.e4m3_encode(qv.numpy()))
    kc = torch.from_numpy(orc.e4m3_encode(kv.numpy()))
    kl = torch.tensor([700, 240], dtype=torch.int32)
    s = shape_of(dsa, batch=B, n_q=T, max_kv=Lmax, idx_dtype="fp8", topk=K)
    got = dsa.index_topk(s, qc.to(DEV), w.to(DEV), kc.to(DEV), kl.to(DEV), q_scale=qs.to(DEV),
                         k_scale=ks.to(DEV)).cpu().numpy()
    scores = orc.index_scores_fp8(qc, qs, w, kc, ks, kl).reshape(B * T, Lmax)
    assert np.array_equal(got.reshape(B * T, K), _expected(orc, scores, kl, T, K))


def test_index_topk_chunked_workspace(dsa, orc):
    """The smallest workspace (one query per pass) gives the same selection."""
    B, T, H, D, Lmax, K = 2, 13, 64, 128, 900, 48
    g = torch.Generator().manual_seed(9)
    q = torch.randint(-3, 4, (B, T, H, D), generator=g).float()
    k = torch.randint(-3, 4, (B, Lmax, D), generator=g).float()
    w = torch.randint(-4, 5, (B, T, H), generator=g).float()
    kl = torch.tensor([900, 500], dtype=torch.int32)
    s = shape_of(dsa, batch=B, n_q=T, max_kv=Lmax, topk=K)
    args = (q.to(torch.bfloat16).to(DEV), w.to(DEV), k.to(torch.bfloat16).to(DEV), kl.to(DEV))
    small = dsa.index_topk_min_workspace_size(s)
    assert 0 < small < dsa.index_topk_workspace_size(s)
    ws = torch.empty(small, dtype=torch.uint8, device=DEV)
    got = dsa.index_topk(s, *args, workspace=ws).cpu().numpy()
    scores = orc.index_scores(q, w, k, kl).reshape(B * T, Lmax)
    assert np.array_equal(got.reshape(B * T, K), _expected(orc, scores, kl, T, K))


def test_index_topk_prefill_4k_sampled(dsa, orc):
    """Gaussian inputs of the prefill_4k workload: sampled rows hold the tie band
    against the oracle's fp64 scores and mostly select the oracle's exact set."""
    wl = get("prefill_4k")
    inp = make_inputs(wl, device=DEV, with_mla=False)
    s = dsa.DsaShape.of(wl)
    announce("index_topk prefill_4k")
    got = dsa.index_topk(s, inp["q_idx"], inp["w"], inp["k_idx"], inp["kv_len"]).cpu().numpy()
    rows = [0, 1, 7, 8, 100, 2046, 2047, 2048, 2049, 3000, 4094, 4095]
    cpu = {k: v.cpu() for k, v in inp.items()}
    ref = orc.index_scores(cpu["q_idx"], cpu["w"], cpu["k_idx"], cpu["kv_len"], rows=rows)
    want = orc.topk(ref, cpu["kv_len"], wl.n_q, wl.topk, rows=rows)
    same = 0
    for i, r in enumerate(rows):
        p = wl.kv_len - wl.n_q + r
        row = got.reshape(-1, wl.topk)[r]
        msg = topk_valid(row, ref[i], p, wl.topk)
        assert msg is None, f"row {r}: {msg}"
        same += int(set(row[row >= 0].tolist()) == set(want[i][want[i] >= 0].tolist()))
    assert same >= len(rows) - 1


CONSISTENCY_CASES = [
    # dt, D, H, B, T, Lmax, lens, K
    ("bf16", 128, 64, 1, 4096, 4096, [4096], 2048),                  # the prefill_4k shape
    ("bf16", 128, 64, 6, 1, 32768, [32768, 30000, 5000, 1, 0, 20000], 2048),  # decode, one query
    ("bf16", 128, 64, 4, 2, 20000, [20000, 15000, 3, 2], 512),        # decode, two queries
    ("fp8", 128, 64, 2, 300, 8192, [8192, 4000], 1024),               # fp8 prefill
    ("fp8", 128, 64, 4, 1, 40000, [40000, 1000, 39000, 7], 2048),     # fp8 decode
    ("f32", 64, 16, 2, 2, 5000, [5000, 4000], 300),
]


@pytest.mark.parametrize("case", CONSISTENCY_CASES)
def test_index_topk_equals_scores_then_topk(dsa, case):
    """On Gaussian inputs dsa_index_topk selects exactly what dsa_index_scores followed by
    dsa_topk select, bit for bit: the fused pass and the score rows (the decode tiling
    included) compute every score in the same order."""
    dt, D, H, B, T, Lmax, lens, K = case
    announce(f"index_topk == index_scores + topk {case}")
    g = torch.Generator().manual_seed(7 * Lmax + T)
    q = torch.randn(B, T, H, D, generator=g)
    k = torch.randn(B, Lmax, D, generator=g)
    w = torch.randn(B, T, H, generator=g)
    kl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    s = shape_of(dsa, batch=B, n_q=T, max_kv=Lmax, idx_heads=H, idx_dim=D, topk=K, idx_dtype=dt)
    w = w.to(DEV)
    if dt == "fp8":
        qc, qs = dsa.rotate_quant_fp8(q.to(DEV, torch.bfloat16))
        kc, ks = dsa.rotate_quant_fp8(k.to(DEV, torch.bfloat16))
        kw = dict(q_scale=qs, k_scale=ks)
        args = (qc, w, kc, kl)
    else:
        tdt = torch.bfloat16 if dt == "bf16" else torch.float32
        kw = {}
        args = (q.to(DEV, tdt), w, k.to(DEV, tdt), kl)
    scores = dsa.index_scores(s, *args, **kw)
    ref = dsa.topk(s, scores, kl)
    got = dsa.index_topk(s, *args, **kw)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
