"""Pins for the oracle's whole path (indexer -> top-k -> sparse MLA).

The DeepSeek-V3.2 model documentation page ("DeepSeek Sparse Attention (DSA)")
says the FP8 indexer is only a precision optimisation of the same scores, and
that each layer runs its own indexer.  Checked here: the fp8 path stays within
5e-2 (relative, per-row max norm) of the unquantised scores; the composition
agrees with its parts; a stored fixture written by tests/golden/make_golden.py
(oracle only) still matches.
"""
import json
import os

import numpy as np

from workloads import get, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rel_rowmax(a, b):
    fin = np.isfinite(b)
    assert np.array_equal(fin, np.isfinite(a))
    d = np.where(fin, np.abs(a - b), 0).max(axis=-1)
    m = np.where(fin, np.abs(b), 0).max(axis=-1)
    return d / np.maximum(m, 1e-30)


def test_forward_composes_its_parts(orc):
    wl = get("tiny_f32")
    inp = make_inputs(wl)
    rows = [0, 5, 63, 64, 200, 255]
    res = orc.forward(inp, wl, rows=rows)
    sc = orc.index_scores(inp["q_idx"], inp["w"], inp["k_idx"], inp["kv_len"], rows=rows)
    assert np.array_equal(res["scores"], sc)
    idx = orc.topk(sc, inp["kv_len"], wl.n_q, wl.topk, rows=rows)
    assert np.array_equal(res["idx"], idx)
    for i, r in enumerate(rows):
        keff = min(wl.topk, r + 1)
        assert np.all(res["idx"][i, :keff] >= 0) and np.all(res["idx"][i, keff:] == -1)
        assert len(set(res["idx"][i, :keff].tolist())) == keff
    o, l = orc.sparse_mla(inp["q"], inp["kv"], idx, wl.sm_scale, rows=rows, v_dim=wl.v_dim)
    assert np.array_equal(res["out"], o) and np.array_equal(res["lse"], l)


def test_fp8_indexer_tracks_unquantised_scores(orc):
    wl = get("decode_128k_fp8").replace(batch=2, max_kv=3000, kv_len=3000, topk=256)
    inp = make_inputs(wl, with_mla=False)
    res_plain = orc.index_scores(inp["q_idx"], inp["w"], inp["k_idx"], inp["kv_len"])
    qc, qs = orc.rotate_quant(inp["q_idx"])
    kc, ks = orc.rotate_quant(inp["k_idx"])
    s8 = orc.index_scores_fp8(qc, qs, inp["w"], kc, ks, inp["kv_len"])
    assert _rel_rowmax(s8, res_plain).max() < 5e-2
    i8 = orc.topk(s8, inp["kv_len"], wl.n_q, wl.topk)
    ip = orc.topk(res_plain, inp["kv_len"], wl.n_q, wl.topk)
    for r in range(wl.rows):
        overlap = len(set(i8[r].tolist()) & set(ip[r].tolist())) / wl.topk
        assert overlap > 0.8


def test_layers_are_independent(orc):
    # Two "layers" with different inputs: the result of each is its solo result,
    # whatever ran before it (the oracle keeps no state between calls).
    wl = get("tiny_f32")
    a = make_inputs(wl, seed=1)
    b = make_inputs(wl, seed=2)
    ra = orc.forward(a, wl, rows=[100, 255])
    orc.forward(b, wl, rows=[100, 255])
    ra2 = orc.forward(a, wl, rows=[100, 255])
    for k in ("scores", "idx", "out", "lse"):
        assert np.array_equal(ra[k], ra2[k])


def test_golden_fixture_tiny(orc):
    with open(os.path.join(GOLDEN, "tiny_f32_rows.json")) as f:
        g = json.load(f)
    wl = get(g["workload"])
    inp = make_inputs(wl)
    res = orc.forward(inp, wl, rows=g["rows"])
    for i, r in enumerate(g["rows"]):
        assert sorted(res["idx"][i][res["idx"][i] >= 0].tolist()) == g["idx_sorted"][str(r)]
        assert np.allclose(res["lse"][i], g["lse"][str(r)], rtol=0, atol=1e-12)
        assert np.allclose(res["out"][i].sum(axis=-1), g["out_rowsum"][str(r)], rtol=0, atol=1e-12)


def test_compact_rows_equal_full_rows(orc):
    # compact inputs (only the listed query rows) give the same results as full inputs
    wl = get("tiny_f32").replace(batch=2, max_kv=300, kv_len=280)
    inp = make_inputs(wl)
    rows = [3, 255, 256, 400, 511]
    full = orc.forward(inp, wl, rows=rows)
    flat = lambda t: t.reshape(wl.rows, *t.shape[2:])[rows]
    cin = dict(inp, q_idx=flat(inp["q_idx"]), w=flat(inp["w"]), q=flat(inp["q"]))
    comp = orc.forward(cin, wl, rows=rows, compact=True)
    for k in ("scores", "idx", "out", "lse"):
        assert np.array_equal(full[k], comp[k]), k
