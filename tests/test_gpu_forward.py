"""End-to-end GPU parity of dsa_forward (indexer -> top-k -> sparse MLA).

Every workload runs on the device at its full size in the launch configuration
the benchmark times (a workspace large enough for one pass); the oracle checks
every decode sequence, every prefill_4k row and 512 stratified prefill_32k rows.
Top-k sets must be valid under the tie band (and, where scores are exact,
identical); outputs of every checked row are compared with the oracle's
attention over the device's own index set (reading R16 (iv)), so a row whose set
differs from the oracle's by a tie swap is checked too.  At most a small share
of rows may select a different set.
"""
import numpy as np
import pytest
import torch

from helpers import TOL, announce, rel_rowmax, topk_valid
from workloads import get, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _prepare(dsa, wl, inp):
    """Device inputs of dsa_forward; an fp8 workload gets its key cache (and, with an fp8
    MLA, its latent cache) quantised by the library."""
    k_idx, k_scale, kv = inp["k_idx"], None, inp["kv"]
    if wl.idx_dtype == "fp8":
        k_idx, k_scale = dsa.rotate_quant_fp8(inp["k_idx"])
    if wl.mla_dtype == "fp8":
        kv = dsa.mla_kv_quant_fp8(inp["kv"])
    return k_idx, k_scale, kv


def _run(dsa, wl, inp, workspace_bytes=None):
    s = dsa.DsaShape.of(wl)
    k_idx, k_scale, kv = _prepare(dsa, wl, inp)
    ws = None
    if workspace_bytes is not None:
        ws = torch.empty(workspace_bytes, dtype=torch.uint8, device=DEV)
    idx, out, lse = dsa.forward(s, inp["q_idx"], inp["w"], k_idx, inp["q"], kv, inp["kv_len"],
                                k_scale=k_scale, workspace=ws)
    torch.cuda.synchronize()
    return idx, out, lse, k_idx, k_scale, kv


def _oracle_inputs(inp, wl, rows, seqs=None):
    """CPU copies the oracle needs: the listed query rows only, whole key/value caches of ``seqs``."""
    seqs = list(range(wl.batch)) if seqs is None else seqs
    flat = lambda t: t.reshape(-1, *t.shape[2:])[torch.as_tensor(rows, device=t.device)].cpu()
    return dict(q_idx=flat(inp["q_idx"]), w=flat(inp["w"]), q=flat(inp["q"]), k_idx=inp["k_idx"][seqs].cpu(),
                kv=inp["kv"][seqs].cpu(), kv_len=inp["kv_len"][seqs].cpu())


def _check(orc, wl, inp_cpu, rows, idx, out, lse, gpu_k_codes=None, gpu_kv_rows=None):
    """Compare device results on query rows ``rows`` (indices into the [B*T] rows of ``wl``);
    ``inp_cpu`` holds compact per-query tensors for exactly those rows.  Outputs are held
    against the oracle's attention over the device's own index set: for rows whose set
    equals the oracle's that is the oracle's forward output, for the others the oracle
    attends again over the device's set.  The fp8 MLA is held to the bf16 tolerance: the
    oracle attends over the same dequantised values."""
    res = orc.forward(inp_cpu, wl, rows=rows, compact=True)
    if gpu_k_codes is not None:
        assert np.array_equal(gpu_k_codes, res["k_codes"]), "device key codes differ from the oracle's"
    if gpu_kv_rows is not None:
        assert np.array_equal(gpu_kv_rows[..., :wl.qk_dim], res["kv_codes"]), "device latent codes differ"
        sc = gpu_kv_rows[..., wl.qk_dim:wl.qk_dim + 4].copy().view("<f4")[..., 0]
        assert np.array_equal(sc, res["kv_scale"]), "device latent scales differ"
    tol = TOL["bf16" if wl.mla_dtype == "fp8" else wl.mla_dtype]
    T, K = wl.n_q, wl.topk
    rows = np.asarray(rows, dtype=np.int64)
    gi = idx.reshape(-1, K)[rows].numpy()
    go = out.float().reshape(-1, wl.heads, wl.v_dim)[rows].numpy()
    gl = lse.reshape(-1, wl.heads)[rows].numpy()
    kl = inp_cpu["kv_len"].numpy()
    same = []
    for i, r in enumerate(rows):
        b, t = divmod(int(r), T)
        p = min(int(kl[b]), wl.max_kv) - T + t
        msg = topk_valid(gi[i], res["scores"][i], p, K)
        assert msg is None, f"row {r}: {msg}"
        same.append(set(gi[i][gi[i] >= 0].tolist()) == set(res["idx"][i][res["idx"][i] >= 0].tolist()))
    same = np.array(same)
    assert same.mean() >= 0.95, f"only {same.mean():.3f} of rows select the oracle's set"
    ref_out, ref_lse = res["out"], res["lse"]
    diff = np.nonzero(~same)[0]
    if diff.size:
        # the oracle's attention over the sets the device selected
        if wl.mla_dtype == "fp8":
            o_d, l_d = orc.sparse_mla_fp8(res["mla_q_codes"][diff], res["mla_q_scale"][diff], res["kv_codes"],
                                          res["kv_scale"], gi[diff], wl.sm_scale, rows=rows[diff], v_dim=wl.v_dim,
                                          T=T)
        else:
            o_d, l_d = orc.sparse_mla(inp_cpu["q"][torch.as_tensor(diff)], inp_cpu["kv"], gi[diff], wl.sm_scale,
                                      rows=rows[diff], v_dim=wl.v_dim, T=T)
        ref_out, ref_lse = ref_out.copy(), ref_lse.copy()
        ref_out[diff] = o_d
        ref_lse[diff] = l_d
    err = rel_rowmax(go.reshape(-1, wl.v_dim), ref_out.reshape(-1, wl.v_dim))
    assert err.max() < tol, err.max()
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(gl)) and np.all(gl[~fin] == -np.inf)
    assert np.abs(gl[fin] - ref_lse[fin]).max(initial=0.0) < tol * max(1.0, np.abs(ref_lse[fin]).max(initial=0.0))
    return same


def _stratified_rows(T, n_random, seed=0):
    """Rows 0-15, 2040-2055 (around the dense-to-sparse crossover at index_topk = 2048),
    the last 16, and n_random further rows drawn uniformly without replacement."""
    fixed = set(range(16)) | set(range(2040, 2056)) | set(range(T - 16, T))
    rest = np.setdiff1d(np.arange(T), np.fromiter(fixed, dtype=np.int64))
    pick = np.random.default_rng(seed).choice(rest, size=n_random, replace=False)
    return sorted(fixed | set(pick.tolist()))


def test_forward_tiny_every_row(dsa, orc):
    wl = get("tiny_f32")
    inp = {k: v.to(DEV) for k, v in make_inputs(wl).items()}
    idx, out, lse, _, _, _ = _run(dsa, wl, inp)
    rows = list(range(wl.rows))
    same = _check(orc, wl, _oracle_inputs(inp, wl, rows), rows, idx.cpu(), out.cpu(), lse.cpu())
    assert same.all()


def test_forward_prefill_4k_every_row(dsa, orc):
    wl = get("prefill_4k")
    inp = make_inputs(wl, device=DEV)
    idx, out, lse, _, _, _ = _run(dsa, wl, inp)
    rows = list(range(wl.rows))
    _check(orc, wl, _oracle_inputs(inp, wl, rows), rows, idx.cpu(), out.cpu(), lse.cpu())


def test_forward_prefill_4k_chunked_matches_single_pass(dsa):
    wl = get("prefill_4k")
    inp = make_inputs(wl, device=DEV)
    idx1, out1, lse1, _, _, _ = _run(dsa, wl, inp)
    s = dsa.DsaShape.of(wl)
    small = dsa.forward_min_workspace_size(s)
    idx2, out2, lse2, _, _, _ = _run(dsa, wl, inp, workspace_bytes=small)
    assert torch.equal(idx1, idx2)
    d = (out1.float() - out2.float()).abs().max().item()
    assert d <= 2e-2 * out1.float().abs().max().item()


@pytest.mark.parametrize("operands", ["integer", "gaussian"])
def test_forward_streaming_fallback_matches_score_rows(dsa, operands):
    """Four decode sequences of 256K keys in their smallest workspace: one query's
    score rows (4 x 1 MiB, with the split top-k's scratch) do not fit, the fused
    scores + top-k (64 KiB of candidate list per row) does, so dsa_forward streams.
    Both paths compute every score in the same order, so the selection, the outputs
    and the lse equal those of the one-pass score-row run bit for bit: on integer-valued
    indexer operands (exact scores, many ties broken by position on both) and on the
    workload's Gaussian ones."""
    wl = get("decode_32k").replace(batch=4, max_kv=1 << 18, kv_len=1 << 18)
    inp = make_inputs(wl, device=DEV)
    if operands == "integer":
        g = torch.Generator(device=DEV).manual_seed(5)
        inp["q_idx"] = torch.randint(-3, 4, inp["q_idx"].shape, generator=g, device=DEV).to(torch.bfloat16)
        inp["k_idx"] = torch.randint(-3, 4, inp["k_idx"].shape, generator=g, device=DEV).to(torch.bfloat16)
        inp["w"] = torch.randint(-4, 5, inp["w"].shape, generator=g, device=DEV).float()
    s = dsa.DsaShape.of(wl)
    small = dsa.forward_min_workspace_size(s)
    assert small < dsa.forward_workspace_size(s)  # T = 1: the score-row path has no smaller layout
    announce(f"forward streaming fallback vs score rows, 4 x 256K decode, {operands} operands")
    idx1, out1, lse1, _, _, _ = _run(dsa, wl, inp)
    idx2, out2, lse2, _, _, _ = _run(dsa, wl, inp, workspace_bytes=small)
    assert torch.equal(idx1, idx2)
    assert torch.equal(out1, out2)
    assert torch.equal(lse1, lse2)


def test_forward_decode_32k_every_sequence(dsa, orc):
    wl = get("decode_32k")
    inp = make_inputs(wl, device=DEV)
    idx, out, lse, _, _, _ = _run(dsa, wl, inp)
    rows = list(range(wl.rows))  # T = 1: row b is sequence b
    _check(orc, wl, _oracle_inputs(inp, wl, rows), rows, idx.cpu(), out.cpu(), lse.cpu())


def test_forward_prefill_32k_stratified_rows(dsa, orc):
    wl = get("prefill_32k")
    inp = make_inputs(wl, device=DEV)
    idx, out, lse, _, _, _ = _run(dsa, wl, inp)
    rows = _stratified_rows(wl.n_q, 512 - 48)
    assert len(rows) == 512
    _check(orc, wl, _oracle_inputs(inp, wl, rows), rows, idx.cpu(), out.cpu(), lse.cpu())


def test_forward_decode_128k_fp8_every_sequence(dsa, orc):
    wl = get("decode_128k_fp8")
    inp = make_inputs(wl, device=DEV)
    idx, out, lse, kc, ks, _ = _run(dsa, wl, inp)
    rows = list(range(wl.rows))
    _check(orc, wl, _oracle_inputs(inp, wl, rows), rows, idx.cpu(), out.cpu(), lse.cpu(),
           gpu_k_codes=kc.cpu().numpy())


def test_forward_decode_128k_fp8_mla_every_sequence(dsa, orc):
    """fp8 indexer and fp8 latent cache: codes of both caches bit-checked, outputs at the
    bf16 tolerance against the oracle's fp8 MLA."""
    wl = get("decode_128k_fp8_mla")
    inp = make_inputs(wl, device=DEV)
    announce("forward decode_128k_fp8_mla")
    idx, out, lse, kc, ks, kv = _run(dsa, wl, inp)
    assert out.dtype == torch.bfloat16
    rows = list(range(wl.rows))
    _check(orc, wl, _oracle_inputs(inp, wl, rows), rows, idx.cpu(), out.cpu(), lse.cpu(),
           gpu_k_codes=kc.cpu().numpy(), gpu_kv_rows=kv.cpu().numpy())


def test_forward_fp8_mla_ragged_and_chunked(dsa, orc):
    """fp8 MLA through dsa_forward with ragged lengths (the last sequence is as short as
    its queries), every row checked; the smallest workspace (query chunks) gives the
    one-pass selection and outputs within the bf16 tolerance."""
    wl = get("decode_128k_fp8_mla").replace(batch=3, n_q=4, max_kv=3000, kv_len=3000)
    lens = [3000, 700, 4]
    inp = make_inputs(wl, device=DEV, kv_len=lens)
    announce("forward fp8 mla ragged")
    idx, out, lse, _, _, _ = _run(dsa, wl, inp)
    rows = list(range(wl.rows))
    _check(orc, wl, _oracle_inputs(inp, wl, rows), rows, idx.cpu(), out.cpu(), lse.cpu())
    small = dsa.forward_min_workspace_size(dsa.DsaShape.of(wl))
    idx2, out2, lse2, _, _, _ = _run(dsa, wl, inp, workspace_bytes=small)
    assert torch.equal(idx, idx2)
    d = (out.float() - out2.float()).abs().max().item()
    assert d <= 2e-2 * out.float().abs().max().item()
    assert torch.allclose(lse, lse2, rtol=1e-4, atol=1e-4)


def test_forward_is_deterministic_and_stateless(dsa):
    wl = get("decode_32k").replace(batch=8, max_kv=8192, kv_len=8192)
    a = make_inputs(wl, device=DEV, seed=1)
    b = make_inputs(wl, device=DEV, seed=2)
    ra = _run(dsa, wl, a)[:3]
    rb = _run(dsa, wl, b)[:3]
    ra2 = _run(dsa, wl, a)[:3]
    rb2 = _run(dsa, wl, b)[:3]
    for x, y in zip(ra + rb, ra2 + rb2):
        assert torch.equal(x, y)
    assert not torch.equal(ra[1], rb[1])


DECODE_SELECTION_CASES = [
    # idx dtype, B, T, Lmax, lens, K, chunked workspace, keys
    ("bf16", 6, 1, 32768, [32768, 30000, 5000, 1, 0, 20000], 2048, False, "gauss"),
    ("bf16", 4, 2, 20000, [20000, 15000, 3, 2], 512, False, "gauss"),
    ("bf16", 3, 2, 16384, [16384, 9000, 2], 1024, True, "gauss"),
    ("fp8", 4, 1, 40000, [40000, 1000, 39000, 7], 2048, False, "gauss"),
    ("fp8", 3, 2, 16384, [16384, 9000, 2], 1024, True, "gauss"),
    # every key of a sequence the same: one threshold bin holds the whole row
    ("bf16", 2, 1, 12000, [12000, 5000], 2048, False, "equal"),
    # a narrow band of scores: many keys in the threshold bin
    ("bf16", 2, 1, 32768, [32768, 25000], 2048, False, "band"),
]


@pytest.mark.parametrize("case", DECODE_SELECTION_CASES)
def test_forward_decode_selection_equals_stage_path(dsa, case):
    """At decode shapes dsa_forward builds the split top-k's row histograms inside the
    indexer launch (the counters cleared by the fp8 query preparation or a fill launch);
    its selection must equal dsa_index_scores followed by dsa_topk bit for bit, for
    ragged, empty and shorter-than-K sequences, one or two queries per sequence, and a
    workspace small enough to run the queries one at a time."""
    dt, B, T, Lmax, lens, K, chunked, keys = case
    announce(f"forward decode selection == index_scores + topk {case}")
    H, D, heads, dqk, dv = 64, 128, 16, 192, 128
    s = dsa.DsaShape(batch=B, n_q=T, max_kv=Lmax, idx_heads=H, idx_dim=D, topk=K, heads=heads, qk_dim=dqk,
                     v_dim=dv, sm_scale=dqk ** -0.5, idx_dtype=dt, mla_dtype="bf16")
    g = torch.Generator().manual_seed(11 * Lmax + T)
    q_idx = torch.randn(B, T, H, D, generator=g).to(DEV, torch.bfloat16)
    k_idx = torch.randn(B, Lmax, D, generator=g)
    if keys == "equal":
        k_idx = k_idx[:, :1].expand(B, Lmax, D).contiguous()
    elif keys == "band":
        k_idx = k_idx[:, :1] + 1e-3 * k_idx
    k_idx = k_idx.to(DEV, torch.bfloat16)
    w = torch.randn(B, T, H, generator=g).to(DEV)
    q = (torch.randn(B, T, heads, dqk, generator=g) * dqk ** -0.5).to(DEV, torch.bfloat16)
    kv = (torch.randn(B, Lmax, dqk, generator=g) * dqk ** -0.5).to(DEV, torch.bfloat16)
    kl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    if dt == "fp8":
        kc, ks = dsa.rotate_quant_fp8(k_idx)
        qc, qs = dsa.rotate_quant_fp8(q_idx)
        scores = dsa.index_scores(s, qc, w, kc, kl, q_scale=qs, k_scale=ks)
        k_fwd, ks_fwd = kc, ks
    else:
        scores = dsa.index_scores(s, q_idx, w, k_idx, kl)
        k_fwd, ks_fwd = k_idx, None
    ref = dsa.topk(s, scores, kl)
    ws = None
    if chunked:
        ws = torch.empty(dsa.forward_min_workspace_size(s), dtype=torch.uint8, device=DEV)
    for _ in range(2):  # a second call on the same workspace starts from what the first left there
        idx, _, _ = dsa.forward(s, q_idx, w, k_fwd, q, kv, kl, k_scale=ks_fwd, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(idx, ref)


def test_forward_ragged_lengths(dsa, orc):
    wl = get("decode_32k").replace(batch=4, n_q=3, max_kv=5000, kv_len=5000)
    lens = [5000, 2049, 1000, 3]
    inp = make_inputs(wl, device=DEV, kv_len=lens)
    idx, out, lse, _, _, _ = _run(dsa, wl, inp)
    rows = list(range(wl.rows))
    _check(orc, wl, _oracle_inputs(inp, wl, rows), rows, idx.cpu(), out.cpu(), lse.cpu())


@pytest.mark.parametrize("name", ["decode_32k", "decode_128k_fp8", "decode_128k_fp8_mla", "prefill_4k"])
def test_forward_graph_replay_matches_eager(dsa, name):
    """dsa_forward captured in a HIP graph (as a serving loop would replay it) gives the
    eager result on every replay, with eager work and synchronisation between replays."""
    wl = get(name)
    if wl.batch > 16:
        wl = wl.replace(batch=16)
    inp = make_inputs(wl, device=DEV)
    s = dsa.DsaShape.of(wl)
    k_idx, k_scale, kv = _prepare(dsa, wl, inp)
    B, T = wl.batch, wl.n_q
    idx = torch.empty((B, T, wl.topk), dtype=torch.int32, device=DEV)
    out = torch.empty((B, T, wl.heads, wl.v_dim), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, T, wl.heads), dtype=torch.float32, device=DEV)
    ws = torch.empty((dsa.forward_workspace_size(s),), dtype=torch.uint8, device=DEV)

    def step():
        dsa.forward(s, inp["q_idx"], inp["w"], k_idx, inp["q"], kv, inp["kv_len"], k_scale=k_scale,
                    idx_out=idx, out=out, lse=lse, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = (idx.clone(), out.clone(), lse.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm the capture stream
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        idx.fill_(-7)
        out.zero_()
        lse.zero_()
        ws.fill_(0xAB)  # scratch holds garbage between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref[0]), f"replay {rep}: idx"
        assert torch.equal(out, ref[1]), f"replay {rep}: out"
        assert torch.equal(lse, ref[2]), f"replay {rep}: lse"


def test_forward_largest_cache_and_topk(dsa, orc):
    """The largest supported shape: a 2^20-key cache and index_topk = 4096 (top-k over
    256 chunks, positions that need all 20 bits, 16-way split MLA)."""
    wl = get("decode_32k").replace(batch=1, max_kv=1 << 20, kv_len=1 << 20, topk=4096)
    inp = make_inputs(wl, device=DEV)
    announce("largest cache: 1 x 2^20 keys, K = 4096")
    idx, out, lse, _, _, _ = _run(dsa, wl, inp)
    assert int(idx.max()) >= 1 << 19  # positions that need the top position bit are selected
    _check(orc, wl, _oracle_inputs(inp, wl, [0]), [0], idx.cpu(), out.cpu(), lse.cpu())
