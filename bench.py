"""DSA forward throughput on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload decode_32k|prefill_32k|decode_128k_fp8|...] [--single]
    python bench.py --sweep-context     (stage times of bf16 decode, batch 16, context 4K..128K)
    python bench.py --mfma-ceiling      (sustained bf16 MFMA rate, constant and random operands;
                                         streaming-read bandwidth)

A step is one dsa_forward call (fp8 workloads: q rotation + quantisation,
index scores, top-k, sparse MLA) over one batch of synthetic inputs already
resident in HBM.  Decode workloads rotate over three independent input sets
so that consecutive steps cannot be served from the 256 MB Infinity Cache.
After the timed forward loop, each stage entry point (same launch
configurations) is timed as back-to-back launches between two HIP events on
the launch stream; the dominant stage is reported against its roofline (every
stage's fraction of its own roofline in "stages_frac"), with the HBM traffic of
its kernel taken from a committed rocprofv3 counter summary under profiles/
while the kernel source still matches it.  FP8 workloads build the index-key
cache through the cache-append entry point and report that kernel's bandwidth
("cache_append"), outside the timed step.  BF16 workloads also time the sparse
MLA backward (dq and dkv for the forward's lse and a random output gradient)
and report it against its own roofline ("mla_bwd"), outside the timed step.
Prefill workloads also time the streaming indexer -> top-k entry point, which
keeps per-row candidate lists instead of the score matrix ("index_topk_stream").
The CPU oracle is timed on a bounded sample of the same workload on the host
cores, and on one thread over a smaller sample (CPU model named).

The default run measures the three points of the metric in one process:
decode_32k (the line's value), prefill_32k and decode_128k_fp8, each with its
own roofline, stage fractions and oracle timing under "points".  It ends by
measuring this GPU's own ceilings ("box_ceilings": a streaming read and the
sustained bf16 MFMA rate from mfma_ceiling.hip, and the vendor GEMM rate for
context), and each roofline adds "frac_of_box", the achieved rate over the ceiling
of its kind, beside "frac" against the published peak.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DSA fwd queries/sec at L=32K/128K + % of MFMA peak / HBM GB/s"
PEAK_HBM_GBS = 8000.0
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}
DEFAULT_STEPS = {"decode_32k": 100, "decode_128k_fp8": 100, "decode_128k_fp8_mla": 100, "prefill_32k": 10,
                 "prefill_4k": 50, "tiny_f32": 100}


def algorithmic(wl) -> dict:
    """Work the method must do per forward, stage by stage (masked work not counted)."""
    B, T, L, K = wl.batch, wl.n_q, wl.kv_len, wl.topk
    HI, DI, H, Dqk, Dv = wl.idx_heads, wl.idx_dim, wl.heads, wl.qk_dim, wl.v_dim
    ib = 1 if wl.idx_dtype == "fp8" else (4 if wl.idx_dtype == "f32" else 2)
    mb = 4 if wl.mla_dtype == "f32" else 2   # q and out element bytes (bf16 for the fp8 MLA)
    row = Dqk * mb if wl.mla_dtype != "fp8" else Dqk + 4  # a gathered latent row (fp8: codes + scale)
    pairs = 0      # causal (query, key) pairs scored
    sel = 0        # selected (query, key) pairs attended
    for t in range(T):
        n = L - T + t + 1
        pairs += n
        sel += min(K, n)
    pairs *= B
    sel *= B
    key_bytes = B * L * DI * ib + (B * L * 4 if wl.idx_dtype == "fp8" else 0)
    idx_flops = 2.0 * pairs * HI * DI
    idx_bytes = key_bytes + B * T * HI * (DI * ib + 4 + (4 if wl.idx_dtype == "fp8" else 0)) + pairs * 4
    topk_bytes = pairs * 4 + B * T * K * 4
    mla_flops = 2.0 * sel * H * (Dqk + Dv)
    gather = sel * row if T == 1 else B * L * row  # prefill rows come from L2 after first touch
    mla_bytes = gather + B * T * H * (Dqk * mb + Dv * mb + 4) + sel * 4
    return dict(indexer=dict(flops=idx_flops, bytes=idx_bytes), topk=dict(flops=0.0, bytes=topk_bytes),
                mla=dict(flops=mla_flops, bytes=mla_bytes))


def mfma_peak(wl, stage: str) -> float:
    """Dense MFMA peak (TFLOP/s) of a stage.  The fp8 MLA runs q.k on fp8 MFMA and the
    value sum on bf16 MFMA: its peak is the rate that does both shares in the time
    they take at their own peaks."""
    if stage == "indexer":
        return PEAK_TFLOPS.get(wl.idx_dtype, PEAK_TFLOPS["bf16"])
    if wl.mla_dtype == "fp8":
        qk, pv = wl.qk_dim, wl.v_dim
        return (qk + pv) / (qk / PEAK_TFLOPS["fp8"] + pv / PEAK_TFLOPS["bf16"])
    return PEAK_TFLOPS.get(wl.mla_dtype, PEAK_TFLOPS["bf16"])


def dominant(wl, stage_us: dict) -> tuple[str, dict]:
    """The longest stage and its roofline object."""
    alg = algorithmic(wl)
    name = max(("indexer", "topk", "mla"), key=lambda k: stage_us.get(k, 0.0))
    us = stage_us[name]
    a = alg[name]
    ai = a["flops"] / max(a["bytes"], 1.0)
    peak = mfma_peak(wl, name)
    ridge = peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    if name != "topk" and ai > ridge:
        achieved = a["flops"] / (us * 1e-6) / 1e12
        return name, {"kernel": stage_kernel(wl, name), "bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                      "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": recorded_traffic(wl, name),
                      "work_per_launch": a["flops"], "avg_launch_us": round(us, 2)}
    achieved = a["bytes"] / (us * 1e-6) / 1e9
    return name, {"kernel": stage_kernel(wl, name), "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                  "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": recorded_traffic(wl, name),
                  "work_per_launch": a["bytes"], "avg_launch_us": round(us, 2)}


def stage_kernel(wl, stage: str) -> str:
    return mla_kernels(wl) if stage == "mla" else STAGE_KERNELS[stage]


def stage_fractions(wl, stage_us: dict) -> dict:
    """Each stage's algorithmic work over its duration, as a fraction of the roofline
    that bounds it (MFMA when its arithmetic intensity is above the ridge, else HBM)."""
    alg = algorithmic(wl)
    out = {}
    for name, us in stage_us.items():
        a = alg[name]
        peak_f = mfma_peak(wl, name)
        ridge = peak_f * 1e12 / (PEAK_HBM_GBS * 1e9)
        if name != "topk" and a["flops"] / max(a["bytes"], 1.0) > ridge:
            out[name] = {"bound": "mfma", "frac": round(a["flops"] / (us * 1e-6) / 1e12 / peak_f, 4)}
        else:
            out[name] = {"bound": "hbm", "frac": round(a["bytes"] / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    return out


class Case:
    """Device inputs, outputs and workspace of one workload."""

    def __init__(self, dsa, wl, seed, torch):
        from workloads import make_inputs
        self.wl = wl
        self.shape = dsa.DsaShape.of(wl)
        inp = make_inputs(wl, device="cuda", seed=seed)
        self.inp = inp
        self.k_idx, self.k_scale = inp["k_idx"], None
        self.append_us = None
        if wl.idx_dtype == "fp8":
            # the fp8 index-key cache, built through the cache-append entry point
            # (every row of every sequence appended at once), timed here
            k_new = inp["k_idx"]
            codes = torch.empty(k_new.shape, dtype=torch.uint8, device="cuda")
            scales = torch.empty(k_new.shape[:2], dtype=torch.float32, device="cuda")
            full = torch.full((wl.batch,), wl.max_kv, dtype=torch.int32, device="cuda")
            dsa.index_cache_append_fp8(k_new, full, codes, scales)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 3
            e0.record()
            for _ in range(reps):
                dsa.index_cache_append_fp8(k_new, full, codes, scales)
            e1.record()
            torch.cuda.synchronize()
            self.append_us = e0.elapsed_time(e1) * 1000.0 / reps
            self.k_idx, self.k_scale = codes, scales
            del inp["k_idx"], k_new
            q_codes, q_scale = dsa.rotate_quant_fp8(inp["q_idx"])
            self.q_codes, self.q_scale = q_codes, q_scale
        self.kv_quant_us = None
        if wl.mla_dtype == "fp8":
            # the fp8 latent cache [B, L_max, D_qk + 16], quantised by the library, timed here
            kv = inp["kv"]
            rows = dsa.mla_kv_quant_fp8(kv)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 3
            e0.record()
            for _ in range(reps):
                dsa.mla_kv_quant_fp8(kv, kv_rows=rows)
            e1.record()
            torch.cuda.synchronize()
            self.kv_quant_us = e0.elapsed_time(e1) * 1000.0 / reps
            inp["kv"] = rows
            del kv
        dev = "cuda"
        B, T = wl.batch, wl.n_q
        self.idx = torch.empty((B, T, wl.topk), dtype=torch.int32, device=dev)
        mdt = torch.float32 if wl.mla_dtype == "f32" else torch.bfloat16  # bf16 for the fp8 MLA too
        self.out = torch.empty((B, T, wl.heads, wl.v_dim), dtype=mdt, device=dev)
        self.lse = torch.empty((B, T, wl.heads), dtype=torch.float32, device=dev)
        self.ws = torch.empty((dsa.forward_workspace_size(self.shape),), dtype=torch.uint8, device=dev)
        self.scores = None

    def forward(self, dsa):
        i = self.inp
        dsa.forward(self.shape, i["q_idx"], i["w"], self.k_idx, i["q"], i["kv"], i["kv_len"], k_scale=self.k_scale,
                    idx_out=self.idx, out=self.out, lse=self.lse, workspace=self.ws)


def capture_graphs(dsa, torch, cases):
    """One HIP graph per input set holding that set's whole dsa_forward call (the
    library's launches go to the capturing stream); None if capture fails."""
    try:
        graphs = []
        for c in cases:
            c.forward(dsa)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                c.forward(dsa)
            graphs.append(g)
        torch.cuda.synchronize()
        return graphs
    except Exception as e:  # noqa: BLE001 -- fall back to eager launches, say so in the output
        print(f"graph capture failed, timing eager launches: {e}", file=sys.stderr)
        return None


def time_forward(dsa, torch, cases, steps, warmup, graphs=None):
    """Average step time over `steps` steps (rotating the input sets) between two HIP
    events on the launch stream; with graphs, each step replays its set's graph."""
    stream = torch.cuda.current_stream()
    step = (lambda s: graphs[s % len(graphs)].replay()) if graphs else (lambda s: cases[s % len(cases)].forward(dsa))
    for s in range(warmup):
        step(s)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    t0 = time.perf_counter()
    for s in range(steps):
        step(s)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall


STAGE_KERNELS = {"indexer": "indexer", "topk": "topk (zero, hist, filter, finish) or topk_kernel"}


def mla_kernels(wl) -> str:
    """The kernels dsa_sparse_mla_fwd launches for this shape: the library splits the index
    list until about 256 workgroups exist (at most K/128 and 16 splits) and takes the
    one-wave-per-SIMD kernels when a split's list has 8 or more 32-key tiles."""
    units = wl.batch * wl.n_q * ((wl.heads + 127) // 128)
    ns = max(1, min(-(-256 // units), max(wl.topk // 128, 1), 16))
    wide = -(-(-(-wl.topk // ns)) // 32) >= 8
    if wl.mla_dtype == "fp8":
        name = "quant_rows_kernel (q) + " + ("mla_fp8w_kernel" if wide else "mla_fp8_kernel")
    elif wl.mla_dtype == "f32":
        name = "mla_f32_kernel"
    else:
        name = "mla_wide_kernel" if wide and wl.qk_dim == 576 else "mla_bf16_kernel"
    return name + (" + mla_combine_kernel" if ns > 1 else "")


def time_stages(dsa, torch, cases, reps):
    """Average duration of each stage entry point, measured as `reps` back-to-back
    launches (alternating input sets) between two HIP events on the launch stream."""
    stream = torch.cuda.current_stream()
    wl = cases[0].wl
    sh = cases[0].shape
    B, T, Lmax = wl.batch, wl.n_q, wl.max_kv
    if wl.n_q > 1 and B * T * Lmax * 4 > (6 << 30):
        return None  # the stage API writes the whole masked score matrix; skip huge prefill shapes
    for c in cases:
        if c.scores is None:
            c.scores = torch.empty((B, T, Lmax), dtype=torch.float32, device="cuda")
        c.mla_ws = torch.empty((max(dsa.sparse_mla_workspace_size(sh), 1),), dtype=torch.uint8, device="cuda")
        c.topk_ws = torch.empty((max(dsa.topk_workspace_size(sh), 1),), dtype=torch.uint8, device="cuda")

    def indexer(c):
        i = c.inp
        qi = c.q_codes if wl.idx_dtype == "fp8" else i["q_idx"]
        dsa.index_scores(sh, qi, i["w"], c.k_idx, i["kv_len"], q_scale=getattr(c, "q_scale", None),
                         k_scale=c.k_scale, scores=c.scores)

    def topk(c):
        dsa.topk(sh, c.scores, c.inp["kv_len"], idx=c.idx, workspace=c.topk_ws)

    def mla(c):
        i = c.inp
        dsa.sparse_mla_fwd(sh, i["q"], i["kv"], c.idx, i["kv_len"], out=c.out, lse=c.lse, workspace=c.mla_ws)

    stages = {"indexer": indexer, "topk": topk, "mla": mla}
    for c in cases:  # every stage reads what the previous one wrote for the same case
        for f in stages.values():
            f(c)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    res = {}
    for name, f in stages.items():
        f(cases[0])
        e0.record(stream)
        for r in range(reps):
            f(cases[r % len(cases)])
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) * 1000.0 / reps
    return res


def bwd_algorithmic(wl) -> dict:
    """Work of one sparse MLA backward: five contractions per selected (query, key)
    pair and head (logits, dP, dq, dk, dv); HBM bytes for the gathered rows, q, dO,
    lse and dq once, and one fp32 update of every touched dkv row element (prefill
    rows: once per cache row, as the forward counts its gather)."""
    B, T, L, K, H, Dqk, Dv = wl.batch, wl.n_q, wl.kv_len, wl.topk, wl.heads, wl.qk_dim, wl.v_dim
    sel = B * sum(min(K, L - T + t + 1) for t in range(T))
    flops = 2.0 * sel * H * (3 * Dqk + 2 * Dv)
    rows = sel if T == 1 else B * L
    nbytes = rows * Dqk * 2 + B * T * H * (Dqk * 2 + Dv * 2 + 4 + Dqk * 4) + rows * Dqk * 4
    return {"flops": flops, "bytes": nbytes, "pairs": sel}


BWD_WS_CAP = 8 << 30  # workspace bound for the backward timing: longer query sets run in chunks


def time_mla_bwd(dsa, torch, case, reps):
    """Average duration of dsa_sparse_mla_bwd (every launch of one call) over `reps`
    back-to-back calls between two HIP events on the launch stream, with the roofline
    of the whole call; None for shapes the backward does not take.  The calls add
    into dkv (accumulate_dkv, as gradient accumulation does); one call that clears
    the dense dkv [B, L_max, D_qk] f32 first is timed on its own ("with_clear_us")."""
    wl, sh = case.wl, case.shape
    if wl.mla_dtype != "bf16" or (wl.qk_dim, wl.v_dim) not in ((576, 512), (192, 128)) or wl.heads > 128:
        return None
    B, T, H = wl.batch, wl.n_q, wl.heads
    g = torch.Generator(device="cuda").manual_seed(1234)
    dout = torch.randn((B, T, H, wl.v_dim), generator=g, device="cuda").to(torch.bfloat16)
    dq = torch.empty((B, T, H, wl.qk_dim), dtype=torch.float32, device="cuda")
    dkv = torch.empty((B, wl.max_kv, wl.qk_dim), dtype=torch.float32, device="cuda")
    ws = torch.empty((min(dsa.sparse_mla_bwd_workspace_size(sh), BWD_WS_CAP),), dtype=torch.uint8, device="cuda")
    i = case.inp

    def call(acc=True):
        dsa.sparse_mla_bwd(sh, i["q"], i["kv"], case.idx, i["kv_len"], case.lse, dout, dq=dq, dkv=dkv,
                           accumulate_dkv=acc, workspace=ws)

    call(False)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    call(False)
    e1.record(stream)
    torch.cuda.synchronize()
    clear_us = e0.elapsed_time(e1) * 1000.0
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / reps
    alg = bwd_algorithmic(wl)
    peak = PEAK_TFLOPS["bf16"]
    tflops = alg["flops"] / (us * 1e-6) / 1e12
    gbs = alg["bytes"] / (us * 1e-6) / 1e9
    ridge = peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    mfma = alg["flops"] / alg["bytes"] > ridge
    return {"kernels": "bwd_prep + bwd_scores + bwd_dq + bwd_dkv per query chunk",
            "avg_call_us": round(us, 2), "with_clear_us": round(clear_us, 2),
            "pairs_per_s": round(alg["pairs"] / (us * 1e-6), 1),
            "bound": "mfma" if mfma else "hbm", "achieved": round(tflops if mfma else gbs, 2 if mfma else 1),
            "peak": peak if mfma else PEAK_HBM_GBS, "unit": "TFLOP/s" if mfma else "GB/s",
            "frac": round((tflops / peak) if mfma else (gbs / PEAK_HBM_GBS), 4),
            "tflops": round(tflops, 2), "gbs": round(gbs, 1), "flops_per_call": alg["flops"],
            "bytes_per_call": alg["bytes"], "workspace_bytes": ws.numel(), "reps": reps}


def time_index_topk(dsa, torch, case, reps):
    """Average duration of dsa_index_topk (indexer scores and top-k in one pass, no
    score matrix) on the case's inputs, and whether it selects what the forward did."""
    wl, sh, i = case.wl, case.shape, case.inp
    qi = case.q_codes if wl.idx_dtype == "fp8" else i["q_idx"]
    qs = getattr(case, "q_scale", None)
    ws = torch.empty((dsa.index_topk_workspace_size(sh),), dtype=torch.uint8, device="cuda")
    idx = torch.empty_like(case.idx)

    def call():
        dsa.index_topk(sh, qi, i["w"], case.k_idx, i["kv_len"], q_scale=qs, k_scale=case.k_scale, idx=idx,
                       workspace=ws)

    call()
    torch.cuda.synchronize()
    same = bool(torch.equal(idx, case.idx))
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / reps
    flops = algorithmic(wl)["indexer"]["flops"]
    tf = flops / (us * 1e-6) / 1e12
    peak = mfma_peak(wl, "indexer")
    return {"kernel": "indexer_prefill_kernel (streaming top-k)", "avg_call_us": round(us, 2),
            "bound": "mfma", "achieved": round(tf, 2), "peak": peak, "unit": "TFLOP/s", "frac": round(tf / peak, 4),
            "workspace_bytes": ws.numel(), "score_matrix_bytes": wl.batch * wl.n_q * wl.max_kv * 4,
            "same_selection_as_forward": same, "reps": reps}


def recorded_traffic(wl, stage: str):
    """HBM bytes per launch of a stage's kernel from a committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, calibrated against a plain copy); None when
    no summary covers this workload or the kernel source has changed since."""
    import glob
    import hashlib
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for line in open(path):
            if not line.startswith("bench-traffic:"):
                continue
            kv = dict(x.split("=", 1) for x in line.split()[1:])
            if kv.get("workload") != wl.name or kv.get("stage") != stage:
                continue
            h = hashlib.sha256()
            for rel in kv["source"].split(","):  # the kernel source and the build script (compile flags)
                src = os.path.join(ROOT, rel)
                if not os.path.exists(src):
                    return None
                h.update(open(src, "rb").read())
            if h.hexdigest() != kv["sha256"]:
                return None
            return int(kv["fetch_bytes"]) + int(kv["write_bytes"])
    return None


CPU_BUDGET_S = 10.0  # oracle work to time, at least (one pass is always completed)
CPU_BUDGET_1T_S = 3.0  # single-thread oracle work to time, at least


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, budget_s: float = CPU_BUDGET_S) -> dict:
    """The oracle, as it stands, on a bounded sample of the workload: on all host
    threads (the reported value), then on one thread over a smaller sample."""
    import numpy as np

    import oracle
    from workloads import make_inputs
    oracle.build()
    threads = oracle.num_threads()
    inp = make_inputs(wl)

    def decode_sample(n_seq, budget):
        # the first n_seq sequences only (the oracle quantises the key caches it is given)
        sub = {k: v[:n_seq] for k, v in inp.items()}
        wsub = wl.replace(batch=n_seq)
        rows = list(range(n_seq))
        passes, dt = 0, 0.0
        while dt < budget and dt < 3 * budget:
            t0 = time.perf_counter()
            oracle.forward(sub, wsub, rows=rows)
            dt += time.perf_counter() - t0
            passes += 1
        return passes * n_seq, dt, passes

    def prefill_sample(n, budget, grow):
        rng = np.random.default_rng(0)
        while True:
            rows = sorted(rng.choice(wl.rows, size=n, replace=False).tolist())
            flat = lambda t: t.reshape(wl.rows, *t.shape[2:])[rows]
            cin = dict(inp, q_idx=flat(inp["q_idx"]), w=flat(inp["w"]), q=flat(inp["q"]))
            t0 = time.perf_counter()
            oracle.forward(cin, wl, rows=rows, compact=True)
            dt = time.perf_counter() - t0
            if not grow or dt >= budget or n >= wl.rows or dt * 2 > 3 * budget:
                return n, dt
            n = min(wl.rows, int(n * max(2.0, min(8.0, budget / max(dt, 1e-3)))))

    if wl.n_q == 1:
        # every sequence of the batch, in repeated passes until the budget is spent
        n, dt, passes = decode_sample(wl.batch, budget_s)
        sample = f"all {wl.batch} sequences (one decode query each, {wl.kv_len}-token context), {passes} passes"
        if wl.idx_dtype == "fp8":
            sample += "; the oracle rotates and quantises the whole index-key cache in every pass"
        used = min(threads, wl.batch)
    else:
        # uniformly drawn query rows, the count raised until one run fills the budget
        n, dt = prefill_sample(min(wl.rows, max(2, threads)), budget_s, True)
        sample = f"{n} uniformly drawn query rows of {wl.rows}"
        used = min(threads, n)
    res = {"value": round(n / dt, 3), "unit": "queries/s", "cores": used, "kind": "oracle", "sample": sample,
           "seconds": round(dt, 2), "cpu_model": cpu_model(), "host_threads": threads}
    # one thread: two sequences (decode) or a handful of rows (prefill)
    oracle.set_num_threads(1)
    try:
        if wl.n_q == 1:
            n1, dt1, _ = decode_sample(min(2, wl.batch), CPU_BUDGET_1T_S)
            s1 = f"first {min(2, wl.batch)} sequences, repeated passes"
        else:
            n1, dt1 = prefill_sample(2, CPU_BUDGET_1T_S, False)
            s1 = "2 uniformly drawn query rows"
    finally:
        oracle.set_num_threads(threads)
    res["single_thread"] = {"value": round(n1 / dt1, 4), "unit": "queries/s", "seconds": round(dt1, 2),
                            "sample": s1}
    return res


def mfma_ceiling() -> dict:
    """Sustained bf16 MFMA rate of this GPU on constant and on random operands
    (mfma_ceiling.hip beside this file, built with hipcc and run as a child
    process), the context for the MFMA fractions of the published peak."""
    import subprocess
    here = os.path.dirname(os.path.abspath(__file__))
    out_dir = os.path.join(here, "_build")
    os.makedirs(out_dir, exist_ok=True)
    exe = os.path.join(out_dir, "mfma_ceiling")
    cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-mllvm", "-amdgpu-mfma-vgpr-form=1",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-o", exe,
           os.path.join(here, "mfma_ceiling.hip")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for mfma_ceiling.hip:\n" + r.stderr)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    if r.returncode != 0:
        raise RuntimeError("mfma_ceiling failed:\n" + r.stderr)
    return json.loads(r.stdout.strip().splitlines()[-1])


def copy_calibration(nbytes: int, reps: int) -> dict:
    """Plain device-to-device copies of a known size, for calibrating HBM counters."""
    import torch
    src = torch.empty((nbytes,), dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"copy_bytes": nbytes, "reps": reps}


SWEEP_BATCH = 16
SWEEP_CONTEXTS = (4096, 8192, 16384, 32768, 65536, 131072)


def sweep_context(args) -> dict:
    """Per-query cost against context length (the O(L) -> O(index_topk) claim of the
    DSA section, item 2): bf16 decode at a fixed batch of 16 sequences, stage times
    of the indexer (linear in L), top-k and sparse MLA (flat once L >= index_topk)
    for L = 4K .. 128K.  Three input sets per length, as in the decode benchmark."""
    import torch

    import sparse_attention_09_amd as dsa
    from workloads import get

    reps = args.steps or 50
    rows = []
    for L in SWEEP_CONTEXTS:
        wl = get("decode_32k").replace(name=f"decode_b{SWEEP_BATCH}_{L // 1024}k", batch=SWEEP_BATCH, max_kv=L,
                                       kv_len=L)
        cases = [Case(dsa, wl, seed, torch) for seed in range(3)]
        torch.cuda.synchronize()
        ms, _ = time_forward(dsa, torch, cases, reps, args.warmup)
        st = time_stages(dsa, torch, cases, reps)
        rows.append({"context": L, "ms_per_step": round(ms, 4), "stages_us": {k: round(v, 2) for k, v in st.items()},
                     "stages_frac": stage_fractions(wl, st)})
        del cases
        torch.cuda.empty_cache()
    return {"sweep": "decode bf16, fixed batch, context length", "batch": SWEEP_BATCH, "topk": 2048,
            "reps": reps, "rows": rows}


# Metric points reported by one default run: L = 32K decode (the headline value),
# L = 32K prefill and L = 128K decode with the fp8 indexer.
POINTS = ("decode_32k", "prefill_32k", "decode_128k_fp8")


def run_point(args, name: str, with_bwd: bool, cpu_budget: float) -> dict:
    """Time one workload: the forward step, the stages and the extras."""
    import torch

    import sparse_attention_09_amd as dsa
    from workloads import get

    wl = get(name)
    steps = args.steps if args.steps is not None else DEFAULT_STEPS.get(wl.name, 20)
    if wl.n_q > 1:
        steps = min(steps, DEFAULT_STEPS.get(wl.name, steps))
    warmup = args.warmup if wl.n_q == 1 else min(args.warmup, 3)
    n_sets = 3 if wl.n_q == 1 else 1
    cases = [Case(dsa, wl, seed, torch) for seed in range(n_sets)]
    torch.cuda.synchronize()
    graphs = capture_graphs(dsa, torch, cases) if args.graph else None
    ms, wall = time_forward(dsa, torch, cases, steps, warmup, graphs)
    queries = wl.batch * wl.n_q
    res = {
        "value": round(queries / (ms * 1e-3), 1), "ms_per_step": round(ms, 4), "steps": steps, "warmup": warmup,
        "dtype": wl.mla_dtype if "fp8" not in (wl.idx_dtype, wl.mla_dtype) else "fp8+bf16",
        "config": {"workload": wl.name, "batch": wl.batch, "queries_per_seq": wl.n_q, "context": wl.kv_len,
                   "index_heads": wl.idx_heads, "index_dim": wl.idx_dim, "topk": wl.topk, "heads": wl.heads,
                   "qk_dim": wl.qk_dim, "v_dim": wl.v_dim, "idx_dtype": wl.idx_dtype, "mla_dtype": wl.mla_dtype,
                   "input_sets": n_sets},
        "wall_s": round(wall, 4),
        "launch": "hip_graph" if graphs else "eager",
    }
    if not args.no_stages:
        st = time_stages(dsa, torch, cases, max(5, min(steps, 50)))
        if st is not None:
            res["stages_us"] = {k: round(v, 2) for k, v in st.items()}
            _, roof = dominant(wl, st)
            res["roofline"] = roof
            res["stages_frac"] = stage_fractions(wl, st)
    if cases[0].append_us is not None:
        rows = wl.batch * wl.max_kv
        nbytes = rows * wl.idx_dim * (2 + 1) + rows * 4  # bf16 keys in, e4m3 codes + f32 scales out
        gbs = nbytes / (cases[0].append_us * 1e-6) / 1e9
        res["cache_append"] = {"kernel": "rotate_quant_kernel (index-key cache append)", "rows": rows,
                               "avg_launch_us": round(cases[0].append_us, 2), "bound": "hbm",
                               "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                               "frac": round(gbs / PEAK_HBM_GBS, 4), "work_per_launch": nbytes}
    if cases[0].kv_quant_us is not None:
        rows = wl.batch * wl.max_kv
        nbytes = rows * (wl.qk_dim * 2 + wl.qk_dim + 16)  # bf16 rows in, fp8 cache rows out
        gbs = nbytes / (cases[0].kv_quant_us * 1e-6) / 1e9
        res["kv_cache_quant"] = {"kernel": "quant_rows_kernel (fp8 latent cache)", "rows": rows,
                                 "avg_launch_us": round(cases[0].kv_quant_us, 2), "bound": "hbm",
                                 "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                 "frac": round(gbs / PEAK_HBM_GBS, 4), "work_per_launch": nbytes}
    if wl.n_q > 2 and not args.no_stages:
        res["index_topk_stream"] = time_index_topk(dsa, torch, cases[0], max(3, min(steps, 20)))
    if with_bwd and not args.no_bwd:
        bwd = time_mla_bwd(dsa, torch, cases[0], 20 if wl.n_q == 1 else 3)
        if bwd is not None:
            res["mla_bwd"] = bwd
    del cases, graphs
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, cpu_budget)
    return res


def box_ceilings(torch) -> dict:
    """This GPU's own ceilings, measured live beside the published peaks: a plain
    streaming read of 1 GiB and the sustained bf16 MFMA rate on random operands (both
    from mfma_ceiling.hip), and, for context, the bf16 GEMM rate of the vendor library
    (torch.matmul, 8192^3, contiguous operands)."""
    probe = mfma_ceiling()
    n = 8192
    g = torch.Generator(device="cuda").manual_seed(0)
    a = torch.randn(n, n, generator=g, device="cuda").to(torch.bfloat16)
    b = torch.randn(n, n, generator=g, device="cuda").to(torch.bfloat16).contiguous()
    torch.matmul(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    mm_tf = 2 * n ** 3 / (e0.elapsed_time(e1) * 1e-3 / 10) / 1e12
    del a, b
    torch.cuda.empty_cache()
    mf = probe["results"]["32x32x16_random"]
    return {"hbm_read": {"achieved": probe["stream_read"]["GBs"], "unit": "GB/s",
                         "how": "grid-stride 16-byte reads of 1 GiB, best of plain and non-temporal loads "
                                "(mfma_ceiling.hip)"},
            "row_gather": {"achieved": probe["row_gather"]["GBs"], "unit": "GB/s",
                           "how": "random 1152-byte rows, 2048 of 32768 per sequence, 64 sequences, "
                                  "best of register and direct-to-LDS, plain and non-temporal loads (mfma_ceiling.hip)",
                           "cases": probe["row_gather"]["cases"]},
            "bf16_mfma": {"achieved": mf["tflops"], "unit": "TFLOP/s",
                          "how": "back-to-back v_mfma_f32_32x32x16_bf16 on random operands (mfma_ceiling.hip)"},
            "bf16_gemm": {"achieved": round(mm_tf, 1), "unit": "TFLOP/s",
                          "how": "torch.matmul 8192 x 8192 x 8192 bf16 (hipBLASLt), for context"}}


def add_box_fraction(roof: dict, box: dict) -> None:
    """roofline["frac_of_box"]: achieved over this box's own measured ceiling of the same kind."""
    if not roof:
        return
    if roof.get("bound") == "hbm":
        roof["frac_of_box"] = round(roof["achieved"] / box["hbm_read"]["achieved"], 4)
    elif roof.get("bound") == "mfma" and roof.get("peak") == PEAK_TFLOPS["bf16"]:
        roof["frac_of_box"] = round(roof["achieved"] / box["bf16_mfma"]["achieved"], 4)


def add_stage_box_fractions(wl_name: str, fr: dict, box: dict) -> None:
    """stages_frac[...]["frac_of_box"]: each stage's rate over this box's measured ceiling
    of its kind.  The decode sparse MLA reads random latent rows, so its HBM figure is
    held to the measured random-row gather rate rather than to the streaming read."""
    from workloads import get
    if not fr:
        return
    decode = get(wl_name).n_q == 1
    for name, f in fr.items():
        if f["bound"] == "hbm":
            ceil = box["row_gather"] if (name == "mla" and decode) else box["hbm_read"]
            f["frac_of_box"] = round(f["frac"] * PEAK_HBM_GBS / ceil["achieved"], 4)
            if name == "mla" and decode:
                f["box_ceiling"] = "row_gather"
        elif f["bound"] == "mfma" and mfma_peak(get(wl_name), name) == PEAK_TFLOPS["bf16"]:
            f["frac_of_box"] = round(f["frac"] * PEAK_TFLOPS["bf16"] / box["bf16_mfma"]["achieved"], 4)


def run(args) -> dict:
    head = run_point(args, args.workload, True, CPU_BUDGET_S)
    res = {"metric": METRIC, "value": head["value"], "unit": "queries/s", "n_gpus": 1, "steps": head["steps"],
           "warmup": head["warmup"], "ms_per_step": head["ms_per_step"], "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": head["dtype"],
           "data": "synthetic (seeded Gaussian, DeepSeek-V3.2 shapes)"}
    res.update({k: v for k, v in head.items() if k not in res and k not in ("value", "steps", "warmup")})
    if args.points and not args.single:
        # the other L = 32K / 128K points of the metric, each with its own roofline
        pts = {args.workload: {k: head[k] for k in ("value", "ms_per_step", "stages_us", "stages_frac", "roofline")
                               if k in head}}
        for name in POINTS:
            if name == args.workload:
                continue
            p = run_point(args, name, False, CPU_BUDGET_S / 2)
            keep = ("value", "ms_per_step", "steps", "dtype", "config", "stages_us", "stages_frac", "roofline",
                    "cache_append", "index_topk_stream", "cpu_baseline")
            pts[name] = {k: p[k] for k in keep if k in p}
            pts[name]["unit"] = "queries/s"
        res["points"] = pts
    import torch

    box = box_ceilings(torch)
    res["box_ceilings"] = box
    add_box_fraction(res.get("roofline"), box)
    add_stage_box_fractions(args.workload, res.get("stages_frac"), box)
    for name, p in res.get("points", {}).items():
        add_box_fraction(p.get("roofline"), box)
        if name != args.workload:
            add_stage_box_fractions(name, p.get("stages_frac"), box)
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode_32k")
    ap.add_argument("--no-stages", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bwd", action="store_true", help="skip the sparse MLA backward timing")
    ap.add_argument("--graph", action="store_true", help="replay each step from a captured HIP graph")
    ap.add_argument("--single", action="store_true", help="time only --workload, not the other metric points")
    ap.add_argument("--sweep-context", action="store_true",
                    help="only time the stages of bf16 decode at a fixed batch over context lengths 4K..128K")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="only measure the sustained bf16 MFMA rate (constant and random operands)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run plain device copies of BYTES bytes (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    args.points = args.workload in POINTS
    if args.sweep_context:
        print(json.dumps(sweep_context(args)), flush=True)
        return
    if args.mfma_ceiling:
        print(json.dumps(mfma_ceiling()), flush=True)
        return
    if args.copy_calibration:
        print(json.dumps(copy_calibration(args.copy_calibration, args.steps or 3)), flush=True)
        return
    print(json.dumps(run(args)), flush=True)


if __name__ == "__main__":
    main()
