"""Seeded synthetic inputs (no arithmetic of the method lives here).

Tensor k of sequence b is drawn from its own generator seeded with
1_000_003 * k + b + seed, in float32, then cast once to the workload dtype; the
oracle and the device consume the same cast values.  Tensor numbers:
0 q_idx, 1 w, 2 k_idx, 3 q, 4 kv, 5 heavy-hitter positions, 6 per-token
lognormal factors.

Distributions: q_idx, k_idx ~ N(0,1)/sqrt(idx_dim); w ~ N(0,1)/sqrt(idx_heads);
q, kv ~ N(0,1)/sqrt(qk_dim).  Optional structure: a share ``heavy_frac`` of the
key positions (drawn without replacement) has both its index-key row and its kv
row multiplied by 4; with ``lognormal_sigma`` every token row of q_idx, k_idx,
q and kv is multiplied by exp(sigma * z_pos), one z per position (a query
uses the factor of its own position kv_len - T + t).

With an fp8 indexer, q_idx and k_idx are still returned in bf16, before any
rotation; with an fp8 MLA, q and kv are returned in bf16 as well: the
quantisation belongs to the method.
"""
from __future__ import annotations

import torch

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _gen(device, k: int, b: int, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(1_000_003 * k + b + seed)
    return g


def _randn(shape, g, device, scale):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * scale


def make_inputs(wl, device="cpu", seqs=None, kv_len=None, seed=None, with_mla=True) -> dict:
    """Inputs of workload ``wl`` for sequences ``seqs`` (default: all).

    Returns q_idx [b,T,H_I,D_I], w [b,T,H_I] f32, k_idx [b,Lmax,D_I], q [b,T,H,Dqk],
    kv [b,Lmax,Dqk], kv_len [b] int32, on ``device``.  ``kv_len`` may override the
    per-sequence context lengths (a list, one per selected sequence).
    """
    seed = wl.seed if seed is None else seed
    seqs = list(range(wl.batch)) if seqs is None else list(seqs)
    idt = _DT["bf16" if wl.idx_dtype == "fp8" else wl.idx_dtype]
    mdt = _DT["bf16" if wl.mla_dtype == "fp8" else wl.mla_dtype]
    T, Lmax = wl.n_q, wl.max_kv
    lens = [wl.kv_len] * len(seqs) if kv_len is None else list(kv_len)
    out = {k: [] for k in ("q_idx", "w", "k_idx", "q", "kv")}
    for b, L in zip(seqs, lens):
        assert T <= L <= Lmax
        q_idx = _randn((T, wl.idx_heads, wl.idx_dim), _gen(device, 0, b, seed), device, wl.idx_dim ** -0.5)
        w = _randn((T, wl.idx_heads), _gen(device, 1, b, seed), device, wl.idx_heads ** -0.5)
        k_idx = _randn((Lmax, wl.idx_dim), _gen(device, 2, b, seed), device, wl.idx_dim ** -0.5)
        if with_mla:
            q = _randn((T, wl.heads, wl.qk_dim), _gen(device, 3, b, seed), device, wl.qk_dim ** -0.5)
            kv = _randn((Lmax, wl.qk_dim), _gen(device, 4, b, seed), device, wl.qk_dim ** -0.5)
        if wl.heavy_frac > 0:
            n_heavy = int(round(wl.heavy_frac * L))
            pos = torch.randperm(L, generator=_gen(device, 5, b, seed), device=device)[:n_heavy]
            k_idx[pos] *= 4.0
            if with_mla:
                kv[pos] *= 4.0
        if wl.lognormal_sigma > 0:
            z = torch.randn((Lmax,), generator=_gen(device, 6, b, seed), device=device)
            f = torch.exp(wl.lognormal_sigma * z)
            qpos = torch.arange(L - T, L, device=device)
            k_idx *= f[:, None]
            q_idx *= f[qpos][:, None, None]
            if with_mla:
                kv *= f[:, None]
                q *= f[qpos][:, None, None]
        out["q_idx"].append(q_idx.to(idt))
        out["w"].append(w)
        out["k_idx"].append(k_idx.to(idt))
        if with_mla:
            out["q"].append(q.to(mdt))
            out["kv"].append(kv.to(mdt))
    res = {k: torch.stack(v) for k, v in out.items() if v}
    res["kv_len"] = torch.tensor(lens, dtype=torch.int32, device=device)
    return res


def make_scores(n_rows: int, Lmax: int, device="cpu", seed: int = 0, kind: str = "gauss") -> torch.Tensor:
    """Synthetic index-score rows for exercising top-k alone.

    kind: "gauss" (continuous), "ties" (a few distinct values, many exact ties),
    "int" (small integers), "const" (every entry equal), "signed_zero" (zeros of
    both signs among negatives and positives), "narrow" (1 + j/65536 for
    j < 4096: values that share sign, exponent and leading mantissa bits, with
    ties).
    """
    g = _gen(device, 7, 0, seed)
    if kind == "gauss":
        return torch.randn((n_rows, Lmax), generator=g, device=device)
    if kind == "ties":
        return torch.randint(0, 7, (n_rows, Lmax), generator=g, device=device).float() * 0.25
    if kind == "int":
        return torch.randint(-50, 50, (n_rows, Lmax), generator=g, device=device).float()
    if kind == "const":
        return torch.full((n_rows, Lmax), 1.5, device=device)
    if kind == "signed_zero":
        x = torch.randint(-2, 3, (n_rows, Lmax), generator=g, device=device).float()
        neg0 = torch.randint(0, 2, (n_rows, Lmax), generator=g, device=device).bool() & (x == 0)
        x[neg0] = -0.0
        return x
    if kind == "narrow":
        j = torch.randint(0, 4096, (n_rows, Lmax), generator=g, device=device).float()
        return 1.0 + j / 65536.0
    raise ValueError(kind)
