"""CPU oracle for the DeepSeek Sparse Attention forward path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It wraps the plain
fp64 C implementation in ``dsa_oracle.c`` (built with gcc + OpenMP) and shares
no code with the HIP library.

Every function takes numpy arrays or CPU torch tensors holding the exact values
the device receives (bf16 values are widened to float32, which is exact) and
returns numpy arrays.

Method source: the DeepSeek-V3.2 model documentation page, section "DeepSeek
Sparse Attention (DSA)" (lightning indexer; top-index_topk token selection;
MLA over the selected tokens; FP8 indexer behind a Hadamard rotation).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dsa_oracle.c")
_SO = os.path.join(_HERE, "_dsa_oracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile dsa_oracle.c into _dsa_oracle.so with gcc (-O2 -fopenmp)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_SO)
            P = ctypes.c_void_p
            I = ctypes.c_int
            L = ctypes.c_long
            D = ctypes.c_double
            lib.orc_num_threads.restype = I
            lib.orc_set_num_threads.argtypes = [I]
            lib.orc_set_num_threads.restype = None
            lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
            lib.orc_e4m3_decode.restype = D
            lib.orc_e4m3_encode.argtypes = [ctypes.c_float]
            lib.orc_e4m3_encode.restype = ctypes.c_uint8
            lib.orc_e4m3_encode_array.argtypes = [L, P, P]
            lib.orc_e4m3_encode_array.restype = None
            lib.orc_hadamard_matrix.argtypes = [I, P]
            lib.orc_rotate.argtypes = [L, I, P, P]
            lib.orc_rotate_quant.argtypes = [L, I, P, P, P]
            lib.orc_quant.argtypes = [L, I, P, P, P]
            lib.orc_index_scores.argtypes = [I, I, I, I, I, P, P, P, P, L, P, I, P]
            lib.orc_index_scores_fp8.argtypes = [I, I, I, I, I, P, P, P, P, P, P, L, P, I, P]
            lib.orc_topk.argtypes = [I, I, I, I, P, L, P, P, P]
            lib.orc_sparse_mla.argtypes = [I, I, I, I, I, I, I, D, P, P, L, P, I, P, P, P]
            lib.orc_masked_dense_mla.argtypes = [I, I, I, I, I, I, I, D, P, P, P, L, P, I, P, P, P]
            lib.orc_sparse_mla_bwd.argtypes = [I, I, I, I, I, I, I, D, P, P, P, L, P, I, P, P, P]
            for f in ("orc_hadamard_matrix", "orc_rotate", "orc_rotate_quant", "orc_quant", "orc_index_scores",
                      "orc_index_scores_fp8", "orc_topk", "orc_sparse_mla", "orc_masked_dense_mla",
                      "orc_sparse_mla_bwd"):
                getattr(lib, f).restype = None
            _lib = lib
    return _lib


def _f32(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor (CPU)
        x = x.detach().to("cpu").float().numpy()
    return np.ascontiguousarray(x, dtype=np.float32)


def _u8(x) -> np.ndarray:
    if hasattr(x, "detach"):
        import torch
        x = x.detach().to("cpu")
        if x.dtype != torch.uint8:
            x = x.view(torch.uint8)
        x = x.numpy()
    return np.ascontiguousarray(x, dtype=np.uint8)


def _i32(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").numpy()
    return np.ascontiguousarray(x, dtype=np.int32)


def _rows(rows, n_all):
    if rows is None:
        return np.arange(n_all, dtype=np.int64)
    return np.ascontiguousarray(np.asarray(rows, dtype=np.int64))


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(_load().orc_num_threads())


def set_num_threads(n: int) -> None:
    """OpenMP threads of the oracle's following calls (for timing it)."""
    _load().orc_set_num_threads(int(n))


# ---------------------------------------------------------------- fp8 codec
def e4m3_decode(codes) -> np.ndarray:
    lib = _load()
    c = _u8(codes)
    table = np.array([lib.orc_e4m3_decode(i) for i in range(256)], dtype=np.float64)
    return table[c]


def e4m3_encode(y) -> np.ndarray:
    y = _f32(y)
    out = np.empty(y.shape, dtype=np.uint8)
    _load().orc_e4m3_encode_array(y.size, _p(y), _p(out))
    return out


# ------------------------------------------------------------ Hadamard / fp8
def hadamard(D: int) -> np.ndarray:
    H = np.empty((D, D), dtype=np.float64)
    _load().orc_hadamard_matrix(D, _p(H))
    return H


def rotate(x) -> np.ndarray:
    x = _f32(x)
    D = x.shape[-1]
    out = np.empty_like(x)
    _load().orc_rotate(x.size // D, D, _p(x), _p(out))
    return out


def rotate_quant(x):
    """Per-row Hadamard rotation + e4m3 quantisation -> (codes uint8, scales f32)."""
    x = _f32(x)
    D = x.shape[-1]
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty(x.shape[:-1], dtype=np.float32)
    _load().orc_rotate_quant(x.size // D, D, _p(x), _p(codes), _p(scales))
    return codes, scales


def index_cache_append(k_new, kv_len, codes, scales):
    """Index-key cache update before the indexer (DeepSeek-V3.2 model documentation,
    "DeepSeek Sparse Attention (DSA)", item 1: the indexer keeps its own key cache,
    which with the FP8 indexer holds rotated e4m3 codes and row scales).

    The t_new newest keys k_new [B, t_new, D] of sequence b are the cache rows
    p = kv_len[b] - t_new + t (the newest tokens are the last ones of the
    sequence); each is rotated and quantised by ``rotate_quant`` and stored there.
    Rows with p outside [0, max_kv) are skipped.  Returns updated copies of
    codes [B, max_kv, D] and scales [B, max_kv].
    """
    k_new = _f32(k_new)
    B, t_new, _ = k_new.shape
    codes = np.array(codes, dtype=np.uint8, copy=True)
    scales = np.array(scales, dtype=np.float32, copy=True)
    max_kv = codes.shape[1]
    kl = np.asarray(kv_len, dtype=np.int64)
    for b in range(B):
        for t in range(t_new):
            p = int(kl[b]) - t_new + t
            if 0 <= p < max_kv:
                c, sc = rotate_quant(k_new[b, t][None, :])
                codes[b, p] = c[0]
                scales[b, p] = sc[0]
    return codes, scales


def quant(x):
    """Per-row e4m3 quantisation without rotation -> (codes uint8, scales f32).

    The codec of ``rotate_quant`` (row scale amax / 448, codes of x * (448 / amax)
    rounded to nearest even) applied to the rows as they are.  It serves the MLA
    latent cache and queries when the attention runs on fp8 codes: the pages run
    the indexer in FP8 and call FP8 a precision optimisation; the latent rows are
    not rotated because their first v_dim columns are the values.
    """
    x = _f32(x)
    D = x.shape[-1]
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty(x.shape[:-1], dtype=np.float32)
    _load().orc_quant(x.size // D, D, _p(x), _p(codes), _p(scales))
    return codes, scales


def kv_rows_fp8(x) -> np.ndarray:
    """The fp8 latent-cache row layout: per row, the D codes of ``quant``, then its
    fp32 scale (little-endian) and 12 zero bytes -> uint8 [..., D + 16]."""
    codes, scales = quant(x)
    tail = np.zeros(codes.shape[:-1] + (16,), dtype=np.uint8)
    tail[..., :4] = scales.astype("<f4").view(np.uint8).reshape(codes.shape[:-1] + (4,))
    return np.concatenate([codes, tail], axis=-1)


def sparse_mla_fp8(q_codes, q_scales, kv_codes, kv_scales, idx, sm_scale: float, rows=None,
                   v_dim: int | None = None, T=None):
    """Sparse MLA on fp8 operands: the attention of ``sparse_mla`` over the
    dequantised queries decode(q_code) * q_scale and latent rows
    decode(kv_code) * kv_scale (keys and values alike)."""
    return sparse_mla(dequant(q_codes, q_scales).astype(np.float32), dequant(kv_codes, kv_scales).astype(np.float32),
                      idx, sm_scale, rows=rows, v_dim=v_dim, T=T)


def dequant(codes, scales) -> np.ndarray:
    """decode(code) * scale in float64 (one scale per row of the last axis)."""
    return e4m3_decode(codes) * _f32(scales).astype(np.float64)[..., None]


# ------------------------------------------------------------------ indexer
def index_scores(q_idx, w, k_idx, kv_len, rows=None, T=None) -> np.ndarray:
    """q_idx [B,T,H,D], w [B,T,H], k_idx [B,Lmax,D], kv_len [B] -> [n_rows, Lmax] f32.

    With ``T`` given, q_idx [n_rows,H,D] and w [n_rows,H] hold only the listed rows.
    """
    q = _f32(q_idx)
    w = _f32(w)
    k = _f32(k_idx)
    kl = _i32(kv_len)
    compact = T is not None
    B = kl.shape[0]
    if compact:
        _, H, D = q.shape
    else:
        _, T, H, D = q.shape
    Lmax = k.shape[1]
    r = _rows(rows, B * T)
    out = np.empty((len(r), Lmax), dtype=np.float32)
    _load().orc_index_scores(B, T, Lmax, H, D, _p(q), _p(w), _p(k), _p(kl), len(r), _p(r), int(compact), _p(out))
    return out


def index_scores_fp8(q_codes, q_scale, w, k_codes, k_scale, kv_len, rows=None, T=None) -> np.ndarray:
    """fp8 operands (codes + row scales); ``T`` as in index_scores."""
    qc = _u8(q_codes)
    qs = _f32(q_scale)
    w = _f32(w)
    kc = _u8(k_codes)
    ks = _f32(k_scale)
    kl = _i32(kv_len)
    compact = T is not None
    B = kl.shape[0]
    if compact:
        _, H, D = qc.shape
    else:
        _, T, H, D = qc.shape
    Lmax = kc.shape[1]
    r = _rows(rows, B * T)
    out = np.empty((len(r), Lmax), dtype=np.float32)
    _load().orc_index_scores_fp8(B, T, Lmax, H, D, _p(qc), _p(qs), _p(w), _p(kc), _p(ks), _p(kl),
                                 len(r), _p(r), int(compact), _p(out))
    return out


# -------------------------------------------------------------------- top-k
def topk(scores, kv_len, T: int, K: int, rows=None) -> np.ndarray:
    """scores [n_rows, Lmax] for query rows ``rows`` -> idx [n_rows, K] int32 (sorted, -1 padded)."""
    s = _f32(scores)
    kl = _i32(kv_len)
    B = kl.shape[0]
    Lmax = s.shape[1]
    r = _rows(rows, B * T)
    assert s.shape[0] == len(r)
    idx = np.empty((len(r), K), dtype=np.int32)
    _load().orc_topk(B, T, Lmax, K, _p(kl), len(r), _p(r), _p(s), _p(idx))
    return idx


# --------------------------------------------------------------- sparse MLA
def sparse_mla(q, kv, idx, sm_scale: float, rows=None, v_dim: int | None = None, T=None):
    """q [B,T,H,Dqk], kv [B,Lmax,Dqk], idx [n_rows,K] -> (out [n_rows,H,Dv] f64, lse [n_rows,H] f64).

    With ``T`` given, q [n_rows,H,Dqk] holds only the listed rows.
    """
    q = _f32(q)
    kv = _f32(kv)
    ix = _i32(idx)
    compact = T is not None
    B = kv.shape[0]
    if compact:
        _, H, Dqk = q.shape
    else:
        _, T, H, Dqk = q.shape
    Lmax = kv.shape[1]
    Dv = Dqk if v_dim is None else v_dim
    r = _rows(rows, B * T)
    K = ix.shape[-1]
    ix = ix.reshape(len(r), K)
    out = np.empty((len(r), H, Dv), dtype=np.float64)
    lse = np.empty((len(r), H), dtype=np.float64)
    _load().orc_sparse_mla(B, T, Lmax, H, Dqk, Dv, K, float(sm_scale), _p(q), _p(kv), len(r), _p(r),
                           int(compact), _p(ix), _p(out), _p(lse))
    return out, lse


def sparse_mla_bwd(q, kv, dout, idx, sm_scale: float, rows=None, v_dim: int | None = None, T=None):
    """Gradients of L = sum(dout * out) for the attention of ``sparse_mla``:
    q [B,T,H,Dqk], kv [B,Lmax,Dqk], dout [B,T,H,Dv], idx [n_rows,K] (entries < 0
    skipped, an index listed twice counts twice) -> (dq [n_rows,H,Dqk] f64,
    dkv [B,Lmax,Dqk] f64, summed over the listed rows).  With ``T`` given, q and
    dout hold only the listed rows ([n_rows,H,·]).

    The page calls DSA trainable (DeepSeek-V3.2 model documentation, model
    description); these are the chain-rule gradients of the softmax attention
    over the selected set: dP_j = dO.v_j, D = dO.O, dz_j = p_j (dP_j - D),
    dq = sm sum_j dz_j k_j, dkv[idx_j] += sm dz_j q, and += p_j dO on the value
    columns.
    """
    q = _f32(q)
    kv = _f32(kv)
    do = _f32(dout)
    ix = _i32(idx)
    compact = T is not None
    B = kv.shape[0]
    if compact:
        _, H, Dqk = q.shape
    else:
        _, T, H, Dqk = q.shape
    Lmax = kv.shape[1]
    Dv = Dqk if v_dim is None else v_dim
    assert do.shape[-1] == Dv and do.shape[-2] == H
    r = _rows(rows, B * T)
    K = ix.shape[-1]
    ix = ix.reshape(len(r), K)
    dq = np.empty((len(r), H, Dqk), dtype=np.float64)
    dkv = np.zeros((B, Lmax, Dqk), dtype=np.float64)
    _load().orc_sparse_mla_bwd(B, T, Lmax, H, Dqk, Dv, K, float(sm_scale), _p(q), _p(kv), _p(do), len(r), _p(r),
                               int(compact), _p(ix), _p(dq), _p(dkv))
    return dq, dkv


def masked_dense_mla(q, kv, kv_len, idx, sm_scale: float, rows=None, v_dim: int | None = None):
    """The additive-mask formulation of the same attention (dense logits + 0/-inf mask)."""
    q = _f32(q)
    kv = _f32(kv)
    kl = _i32(kv_len)
    ix = _i32(idx)
    B, T, H, Dqk = q.shape
    Lmax = kv.shape[1]
    Dv = Dqk if v_dim is None else v_dim
    r = _rows(rows, B * T)
    K = ix.shape[-1]
    ix = ix.reshape(len(r), K)
    out = np.empty((len(r), H, Dv), dtype=np.float64)
    lse = np.empty((len(r), H), dtype=np.float64)
    _load().orc_masked_dense_mla(B, T, Lmax, H, Dqk, Dv, K, float(sm_scale), _p(q), _p(kv), _p(kl),
                                 len(r), _p(r), 0, _p(ix), _p(out), _p(lse))
    return out, lse


# -------------------------------------------------------------- whole path
def forward(inp: dict, shape, rows=None, compact: bool = False) -> dict:
    """The whole path on the listed query rows.

    ``inp`` holds q_idx, w, k_idx (raw, pre-rotation), q, kv, kv_len.  With
    ``compact`` the per-query tensors q_idx [n,H_I,D_I], w [n,H_I] and q [n,H,Dqk]
    hold only the listed rows.  With an fp8 indexer the oracle rotates and
    quantises q_idx and k_idx itself, and with an fp8 MLA it quantises q and kv
    (``quant``, no rotation).  Returns scores [n,Lmax] f32, idx [n,K] i32,
    out [n,H,Dv] f64, lse [n,H] f64 and, for fp8, the codes and scales it used.
    """
    B, T = shape.batch, shape.n_q
    r = _rows(rows, B * T)
    Tc = T if compact else None
    res = {}
    if shape.idx_dtype == "fp8":
        qc, qs = rotate_quant(inp["q_idx"])
        kc, ks = rotate_quant(inp["k_idx"])
        res.update(q_codes=qc, q_scale=qs, k_codes=kc, k_scale=ks)
        sc = index_scores_fp8(qc, qs, inp["w"], kc, ks, inp["kv_len"], rows=r, T=Tc)
    else:
        sc = index_scores(inp["q_idx"], inp["w"], inp["k_idx"], inp["kv_len"], rows=r, T=Tc)
    idx = topk(sc, inp["kv_len"], T, shape.topk, rows=r)
    if getattr(shape, "mla_dtype", None) == "fp8":
        mqc, mqs = quant(inp["q"])
        kvc, kvs = quant(inp["kv"])
        res.update(mla_q_codes=mqc, mla_q_scale=mqs, kv_codes=kvc, kv_scale=kvs)
        out, lse = sparse_mla_fp8(mqc, mqs, kvc, kvs, idx, shape.sm_scale, rows=r, v_dim=shape.v_dim, T=Tc)
    else:
        out, lse = sparse_mla(inp["q"], inp["kv"], idx, shape.sm_scale, rows=r, v_dim=shape.v_dim, T=Tc)
    res.update(scores=sc, idx=idx, out=out, lse=lse, rows=r)
    return res
