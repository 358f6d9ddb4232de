"""ctypes binding of libdsa.so (include/dsa.h).

Argument marshalling only: tensors are passed as raw device pointers with the
current HIP stream of torch; every step of the path runs in the library's
kernels.  Output tensors are allocated here with torch (device memory only).
The binding fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdsa.so")

F32, BF16, FP8_E4M3 = 0, 1, 2
_DT = {"f32": F32, "bf16": BF16, "fp8": FP8_E4M3}

STATUS = {0: "DSA_OK", -1: "DSA_ERR_NULL", -2: "DSA_ERR_SHAPE", -3: "DSA_ERR_DTYPE", -4: "DSA_ERR_ALIGN",
          -5: "DSA_ERR_WORKSPACE", -6: "DSA_ERR_UNSUPPORTED", -7: "DSA_ERR_HIP",
          -8: "DSA_ERR_SCRATCH"}

EXPORTS = ["dsa_index_scores", "dsa_topk_workspace_size", "dsa_topk", "dsa_sparse_mla_workspace_size",
           "dsa_sparse_mla_fwd", "dsa_rotate_quant_fp8", "dsa_index_cache_append_fp8", "dsa_forward_workspace_size",
           "dsa_mla_kv_quant_fp8", "dsa_forward_min_workspace_size", "dsa_forward", "dsa_status_string",
           "dsa_sparse_mla_bwd_workspace_size", "dsa_sparse_mla_bwd_min_workspace_size", "dsa_sparse_mla_bwd",
           "dsa_index_topk_workspace_size", "dsa_index_topk_min_workspace_size", "dsa_index_topk",
           "dsa_forward_noalloc"]


class DsaError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({text})")
        self.status = status


class CShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q", ctypes.c_int32), ("max_kv", ctypes.c_int32),
                ("idx_heads", ctypes.c_int32), ("idx_dim", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("heads", ctypes.c_int32), ("qk_dim", ctypes.c_int32), ("v_dim", ctypes.c_int32),
                ("sm_scale", ctypes.c_float), ("idx_dtype", ctypes.c_int32), ("mla_dtype", ctypes.c_int32)]


@dataclass
class DsaShape:
    batch: int
    n_q: int
    max_kv: int
    idx_heads: int
    idx_dim: int
    topk: int
    heads: int
    qk_dim: int
    v_dim: int
    sm_scale: float
    idx_dtype: str = "bf16"
    mla_dtype: str = "bf16"

    @classmethod
    def of(cls, obj) -> "DsaShape":
        """Copy the shape fields of any object carrying them (e.g. a workload)."""
        return cls(**{f: getattr(obj, f) for f in cls.__dataclass_fields__})

    def c(self) -> CShape:
        return CShape(self.batch, self.n_q, self.max_kv, self.idx_heads, self.idx_dim, self.topk, self.heads,
                      self.qk_dim, self.v_dim, float(self.sm_scale), _DT[self.idx_dtype], _DT[self.mla_dtype])


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m sparse_attention_09_amd.build` "
                               "(or __graft_entry__.build()); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        P, SZ, I32, I64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
        SP = ctypes.POINTER(CShape)
        sig = {
            "dsa_index_scores": ([SP, P, P, P, P, P, P, P, P], I32),
            "dsa_index_topk_workspace_size": ([SP], SZ),
            "dsa_index_topk_min_workspace_size": ([SP], SZ),
            "dsa_index_topk": ([SP, P, P, P, P, P, P, P, P, SZ, P], I32),
            "dsa_topk_workspace_size": ([SP], SZ),
            "dsa_topk": ([SP, P, P, P, P, SZ, P], I32),
            "dsa_sparse_mla_workspace_size": ([SP], SZ),
            "dsa_sparse_mla_fwd": ([SP, P, P, P, P, P, P, P, SZ, P], I32),
            "dsa_rotate_quant_fp8": ([I64, I32, P, I32, P, P, P], I32),
            "dsa_index_cache_append_fp8": ([I32, I32, I32, I32, P, I32, P, P, P, P], I32),
            "dsa_mla_kv_quant_fp8": ([I64, I32, P, I32, P, P], I32),
            "dsa_sparse_mla_bwd_workspace_size": ([SP], SZ),
            "dsa_sparse_mla_bwd_min_workspace_size": ([SP], SZ),
            "dsa_sparse_mla_bwd": ([SP, P, P, P, P, P, P, P, P, I32, P, SZ, P], I32),
            "dsa_forward_workspace_size": ([SP], SZ),
            "dsa_forward_min_workspace_size": ([SP], SZ),
            "dsa_forward": ([SP, P, P, P, P, P, P, P, P, P, P, P, SZ, P], I32),
            "dsa_forward_noalloc": ([SP, P, P, P, P, P, P, P, P, P, P, P], I32),
            "dsa_status_string": ([I32], ctypes.c_char_p),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to libdsa must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to libdsa must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _check(fn: str, st: int):
    if st != 0:
        raise DsaError(fn, st, lib().dsa_status_string(st).decode())


def _empty(shape, dt, device):
    return torch.empty(shape, dtype=dt, device=device)


def _out_dtype(shape: DsaShape):
    """MLA output dtype: f32 for the f32 path, bf16 for the bf16 and fp8 paths."""
    return torch.float32 if shape.mla_dtype == "f32" else torch.bfloat16


def _view_u8(t):
    if t is None:
        return None
    return t if t.dtype == torch.uint8 else t.view(torch.uint8)


# ------------------------------------------------------------------ entry points
def index_scores(shape: DsaShape, q_idx, w, k_idx, kv_len, q_scale=None, k_scale=None, scores=None, stream=None):
    """Lightning-indexer scores [B,T,L_max] f32 (-inf where masked)."""
    if shape.idx_dtype == "fp8":
        q_idx, k_idx = _view_u8(q_idx), _view_u8(k_idx)
    if scores is None:
        scores = _empty((shape.batch, shape.n_q, shape.max_kv), torch.float32, q_idx.device)
    cs = shape.c()
    _check("dsa_index_scores", lib().dsa_index_scores(ctypes.byref(cs), _ptr(q_idx), _ptr(q_scale), _ptr(w),
                                                       _ptr(k_idx), _ptr(k_scale), _ptr(kv_len), _ptr(scores),
                                                       _stream(stream)))
    return scores


def index_topk_workspace_size(shape: DsaShape) -> int:
    return int(lib().dsa_index_topk_workspace_size(ctypes.byref(shape.c())))


def index_topk_min_workspace_size(shape: DsaShape) -> int:
    return int(lib().dsa_index_topk_min_workspace_size(ctypes.byref(shape.c())))


def index_topk(shape: DsaShape, q_idx, w, k_idx, kv_len, q_scale=None, k_scale=None, idx=None, workspace=None,
               stream=None):
    """Indexer scores and top-k in one pass (no score matrix) -> idx [B,T,K] int32."""
    if shape.idx_dtype == "fp8":
        q_idx, k_idx = _view_u8(q_idx), _view_u8(k_idx)
    dev = q_idx.device
    if idx is None:
        idx = _empty((shape.batch, shape.n_q, shape.topk), torch.int32, dev)
    if workspace is None:
        workspace = _empty((max(1, index_topk_workspace_size(shape)),), torch.uint8, dev)
    cs = shape.c()
    _check("dsa_index_topk", lib().dsa_index_topk(ctypes.byref(cs), _ptr(q_idx), _ptr(q_scale), _ptr(w),
                                                   _ptr(k_idx), _ptr(k_scale), _ptr(kv_len), _ptr(idx),
                                                   _ptr(workspace), workspace.numel(), _stream(stream)))
    return idx


def topk_workspace_size(shape: DsaShape) -> int:
    return int(lib().dsa_topk_workspace_size(ctypes.byref(shape.c())))


def topk(shape: DsaShape, scores, kv_len, idx=None, workspace=None, stream=None):
    """Top-index_topk positions [B,T,K] int32, ascending, -1 padded."""
    if idx is None:
        idx = _empty((shape.batch, shape.n_q, shape.topk), torch.int32, scores.device)
    need = topk_workspace_size(shape)
    if workspace is None and need > 0:
        workspace = _empty((need,), torch.uint8, scores.device)
    cs = shape.c()
    _check("dsa_topk", lib().dsa_topk(ctypes.byref(cs), _ptr(scores), _ptr(kv_len), _ptr(idx), _ptr(workspace),
                                      0 if workspace is None else workspace.numel(), _stream(stream)))
    return idx


def sparse_mla_workspace_size(shape: DsaShape) -> int:
    return int(lib().dsa_sparse_mla_workspace_size(ctypes.byref(shape.c())))


def sparse_mla_fwd(shape: DsaShape, q, kv, idx, kv_len, out=None, lse=None, want_lse=True, workspace=None,
                   stream=None):
    """Sparse absorbed MLA -> (out [B,T,H,Dv], lse [B,T,H] f32).  For mla_dtype fp8, q is
    bf16 and kv the fp8 latent cache of ``mla_kv_quant_fp8`` ([B, L_max, D_qk + 16] u8)."""
    dt = _out_dtype(shape)
    if shape.mla_dtype == "fp8":
        kv = _view_u8(kv)
    if out is None:
        out = _empty((shape.batch, shape.n_q, shape.heads, shape.v_dim), dt, q.device)
    if lse is None and want_lse:
        lse = _empty((shape.batch, shape.n_q, shape.heads), torch.float32, q.device)
    need = sparse_mla_workspace_size(shape)
    if workspace is None and need > 0:
        workspace = _empty((need,), torch.uint8, q.device)
    cs = shape.c()
    _check("dsa_sparse_mla_fwd", lib().dsa_sparse_mla_fwd(ctypes.byref(cs), _ptr(q), _ptr(kv), _ptr(idx),
                                                           _ptr(kv_len), _ptr(out), _ptr(lse), _ptr(workspace),
                                                           0 if workspace is None else workspace.numel(),
                                                           _stream(stream)))
    return out, lse


def rotate_quant_fp8(x, codes=None, scales=None, stream=None):
    """Per-row Hadamard rotation + e4m3 quantisation of x [..., dim] -> (codes u8, scales f32)."""
    dim = x.shape[-1]
    rows = x.numel() // dim
    xt = {torch.float32: F32, torch.bfloat16: BF16}[x.dtype]
    if codes is None:
        codes = _empty(x.shape, torch.uint8, x.device)
    if scales is None:
        scales = _empty(x.shape[:-1], torch.float32, x.device)
    _check("dsa_rotate_quant_fp8", lib().dsa_rotate_quant_fp8(rows, dim, _ptr(x), xt, _ptr(codes), _ptr(scales),
                                                               _stream(stream)))
    return codes, scales


def index_cache_append_fp8(k_new, kv_len, codes, scales, stream=None):
    """Rotate + quantise the newest keys k_new [B, t_new, dim] into the fp8 index-key
    cache codes [B, max_kv, dim] u8 / scales [B, max_kv] f32 (in place) at rows
    kv_len[b] - t_new + t.  Returns (codes, scales)."""
    B, t_new, dim = k_new.shape
    xt = {torch.float32: F32, torch.bfloat16: BF16}[k_new.dtype]
    if codes.shape[0] != B or codes.shape[2] != dim or tuple(scales.shape) != tuple(codes.shape[:2]):
        raise ValueError("cache shape mismatch")
    _check("dsa_index_cache_append_fp8",
           lib().dsa_index_cache_append_fp8(B, t_new, codes.shape[1], dim, _ptr(k_new), xt, _ptr(kv_len),
                                            _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def mla_kv_quant_fp8(x, kv_rows=None, stream=None):
    """Per-row e4m3 quantisation (no rotation) of x [..., dim] into fp8 latent-cache
    rows [..., dim + 16] u8: the codes, the fp32 row scale, 12 zero bytes."""
    dim = x.shape[-1]
    rows = x.numel() // dim
    xt = {torch.float32: F32, torch.bfloat16: BF16}[x.dtype]
    if kv_rows is None:
        kv_rows = _empty(tuple(x.shape[:-1]) + (dim + 16,), torch.uint8, x.device)
    _check("dsa_mla_kv_quant_fp8", lib().dsa_mla_kv_quant_fp8(rows, dim, _ptr(x), xt, _ptr(kv_rows),
                                                               _stream(stream)))
    return kv_rows


def sparse_mla_bwd_workspace_size(shape: DsaShape) -> int:
    return int(lib().dsa_sparse_mla_bwd_workspace_size(ctypes.byref(shape.c())))


def sparse_mla_bwd_min_workspace_size(shape: DsaShape) -> int:
    return int(lib().dsa_sparse_mla_bwd_min_workspace_size(ctypes.byref(shape.c())))


def sparse_mla_bwd(shape: DsaShape, q, kv, idx, kv_len, lse, dout, dq=None, dkv=None, accumulate_dkv=False,
                   workspace=None, stream=None):
    """Backward of sparse_mla_fwd -> (dq [B,T,H,Dqk] f32, dkv [B,L_max,Dqk] f32)."""
    dev = q.device
    if dq is None:
        dq = _empty((shape.batch, shape.n_q, shape.heads, shape.qk_dim), torch.float32, dev)
    if dkv is None:
        dkv = _empty((shape.batch, shape.max_kv, shape.qk_dim), torch.float32, dev)
    if workspace is None:
        workspace = _empty((max(1, sparse_mla_bwd_workspace_size(shape)),), torch.uint8, dev)
    cs = shape.c()
    _check("dsa_sparse_mla_bwd", lib().dsa_sparse_mla_bwd(ctypes.byref(cs), _ptr(q), _ptr(kv), _ptr(idx),
                                                           _ptr(kv_len), _ptr(lse), _ptr(dout),
                                                           _ptr(dq), _ptr(dkv), int(bool(accumulate_dkv)),
                                                           _ptr(workspace), workspace.numel(), _stream(stream)))
    return dq, dkv


def forward_workspace_size(shape: DsaShape) -> int:
    return int(lib().dsa_forward_workspace_size(ctypes.byref(shape.c())))


def forward_min_workspace_size(shape: DsaShape) -> int:
    return int(lib().dsa_forward_min_workspace_size(ctypes.byref(shape.c())))


def forward(shape: DsaShape, q_idx, w, k_idx, q, kv, kv_len, k_scale=None, idx_out=None, out=None, lse=None,
            want_idx=True, want_lse=True, workspace=None, stream=None):
    """The whole path -> (idx [B,T,K] or None, out [B,T,H,Dv], lse [B,T,H] or None)."""
    dev = q.device
    if shape.idx_dtype == "fp8":
        k_idx = _view_u8(k_idx)
    if shape.mla_dtype == "fp8":
        kv = _view_u8(kv)
    if idx_out is None and want_idx:
        idx_out = _empty((shape.batch, shape.n_q, shape.topk), torch.int32, dev)
    if out is None:
        out = _empty((shape.batch, shape.n_q, shape.heads, shape.v_dim), _out_dtype(shape), dev)
    if lse is None and want_lse:
        lse = _empty((shape.batch, shape.n_q, shape.heads), torch.float32, dev)
    if workspace is None:
        workspace = _empty((forward_workspace_size(shape),), torch.uint8, dev)
    cs = shape.c()
    _check("dsa_forward", lib().dsa_forward(ctypes.byref(cs), _ptr(q_idx), _ptr(w), _ptr(k_idx), _ptr(k_scale),
                                            _ptr(q), _ptr(kv), _ptr(kv_len), _ptr(idx_out), _ptr(out), _ptr(lse),
                                            _ptr(workspace), workspace.numel(), _stream(stream)))
    return idx_out, out, lse


NOALLOC_SCRATCH_BYTES = 64 << 20  # DSA_NOALLOC_SCRATCH_BYTES


def forward_noalloc(shape: DsaShape, q_idx, w, k_idx, q, kv, kv_len, idx_out, out, lse=None, k_scale=None,
                    stream=None):
    """dsa_forward_noalloc: the whole path on the library's static scratch; the caller
    passes every output (this wrapper allocates nothing either)."""
    if shape.idx_dtype == "fp8":
        k_idx = _view_u8(k_idx)
    if shape.mla_dtype == "fp8":
        kv = _view_u8(kv)
    cs = shape.c()
    _check("dsa_forward_noalloc",
           lib().dsa_forward_noalloc(ctypes.byref(cs), _ptr(q_idx), _ptr(w), _ptr(k_idx), _ptr(k_scale), _ptr(q),
                                     _ptr(kv), _ptr(kv_len), _ptr(idx_out), _ptr(out), _ptr(lse), _stream(stream)))
    return idx_out, out, lse
