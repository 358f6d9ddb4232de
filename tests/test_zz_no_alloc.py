"""dsa_forward_noalloc (the whole path on the library's static scratch) against
dsa_forward with a caller-owned workspace, through the C ABI.

Both run the same kernels with the same query chunking when dsa_forward gets a
workspace of the scratch's size, so the results must be identical bit for bit;
with a one-pass workspace the decode shapes are identical too (they fit the
scratch in one pass).  Calls run back to back, the second on a smaller input,
so a stale scratch from the first call would show.
"""
import pytest
import torch

from helpers import announce
from workloads import get, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _pair(dsa, wl, seed=0, own_idx=False, ws_bytes=None):
    inp = make_inputs(wl, device=DEV, seed=seed)
    s = dsa.DsaShape.of(wl)
    k_idx, k_scale, kv = inp["k_idx"], None, inp["kv"]
    if wl.idx_dtype == "fp8":
        k_idx, k_scale = dsa.rotate_quant_fp8(inp["k_idx"])
    if wl.mla_dtype == "fp8":
        kv = dsa.mla_kv_quant_fp8(inp["kv"])
    B, T = wl.batch, wl.n_q
    odt = torch.float32 if wl.mla_dtype == "f32" else torch.bfloat16
    ws = None if ws_bytes is None else torch.empty((ws_bytes,), dtype=torch.uint8, device=DEV)
    ref = dsa.forward(s, inp["q_idx"], inp["w"], k_idx, inp["q"], kv, inp["kv_len"], k_scale=k_scale,
                      workspace=ws)
    idx = None if own_idx else torch.full((B, T, wl.topk), -7, dtype=torch.int32, device=DEV)
    out = torch.full((B, T, wl.heads, wl.v_dim), 3.0, dtype=odt, device=DEV)
    lse = torch.full((B, T, wl.heads), 5.0, dtype=torch.float32, device=DEV)
    got = dsa.forward_noalloc(s, inp["q_idx"], inp["w"], k_idx, inp["q"], kv, inp["kv_len"], idx, out, lse,
                              k_scale=k_scale)
    torch.cuda.synchronize()
    return ref, got


def _same(ref, got, own_idx=False):
    if not own_idx:
        assert torch.equal(ref[0], got[0]), "idx"
    assert torch.equal(ref[1], got[1]), "out"
    assert torch.equal(ref[2], got[2]), "lse"


def test_noalloc_matches_forward_on_two_calls_in_a_row(dsa):
    """decode_32k at its full size, then a smaller decode (8 sequences of 8K): each
    equal to dsa_forward bit for bit."""
    announce("noalloc: decode_32k full size")
    _same(*_pair(dsa, get("decode_32k")))
    announce("noalloc: decode 8 x 8K after the full-size call")
    _same(*_pair(dsa, get("decode_32k").replace(batch=8, max_kv=8192, kv_len=8192), seed=3))


def test_noalloc_fp8_and_internal_index_list(dsa):
    """fp8 indexer and fp8 latent cache at 16 x 128K, then the same path at 4 x 16K with the
    index list kept in the scratch (idx_out NULL)."""
    announce("noalloc: decode_128k_fp8_mla")
    _same(*_pair(dsa, get("decode_128k_fp8_mla")))
    announce("noalloc: fp8 4 x 16K, idx in scratch")
    _same(*_pair(dsa, get("decode_128k_fp8_mla").replace(batch=4, max_kv=16384, kv_len=16384), seed=5,
                 own_idx=True), own_idx=True)


def test_noalloc_chunked_prefill(dsa):
    """prefill_4k needs two query chunks inside the scratch: identical to dsa_forward on a
    workspace of the scratch's size; then a small prefill in one pass."""
    announce("noalloc: prefill_4k in query chunks")
    _same(*_pair(dsa, get("prefill_4k"), ws_bytes=dsa.NOALLOC_SCRATCH_BYTES))
    announce("noalloc: prefill 1 x 1K")
    _same(*_pair(dsa, get("prefill_4k").replace(n_q=1024, max_kv=1024, kv_len=1024), seed=2))
