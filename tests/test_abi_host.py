"""Host-only checks of the C ABI (no GPU call is made).

libdsa.so must load, export every function that include/dsa.h declares, and
reject bad arguments on the host before anything is enqueued.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")
LIB = os.path.join(ROOT, "sparse_attention_09_amd", "libdsa.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libdsa.so not built (run __graft_entry__.build())")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z0-9_]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def dsa():
    from sparse_attention_09_amd import _lib
    return _lib


def test_every_declared_symbol_is_exported(dsa):
    names = _declared()
    assert set(dsa.EXPORTS) == set(names), (set(dsa.EXPORTS) ^ set(names))
    lib = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(lib, n), n


def test_no_other_symbols_exported():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    ours = [l.split()[-1] for l in out.splitlines() if " T " in l and "dsa" in l]
    assert sorted(ours) == _declared()


def _shape(dsa, **kw):
    base = dict(batch=2, n_q=4, max_kv=256, idx_heads=64, idx_dim=128, topk=64, heads=128, qk_dim=576, v_dim=512,
                sm_scale=0.07, idx_dtype="bf16", mla_dtype="bf16")
    base.update(kw)
    return dsa.DsaShape(**base)


FAKE = 0x10000  # a 16-byte aligned non-null address that is never dereferenced on these paths


def _call_scores(dsa, shape, q=FAKE, w=FAKE, k=FAKE, kl=FAKE, out=FAKE, qs=None, ks=None):
    L = dsa.lib()
    return L.dsa_index_scores(ctypes.byref(shape.c()), q, qs, w, k, ks, kl, out, None)


def test_status_strings(dsa):
    L = dsa.lib()
    for st in range(0, -9, -1):
        assert L.dsa_status_string(st)
    assert L.dsa_status_string(-99) == b"unknown status"


def test_index_scores_rejects_bad_arguments(dsa):
    L = dsa.lib()
    assert L.dsa_index_scores(None, FAKE, None, FAKE, FAKE, None, FAKE, FAKE, None) == -1
    assert _call_scores(dsa, _shape(dsa), q=None) == -1
    assert _call_scores(dsa, _shape(dsa), q=FAKE + 8) == -4
    assert _call_scores(dsa, _shape(dsa, batch=0)) == -2
    assert _call_scores(dsa, _shape(dsa, n_q=300)) == -2
    assert _call_scores(dsa, _shape(dsa, idx_heads=65)) == -6
    assert _call_scores(dsa, _shape(dsa, idx_dim=96)) == -6
    assert _call_scores(dsa, _shape(dsa, idx_dtype="fp8")) == -1  # scales missing
    s = _shape(dsa)
    cs = s.c()
    cs.idx_dtype = 7
    assert L.dsa_index_scores(ctypes.byref(cs), FAKE, None, FAKE, FAKE, None, FAKE, FAKE, None) == -3


def test_topk_and_mla_reject_bad_arguments(dsa):
    L = dsa.lib()
    s = _shape(dsa, topk=5000)
    assert L.dsa_topk(ctypes.byref(s.c()), FAKE, FAKE, FAKE, None, 0, None) == -6
    s = _shape(dsa, topk=0)
    assert L.dsa_topk(ctypes.byref(s.c()), FAKE, FAKE, FAKE, None, 0, None) == -2
    s = _shape(dsa, qk_dim=512, v_dim=576)
    assert L.dsa_sparse_mla_fwd(ctypes.byref(s.c()), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == -2
    s = _shape(dsa, qk_dim=320, v_dim=256)
    assert L.dsa_sparse_mla_fwd(ctypes.byref(s.c()), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == -6
    s = _shape(dsa, mla_dtype="fp8", qk_dim=192, v_dim=128)
    assert L.dsa_sparse_mla_fwd(ctypes.byref(s.c()), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == -6
    cs = _shape(dsa).c()
    cs.mla_dtype = 7
    assert L.dsa_sparse_mla_fwd(ctypes.byref(cs), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == -3
    # the fp8 path quantises the queries into the workspace, so it always needs one
    s = _shape(dsa, mla_dtype="fp8")
    need = dsa.sparse_mla_workspace_size(s)
    assert need >= 2 * 4 * 128 * (576 + 4)
    assert L.dsa_sparse_mla_fwd(ctypes.byref(s.c()), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == -5
    assert L.dsa_sparse_mla_fwd(ctypes.byref(s.c()), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, need - 1, None) == -5
    assert L.dsa_sparse_mla_fwd(ctypes.byref(s.c()), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE + 8, need, None) == -4
    sb = _shape(dsa, mla_dtype="bf16")
    assert dsa.sparse_mla_workspace_size(sb) < need
    for bad_scale in (float("nan"), 0.0, -0.07):
        s = _shape(dsa, sm_scale=bad_scale)
        assert L.dsa_sparse_mla_fwd(ctypes.byref(s.c()), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == -2
    # decode shapes split the index list and need a workspace
    s = _shape(dsa, batch=4, n_q=1, topk=2048, max_kv=4096)
    assert dsa.sparse_mla_workspace_size(s) > 0
    assert L.dsa_sparse_mla_fwd(ctypes.byref(s.c()), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == -5


def test_topk_workspace_only_for_few_long_rows(dsa):
    L = dsa.lib()
    # few long rows are split over many workgroups and need scratch
    s = _shape(dsa, batch=64, n_q=1, topk=2048, max_kv=32768)
    need = dsa.topk_workspace_size(s)
    assert need >= 64 * (4096 * 4 + 2048 * 4)
    assert L.dsa_topk(ctypes.byref(s.c()), FAKE, FAKE, FAKE, None, 0, None) == -5
    assert L.dsa_topk(ctypes.byref(s.c()), FAKE, FAKE, FAKE, FAKE, need - 1, None) == -5
    assert L.dsa_topk(ctypes.byref(s.c()), FAKE, FAKE, FAKE, FAKE + 4, need, None) == -4
    # many rows, or short rows: one workgroup per row, no scratch
    assert dsa.topk_workspace_size(_shape(dsa, batch=1, n_q=4096, topk=2048, max_kv=32768)) == 0
    assert dsa.topk_workspace_size(_shape(dsa, batch=64, n_q=1, topk=2048, max_kv=4096)) == 0


def test_rotate_quant_rejects_bad_arguments(dsa):
    L = dsa.lib()
    assert L.dsa_rotate_quant_fp8(0, 128, FAKE, 1, FAKE, FAKE, None) == -2
    assert L.dsa_rotate_quant_fp8(4, 96, FAKE, 1, FAKE, FAKE, None) == -6
    assert L.dsa_rotate_quant_fp8(4, 512, FAKE, 1, FAKE, FAKE, None) == -6
    assert L.dsa_rotate_quant_fp8(4, 128, FAKE, 2, FAKE, FAKE, None) == -3
    assert L.dsa_rotate_quant_fp8(4, 128, None, 1, FAKE, FAKE, None) == -1


def test_cache_append_rejects_bad_arguments(dsa):
    L = dsa.lib()
    f = L.dsa_index_cache_append_fp8
    assert f(0, 1, 16, 128, FAKE, 1, FAKE, FAKE, FAKE, None) == -2
    assert f(2, 0, 16, 128, FAKE, 1, FAKE, FAKE, FAKE, None) == -2
    assert f(2, 1, 0, 128, FAKE, 1, FAKE, FAKE, FAKE, None) == -2
    assert f(2, 1, 16, 96, FAKE, 1, FAKE, FAKE, FAKE, None) == -6
    assert f(2, 1, 16, 128, FAKE, 2, FAKE, FAKE, FAKE, None) == -3
    assert f(2, 1, 16, 128, FAKE, 1, None, FAKE, FAKE, None) == -1
    assert f(2, 1, 16, 128, FAKE, 1, FAKE, FAKE, None, None) == -1
    assert f(2, 1, 16, 128, FAKE + 4, 1, FAKE, FAKE, FAKE, None) == -4
    assert f(2, 1, 16, 128, FAKE, 1, FAKE, FAKE + 8, FAKE, None) == -4
    assert L.dsa_rotate_quant_fp8(4, 128, FAKE + 4, 1, FAKE, FAKE, None) == -4


def test_mla_kv_quant_rejects_bad_arguments(dsa):
    f = dsa.lib().dsa_mla_kv_quant_fp8
    assert f(0, 576, FAKE, 1, FAKE, None) == -2
    assert f(4, 0, FAKE, 1, FAKE, None) == -2
    assert f(4, 584, FAKE, 1, FAKE, None) == -6
    assert f(4, 1040, FAKE, 1, FAKE, None) == -6
    assert f(4, 576, FAKE, 2, FAKE, None) == -3
    assert f(4, 576, None, 1, FAKE, None) == -1
    assert f(4, 576, FAKE, 1, None, None) == -1
    assert f(4, 576, FAKE + 8, 1, FAKE, None) == -4
    assert f(4, 576, FAKE, 0, FAKE + 4, None) == -4


def test_mla_bwd_rejects_bad_arguments(dsa):
    L = dsa.lib()
    f = L.dsa_sparse_mla_bwd
    args = [FAKE] * 8  # q, kv, idx, kv_len, lse, dout, dq, dkv

    def call(shape, *, ws=FAKE, nbytes=1 << 40, a=args):
        return f(ctypes.byref(shape.c()), *a, 0, ws, nbytes, None)

    assert call(_shape(dsa, mla_dtype="fp8")) == -3
    assert call(_shape(dsa, mla_dtype="f32", qk_dim=80, v_dim=64)) == -3
    assert call(_shape(dsa, heads=129)) == -6
    assert call(_shape(dsa, qk_dim=320, v_dim=256)) == -6
    assert call(_shape(dsa), ws=None) == -5
    assert call(_shape(dsa), ws=FAKE + 16) == -4
    assert call(_shape(dsa), nbytes=16) == -5
    bad = list(args)
    bad[6] = FAKE + 4  # dq
    assert call(_shape(dsa), a=bad) == -4
    bad = list(args)
    bad[4] = None  # lse
    assert call(_shape(dsa), a=bad) == -1
    s = _shape(dsa, batch=2, n_q=4, topk=64, heads=20)
    full, small = dsa.sparse_mla_bwd_workspace_size(s), dsa.sparse_mla_bwd_min_workspace_size(s)
    # per query: p and dP for K entries x 32 padded heads, the split sums of p dP,
    # and the transposed q and dout
    assert small >= 2 * (2 * 64 * 32 * 4 + 32 * 4 + 576 * 32 * 2 + 512 * 32 * 2)
    assert full >= 4 * small - 4 * 5 * 256
    assert dsa.sparse_mla_bwd_workspace_size(_shape(dsa, mla_dtype="fp8")) == 0


def test_forward_workspace_sizes_and_checks(dsa):
    from workloads import WORKLOADS
    L = dsa.lib()
    for wl in WORKLOADS.values():
        s = dsa.DsaShape.of(wl)
        full = dsa.forward_workspace_size(s)
        small = dsa.forward_min_workspace_size(s)
        assert 0 < small
        # the full-size buffer holds at least the scores of every query
        assert full >= wl.batch * wl.n_q * wl.max_kv * 4
    s = dsa.DsaShape.of(WORKLOADS["prefill_32k"])
    args = [FAKE] * 7
    st = L.dsa_forward(ctypes.byref(s.c()), *args, None, FAKE, None, FAKE, 16, None)
    assert st == -5
    st = L.dsa_forward(ctypes.byref(s.c()), *args, None, FAKE, None, FAKE + 16, 1 << 40, None)
    assert st == -4  # workspace must be 256-byte aligned
    bad = dsa.DsaShape.of(WORKLOADS["decode_32k"])
    bad.heads = 0
    assert dsa.forward_workspace_size(bad) == 0


def test_launch_size_limits(dsa):
    """batch <= 65535, B * T <= 2^30 and B * T * H <= 2^30 keep every launch size and kernel
    row index inside int; beyond them the host returns DSA_ERR_UNSUPPORTED (-6)."""
    assert _call_scores(dsa, _shape(dsa, batch=65536, n_q=1)) == -6
    assert _call_scores(dsa, _shape(dsa, batch=65535, n_q=20000, max_kv=20000)) == -6  # B*T > 2^30
    assert dsa.forward_workspace_size(_shape(dsa, batch=65536, n_q=1)) == 0
    # B*T*H beyond 2^30 with an MLA: 4096 x 256 queries x 2048 heads = 2^31
    big = _shape(dsa, batch=4096, n_q=256, max_kv=256, heads=2048)
    assert dsa.forward_workspace_size(big) == 0
    assert dsa.sparse_mla_workspace_size(big) == 0
    # the same query count with 128 heads is within the limits
    assert dsa.forward_workspace_size(_shape(dsa, batch=4096, n_q=256, max_kv=256)) > 0
    L = dsa.lib()
    for st in (-2147483648, -100, -9, 1, 2147483647):  # any int32 is a valid status value
        assert L.dsa_status_string(st) == b"unknown status"


def test_index_topk_rejects_bad_arguments(dsa):
    L = dsa.lib()
    f = L.dsa_index_topk
    args = [FAKE] * 7  # q_idx, q_scale, w, k_idx, k_scale, kv_len, idx

    def call(shape, *, ws=FAKE, nbytes=1 << 40, a=args):
        return f(ctypes.byref(shape.c()), *a, ws, nbytes, None)

    assert call(_shape(dsa, topk=0)) == -2
    assert call(_shape(dsa, topk=4097)) == -6
    assert call(_shape(dsa, idx_heads=65)) == -6
    assert call(_shape(dsa, n_q=300, max_kv=256)) == -2
    assert call(_shape(dsa), ws=None) == -5
    assert call(_shape(dsa), ws=FAKE + 16) == -4
    assert call(_shape(dsa), nbytes=16) == -5
    for i, name in ((0, "q_idx"), (2, "w"), (3, "k_idx"), (5, "kv_len"), (6, "idx")):
        bad = list(args)
        bad[i] = None
        assert call(_shape(dsa), a=bad) == -1, name
    bad = list(args)
    bad[6] = FAKE + 2  # idx
    assert call(_shape(dsa), a=bad) == -4
    bad = list(args)
    bad[1] = None  # fp8 needs the query scales
    assert call(_shape(dsa, idx_dtype="fp8"), a=bad) == -1
    # sizes: one pass for every query, or one query at a time; 8-byte list words per row
    s = _shape(dsa, batch=2, n_q=4, topk=64)
    full, small = dsa.index_topk_workspace_size(s), dsa.index_topk_min_workspace_size(s)
    cap = max(4 * 64, 64 + 64)
    assert full >= 2 * 4 * cap * 8 and small >= 2 * cap * 8 and small < full
    assert dsa.index_topk_workspace_size(_shape(dsa, topk=0)) == 0


def test_forward_noalloc_rejects_on_the_host(dsa):
    """dsa_forward_noalloc checks its arguments as dsa_forward does and rejects a shape
    whose smallest workspace exceeds the static scratch with DSA_ERR_SCRATCH, all
    before any GPU call (these run without a GPU)."""
    from workloads import WORKLOADS
    L = dsa.lib()
    f = L.dsa_forward_noalloc
    assert L.dsa_status_string(-8)
    args = [FAKE] * 7  # q_idx, w, k_idx, k_scale, q, kv, kv_len

    def call(shape, a=args, idx=FAKE, out=FAKE, lse=FAKE):
        return f(ctypes.byref(shape.c()), *a, idx, out, lse, None)

    assert f(None, *args, FAKE, FAKE, FAKE, None) == -1
    s = dsa.DsaShape.of(WORKLOADS["decode_32k"])
    bad = list(args)
    bad[0] = None
    assert call(s, a=bad) == -1
    assert call(s, out=None) == -1
    bad = list(args)
    bad[4] = FAKE + 8  # q
    assert call(s, a=bad) == -4
    z = dsa.DsaShape.of(WORKLOADS["decode_32k"])
    z.heads = 0
    assert call(z) == -2
    # one decode query per sequence cannot be chunked: 64 rows of 2^20 scores need 256 MiB,
    # but the fused scores + top-k needs 64 KiB of candidate list per row, which fits
    big = dsa.DsaShape.of(WORKLOADS["decode_32k"])
    big.max_kv = 1 << 20
    assert dsa.forward_workspace_size(big) > dsa.NOALLOC_SCRATCH_BYTES
    assert dsa.forward_min_workspace_size(big) <= dsa.NOALLOC_SCRATCH_BYTES
    # 4096 such rows need 256 MiB of candidate lists and 16 GiB of score rows: rejected
    big.batch = 4096
    assert dsa.forward_min_workspace_size(big) > dsa.NOALLOC_SCRATCH_BYTES
    assert call(big) == -8
    # the fp8 MLA quantises every query before the chunk loop: 2.4 GB of codes at prefill_32k
    p = dsa.DsaShape.of(WORKLOADS["prefill_32k"])
    p.mla_dtype = "fp8"
    assert call(p) == -8
    # the decode workloads fit the scratch in one pass (the checks above stop before it)
    for name in ("decode_32k", "decode_128k_fp8", "decode_128k_fp8_mla"):
        s = dsa.DsaShape.of(WORKLOADS[name])
        assert dsa.forward_workspace_size(s) <= dsa.NOALLOC_SCRATCH_BYTES, name
