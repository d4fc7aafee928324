"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports every function
include/dsa.h declares, and its argument validation returns the documented status codes
before touching the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")


@pytest.fixture(scope="module")
def lib():
    import sparse_indexed_attention_amd as m
    if not os.path.exists(m.LIB_PATH):
        from sparse_indexed_attention_amd.build import build
        build()
    return m.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert "dsa_indexer_topk" in names and "dsa_sparse_attn" in names
    for n in names:
        assert hasattr(lib, n), n


@pytest.mark.parametrize("L,G", [(0, 1), (1, 1), (16, 2), (24, 4), (17, 2), (1000, 3), (4099, 8),
                                 (5, 4), (16384, 8), (3 * 10 ** 12 + 7, 5)])
def test_zigzag_ranges_match_the_oracle(L, G):
    import sparse_indexed_attention_amd as m
    import oracle
    for g in range(G):
        (b0, e0), (b1, e1) = m.zigzag_ranges(L, G, g)
        seg = oracle.zigzag_segments(L, G)
        assert (b0, e0) == seg[g] and (b1, e1) == seg[2 * G - 1 - g]


def test_zigzag_ranges_reject_bad_arguments(lib):
    import ctypes
    r = (ctypes.c_int64 * 4)()
    p = ctypes.cast(r, ctypes.c_void_p)
    assert lib.dsa_zigzag_ranges(16, 2, 0, None) == 1
    assert lib.dsa_zigzag_ranges(-1, 2, 0, p) == 2
    assert lib.dsa_zigzag_ranges(16, 0, 0, p) == 2
    assert lib.dsa_zigzag_ranges(16, 2, 2, p) == 2
    assert lib.dsa_zigzag_ranges(16, 2, -1, p) == 2


def test_prolog_rejects_bad_arguments(lib):
    import sparse_indexed_attention_amd as m
    P = lambda i: ctypes.c_void_p(A[i])
    ws_ok = m.prolog_workspace_bytes(8, 64, 128)

    def call(x=P(0), T=8, dx=7168, W=P(1), g=P(2), eps=1e-6, H=64, D=128, q=P(3), w=P(4), k=None,
             slot=P(5), pool=P(6), kd=2, ks=P(7), ws=P(8), wsb=ws_ok):
        return lib.dsa_indexer_prolog(x, T, dx, W, g, eps, H, D, q, w, k, slot, pool, kd, ks, ws,
                                      wsb, None)
    assert call(x=None) == 1
    assert call(slot=None) == 1                      # a pool without slots
    assert call(ks=None) == 1                        # fp8 keys need their scales
    assert call(kd=7) == 3
    assert call(T=0) == 2
    assert call(eps=-1.0) == 2
    assert call(eps=float("nan")) == 2
    assert call(kd=3, D=40, H=2) == 2                # MXFP8 keys: head_dim % 32
    assert call(D=2048, H=1, wsb=1 << 30) == 4
    assert call(wsb=ws_ok - 1) == 5
    assert call(ws=None) == 5
    assert call(x=ctypes.c_void_p(A[0] + 2)) == 6
    assert m.prolog_workspace_bytes(8, 64, 128) >= 8 * (64 * 128 + 128 + 64) * 4


def test_version_and_status_strings(lib):
    assert lib.dsa_abi_version() == 3
    for s in range(9):
        assert lib.dsa_status_string(s).startswith(b"DSA_")


# fake, never dereferenced, 16-byte aligned device addresses
A = [0x10000 * (i + 1) for i in range(16)]


def _lq(m, bt=A[8], bs=64, maxb=4, T=2, maxv=200, stride=0, rows=10000):
    layout = m.DsaLayout(bs, maxb, bt, stride, 2, rows)
    queries = m.DsaQueries(T, A[9], A[10], maxv)
    return layout, queries


def _idx_call(lib, m, **kw):
    args = dict(q=A[0], qd=1, w=A[1], k=A[2], kd=2, ks=A[3], H=64, D=128, K=2048,
                out=A[4], sc=A[5], ws=A[6], wsb=1 << 40)
    lay = kw.pop("layout", None)
    qs = kw.pop("queries", None)
    args.update(kw)
    if lay is None:
        lay, qs = _lq(m)
    return lib.dsa_indexer_topk(args["q"], args["qd"], args["w"], args["k"], args["kd"], args["ks"],
                                args["H"], args["D"], ctypes.byref(lay), ctypes.byref(qs), args["K"],
                                args["out"], args["sc"], args["ws"], args["wsb"], None)


def test_indexer_validation(lib):
    import sparse_indexed_attention_amd as m
    assert _idx_call(lib, m, q=None) == 1
    assert _idx_call(lib, m, ks=None) == 1                    # fp8 keys need scales
    assert _idx_call(lib, m, out=None) == 1
    assert _idx_call(lib, m, qd=2) == 3                       # fp8 queries not accepted
    assert _idx_call(lib, m, kd=9) == 3
    assert _idx_call(lib, m, kd=3, ks=None) == 1              # MXFP8 keys need their scale bytes
    assert _idx_call(lib, m, kd=3, D=136, H=32) == 2          # MXFP8: head_dim % 32
    assert _idx_call(lib, m, D=100) == 2                      # head_dim % 8
    assert _idx_call(lib, m, H=128, D=128) == 4               # above the reference limit
    assert _idx_call(lib, m, K=0) == 2
    assert _idx_call(lib, m, K=4096) == 4
    assert _idx_call(lib, m, q=A[0] + 2) == 6
    assert _idx_call(lib, m, ws=None) == 5
    assert _idx_call(lib, m, wsb=16) == 5
    lay, qs = _lq(m, maxb=3, maxv=200)                        # 3*64 < 200 visible
    assert _idx_call(lib, m, layout=lay, queries=qs) == 2
    lay, qs = _lq(m, bs=48)                                   # not a power of two
    assert _idx_call(lib, m, layout=lay, queries=qs) == 2
    lay, qs = _lq(m, T=0)
    assert _idx_call(lib, m, layout=lay, queries=qs) == 2
    lay, qs = _lq(m, maxv=0)
    assert _idx_call(lib, m, layout=lay, queries=qs) == 2
    lay, qs = _lq(m, maxv=(1 << 22) + 1, maxb=1 << 20)
    assert _idx_call(lib, m, layout=lay, queries=qs) == 2
    lay, qs = _lq(m, bt=None, stride=100, maxv=200)           # contiguous stride too short
    assert _idx_call(lib, m, layout=lay, queries=qs) == 2
    lay, qs = _lq(m, bt=None, stride=200, maxv=200, rows=300) # pool too short for 2 seqs
    assert _idx_call(lib, m, layout=lay, queries=qs) == 2


def test_workspace_sizes_are_monotone(lib):
    a = lib.dsa_indexer_topk_workspace_size(8, 131072, 2048)
    b = lib.dsa_indexer_topk_workspace_size(8, 65536, 2048)
    assert a >= b > 0
    assert lib.dsa_indexer_topk_workspace_size(0, 10, 10) == 0
    assert lib.dsa_sparse_attn_workspace_size(8, 128, 2048, 512) > 0


def _sfa_call(lib, m, **kw):
    args = dict(q=A[0], dt=1, kv=A[2], kvd=None, H=128, dqk=576, dv=512, scale=1 / 24, idx=A[3],
                K=2048, out=A[4], lse=A[5], ws=A[6], wsb=1 << 40)
    args.update(kw)
    if args["kvd"] is None:
        args["kvd"] = args["dt"]
    lay, qs = _lq(m)
    return lib.dsa_sparse_attn(args["q"], args["dt"], args["kv"], args["kvd"], args["H"], args["dqk"],
                               args["dv"],
                               args["scale"], ctypes.byref(lay), ctypes.byref(qs), args["idx"],
                               args["K"], args["out"], args["lse"], args["ws"], args["wsb"], None)


def test_sparse_attn_validation(lib):
    import sparse_indexed_attention_amd as m
    assert _sfa_call(lib, m, q=None) == 1
    assert _sfa_call(lib, m, idx=None) == 1
    assert _sfa_call(lib, m, dt=2) == 3
    assert _sfa_call(lib, m, dqk=500) == 2
    assert _sfa_call(lib, m, dv=640) == 2
    assert _sfa_call(lib, m, dqk=2048, dv=512) == 4
    assert _sfa_call(lib, m, K=0) == 2
    assert _sfa_call(lib, m, K=3000) == 4
    assert _sfa_call(lib, m, H=0) == 2
    assert _sfa_call(lib, m, out=A[4] + 4) == 6
    assert _sfa_call(lib, m, wsb=8) == 5
    assert _sfa_call(lib, m, scale=float("nan")) == 2
    # fp8 latent rows: bf16 queries and the 576/512 geometry only
    assert _sfa_call(lib, m, kvd=2, dt=0) == 3
    assert _sfa_call(lib, m, kvd=0, dt=1) == 3
    assert _sfa_call(lib, m, kvd=2, dqk=640, dv=512) == 4
    assert _sfa_call(lib, m, kvd=2, dqk=576, dv=448) == 4


def test_store_validation(lib):
    assert lib.dsa_store_index_keys(None, 4, 128, A[1], A[2], 2, A[3], None) == 1
    assert lib.dsa_store_index_keys(A[0], 4, 128, A[1], A[2], 2, None, None) == 1
    assert lib.dsa_store_index_keys(A[0], 0, 128, A[1], A[2], 2, A[3], None) == 2
    assert lib.dsa_store_index_keys(A[0], 4, 128, A[1], A[2], 7, A[3], None) == 3
    assert lib.dsa_store_index_keys(A[0], 4, 128, A[1], A[2], 3, None, None) == 1
    assert lib.dsa_store_index_keys(A[0], 4, 120, A[1], A[2], 3, A[3], None) == 2
    assert lib.dsa_store_kv(A[0], 2, 4, 576, A[1], A[2], 1, None) == 3
    assert lib.dsa_store_kv(A[0], 1, 4, 576, A[1] + 8, A[2], 1, None) == 6
    assert lib.dsa_store_kv(A[0], 1, 4, 512, A[1], A[2], 2, None) == 4   # fp8 rows: d_qk 576 only


def _noalloc_call(lib, m, layout=None, queries=None, **kw):
    args = dict(q=A[0], qd=1, w=A[1], k=A[2], kd=2, ks=A[3], H=64, D=128, K=2048,
                out=A[4], sc=A[5])
    args.update(kw)
    if layout is None:
        layout, queries = _lq(m)
    return lib.dsa_indexer_topk_noalloc(args["q"], args["qd"], args["w"], args["k"], args["kd"],
                                        args["ks"], args["H"], args["D"], ctypes.byref(layout),
                                        ctypes.byref(queries), args["K"], args["out"], args["sc"],
                                        None)


def test_indexer_noalloc_validation(lib):
    """Argument errors and plans larger than the scratch array return before any device call."""
    import sparse_indexed_attention_amd as m
    assert _noalloc_call(lib, m, q=None) == 1
    assert _noalloc_call(lib, m, ks=None) == 1
    assert _noalloc_call(lib, m, qd=2) == 3
    assert _noalloc_call(lib, m, K=4096) == 4
    assert _noalloc_call(lib, m, out=A[4] + 4) == 6
    lay, qs = _lq(m, maxb=3, maxv=200)
    assert _noalloc_call(lib, m, layout=lay, queries=qs) == 2
    # a chunked-prefill launch (4096 queries over a 69632-token context) needs far more
    # candidate space than the scratch array holds
    need = lib.dsa_indexer_topk_workspace_size(4096, 69632, 2048)
    assert need > 32 << 20
    lay = m.DsaLayout(64, 1088, A[8], 0, 1, 69632)
    qs = m.DsaQueries(4096, A[9], A[10], 69632, 0)
    assert _noalloc_call(lib, m, layout=lay, queries=qs) == 5
