"""GPU parity of dsa_indexer_prolog through the C ABI.

Each stage is checked in the precision it is computed in.  The projections (one rocBLAS GEMM,
fp32 sums of bf16 products, read back from the workspace where they land) must lie within
the worst-case fp32 summation bound gamma_n * (|x| |W|) of the oracle's float64 product,
gamma_n = n u / (1 - n u), u = 2^-24, n = d_x.  The epilogue then decides bf16 roundings and
fp8 codes from those fp32 values, so the oracle takes the same decisions from the same
values: the query must be exactly their bf16 rounding (or their MXFP8 quantization), the head
weights exactly the fp32 values, the key the oracle's RMSNorm of them within (D + 8) u
relative, and the stored bytes exactly the oracle's quantizer applied to the key the call
returns."""
import numpy as np
import pytest

import oracle
from synth import make_prolog_inputs
from tests.gpu_util import log

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
SENTINEL = 0x5A

CASES = {
    "decode_dx7168_fp8": (8, 7168, 64, 128, "fp8"),
    "decode_dx7168_mxfp8": (8, 7168, 64, 128, "mxfp8"),
    "prefill_t512_bf16": (512, 2048, 64, 128, "bf16"),
    "odd_shapes_f32": (3, 100, 5, 32, "f32"),
    "no_store_bf16": (5, 256, 8, 64, None),
    "no_store_mx_query": (4, 320, 4, 64, "mxfp8-nostore"),
}


def make_pool(torch, fmt, rows, D):
    if fmt == "f32":
        return torch.full((rows, D), float("nan"), device="cuda"), None
    if fmt == "bf16":
        return torch.full((rows, D), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16), None
    pool = torch.full((rows, D), SENTINEL, dtype=torch.uint8, device="cuda")
    if fmt == "fp8":
        return pool, torch.full((rows,), -1.0, device="cuda")
    return pool, torch.full((rows, D // 32), SENTINEL, dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("case", sorted(CASES))
def test_prolog_matches_oracle(dsa, case):
    import torch
    T, d_x, H, D, fmt = CASES[case]
    log(f"case prolog {case}: T={T} d_x={d_x} H={H} D={D} keys={fmt}")
    pi = make_prolog_inputs(T, d_x, H, D, seed=T * 7 + d_x)
    x = torch.from_numpy(pi.x.view(np.int16)).cuda().view(torch.bfloat16)
    W = torch.from_numpy(pi.w_proj.view(np.int16)).cuda().view(torch.bfloat16)
    g = torch.from_numpy(pi.gain).cuda()
    N = H * D + D + H
    ws = torch.full((dsa.prolog_workspace_bytes(T, H, D),), 0x7F, dtype=torch.uint8, device="cuda")
    store = fmt in ("f32", "bf16", "fp8", "mxfp8")
    rows = 3 * T + 7
    slot_np = np.random.default_rng(T).permutation(rows)[:T].astype(np.int64)
    kw = {}
    if store:
        pool, ks = make_pool(torch, fmt, rows, D)
        kw = dict(slot=torch.from_numpy(slot_np).cuda(), k_pool=pool, k_scale=ks)
    else:
        kw = dict(key_format="mxfp8" if fmt == "mxfp8-nostore" else "bf16")
    q, w, k = dsa.indexer_prolog(x, W, g, pi.eps, H, D, want_k=True, workspace=ws, **kw)
    torch.cuda.synchronize()
    Y = ws[:T * N * 4].view(torch.float32).reshape(T, N).cpu().numpy()
    qb = q.view(torch.int16).cpu().numpy().view(np.uint16)
    w_np, k_np = w.cpu().numpy(), k.cpu().numpy()

    # the GEMM against the float64 product
    Yref = oracle.project(pi.x, pi.w_proj)
    S = np.abs(oracle.decode_bf16(pi.x)) @ np.abs(oracle.decode_bf16(pi.w_proj))
    gam = d_x * U / (1 - d_x * U)
    err = np.abs(Y - Yref)
    log(f"  GEMM max err {err.max():.2e}, worst err / bound {np.max(err / (gam * S + 1e-300)):.3f}")
    assert np.all(err <= gam * S)
    # the epilogue from the same fp32 values
    HD = H * D
    if fmt in ("mxfp8", "mxfp8-nostore"):
        codes, sb = oracle.quantize_mxfp8(Y[:, :HD].reshape(T, H, D))
        assert int(sb.min()) >= 3
        want_q = oracle.decode_mxfp8(codes, sb).reshape(T, H, D)
        assert np.array_equal(oracle.decode_bf16(qb), want_q)
    else:
        assert np.array_equal(qb.reshape(T, HD), oracle.encode_bf16_rne(Y[:, :HD]))
    assert np.array_equal(w_np.view(np.uint32), Y[:, HD + D:].view(np.uint32))
    kref = oracle.rms_norm(Y[:, HD:HD + D].astype(np.float64), pi.gain, pi.eps)
    assert np.all(np.abs(k_np - kref) <= (D + 8) * U * np.abs(kref) + 1e-30)
    # the store: the oracle's quantizer on the returned key
    if store:
        pool_np = (pool.view(torch.int16) if fmt == "bf16" else pool).cpu().numpy()
        others = np.setdiff1d(np.arange(rows), slot_np)
        got = pool_np[slot_np]
        if fmt == "f32":
            assert np.array_equal(got.view(np.uint32), k_np.view(np.uint32))
            assert np.all(np.isnan(pool_np[others]))
        elif fmt == "bf16":
            assert np.array_equal(got.view(np.uint16), oracle.encode_bf16_rne(k_np))
            assert np.all(pool_np[others] == SENTINEL)
        elif fmt == "fp8":
            c, s = oracle.quantize_fp8_per_token(k_np)
            assert np.array_equal(got, c)
            sc = ks.cpu().numpy()
            assert np.array_equal(sc[slot_np].view(np.uint32), s.view(np.uint32))
            assert np.all(sc[others] == -1.0) and np.all(pool_np[others] == SENTINEL)
        else:
            c, s = oracle.quantize_mxfp8(k_np)
            assert np.array_equal(got, c)
            sc = ks.cpu().numpy()
            assert np.array_equal(sc[slot_np], s)
            assert np.all(sc[others] == SENTINEL) and np.all(pool_np[others] == SENTINEL)


@pytest.mark.parametrize("fmt", ["fp8", "mxfp8"])
def test_prolog_feeds_the_indexer(dsa, fmt):
    """A prefill chunk end to end: the prolog projects the chunk's hidden vectors and writes
    their keys into the paged cache after a prefix, then the indexer scores the chunk's
    queries (the prolog's q and head weights) causally over prefix and chunk.  The oracle
    gets the same cache by quantizing the keys the prolog returned (its bytes must equal the
    GPU's) and the same q and w, and its Top-K must match the indexer's."""
    import dataclasses
    import torch
    from synth import make_inputs
    from synth.configs import Spec
    from synth.device import bits_of, to_device
    from tests.gpu_util import run_indexer, score_error
    from tests.helpers import rows_of
    P, L, H, D = 6000, 300, 64, 128
    spec = Spec(name=f"prolog_chunk_{fmt}", seq_lens=(P + L,), q_seq=(0,) * L,
                q_visible=tuple(P + i + 1 for i in range(L)),
                k_dtype="fp8" if fmt == "fp8" else "f32", k_std=1.0)
    inp = make_inputs(spec, seed=61, with_sfa=False)
    if fmt == "mxfp8":
        with np.errstate(invalid="ignore"):
            codes, sb = oracle.quantize_mxfp8(inp.k_pool)
        inp = dataclasses.replace(inp, spec=dataclasses.replace(spec, k_dtype="mxfp8"),
                                  k_pool=codes, k_scale=sb)
    d = to_device(inp)
    pi = make_prolog_inputs(L, 1024, H, D, seed=62)
    x = torch.from_numpy(pi.x.view(np.int16)).cuda().view(torch.bfloat16)
    W = torch.from_numpy(pi.w_proj.view(np.int16)).cuda().view(torch.bfloat16)
    g = torch.from_numpy(pi.gain).cuda()
    slots = rows_of(inp, 0, np.arange(P, P + L)).astype(np.int64)
    q, w, k = dsa.indexer_prolog(x, W, g, pi.eps, H, D, slot=torch.from_numpy(slots).cuda(),
                                 k_pool=d.k_pool, k_scale=d.k_scale, want_k=True)
    torch.cuda.synchronize()
    k_np = k.cpu().numpy()
    if fmt == "fp8":
        c, s = oracle.quantize_fp8_per_token(k_np)
    else:
        c, s = oracle.quantize_mxfp8(k_np)
    assert np.array_equal(d.k_pool.cpu().numpy()[slots], c)
    assert np.array_equal(d.k_scale.cpu().numpy()[slots].view(np.uint8), s.view(np.uint8))
    inp.k_pool[slots], inp.k_scale[slots] = c, s
    inp.q_idx[...] = bits_of(q)
    inp.w[...] = w.cpu().numpy()
    d.q_idx, d.w = q, w
    idx, score = run_indexer(dsa, inp, d)
    sample = [0, 1, 150, 298, 299]
    refs = oracle.indexer_topk(inp, sample)
    res = oracle.check_topk(idx, refs)
    err = max(score_error(score[r.t], idx[r.t], r) for r in refs)
    log(f"  prolog -> indexer ({fmt}): score err {err:.2e}")
    assert res.ok, res.msgs[:5]
    assert err <= 2e-6
