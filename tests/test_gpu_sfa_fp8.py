"""GPU parity of the fp8 latent KV path (rows quantized per token and per 128-column tile,
include/dsa.h DSA_KV_FP8_ROW_BYTES) through the C ABI.

The cache writer dsa_store_kv quantizes on the GPU and must give the oracle's bytes exactly;
dsa_sparse_attn then reads the GPU-written rows and is compared with the oracle's attention
over the oracle-quantized rows, within the bf16 bound (2e-2 on O, 1e-4 on LSE): the kernel
widens codes times power-of-two scales exactly, so the arithmetic is the bf16 path's."""
import dataclasses
import zlib

import numpy as np
import pytest

import oracle
from synth import make_inputs, scaled_spec, workload
from synth.device import to_device
from tests.gpu_util import log, run_indexer, run_sfa
from tests.helpers import rows_of
from tests.test_gpu_sfa import check, oracle_idx

pytestmark = pytest.mark.gpu


def live_rows(inp):
    return np.concatenate([rows_of(inp, b, np.arange(n)) for b, n in enumerate(inp.spec.seq_lens)])


def fp8_pair(dsa, inp):
    """(oracle-side inputs holding the oracle's fp8 rows, device inputs holding the rows that
    the GPU writer produced from the same bf16 pool)."""
    import torch
    kv = oracle.decode(inp.kv_pool, "bf16").astype(np.float32)
    with np.errstate(invalid="ignore"):
        rows8 = oracle.quantize_kv_fp8_rows(kv)
    inp8 = dataclasses.replace(inp, spec=dataclasses.replace(inp.spec, kv_dtype="fp8"), kv_pool=rows8)
    d = to_device(inp)
    n = d.kv_pool.shape[0]
    pool8 = torch.zeros((n, oracle.KV_FP8_ROW_BYTES), dtype=torch.uint8, device=d.kv_pool.device)
    dsa.store_kv(d.kv_pool, torch.arange(n, dtype=torch.int64, device=pool8.device), pool8)
    torch.cuda.synchronize()
    live = live_rows(inp)
    got = pool8.cpu().numpy()
    assert np.array_equal(got[live], rows8[live]), "GPU fp8 rows differ from the oracle's"
    d.kv_pool = pool8
    return inp8, d


def test_store_kv_fp8_is_bit_exact_on_edge_values(dsa):
    """fp32 and bf16 sources with zero tiles, tile maxima on and next to the scale
    boundaries 448 * 2^k and 1.75 * 2^k, subnormal and huge magnitudes, rounding ties."""
    import torch
    rng = np.random.default_rng(21)
    n = 512
    x = (rng.standard_normal((n, 576)) * np.exp(rng.uniform(-40, 40, (n, 1)))).astype(np.float32)
    x[0, :] = 0.0
    x[1, :128] = 0.0
    x[2, 0] = 448.0 * 2.0 ** -10
    x[3, 130] = np.nextafter(np.float32(448.0 * 2.0 ** 5), np.float32(np.inf))
    x[4, 300] = 1.75 * 2.0 ** 3
    x[5, 400] = np.nextafter(np.float32(1.75 * 2.0 ** 3), np.float32(0))
    x[6, :] *= np.float32(1e-36)
    x[7, :] = np.float32(3e38) * np.sign(x[7, :])
    x[8, :128] = np.float32(448.0) * (np.arange(128) % 2 * 2 - 1)
    # e4m3 rounding ties at scale 1: midpoints between neighbouring codes
    vals = oracle.fp8_e4m3_table()[:127]
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    x[9, :126] = mids
    x[9, 127] = 448.0
    x = x[np.isfinite(x).all(axis=1)]
    ref = oracle.quantize_kv_fp8_rows(x)
    for src in ("f32", "bf16"):
        xs = x if src == "f32" else oracle.decode_bf16(oracle.encode_bf16_rne(x)).astype(np.float32)
        refs = ref if src == "f32" else oracle.quantize_kv_fp8_rows(xs)
        if src == "f32":
            t = torch.from_numpy(xs).cuda()
        else:
            t = torch.from_numpy(oracle.encode_bf16_rne(xs).view(np.int16)).cuda().view(torch.bfloat16)
        slot = torch.from_numpy(np.arange(len(xs))[::-1].copy()).cuda()
        pool = torch.zeros((len(xs), oracle.KV_FP8_ROW_BYTES), dtype=torch.uint8, device="cuda")
        dsa.store_kv(t, slot, pool)
        torch.cuda.synchronize()
        got = pool.cpu().numpy()[::-1]
        bad = np.nonzero((got != refs).any(axis=1))[0]
        log(f"  store fp8 from {src}: {len(xs)} rows, {len(bad)} differ")
        assert len(bad) == 0, bad[:8]


CASES = {
    "h128_T3": (lambda: scaled_spec(workload(2), seq_lens=[5000, 2500, 40000]), "sharp"),
    "h128_T40": (lambda: scaled_spec(workload(2), seq_lens=[3000] * 40), "sharp"),
    "h32_k100": (lambda: scaled_spec(workload(2), seq_lens=[500, 700], sfa_heads=32, top_k=100),
                 "sharp"),
    "h64_config": (lambda: scaled_spec(workload(4), seq_lens=[9000, 4000], sfa_heads=64), "config"),
    "h128_T260_whole": (lambda: scaled_spec(workload(2), seq_lens=[300] * 260, top_k=256), "sharp"),
    "ref_h8": (lambda: scaled_spec(workload(2), seq_lens=[900], sfa_heads=8, top_k=300), "sharp"),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_sfa_fp8_kv_matches_oracle(dsa, case):
    mk, dist = CASES[case]
    spec = mk()
    inp = make_inputs(spec, seed=zlib.crc32(case.encode()) % 997, sfa_dist=dist)
    idx = oracle_idx(inp, seed=3, minus_one_frac=0.05)
    log(f"case fp8 {case}: T={spec.num_queries} H={spec.sfa_heads} K={spec.top_k}")
    inp8, d = fp8_pair(dsa, inp)
    O, lse = run_sfa(dsa, inp8, idx, d)
    check(inp8, idx, O, lse)


def test_sfa_fp8_kv_far_maximum_takes_the_reference_fixup(dsa):
    """As for bf16 rows: a late-selected row scaled by 64 pushes its logits far past the
    exponent headroom, its heads are recomputed by the reference method (which reads the fp8
    rows too), and a second call on the same workspace gives the same result.  |O| reaches
    ~50, so the bound is relative, as in the bf16 test."""
    spec = scaled_spec(workload(2), seq_lens=[5000, 4000])
    inp = make_inputs(spec, seed=11, sfa_dist="sharp")
    idx = oracle_idx(inp, seed=5)
    r = rows_of(inp, 0, [int(idx[0, spec.top_k - 1])])[0]
    inp.kv_pool[r] = oracle.encode_bf16_rne(oracle.decode(inp.kv_pool[r], "bf16") * 64.0)
    inp8, d = fp8_pair(dsa, inp)
    ws = dsa.zeroed_workspace(dsa.sfa_workspace_bytes(spec.num_queries, spec.sfa_heads,
                                                      spec.top_k, spec.d_v), "cuda")
    O1, L1 = run_sfa(dsa, inp8, idx, d, workspace=ws)
    O2, L2 = run_sfa(dsa, inp8, idx, d, workspace=ws)
    Oref, Lref = oracle.sfa(inp8, idx, list(range(spec.num_queries)))
    scale = np.maximum(np.abs(Oref).max(axis=-1, keepdims=True), 1.0)
    rel = np.abs(O1 - Oref) / scale
    log(f"  fp8: max |dO|/max|O| per head {rel.max():.2e}, max |dLSE| {np.abs(L1 - Lref).max():.2e}")
    assert rel.max() <= 2e-2 / 4
    assert np.all(np.abs(L1 - Lref) <= 1e-4 * np.maximum(1.0, np.abs(Lref)))
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


@pytest.mark.slow
def test_full_size_decode_fp8_kv_sampled(dsa):
    """The 128K quantized-decode workload with its latent cache stored as fp8 rows; the
    indexer's own index list drives SFA; two queries checked."""
    inp = make_inputs(workload(4), seed=4)
    idx, _ = run_indexer(dsa, inp)
    inp8, d = fp8_pair(dsa, inp)
    sample = [0, inp.spec.num_queries - 1]
    O, lse = run_sfa(dsa, inp8, idx, d)
    check(inp8, idx, O, lse, queries=sample)
