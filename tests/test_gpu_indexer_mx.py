"""GPU parity of the MXFP8 indexer path (queries and keys quantized per group of 32 dims with
E8M0 scales; the kernel widens both exactly and scores them with bf16 MFMA products and fp32
sums) through the C ABI.

dsa_store_index_keys quantizes the keys on the GPU and must give the oracle's bytes
exactly; dsa_indexer_topk then reads the GPU-written keys, quantizes the query itself, and its
Top-K is compared with the oracle's over the oracle-quantized keys: bit-exact except for
positions within 1e-6 relative of the K-th score."""
import dataclasses
import zlib

import numpy as np
import pytest

import oracle
from synth import make_inputs, scaled_spec, workload
from synth.configs import Spec
from synth.device import to_device
from tests.gpu_util import log, run_indexer, score_error
from tests.helpers import rows_of

pytestmark = pytest.mark.gpu


def live_rows(inp):
    return np.concatenate([rows_of(inp, b, np.arange(n)) for b, n in enumerate(inp.spec.seq_lens)])


def mx_pair(dsa, inp):
    """(oracle-side inputs with the oracle's MXFP8 keys, device inputs with the keys the GPU
    writer produced from the same fp32 keys)."""
    import torch
    assert inp.spec.k_dtype == "f32"
    with np.errstate(invalid="ignore"):
        codes, sb = oracle.quantize_mxfp8(inp.k_pool)
    inp_mx = dataclasses.replace(inp, spec=dataclasses.replace(inp.spec, k_dtype="mxfp8"),
                                 k_pool=codes, k_scale=sb)
    d = to_device(inp)
    n, D = d.k_pool.shape
    kp = torch.zeros((n, D), dtype=torch.uint8, device=d.k_pool.device)
    ks = torch.zeros((n, D // 32), dtype=torch.uint8, device=d.k_pool.device)
    dsa.store_index_keys(d.k_pool, torch.arange(n, dtype=torch.int64, device=kp.device), kp, ks)
    torch.cuda.synchronize()
    live = live_rows(inp)
    assert np.array_equal(kp.cpu().numpy()[live], codes[live]), "GPU MXFP8 codes differ"
    assert np.array_equal(ks.cpu().numpy()[live], sb[live]), "GPU E8M0 bytes differ"
    d.k_pool, d.k_scale = kp, ks
    return inp_mx, d


def check(inp_mx, idx, score, strict=False):
    refs = oracle.indexer_topk(inp_mx)
    res = oracle.check_topk(idx, refs, strict=strict)
    err = max(score_error(score[t], idx[t], refs[t]) for t in range(len(refs)))
    log(f"  {inp_mx.spec.name}: score err {err:.2e}")
    assert res.ok, res.msgs[:5]
    assert err <= 1e-6


def test_store_index_keys_mx_is_bit_exact_on_edge_values(dsa):
    import torch
    rng = np.random.default_rng(31)
    n, D = 400, 128
    x = (rng.standard_normal((n, D)) * np.exp(rng.uniform(-60, 60, (n, 1)))).astype(np.float32)
    x[0] = 0.0
    x[1, :32] = 0.0
    x[2, :32] = np.ldexp(np.float32(1), np.arange(-20, 12))          # exact powers of two
    x[3, 32:64] = np.float32(500.0) * (np.arange(32) % 2 * 2 - 1)      # saturates: 500 > 448
    x[4, :] *= np.float32(1e-38)                                       # subnormal groups
    x[5, :] = np.float32(3e38) * np.sign(x[5, :])
    vals = oracle.fp8_e4m3_table()[:127]
    x[6, :32] = ((vals[90:122] + vals[91:123]) / 2).astype(np.float32)  # e4m3 rounding ties
    x[6, 31] = 256.0                                                  # scale 2^0
    x = x[np.isfinite(x).all(axis=1)]
    codes, sb = oracle.quantize_mxfp8(x)
    t = torch.from_numpy(x).cuda()
    slot = torch.from_numpy(np.arange(len(x))[::-1].copy()).cuda()
    kp = torch.zeros((len(x), D), dtype=torch.uint8, device="cuda")
    ks = torch.zeros((len(x), D // 32), dtype=torch.uint8, device="cuda")
    dsa.store_index_keys(t, slot, kp, ks)
    torch.cuda.synchronize()
    gc, gs = kp.cpu().numpy()[::-1], ks.cpu().numpy()[::-1]
    bad = np.nonzero((gc != codes).any(axis=1) | (gs != sb).any(axis=1))[0]
    log(f"  store MXFP8: {len(x)} rows, {len(bad)} differ")
    assert len(bad) == 0, bad[:8]


CASES = {
    "paged_bs64": lambda: scaled_spec(workload(4), seq_lens=[9000, 4000, 700], k_dtype="f32", k_std=1.0),
    "paged_bs32_k256": lambda: scaled_spec(workload(4), seq_lens=[6000, 2500], k_dtype="f32",
                                           block_size=32, top_k=256),
    "contiguous": lambda: scaled_spec(workload(4), seq_lens=[5000, 3000], k_dtype="f32",
                                      block_size=0, permute=False, extra_blocks=0),
    "ref_f32q": lambda: scaled_spec(workload(4), seq_lens=[3000], k_dtype="f32", q_dtype="f32"),
    "ref_h8_d64": lambda: scaled_spec(workload(4), seq_lens=[2000, 900], k_dtype="f32",
                                      idx_heads=8, idx_dim=64, top_k=100),
    # a chunk of 300 new queries over a 6000-token prefix (many queries, one sequence)
    "prefill_chunk_300": lambda: Spec(name="mx_chunk", seq_lens=(6300,), q_seq=(0,) * 300,
                                      q_visible=tuple(6000 + i + 1 for i in range(300)),
                                      k_dtype="f32", k_std=1.0),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_indexer_mx_matches_oracle(dsa, case):
    spec = CASES[case]()
    inp = make_inputs(spec, seed=zlib.crc32(case.encode()) % 997, with_sfa=False)
    log(f"case mx {case}: T={spec.num_queries} H={spec.idx_heads} D={spec.idx_dim} K={spec.top_k}")
    inp_mx, d = mx_pair(dsa, inp)
    idx, score = run_indexer(dsa, inp_mx, d)
    check(inp_mx, idx, score)


def test_indexer_mx_integer_exact_is_bit_exact(dsa):
    """Small-integer queries and keys quantize losslessly and every product sum is exact in
    fp32, so the Top-K (ties included) must match the oracle exactly."""
    from synth.generate import to_bf16_bits
    spec = scaled_spec(workload(4), seq_lens=[8000, 3000], k_dtype="f32")
    inp = make_inputs(spec, seed=5, with_sfa=False)
    rng = np.random.default_rng(6)
    inp.q_idx[...] = to_bf16_bits(rng.integers(-8, 9, size=inp.q_idx.shape).astype(np.float32))
    inp.w[...] = rng.choice(np.array([-2, -1, -0.5, 0.5, 1, 2], np.float32), size=inp.w.shape)
    for b, n in enumerate(spec.seq_lens):
        inp.k_pool[rows_of(inp, b, np.arange(n))] = rng.integers(-8, 9, size=(n, 128)).astype(np.float32)
    inp_mx, d = mx_pair(dsa, inp)
    idx, score = run_indexer(dsa, inp_mx, d)
    check(inp_mx, idx, score, strict=True)


@pytest.mark.slow
def test_full_size_decode_mx_sampled(dsa):
    """The 128K quantized-decode shape with MXFP8 keys (values N(0,1) before quantization);
    two queries checked."""
    spec = dataclasses.replace(workload(4), k_dtype="f32")
    inp = make_inputs(spec, seed=4, with_sfa=False)
    inp_mx, d = mx_pair(dsa, inp)
    idx, score = run_indexer(dsa, inp_mx, d)
    sample = [0, spec.num_queries - 1]
    refs = oracle.indexer_topk(inp_mx, sample)
    res = oracle.check_topk(idx, refs)
    assert res.ok, res.msgs[:5]
