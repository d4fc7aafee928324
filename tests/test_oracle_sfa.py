"""Pins of the oracle's sparse attention against a hand-worked example, torch's CPU scaled
dot-product attention in float64 (a library routine) when every position is selected,
closed forms (one row, identical rows, two rows with a known logit gap), a long-double
softmax without max subtraction, and mutation checks showing the 2e-2 bf16 bound rejects
plausible mistakes on the sharp parity distribution."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from synth import make_inputs, scaled_spec, workload
from tests.helpers import rows_of

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _num(x):
    if isinstance(x, str):
        if x.startswith("ln"):
            return math.log(float(x[2:]))
        return float(Fraction(x))
    return float(x)


def test_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "sfa_worked_example.json")))
    q = np.array([[_num(v) for v in r] for r in g["q"]])
    rows = np.array([[_num(v) for v in r] for r in g["rows"]])
    O, lse = oracle.sfa_dense(q, rows, g["scale"], g["d_v"])
    want = np.array([[_num(v) for v in r] for r in g["O"]])
    assert np.allclose(O, want, rtol=1e-14, atol=1e-14)
    assert np.allclose(lse, [_num(v) for v in g["lse"]], rtol=1e-14)


def test_all_selected_equals_dense_sdpa():
    rng = np.random.default_rng(0)
    H, n, dqk, dv = 6, 77, 576, 512
    q = rng.standard_normal((H, dqk)) * 2
    rows = rng.standard_normal((n, dqk)) * 0.3
    scale = 1 / 24
    O, lse = oracle.sfa_dense(q, rows, scale, dv)
    tq = torch.from_numpy(q)[None, :, None, :]                   # [1, H, 1, dqk]
    tk = torch.from_numpy(rows)[None, None].expand(1, H, n, dqk)
    tv = torch.from_numpy(rows[:, :dv])[None, None].expand(1, H, n, dv)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)[0, :, 0].numpy()
    assert np.allclose(O, ref, rtol=1e-12, atol=1e-13)
    from scipy.special import logsumexp
    assert np.allclose(lse, logsumexp(scale * q @ rows.T, axis=1), rtol=1e-13)


def test_single_row_and_identical_rows():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((4, 576)) * 8
    r = rng.standard_normal((1, 576))
    O, lse = oracle.sfa_dense(q, r, 1 / 24, 512)
    assert np.array_equal(O, np.broadcast_to(r[:, :512], (4, 512)))
    assert np.allclose(lse, (q @ r[0]) / 24)
    O3, lse3 = oracle.sfa_dense(q, np.repeat(r, 5, axis=0), 1 / 24, 512)
    assert np.allclose(O3, O, rtol=1e-15, atol=0)
    assert np.allclose(lse3, lse + math.log(5))


def test_two_rows_logit_gap():
    q = np.zeros((1, 576))
    q[0, 575] = 1.0
    a = np.zeros(576)
    b = np.zeros(576)
    a[0], b[0] = 1.0, 0.0
    for delta in (0.0, 0.7, 3.0):
        b[575] = delta * 24                         # logit gap delta at scale 1/24
        O, _ = oracle.sfa_dense(q, np.stack([a, b]), 1 / 24, 512)
        sig = 1 / (1 + math.exp(delta))             # weight of row a
        assert abs(O[0, 0] - sig) < 1e-15


def test_long_double_naive_softmax():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((3, 8))
    rows = rng.standard_normal((9, 8))
    O, lse = oracle.sfa_dense(q, rows, 0.5, 5)
    ql, rl = q.astype(np.longdouble), rows.astype(np.longdouble)
    e = np.exp(np.longdouble(0.5) * (ql @ rl.T))
    ref = (e @ rl[:, :5]) / e.sum(axis=1, keepdims=True)
    assert np.allclose(O, ref.astype(np.float64), rtol=1e-14, atol=1e-15)
    assert np.allclose(lse, np.log(e.sum(axis=1)).astype(np.float64), rtol=1e-14)


def test_empty_selection():
    O, lse = oracle.sfa_dense(np.ones((2, 4)), np.zeros((0, 4)), 1.0, 3)
    assert np.all(O == 0) and np.all(np.isneginf(lse))


def test_sfa_query_skips_minus_one_and_reads_through_block_table():
    spec = scaled_spec(workload(2), seq_lens=[300, 200], sfa_heads=4, top_k=8)
    inp = make_inputs(spec, seed=4, sfa_dist="sharp")
    idx = np.array([5, -1, 250, 7, -1, 0, 299, 64], np.int64)
    O, lse = oracle.sfa_query(inp, 0, idx)
    keep = idx[idx != -1]
    R = oracle.decode(inp.kv_pool[rows_of(inp, 0, keep)], "bf16")
    assert not np.isnan(R).any()
    O2, lse2 = oracle.sfa_dense(oracle.decode(inp.q_sfa[0], "bf16"), R, spec.softmax_scale, 512)
    assert np.array_equal(O, O2) and np.array_equal(lse, lse2)


def test_mutations_fail_the_bf16_bound_on_sharp_inputs():
    """The sharp SFA distribution makes the 2e-2 bound discriminating: a zero output, a
    dropped softmax scale and values taken 64 columns off all fail it, while rounding the
    correct output to bf16 passes with a wide margin."""
    spec = scaled_spec(workload(2), seq_lens=[3000], sfa_heads=16, top_k=2048)
    inp = make_inputs(spec, seed=8, sfa_dist="sharp")
    rng = np.random.default_rng(0)
    idx = np.sort(rng.choice(3000, 2048, replace=False))
    O, lse = oracle.sfa_query(inp, 0, idx)
    rows = oracle.decode(inp.kv_pool[rows_of(inp, 0, idx)], "bf16")
    q = oracle.decode(inp.q_sfa[0], "bf16")
    assert np.abs(O).max() < 2.0
    o_bf16 = oracle.decode_bf16(oracle.encode_bf16_rne(O.astype(np.float32)))
    assert oracle.check_attention(o_bf16, O, 2e-2).max_abs < 2e-3
    assert not oracle.check_attention(np.zeros_like(O), O, 2e-2).ok
    O_noscale, _ = oracle.sfa_dense(q, rows, 1.0, 512)
    assert not oracle.check_attention(O_noscale, O, 2e-2).ok
    O_shift, _ = oracle.sfa_dense(q, np.roll(rows, -64, axis=1), spec.softmax_scale, 512)
    assert not oracle.check_attention(O_shift, O, 2e-2).ok


def test_fp8_rows_path_equals_the_f32_path_on_representable_rows():
    """SFA over fp8 latent rows reads the row through the tile scales: with rows whose values
    are exactly representable (e4m3 codes times powers of two, bf16 rope), the fp8 path and
    the fp32 path over the same values give identical results; a row read with a wrong tile
    scale, or with the rope columns misplaced, would not."""
    import dataclasses
    spec = scaled_spec(workload(1), seq_lens=[700], sfa_heads=16, top_k=64, block_size=64,
                       permute=True, extra_blocks=1)
    inp = make_inputs(spec, seed=11, sfa_dist="sharp")
    rng = np.random.default_rng(12)
    rows = rows_of(inp, 0, np.arange(700))
    codes = rng.integers(0, 127, size=(700, 512)) | (rng.integers(0, 2, (700, 512)) << 7)
    codes[:, ::128] = 0x7E
    e = rng.integers(-12, -4, size=(700, 4))
    vals = oracle.decode_fp8_e4m3(codes.astype(np.uint8)).reshape(700, 4, 128) * np.ldexp(1.0, e)[:, :, None]
    rope = oracle.decode_bf16(oracle.encode_bf16_rne(rng.standard_normal((700, 64)).astype(np.float32) * 0.05))
    x = np.concatenate([vals.reshape(700, 512), rope], axis=1).astype(np.float32)
    inp.kv_pool[rows] = x
    pool8 = np.zeros((inp.kv_pool.shape[0], oracle.KV_FP8_ROW_BYTES), np.uint8)
    pool8[rows] = oracle.quantize_kv_fp8_rows(x)
    q_bf16 = oracle.encode_bf16_rne(inp.q_sfa)
    inp.q_sfa[...] = oracle.decode_bf16(q_bf16)
    inp8 = dataclasses.replace(inp, spec=dataclasses.replace(spec, kv_dtype="fp8"), kv_pool=pool8,
                               q_sfa=q_bf16)
    idx = rng.choice(700, size=(1, 64), replace=False)
    O32, L32 = oracle.sfa(inp, idx)
    O8, L8 = oracle.sfa(inp8, idx)
    assert np.array_equal(O8, O32) and np.array_equal(L8, L32)
    # a swapped pair of tile scales changes the result
    bad = pool8.copy()
    bad[rows, 640:644], bad[rows, 644:648] = pool8[rows, 644:648], pool8[rows, 640:644]
    Ob, _ = oracle.sfa(dataclasses.replace(inp8, kv_pool=bad), idx)
    assert np.abs(Ob - O32).max() > 1e-3
