"""The benchmark's algorithmic byte and flop counts (the numerators of its roofline figures),
recomputed by hand for small workloads, and its one-GPU contract."""
import math
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synth import scaled_spec, workload  # noqa: E402


def test_indexer_bytes_by_hand():
    # fp8 keys: 128 code bytes + a 4-byte scale per visible token, one 4-byte block-table entry
    # per 64-token page, the bf16 query (64 x 128 x 2) and fp32 head weights (64 x 4), the
    # 2048-entry index list
    spec = scaled_spec(workload(4), seq_lens=[1000, 64])
    want = (1000 * 132 + 4 * 16 + 64 * (256 + 4) + 4 * 2048) + (64 * 132 + 4 * 1 + 64 * 260 + 4 * 2048)
    assert bench.indexer_bytes(spec, [1000, 64]) == want
    # bf16 keys, contiguous layout: 256 bytes per token, no block table
    spec = scaled_spec(workload(2), seq_lens=[777], block_size=0, permute=False, extra_blocks=0)
    assert bench.indexer_bytes(spec, [777]) == 777 * 256 + 64 * 260 + 4 * 2048
    # MXFP8 keys: 128 codes + 4 scale bytes (one per 32 dims)
    spec = scaled_spec(workload(4), seq_lens=[100], k_dtype="mxfp8")
    assert bench.indexer_bytes(spec, [100]) == 100 * 132 + 4 * 2 + 64 * 260 + 4 * 2048


def test_sfa_bytes_and_flops_by_hand():
    spec = scaled_spec(workload(4), seq_lens=[5000, 100])
    # index list, K_eff selected 1152-byte bf16 rows, bf16 queries (128 x 576) and outputs (128 x 512)
    want = sum(4 * 2048 + min(2048, v) * 1152 + 128 * (576 * 2 + 512 * 2) for v in (5000, 100))
    assert bench.sfa_bytes(spec, [5000, 100]) == want
    assert bench.sfa_flops(spec, [5000, 100]) == sum(2 * 128 * min(2048, v) * (576 + 512) for v in (5000, 100))
    # fp8 latent rows are 656 bytes
    spec8 = scaled_spec(workload(4), seq_lens=[5000], kv_dtype="fp8")
    assert bench.sfa_bytes(spec8, [5000]) == 4 * 2048 + 2048 * 656 + 128 * (576 * 2 + 512 * 2)


def test_indexer_flops_by_hand():
    spec = scaled_spec(workload(3), seq_lens=[70000], q_seq=(0, 0), q_visible=(65537, 65538))
    assert bench.indexer_flops(spec, [65537, 65538]) == 2 * 64 * 128 * (65537 + 65538)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_committed_counter_summary_matches_the_kernel_sources():
    """The committed rocprofv3 counter summary (FETCH_SIZE and WRITE_SIZE, scaled by a copy
    kernel's reading) was taken on the current kernel sources, so the bench line of its workload
    carries counter-measured HBM traffic for both calls of the decode step."""
    idx, wl = bench.counter_traffic("indexer")
    sfa, wl_sfa = bench.counter_traffic("sparse_attn")
    assert wl == wl_sfa == workload(4).name
    assert idx is not None and sfa is not None, "counters were taken on other kernel sources"
    spec = workload(4)
    from synth import make_inputs
    V = [int(v) for v in make_inputs(spec, seed=4, with_sfa=False).q_visible]
    alg = bench.indexer_bytes(spec, V)
    # the keys are read once: the measured traffic is the algorithmic bytes plus a few percent
    assert alg <= idx <= 1.25 * alg
