"""GPU parity of the cache writers against the oracle's codecs (bit-exact)."""
import numpy as np
import pytest
import torch

import oracle
from synth.device import bits_of

pytestmark = pytest.mark.gpu


def _slots(n, rows, rng):
    return torch.from_numpy(rng.choice(rows, size=n, replace=False).astype(np.int64)).cuda()


def test_store_index_keys_fp8_per_token(dsa):
    rng = np.random.default_rng(0)
    n, D, rows = 3000, 128, 4096
    x = rng.standard_normal((n, D)).astype(np.float32)
    x[0] = 0.0
    x[1] *= 1e-6
    x[2] *= 3e4
    x[3, :] = 2.0 ** -12                                  # subnormal codes after scaling
    x[4] = rng.integers(-8, 9, D).astype(np.float32)      # exact ties in the quotient
    slot = _slots(n, rows, rng)
    pool = torch.zeros((rows, D), dtype=torch.uint8, device="cuda")
    scale = torch.zeros(rows, dtype=torch.float32, device="cuda")
    dsa.store_index_keys(torch.from_numpy(x).cuda(), slot, pool, scale)
    torch.cuda.synchronize()
    codes, sc = oracle.quantize_fp8_per_token(x)
    s = slot.cpu().numpy()
    assert np.array_equal(bits_of(pool)[s], codes)
    assert np.array_equal(scale.cpu().numpy()[s], sc)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_store_index_keys_plain(dsa, dt):
    rng = np.random.default_rng(1)
    n, D, rows = 500, 64, 1000
    x = (rng.standard_normal((n, D)) * 10).astype(np.float32)
    slot = _slots(n, rows, rng)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    pool = torch.zeros((rows, D), dtype=tdt, device="cuda")
    dsa.store_index_keys(torch.from_numpy(x).cuda(), slot, pool)
    torch.cuda.synchronize()
    got = bits_of(pool)[slot.cpu().numpy()]
    want = oracle.encode_bf16_rne(x) if dt == "bf16" else x
    assert np.array_equal(got.view(np.uint8), want.view(np.uint8))


def test_store_kv_f32_to_bf16_and_copy(dsa):
    rng = np.random.default_rng(2)
    n, dqk, rows = 200, 576, 512
    x = rng.standard_normal((n, dqk)).astype(np.float32)
    slot = _slots(n, rows, rng)
    pool = torch.zeros((rows, dqk), dtype=torch.bfloat16, device="cuda")
    dsa.store_kv(torch.from_numpy(x).cuda(), slot, pool)
    torch.cuda.synchronize()
    s = slot.cpu().numpy()
    assert np.array_equal(bits_of(pool)[s], oracle.encode_bf16_rne(x))
    pool2 = torch.zeros_like(pool)
    src = pool[slot]
    dsa.store_kv(src, slot, pool2)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(pool2)[s], bits_of(pool)[s])
