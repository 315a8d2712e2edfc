"""Shapes off the workload grid, against the oracle: seeded random
configurations (heads, head_dim, capacity, write lengths, a rebase, both
storages, both entry points) checked in full after every call, and one large
ring whose offsets pass 2^27 bytes, checked on sampled query rows.
"""
import numpy as np
import pytest
import torch

from streaming_fp8_kv_amd import workloads as W
from tests.gpu_helpers import Mirror, attention_error, A_MAX, B_MEAN, say, spread_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sfkv():
    from streaming_fp8_kv_amd import sfkv as lib
    return lib


def _random_case(seed):
    rng = np.random.default_rng(seed)
    heads = int(rng.integers(1, 7))
    d = int(rng.choice([64, 128]))
    cap = int(rng.integers(1, 700))
    max_new = int(rng.integers(1, cap + 1))
    lens = [int(rng.integers(1, max_new + 1)) for _ in range(int(rng.integers(2, 7)))]
    rebase_at = int(rng.integers(1, len(lens)))
    storage = "bf16" if rng.integers(0, 2) else "fp8"
    dtype = torch.bfloat16 if rng.integers(0, 2) else torch.float32
    return heads, d, cap, max_new, lens, rebase_at, storage, dtype


@pytest.mark.parametrize("seed", range(12))
def test_random_shapes(sfkv, seed):
    heads, d, cap, max_new, lens, rebase_at, storage, dtype = _random_case(1000 + seed)
    say(f"case random seed {seed}: h{heads} d{d} c{cap} max{max_new} lens {lens} rebase before {rebase_at} "
        f"{storage} {str(dtype).split('.')[-1]}")
    shape = W.CacheShape(heads, d, cap, max_new, max_position=8192)
    spec = W.WorkloadSpec(name="random", shape=shape, seed=2000 + seed, dtype=dtype, dist="normal",
                          sigma_q=(0.5, 4.0), sigma_kv=(0.5, 4.0), steps=len(lens))
    rope = sfkv.Rope(d, shape.max_position)
    m = Mirror(sfkv, rope, spec, storage=storage)
    fs = W.FrameStream(spec)
    for step, n in enumerate(lens):
        q, k, v = fs.frame(n)
        if step == 0:
            m.calibrate(k, v)
        if step == rebase_at:
            m.rebase(int(np.random.default_rng(seed).integers(0, m.ora.next_pos + 1)))
            m.check_cache(f"step {step} after rebase")
        if step % 2:
            out = m.gpu.write_attend(k.cuda(), v.cuda(), q.cuda())
            m.ora.write(m._sub(k), m._sub(v))
            m.check_cache(f"step {step}")
            torch.cuda.synchronize()
            got = out.cpu().numpy()
            ref = m.reference_from_gpu_cache(q, np.arange(n))
            a, b = attention_error(got, ref)
            say(f"  step {step} n={n} (fused): A={a:.2e} B={b:.2e}")
            assert a <= A_MAX and b <= B_MEAN
        else:
            m.write(k, v)
            m.check_cache(f"step {step}")
            m.check_attend(q, tag=f"step {step} n={n}")


def test_large_ring_sampled(sfkv):
    """2 heads x 128 dims, 600,000 slots (a 153.6 MB plane, offsets past 2^27),
    filled by five 120,000-token writes then wrapped by a sixth; the last
    write's attention is checked on 24 sampled query rows."""
    heads, d, cap, n = 2, 128, 600_000, 120_000
    shape = W.CacheShape(heads, d, cap, n, max_position=1 << 20)
    spec = W.WorkloadSpec(name="large", shape=shape, seed=31, dtype=torch.bfloat16, dist="normal",
                          sigma_q=(0.5, 2.0), sigma_kv=(0.5, 2.0), steps=6)
    say(f"case large ring h{heads} d{d} c{cap} n{n}")
    rope = sfkv.Rope(d, shape.max_position)
    m = Mirror(sfkv, rope, spec)
    fs = W.FrameStream(spec)
    for step in range(6):
        q, k, v = fs.frame()
        if step == 0:
            m.calibrate(k, v)
        m.write(k, v)
    st = m.gpu.state()
    assert st["n_valid"] == cap and st["write_slot"] == (6 * n) % cap
    m.check_cache("after 6 writes")
    m.check_attend(q, rows=spread_rows(n, 24), tag="last write")


@pytest.mark.parametrize("storage", ["fp8", "bf16"])
def test_degenerate_heads(sfkv, storage):
    """Head 0 all zeros (scale 1, every score 0, uniform weights over zero
    values: output exactly 0), head 1 with the same raw key at every position
    and one constant value (whatever the weights, the output is that value),
    head 2 ordinary; four writes that wrap a 96-slot ring, checked in full
    against the oracle."""
    heads, d, cap, n = 3, 64, 96, 40
    shape = W.CacheShape(heads, d, cap, n, max_position=4096)
    spec = W.WorkloadSpec(name="degenerate", shape=shape, seed=51, dtype=torch.float32, dist="normal",
                          sigma_q=None, sigma_kv=None, steps=4)
    say(f"case degenerate heads {storage}")
    rope = sfkv.Rope(d, shape.max_position)
    m = Mirror(sfkv, rope, spec, storage=storage)
    fs = W.FrameStream(spec)
    key = torch.linspace(-1.5, 1.5, d)
    for step in range(spec.steps):
        q, k, v = fs.frame()
        q[:, 0], k[:, 0], v[:, 0] = 0.0, 0.0, 0.0
        k[:, 1] = key                    # the same raw key at every position (rotated differently)
        v[:, 1] = 0.75
        if step == 0:
            m.calibrate(k, v)
        m.write(k, v)
        m.check_cache(f"step {step}")
        out = m.check_attend(q, tag=f"step {step}")
        o = out.cpu()
        assert torch.all(o[:, 0] == 0.0), "an all-zero head must attend to zeros"
        assert torch.allclose(o[:, 1], torch.full_like(o[:, 1], 0.75), rtol=0, atol=1e-6)
