"""GPU parity of the non-FP8 (bfloat16) ring against the oracle's bf16 mode.

The same call sequences as the FP8 parity cases, with the cache storing the
rotated keys and the values as bfloat16. Stored bf16 bit patterns, positions,
the power-of-two factors in the scale slots and the ring counters must match
bit for bit; attention must meet the bar stated in gpu_helpers (against fp64
attention over the GPU's own bf16 cache).
"""
import numpy as np
import pytest
import torch

from streaming_fp8_kv_amd import workloads as W
from tests.gpu_helpers import Mirror, say, spread_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sfkv():
    from streaming_fp8_kv_amd import sfkv as lib
    return lib


_ROPES = {}


def rope_for(sfkv, shape):
    key = (shape.head_dim, shape.max_position, shape.rope_base)
    if key not in _ROPES:
        _ROPES[key] = sfkv.Rope(shape.head_dim, shape.max_position, shape.rope_base)
    return _ROPES[key]


def test_bf16_tiny_session_wrap_and_resets(sfkv):
    """1 head, d=64, 16 tokens per frame into 64 slots, resets every 3 steps."""
    spec = W.TINY
    say(f"case bf16 {spec.name}")
    m = Mirror(sfkv, rope_for(sfkv, spec.shape), spec, storage="bf16")
    fs = W.FrameStream(spec)
    for step in range(spec.steps):
        q, k, v = fs.frame()
        if step == 0:
            m.calibrate(k, v)
        if step > 0 and step % spec.reset_period == 0:
            m.rebase(m.ora.next_pos)
            m.check_cache(f"step {step} after rebase")
        m.write(k, v)
        m.check_cache(f"step {step}")
        m.check_attend(q, tag=f"step {step}")


def test_bf16_production_call(sfkv):
    """24 heads x 128, 757 new tokens into 5,788 slots after 8 prefill frames."""
    spec = W.PROD
    say(f"case bf16 {spec.name}")
    m = Mirror(sfkv, rope_for(sfkv, spec.shape), spec, storage="bf16")
    fs = W.FrameStream(spec)
    for step in range(spec.steps):
        q, k, v = fs.frame()
        if step == 0:
            m.calibrate(k, v)
        m.write(k, v)
        m.check_cache(f"frame {step}")
        if step in (0, 7, spec.steps - 1):
            m.check_attend(q, rows=spread_rows(q.shape[0], 96), tag=f"frame {step}")
    st = m.gpu.state()
    assert st["n_valid"] == 5788 and st["write_slot"] == (9 * 757) % 5788


def test_bf16_long_session_with_resets(sfkv):
    """200 steps of 757 tokens with a rebase to 0 every 42 steps; three heads
    mirrored, attention around every reset."""
    spec = W.LONG
    heads = [0, 11, 23]
    say(f"case bf16 {spec.name}")
    m = Mirror(sfkv, rope_for(sfkv, spec.shape), spec, heads=heads, storage="bf16")
    fs = W.FrameStream(spec)
    attend_steps = {0, 41, 42, 43, 84, 126, 168, 199}
    for step in range(spec.steps):
        q, k, v = fs.frame()
        if step == 0:
            m.calibrate(k, v)
        if step > 0 and step % spec.reset_period == 0:
            m.rebase(m.ora.next_pos)
        m.write(k, v)
        m.check_cache(f"step {step}")
        if step in attend_steps:
            m.check_attend(q, rows=spread_rows(q.shape[0], 48), tag=f"step {step}")


def test_bf16_stress_heavy_tails(sfkv):
    """40 heads, Student-t(3) inputs with per-head std up to 8 and a variable
    first write: values far beyond the calibration frame's absmax stay exact
    in bf16 and inside the fp16 range the attention moves them to."""
    spec = W.STRESS
    heads = [0, 13, 26, 39]
    say(f"case bf16 {spec.name}")
    fs = W.FrameStream(spec)
    n0 = fs.first_length()
    m = Mirror(sfkv, rope_for(sfkv, spec.shape), spec, heads=heads, storage="bf16")
    for step in range(spec.steps):
        q, k, v = fs.frame(n0 if step == 0 else None)
        if step == 0:
            m.calibrate(k, v)
        m.write(k, v)
        if step in (0, 1, 25, spec.steps - 1):
            m.check_cache(f"step {step}")
            m.check_attend(q, rows=spread_rows(q.shape[0], 48), tag=f"step {step}")


def test_bf16_values_far_above_calibration(sfkv):
    """Frames after calibration carry values 64x the calibration frame's: the
    power-of-two factor leaves that much headroom below the fp16 limit, so the
    attention over them is still exact to the bar."""
    shape = W.CacheShape(4, 128, 512, 128, max_position=4096)
    spec = W.WorkloadSpec(name="bf16_growth", shape=shape, seed=21, dtype=torch.float32, dist="normal",
                          sigma_q=(0.5, 2.0), sigma_kv=(0.5, 2.0), steps=5)
    say("case bf16_growth_h4_d128_c512")
    m = Mirror(sfkv, rope_for(sfkv, shape), spec, storage="bf16")
    fs = W.FrameStream(spec)
    for step in range(spec.steps):
        q, k, v = fs.frame()
        if step == 0:
            m.calibrate(k, v)
        else:
            v = v * 64.0
        m.write(k, v)
        m.check_cache(f"step {step}")
        m.check_attend(q, tag=f"step {step}")
    sc = m.gpu.scales().cpu().numpy()
    assert np.all(sc[0] * sc[1] == 1.0) and np.all(sc[2] * sc[3] == 1.0)


@pytest.mark.parametrize("heads,d,cap,max_new,lens", [
    (3, 128, 1000, 1000, [1000, 1, 37, 999]),
    (5, 128, 333, 64, [1, 1, 64, 63, 64, 64, 64, 64, 2]),
    (2, 64, 4096, 700, [700, 129, 700, 700, 700, 700, 700]),
])
def test_bf16_ragged_shapes(sfkv, heads, d, cap, max_new, lens):
    """Single-token and whole-ring writes, capacities off the 64-key tile,
    head_dim 64, a rebase in the middle; every call checked in full."""
    say(f"case bf16 ragged_h{heads}_d{d}_c{cap}_max{max_new}")
    shape = W.CacheShape(heads, d, cap, max_new, max_position=16384)
    spec = W.WorkloadSpec(name="ragged", shape=shape, seed=31 + heads, dtype=torch.bfloat16, dist="normal",
                          sigma_q=(0.5, 4.0), sigma_kv=(0.5, 4.0), steps=len(lens))
    m = Mirror(sfkv, rope_for(sfkv, shape), spec, storage="bf16")
    fs = W.FrameStream(spec)
    for step, n in enumerate(lens):
        q, k, v = fs.frame(n)
        if step == 0:
            m.calibrate(k, v)
        if step == len(lens) // 2:
            m.rebase(7)
            m.check_cache(f"step {step} after rebase")
        m.write(k, v)
        m.check_cache(f"step {step}")
        m.check_attend(q, tag=f"step {step} n={n}")
