"""GPU parity of the HIP path against the oracle, through the C ABI.

Cases follow the synthetic workloads: the tiny wrap-and-reset session, the
production-shape call, the long session with resets every 42 steps, the
heavy-tailed 40-head stress session with a variable first write, and the
240-call sweep in the launch configuration the benchmark times. Bytes,
positions, scales and ring counters must match bit for bit; attention must meet
the bar stated in gpu_helpers.
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


def test_tiny_session_wrap_and_resets(sfkv):
    """1 head, d=64, 16 tokens per frame, 64 slots (wraps after 4 frames), 10 steps,
    positions reset before steps 3, 6 and 9; every call checked in full."""
    spec = W.TINY
    say(f"case {spec.name}")
    m = Mirror(sfkv, rope_for(sfkv, spec.shape), spec)
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


def test_production_call(sfkv):
    """24 heads x 128, 757 new tokens into 5,788 slots after 8 prefill frames."""
    spec = W.PROD
    say(f"case {spec.name}")
    m = Mirror(sfkv, rope_for(sfkv, spec.shape), spec)
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


def test_long_session_with_resets(sfkv):
    """200 steps of 757 tokens, rebase to 0 before steps 42, 84, 126 and 168.
    Bytes of three heads are checked every step; attention at every reset step,
    the step before it and a few ordinary steps."""
    spec = W.LONG
    heads = [0, 11, 23]
    say(f"case {spec.name}")
    m = Mirror(sfkv, rope_for(sfkv, spec.shape), spec, heads=heads)
    fs = W.FrameStream(spec)
    attend_steps = {0, 7, 41, 42, 43, 83, 84, 125, 126, 167, 168, 199}
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
    assert m.ora.next_pos == (spec.steps - 168) * 757


def test_rebase_partial_ring_all_heads(sfkv):
    """Delta rotation before the ring wraps (3 frames = 2,271 valid slots, not a
    multiple of any launch tile), checked on all 24 heads: a small delta, then a
    reset to position 0, each followed by a write and an attention check."""
    spec = W.PROD
    say("case rebase_partial_h24_d128_n757_c5788")
    m = Mirror(sfkv, rope_for(sfkv, spec.shape), spec)
    fs = W.FrameStream(spec)
    for step in range(3):
        q, k, v = fs.frame()
        if step == 0:
            m.calibrate(k, v)
        m.write(k, v)
    assert m.gpu.state()["n_valid"] == 3 * 757
    for delta in (5, None):
        m.rebase(m.ora.next_pos if delta is None else delta)
        m.check_cache(f"after rebase {delta}")
        q, k, v = fs.frame()
        m.write(k, v)
        m.check_cache(f"write after rebase {delta}")
        m.check_attend(q, rows=spread_rows(q.shape[0], 32), tag=f"attend after rebase {delta}")


def test_stress_heavy_tails_variable_first_write(sfkv):
    """40 heads, Student-t(3) keys and values with per-head std up to 8 (so later
    frames saturate the E4M3 range of the step-0 scales), a first write of
    100..757 tokens, then 50 steady frames."""
    spec = W.STRESS
    heads = [0, 13, 26, 39]
    say(f"case {spec.name}")
    fs = W.FrameStream(spec)
    n0 = fs.first_length()
    say(f"  first write {n0} tokens")
    m = Mirror(sfkv, rope_for(sfkv, spec.shape), spec, heads=heads)
    for step in range(spec.steps):
        q, k, v = fs.frame(n0 if step == 0 else None)
        if step == 0:
            m.calibrate(k, v)
        m.write(k, v)
        m.check_cache(f"step {step}")
        if step in (0, 1, 8, 25, spec.steps - 1):
            m.check_attend(q, rows=spread_rows(q.shape[0], 48), tag=f"step {step}")
    k8 = m.gpu.k_codes()[torch.tensor(heads)].cpu().numpy()
    sat = np.count_nonzero((k8 & 0x7F) == 0x7E)
    say(f"  saturated K codes in checked heads: {sat}")
    assert sat > 0


def test_sweep_launch_configuration(sfkv):
    """The 240-call step as the benchmark runs it (device-drawn inputs, one stream,
    each cache prefilled with 8 frames); three caches are mirrored in the oracle."""
    from streaming_fp8_kv_amd.sweep import Sweep
    say("case step_240x_h24_d128_n757_c5788")
    sw = Sweep(sfkv, n_caches=W.CALLS_PER_STEP, keep_frames_of=(0, 119, 239))
    sw.prefill()
    sw.step()
    torch.cuda.synchronize()
    for ci in (0, 119, 239):
        say(f"  mirror cache {ci}")
        m = Mirror(sfkv, sw.rope, W.SWEEP)
        m.gpu = sw.caches[ci]
        frames = sw.kept[ci]
        for step, (q, k, v) in enumerate(frames):
            if step == 0:
                m.ora.calibrate(m._sub(k), m._sub(v))
            m.ora.write(m._sub(k), m._sub(v))
        m.check_cache(f"cache {ci}")
        q = frames[-1][0]
        out = sw.outs[ci]
        rows = spread_rows(q.shape[0], 64)
        got = out[torch.as_tensor(rows)].cpu().numpy()
        ref = m.reference_from_gpu_cache(q, rows)
        from tests.gpu_helpers import attention_error, A_MAX, B_MEAN
        a, b = attention_error(got, ref)
        say(f"  cache {ci}: A={a:.2e} B={b:.2e}")
        assert a <= A_MAX and b <= B_MEAN


@pytest.mark.parametrize("heads,d,cap,max_new,lens", [
    (3, 128, 1000, 1000, [1000, 1, 37, 999]),   # a write that fills the whole ring, then ragged ones
    (5, 128, 333, 64, [1, 1, 64, 63, 64, 64, 64, 64, 2]),   # capacity not a multiple of the key tile
    (2, 64, 4096, 700, [700, 129, 700, 700, 700, 700, 700]),   # head_dim 64 at a long ring, wrapped
    (1, 128, 64, 64, [64, 64, 64]),             # a single key tile, fully replaced each write
])
def test_ragged_shapes(sfkv, heads, d, cap, max_new, lens):
    """Shapes off the production grid: a single-token write, a whole-ring write,
    capacities and token counts that are not multiples of the 64-key tile or the
    32-query block, head_dim 64, and every call checked in full."""
    say(f"case ragged_h{heads}_d{d}_c{cap}_max{max_new}")
    shape = W.CacheShape(heads, d, cap, max_new, max_position=16384)
    spec = W.WorkloadSpec(name="ragged", shape=shape, seed=11 + heads, dtype=torch.bfloat16, dist="normal",
                          sigma_q=(0.5, 4.0), sigma_kv=(0.5, 4.0), steps=len(lens))
    m = Mirror(sfkv, rope_for(sfkv, shape), spec)
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
