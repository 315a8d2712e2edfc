"""The fused write + attend call against the two separate calls and the oracle.

sfkv_write_attend runs the query preparation inside the write's launch; the
arithmetic is the same functions, so the cache bytes and the attention output
must equal those of cache_write followed by attend bit for bit, for both
storages, both head dims and both input dtypes. The production-shape case is
also checked against the oracle.
"""
import pytest
import torch

from streaming_fp8_kv_amd import workloads as W
from tests.gpu_helpers import Mirror, attention_error, A_MAX, B_MEAN, say, spread_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sfkv():
    from streaming_fp8_kv_amd import sfkv as lib
    return lib


@pytest.mark.parametrize("storage", ["fp8", "bf16"])
@pytest.mark.parametrize("heads,d,cap,max_new,lens,dtype", [
    (24, 128, 5788, 757, [757] * 9, torch.bfloat16),       # production shape, wrapped
    (3, 64, 333, 100, [100, 1, 57, 100, 100, 99], torch.float32),
    (2, 128, 200, 200, [200, 13, 200], torch.float32),
])
def test_fused_equals_separate_calls(sfkv, storage, heads, d, cap, max_new, lens, dtype):
    say(f"case write_attend vs separate: {storage} h{heads} d{d} c{cap} {dtype}")
    code = sfkv.STORE_BF16 if storage == "bf16" else sfkv.STORE_E4M3
    rope = sfkv.Rope(d, 16384)
    a = sfkv.RingCache(rope, heads, cap, max_new, storage=code)
    b = sfkv.RingCache(rope, heads, cap, max_new, storage=code)
    ws = torch.empty(a.workspace_bytes(), dtype=torch.uint8, device="cuda")
    spec = W.WorkloadSpec(name="fused", shape=W.CacheShape(heads, d, cap, max_new, max_position=16384),
                          seed=41 + heads, dtype=dtype, dist="normal", sigma_q=(0.5, 4.0),
                          sigma_kv=(0.5, 4.0), steps=len(lens))
    fs = W.FrameStream(spec)
    for step, n in enumerate(lens):
        q, k, v = (t.cuda() for t in fs.frame(n))
        if step == 0:
            a.calibrate_scales(k, v)
            b.calibrate_scales(k, v)
        if step == len(lens) // 2:
            a.rebase_positions(a.state()["next_pos"])
            b.rebase_positions(b.state()["next_pos"])
        a.cache_write(k, v)
        oa = a.attend(q, workspace=ws)
        ob = b.write_attend(k, v, q, workspace=ws)
        torch.cuda.synchronize()
        assert a.state() == b.state(), f"step {step}"
        assert torch.equal(a.buf, b.buf), f"step {step}: cache buffers differ"
        assert torch.equal(oa, ob), f"step {step}: outputs differ (max {float((oa - ob).abs().max()):.3e})"
    say(f"  {len(lens)} calls identical")


def test_fused_production_against_oracle(sfkv):
    """The production call through the fused entry point, 24 heads, checked
    against the oracle after 8 prefill frames."""
    spec = W.PROD
    say("case write_attend production against the oracle")
    rope = sfkv.Rope(spec.shape.head_dim, spec.shape.max_position, spec.shape.rope_base)
    m = Mirror(sfkv, rope, spec)
    fs = W.FrameStream(spec)
    for step in range(spec.steps):
        q, k, v = fs.frame()
        if step == 0:
            m.calibrate(k, v)
        out = m.gpu.write_attend(k.cuda(), v.cuda(), q.cuda())
        m.ora.write(m._sub(k), m._sub(v))
        if step in (0, spec.steps - 1):
            m.check_cache(f"frame {step}")
            torch.cuda.synchronize()
            rows = spread_rows(q.shape[0], 96)
            got = out[torch.as_tensor(rows)].cpu().numpy()
            ref = m.reference_from_gpu_cache(q, rows)
            a_err, b_err = attention_error(got, ref)
            say(f"  frame {step}: A={a_err:.2e} B={b_err:.2e}")
            assert a_err <= A_MAX and b_err <= B_MEAN


def test_fused_errors_leave_state(sfkv):
    """Validation failures of the fused call enqueue nothing and leave the ring
    as it was: a missing output, a short workspace, a call before calibration."""
    rope = sfkv.Rope(64, 1024)
    c = sfkv.RingCache(rope, 2, 64, 16)
    k = torch.randn(16, 2, 64, device="cuda")
    ws = torch.empty(c.workspace_bytes(), dtype=torch.uint8, device="cuda")
    out = torch.empty(16, 2, 64, device="cuda")
    lib = sfkv._lib
    st = lib.sfkv_write_attend(c.handle, k.data_ptr(), k.data_ptr(), k.data_ptr(), sfkv.FP32, 16,
                               out.data_ptr(), ws.data_ptr(), ws.numel(), None)
    assert st == sfkv.ESTATE
    c.calibrate_scales(k, k)
    before = c.state()
    st = lib.sfkv_write_attend(c.handle, k.data_ptr(), k.data_ptr(), k.data_ptr(), sfkv.FP32, 16,
                               None, ws.data_ptr(), ws.numel(), None)
    assert st == sfkv.EINVAL and c.state() == before
    st = lib.sfkv_write_attend(c.handle, k.data_ptr(), k.data_ptr(), k.data_ptr(), sfkv.FP32, 16,
                               out.data_ptr(), ws.data_ptr(), 256, None)
    assert st == sfkv.EINVAL and c.state() == before
    st = lib.sfkv_write_attend(c.handle, k.data_ptr(), k.data_ptr(), k.data_ptr(), sfkv.FP32, 17,
                               out.data_ptr(), ws.data_ptr(), ws.numel(), None)
    assert st == sfkv.EINVAL and c.state() == before
    torch.cuda.synchronize()
    assert int(c.positions().abs().sum()) == 0


@pytest.mark.parametrize("storage", ["fp8", "bf16"])
def test_fused_long_session_with_resets(sfkv, storage):
    """The 200-step session with a reset to position 0 every 42 steps, every
    step through the fused call; three heads mirrored, attention checked around
    every reset."""
    spec = W.LONG
    heads = [0, 11, 23]
    say(f"case write_attend long session {storage}")
    rope = sfkv.Rope(spec.shape.head_dim, spec.shape.max_position, spec.shape.rope_base)
    m = Mirror(sfkv, rope, spec, heads=heads, storage=storage)
    fs = W.FrameStream(spec)
    ws = torch.empty(m.gpu.workspace_bytes(), dtype=torch.uint8, device="cuda")
    check = {0, 41, 42, 43, 84, 126, 168, 199}
    for step in range(spec.steps):
        q, k, v = fs.frame()
        if step == 0:
            m.calibrate(k, v)
        if step > 0 and step % spec.reset_period == 0:
            m.rebase(m.ora.next_pos)
        out = m.gpu.write_attend(k.cuda(), v.cuda(), q.cuda(), workspace=ws)
        m.ora.write(m._sub(k), m._sub(v))
        if step in check:
            m.check_cache(f"step {step}")
            torch.cuda.synchronize()
            rows = spread_rows(q.shape[0], 48)
            got = out[torch.as_tensor(rows)][:, heads].cpu().numpy()
            ref = m.reference_from_gpu_cache(q, rows)
            a_err, b_err = attention_error(got, ref)
            say(f"  step {step}: A={a_err:.2e} B={b_err:.2e}")
            assert a_err <= A_MAX and b_err <= B_MEAN
