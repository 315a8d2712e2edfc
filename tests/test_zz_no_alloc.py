"""The allocation-free fused call (sfkv_write_attend_noalloc) through the C ABI,
against the fused call with a caller workspace (sfkv_write_attend): the same
kernels, so cache bytes, ring state and outputs must be identical bit for bit.
Two calls in a row, the second with fewer tokens, on both storages; a second
cache on the same GPU after them (the static scratch keeps the last call's
contents and nothing in it may be assumed zero); a configuration needing more
scratch than the maximum is rejected with the state unchanged; and no device
memory is allocated by the calls."""

import pytest
import torch

from streaming_fp8_kv_amd import workloads as W
from tests.gpu_helpers import Mirror, attention_error, A_MAX, B_MEAN, say, spread_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sfkv():
    from streaming_fp8_kv_amd import sfkv as lib
    return lib


def _noalloc(sfkv, handle, k, v, q, out):
    st = sfkv._lib.sfkv_write_attend_noalloc(handle, k.data_ptr(), v.data_ptr(), q.data_ptr(),
                                             sfkv._dtype_code(k), k.shape[0], out.data_ptr(), None)
    if st != sfkv.OK:
        raise sfkv.SfkvError(st, sfkv._lib.sfkv_last_error().decode())


@pytest.mark.parametrize("storage", ["fp8", "bf16"])
def test_noalloc_equals_workspace_call(sfkv, storage):
    say(f"case write_attend_noalloc vs write_attend ({storage})")
    spec = W.PROD
    s = spec.shape
    code = sfkv.STORE_BF16 if storage == "bf16" else sfkv.STORE_E4M3
    rope = sfkv.Rope(s.head_dim, 16384)
    a = sfkv.RingCache(rope, s.heads, s.capacity, s.new_tokens, storage=code)
    b = sfkv.RingCache(rope, s.heads, s.capacity, s.new_tokens, storage=code)
    ws = torch.empty(a.workspace_bytes(), dtype=torch.uint8, device="cuda")
    fs = W.FrameStream(spec, seed=61)
    q, k, v = (t.cuda() for t in fs.frame())
    a.calibrate_scales(k, v)
    b.calibrate_scales(k, v)
    for _ in range(7):
        q, k, v = (t.cuda() for t in fs.frame())
        a.cache_write(k, v)
        b.cache_write(k, v)
    torch.cuda.synchronize()
    for n in (757, 300):                      # two calls in a row, the second smaller
        q, k, v = (t.cuda() for t in fs.frame(n))
        oa = torch.full((n, s.heads, s.head_dim), float("nan"), device="cuda")
        ob = torch.full((n, s.heads, s.head_dim), float("nan"), device="cuda")
        # the workspace call first: it launches the same kernels, so whatever the
        # runtime sets up on a kernel's first launch is done before the
        # allocation-free call is measured
        sfkv.write_attend(b.handle, k, v, q, ob, ws)
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        _noalloc(sfkv, a.handle, k, v, q, oa)
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info()[0] == free0, "the call allocated device memory"
        assert a.state() == b.state()
        assert torch.equal(a.buf, b.buf), f"n={n}: cache buffers differ"
        assert torch.equal(oa, ob), f"n={n}: outputs differ"
        say(f"  n={n}: identical")


def test_noalloc_second_cache_and_oracle(sfkv):
    """A tiny cache after the production-size calls above (the scratch holds
    their leftovers): every call matches the oracle and the workspace call."""
    say("case write_attend_noalloc tiny session against the oracle")
    spec = W.TINY
    s = spec.shape
    rope = sfkv.Rope(s.head_dim, s.max_position, s.rope_base)
    m = Mirror(sfkv, rope, spec)
    twin = sfkv.RingCache(rope, s.heads, s.capacity, s.new_tokens)
    ws = torch.empty(twin.workspace_bytes(), dtype=torch.uint8, device="cuda")
    fs = W.FrameStream(spec)
    for step in range(6):
        q, k, v = fs.frame()
        if step == 0:
            m.calibrate(k, v)
            twin.calibrate_scales(k.cuda(), v.cuda())
        out = torch.empty(q.shape, device="cuda")
        ref_out = torch.empty(q.shape, device="cuda")
        _noalloc(sfkv, m.gpu.handle, k.cuda(), v.cuda(), q.cuda(), out)
        sfkv.write_attend(twin.handle, k.cuda(), v.cuda(), q.cuda(), ref_out, ws)
        m.ora.write(m._sub(k), m._sub(v))
        m.check_cache(f"step {step}")
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out)
        rows = spread_rows(q.shape[0], 16)
        a, b = attention_error(out.cpu().numpy()[rows], m.reference_from_gpu_cache(q, rows))
        assert a <= A_MAX and b <= B_MEAN, f"step {step}: A={a:.2e} B={b:.2e}"


def test_noalloc_rejects_configurations_beyond_the_maximum(sfkv):
    say("case write_attend_noalloc size limit")
    rope = sfkv.Rope(128, 4096)
    big = sfkv.RingCache(rope, 96, 4096, 2048)          # workspace far above 64 MiB
    assert big.workspace_bytes() > (64 << 20)
    x = torch.randn(16, 96, 128, device="cuda", dtype=torch.bfloat16)
    big.calibrate_scales(x, x)
    before = big.state()
    out = torch.empty(16, 96, 128, device="cuda")
    with pytest.raises(sfkv.SfkvError) as e:
        _noalloc(sfkv, big.handle, x, x, x, out)
    assert e.value.status == sfkv.EINVAL and "static maximum" in str(e.value)
    assert big.state() == before
    torch.cuda.synchronize()
