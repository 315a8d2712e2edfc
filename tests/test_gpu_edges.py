"""Edge cases of the ring against the oracle: a single-slot ring (every call
attends to exactly one key, so the output is that key's value), a one-token
query frame over a long ring (each (head, query tile) pair split into dozens of
key ranges, which the merge handles with its general loop), and writes whose
positions run up to the last row of the RoPE table, followed by a reset."""
import numpy as np
import pytest
import torch

from oracle import bf16 as obf16, e4m3
from streaming_fp8_kv_amd import workloads as W
from tests.gpu_helpers import Mirror, say, spread_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sfkv():
    from streaming_fp8_kv_amd import sfkv as lib
    return lib


@pytest.mark.parametrize("storage", ["fp8", "bf16"])
@pytest.mark.parametrize("heads,d", [(1, 64), (3, 128)])
def test_single_slot_ring(sfkv, storage, heads, d):
    """Capacity 1, one token per write: after every write the ring holds only
    that token, and attention over one key returns its value (decoded, times the
    head's scale for E4M3) whatever the query; a rebase in the middle."""
    shape = W.CacheShape(heads, d, 1, 1, max_position=512)
    spec = W.WorkloadSpec(name="one_slot", shape=shape, seed=71 + heads, dtype=torch.float32, dist="normal",
                          sigma_q=(0.5, 4.0), sigma_kv=(0.5, 4.0), steps=8)
    say(f"case single-slot ring h{heads} d{d} {storage}")
    m = Mirror(sfkv, sfkv.Rope(d, shape.max_position), spec, storage=storage)
    fs = W.FrameStream(spec)
    for step in range(spec.steps):
        q, k, v = fs.frame()
        if step == 0:
            m.calibrate(k, v)
        if step == 4:
            m.rebase(m.ora.next_pos)
            m.check_cache("after rebase")
        m.write(k, v)
        m.check_cache(f"step {step}")
        out = m.check_attend(q, tag=f"step {step}").cpu().numpy()
        assert m.gpu.state()["n_valid"] == 1 and m.gpu.state()["write_slot"] == 0
        if storage == "bf16":
            want = obf16.decode(m.codes("v", 1)).astype(np.float64)[:, 0, :]          # [H, d]
        else:
            sv = m.gpu.scales().cpu().numpy()[2].astype(np.float64)
            want = e4m3.decode(m.codes("v", 1))[:, 0, :] * sv[:, None]
        # one key: every weight is 1, so the output is the stored value itself
        np.testing.assert_allclose(out[0], want, rtol=2e-6, atol=0)


@pytest.mark.parametrize("storage", ["fp8", "bf16"])
def test_one_query_over_a_long_ring(sfkv, storage):
    """2 heads x 128, 20,000 slots filled by four 5,000-token writes, then
    one-token writes: each attend call splits every pair into 78 key ranges."""
    heads, d, cap, big = 2, 128, 20_000, 5_000
    shape = W.CacheShape(heads, d, cap, big, max_position=32768)
    spec = W.WorkloadSpec(name="long_ring", shape=shape, seed=81, dtype=torch.bfloat16, dist="normal",
                          sigma_q=(0.5, 4.0), sigma_kv=(0.5, 4.0), steps=7)
    say(f"case one query over 20,000 slots {storage}")
    m = Mirror(sfkv, sfkv.Rope(d, shape.max_position), spec, storage=storage)
    fs = W.FrameStream(spec)
    for step in range(4):
        q, k, v = fs.frame(big)
        if step == 0:
            m.calibrate(k, v)
        m.write(k, v)
    m.check_attend(q, rows=spread_rows(big, 8), tag="5,000 queries")
    for step in range(3):
        q, k, v = fs.frame(1)
        m.write(k, v)
        m.check_cache(f"one-token write {step}")
        m.check_attend(q, tag=f"one query, write {step}")
    assert m.gpu.state()["n_valid"] == cap


@pytest.mark.parametrize("storage", ["fp8", "bf16"])
def test_positions_up_to_the_table_end(sfkv, storage):
    """A table of max_position 300 and 75-token writes: the fourth write takes
    positions 225 .. 299, the last rows the table holds (a fifth is refused
    with ERANGE, nothing changed); a reset then brings the next write back to
    position 0. Every call against the oracle."""
    heads, d, cap, n = 2, 64, 200, 75
    shape = W.CacheShape(heads, d, cap, n, max_position=300)
    spec = W.WorkloadSpec(name="table_end", shape=shape, seed=91, dtype=torch.float32, dist="normal",
                          sigma_q=(0.5, 4.0), sigma_kv=(0.5, 4.0), steps=6)
    say(f"case positions up to the table end {storage}")
    m = Mirror(sfkv, sfkv.Rope(d, shape.max_position), spec, storage=storage)
    fs = W.FrameStream(spec)
    for step in range(4):
        q, k, v = fs.frame()
        if step == 0:
            m.calibrate(k, v)
        m.write(k, v)
        m.check_cache(f"write {step}")
        m.check_attend(q, tag=f"write {step}")
    assert m.ora.next_pos == 300
    q, k, v = fs.frame()
    before = m.gpu.state()
    with pytest.raises(sfkv.SfkvError) as e:
        m.gpu.cache_write(k.cuda(), v.cuda())
    assert e.value.status == sfkv.ERANGE and m.gpu.state() == before
    m.rebase(m.ora.next_pos)
    m.write(k, v)
    m.check_cache("write after reset")
    m.check_attend(q, tag="write after reset")


@pytest.mark.parametrize("storage", ["fp8", "bf16"])
def test_one_key_dominates(sfkv, storage):
    """Small keys everywhere except one token per head whose key points along a
    unit direction the frame's queries share, scaled so that, fully aligned,
    its score is about 40 log2 units above the rest: for the queries it lines up
    with, the running maximum jumps far past its reference and every other
    weight underflows in fp16 (a one-hot output), for the others it sits
    anywhere between; key ranges whose maxima differ by tens of units are
    merged. Calibrated on a frame that holds the large key with headroom, so
    the E4M3 cache does not clip it. Every call against the oracle; a reset in
    between."""
    heads, d, cap, n = 2, 128, 512, 96
    shape = W.CacheShape(heads, d, cap, n, max_position=4096)
    spec = W.WorkloadSpec(name="one_key", shape=shape, seed=97, dtype=torch.float32, dist="normal",
                          sigma_q=None, sigma_kv=None, steps=7)
    say(f"case one dominating key {storage}")
    m = Mirror(sfkv, sfkv.Rope(d, shape.max_position), spec, storage=storage)
    fs = W.FrameStream(spec)
    g = torch.Generator().manual_seed(98)
    u = torch.randn(heads, d, generator=g)
    u = u / u.norm(dim=1, keepdim=True)
    big = 17.7                              # |q||k| = 313: 40 log2 units once divided by sqrt(d), times log2(e)
    for step in range(spec.steps):
        q, k, v = fs.frame()
        k *= 0.05
        q = big * u[None].expand(n, heads, d).contiguous() + 0.05 * q
        if step == 0:
            cal = k.clone()
            cal[0] = 1.5 * big * u
            m.calibrate(cal, v)
        if step == 2:
            k[37] = big * u                 # the dominating key, one token of the third frame
            v[37] = torch.linspace(-3.0, 3.0, d)
        if step == 5:
            m.rebase(m.ora.next_pos)
            m.check_cache("after reset")
        m.write(k, v)
        m.check_cache(f"step {step}")
        m.check_attend(q, tag=f"step {step}")
