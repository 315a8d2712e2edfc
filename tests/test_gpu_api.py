"""C-ABI behaviour on the GPU: error statuses with the state left unchanged, the
E4M3 encoder at every rounding boundary through the real write kernel, chained
calls replayed from a captured graph, no host synchronisation in the per-step
path, no allocation keyed by token count, and the binding's refusal of tensors
that would let a kernel read or write past an end."""
import numpy as np
import pytest
import torch

from oracle import e4m3
from oracle.cache import RingCache as OracleCache
from streaming_fp8_kv_amd import workloads as W
from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sfkv():
    from streaming_fp8_kv_amd import sfkv as lib
    return lib


@pytest.fixture(scope="module")
def rope128(sfkv):
    return sfkv.Rope(128, 4096)


def test_errors_leave_state_unchanged(sfkv, rope128):
    say("case api errors")
    c = sfkv.RingCache(rope128, 2, 64, 16)
    x = torch.randn(8, 2, 128, device="cuda", dtype=torch.bfloat16)
    with pytest.raises(sfkv.SfkvError) as e:
        c.cache_write(x, x)
    assert e.value.status == sfkv.ESTATE
    with pytest.raises(sfkv.SfkvError) as e:
        c.attend(x)
    assert e.value.status == sfkv.ESTATE
    c.calibrate_scales(x, x)
    big = torch.randn(17, 2, 128, device="cuda", dtype=torch.bfloat16)
    with pytest.raises(sfkv.SfkvError) as e:
        c.cache_write(big, big)
    assert e.value.status == sfkv.EINVAL
    c.cache_write(x, x)
    before = c.state()
    with pytest.raises(sfkv.SfkvError) as e:
        c.attend(x[:4].contiguous())                 # n_q differs from the last write
    assert e.value.status == sfkv.EINVAL
    with pytest.raises(sfkv.SfkvError) as e:
        c.rebase_positions(before["next_pos"] + 1)
    assert e.value.status == sfkv.ERANGE
    with pytest.raises(sfkv.SfkvError) as e:
        c.rebase_positions(-1)
    assert e.value.status == sfkv.ERANGE
    assert c.state() == before
    # positions reaching the end of the rope table
    small = sfkv.Rope(128, 20)
    c2 = sfkv.RingCache(small, 2, 64, 16)
    c2.calibrate_scales(x, x)
    c2.cache_write(x, x)
    c2.cache_write(x, x)                         # positions 0..15 of 0..19
    st = c2.state()
    with pytest.raises(sfkv.SfkvError) as e:
        c2.cache_write(x, x)
    assert e.value.status == sfkv.ERANGE and c2.state() == st
    # an empty frame: n_tokens must be at least 1
    empty = x[:0]
    for call in (lambda: c.cache_write(empty, empty), lambda: c.calibrate_scales(empty, empty)):
        with pytest.raises(sfkv.SfkvError) as e:
            call()
        assert e.value.status == sfkv.EINVAL and c.state() == before
    # an empty batched reset changes nothing
    sfkv.rebase_positions_many([], [])
    assert c.state() == before
    # a workspace that is too small
    c3 = sfkv.RingCache(sfkv.Rope(128, 8192), 24, 5788, 757)
    need = c3.workspace_bytes()
    y = torch.randn(757, 24, 128, device="cuda", dtype=torch.bfloat16)
    c3.calibrate_scales(y, y)
    for _ in range(8):
        c3.cache_write(y, y)
    if need:
        with pytest.raises(sfkv.SfkvError) as e:
            c3.attend(y, workspace=torch.empty(need - 256, dtype=torch.uint8, device="cuda"))
        assert e.value.status == sfkv.EINVAL
    torch.cuda.synchronize()


def _boundary_values():
    """Every rounding class of the E4M3 encoder: the codes themselves, the
    midpoints between adjacent codes and one and two fp32 ulps either side, the
    subnormal range, saturation, signed zero, and a log-uniform random sample."""
    codes = np.arange(0, 0x7F)
    vals = e4m3.decode(codes)
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    parts = [vals.astype(np.float32), mids]
    for k in (1, 2):
        up, dn = mids.copy(), mids.copy()
        for _ in range(k):
            up = np.nextafter(up, np.float32(np.inf))
            dn = np.nextafter(dn, np.float32(0))
        parts += [up, dn]
    parts.append(np.array([448.0, 448.5, 464.0, 480.0, 1e6, 3.0e38, 1e-30, 1e-40, 0.0], np.float32))
    rng = np.random.default_rng(3)
    parts.append(np.exp2(rng.uniform(-14, 9.0, size=200_000)).astype(np.float32))
    pos = np.concatenate(parts)
    allv = np.concatenate([pos, -pos]).astype(np.float32)
    return allv


def test_encoder_boundaries_through_write(sfkv, rope128):
    """Values stored with scale 1 (the calibration frame's absmax is 448) come out
    as the oracle's E4M3 codes of the values themselves."""
    say("case e4m3 boundary classes via cache_write")
    vals = _boundary_values()
    per_tok = 128
    n = -(-vals.size // per_tok)
    buf = np.zeros(n * per_tok, np.float32)
    buf[:vals.size] = vals
    v = torch.from_numpy(buf.reshape(n, 1, per_tok))
    cap = 4096
    assert n <= cap
    c = sfkv.RingCache(sfkv.Rope(128, cap + 8), 1, cap, cap)
    cal = torch.zeros(1, 1, 128)
    cal[0, 0, 0] = 448.0                      # position 0: rotation is the identity
    c.calibrate_scales(cal.cuda(), cal.cuda())
    assert c.scales().cpu().numpy().ravel().tolist() == [1.0, 1.0, 1.0, 1.0]
    c.cache_write(v.cuda(), v.cuda())
    got_v = c.v_codes()[0, :n].cpu().numpy().reshape(-1)[:vals.size]
    want = e4m3.encode(vals)
    bad = np.nonzero(got_v != want)[0]
    assert bad.size == 0, f"{bad.size} codes differ, first {vals[bad[:5]]}: {got_v[bad[:5]]} vs {want[bad[:5]]}"
    # keys: rotated at positions 0..n-1 in fp32 first; compare with the oracle
    ora = OracleCache(1, 128, cap, cap, 10000.0, cap + 8)
    ora.calibrate(cal.numpy(), cal.numpy())
    ora.write(v.numpy(), v.numpy())
    assert np.array_equal(c.k_codes()[0, :n].cpu().numpy(), ora.k[0, :n])


@pytest.mark.parametrize("fused", [False, True])
def test_graph_captured_chain_matches_eager(sfkv, fused):
    """write -> attend -> write -> attend ... captured once into a graph and
    replayed; every replay must reproduce the eager run bit for bit, with eager
    work between replays (the chained-call tests the pages describe). With
    fused=True the graph holds sfkv_write_attend calls, checked against eager
    separate calls."""
    say(f"case graph-captured chain (fused={fused})")
    spec = W.PROD
    s = spec.shape
    rope = sfkv.Rope(s.head_dim, 16384)
    fs = W.FrameStream(spec, seed=77)
    frames = [tuple(t.cuda() for t in fs.frame()) for _ in range(6)]

    def fresh():
        c = sfkv.RingCache(rope, s.heads, s.capacity, s.new_tokens)
        c.calibrate_scales(frames[0][1], frames[0][2])
        for q, k, v in frames[:3]:
            c.cache_write(k, v)
        return c

    eager = fresh()
    ws = torch.empty(max(eager.workspace_bytes(), 256), dtype=torch.uint8, device="cuda")
    e_outs = []
    for q, k, v in frames[3:]:
        eager.cache_write(k, v)
        e_outs.append(eager.attend(q, workspace=ws).clone())
    torch.cuda.synchronize()

    g_cache = fresh()
    g_outs = [torch.empty(757, s.heads, s.head_dim, device="cuda") for _ in frames[3:]]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for (q, k, v), o in zip(frames[3:], g_outs):
                if fused:
                    g_cache.write_attend(k, v, q, out=o, workspace=ws)
                else:
                    g_cache.cache_write(k, v)
                    g_cache.attend(q, out=o, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        for o in g_outs:
            o.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda").sum()      # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(e_outs, g_outs)):
            assert torch.equal(a, b), f"replay {rep}: output {i} differs"
        assert torch.equal(eager.k_codes(), g_cache.k_codes())
        assert torch.equal(eager.v_codes(), g_cache.v_codes())
        assert torch.equal(eager.positions(), g_cache.positions())
        del junk


def test_no_host_synchronisation_in_step(sfkv):
    """With the stream held busy by a long device-side sleep, a full 24-call slice
    of the step (write + attend, half of the calls through the fused entry point)
    and a reset must all return on the host while the GPU is still asleep: no
    call waits for the device."""
    say("case no host sync")
    spec = W.PROD
    s = spec.shape
    rope = sfkv.Rope(s.head_dim, 16384)
    fs = W.FrameStream(spec, seed=5, device="cuda")
    caches, frames = [], []
    for _ in range(24):
        c = sfkv.RingCache(rope, s.heads, s.capacity, s.new_tokens)
        q, k, v = fs.frame()
        c.calibrate_scales(k, v)
        c.cache_write(k, v)
        caches.append(c)
        frames.append((q, k, v))
    ws = torch.empty(max(caches[0].workspace_bytes(), 256), dtype=torch.uint8, device="cuda")
    outs = [torch.empty(757, s.heads, s.head_dim, device="cuda") for _ in caches]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    torch.cuda._sleep(int(3e8))              # a bounded device-side spin (0.1 s or more)
    for i, (c, (q, k, v), o) in enumerate(zip(caches, frames, outs)):
        c.rebase_positions(c.state()["next_pos"])
        if i % 2:
            c.write_attend(k, v, q, out=o, workspace=ws)
        else:
            c.cache_write(k, v)
            c.attend(q, out=o, workspace=ws)
    still_busy = not stream.query()
    torch.cuda.synchronize()
    assert still_busy, "the host waited for the device during the step"
    assert all(torch.isfinite(o).all() for o in outs)


def test_variable_first_lengths_allocate_nothing(sfkv):
    """Sessions whose first write length varies (100..757 tokens) reuse the memory
    given at init: free device memory is the same after every session."""
    say("case no per-length allocation")
    spec = W.STRESS
    s = spec.shape
    rope = sfkv.Rope(s.head_dim, 65536)
    c = sfkv.RingCache(rope, s.heads, s.capacity, s.new_tokens)
    ws = torch.empty(max(c.workspace_bytes(), 256), dtype=torch.uint8, device="cuda")
    lengths = [100, 757, 433, 101, 650, 312, 757, 128]
    data = torch.randn(757, s.heads, s.head_dim, device="cuda", dtype=torch.bfloat16)
    outs = {n: torch.empty(n, s.heads, s.head_dim, device="cuda") for n in set(lengths)}
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for n in lengths:
        x = data[:n]
        c.calibrate_scales(x, x)
        c.cache_write(x, x)
        c.attend(x, out=outs[n], workspace=ws)
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info()[0] == free0


def test_binding_refuses_mismatched_tensors(sfkv, rope128):
    """The library reads every input with k's (or q's) dtype and row count and
    writes n_q rows of float32 to out: the binding refuses a v, q, out or
    workspace that does not match, before anything is launched."""
    say("case binding argument checks")
    c = sfkv.RingCache(rope128, 2, 64, 16)
    x = torch.randn(8, 2, 128, device="cuda", dtype=torch.bfloat16)
    c.calibrate_scales(x, x)
    c.cache_write(x, x)
    before = c.state()
    short, wide = x[:4].contiguous(), x.float()
    for k, v in ((x, short), (short, x), (x, wide), (wide, x), (x, x.cpu()), (x, x.transpose(0, 1))):
        for call in (c.cache_write, c.calibrate_scales):
            with pytest.raises(ValueError):
                call(k, v)
    ws = torch.empty(max(c.workspace_bytes(), 256), dtype=torch.uint8, device="cuda")
    bad_outs = [torch.empty(4, 2, 128, device="cuda"), torch.empty(8, 2, 128, device="cuda", dtype=torch.bfloat16),
                torch.empty(8, 2, 128), torch.empty(2, 8, 128, device="cuda").transpose(0, 1)]
    for o in bad_outs:
        with pytest.raises(ValueError):
            c.attend(x, out=o, workspace=ws)
        with pytest.raises(ValueError):
            c.write_attend(x, x, x, out=o, workspace=ws)
        with pytest.raises(ValueError):
            sfkv.write_attend_noalloc(c.handle, x, x, x, o)
    with pytest.raises(ValueError):
        c.attend(x, workspace=ws.cpu())
    with pytest.raises(ValueError):
        c.write_attend(x, x, wide, workspace=ws)
    torch.cuda.synchronize()
    assert c.state() == before
    # the same cache still works after the refusals
    out = c.attend(x, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
