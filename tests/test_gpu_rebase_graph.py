"""GPU parity of the reset paths and of graph-replayed calls against the oracle.

* Attention issued right after a position reset, with no write in between: the
  last write's queries then sit at negative positions (its positions minus the
  delta), which the kernels rotate with the table row of |p| and a negated
  sine; the oracle evaluates that rotation directly. Both storages, the tiny
  and the production shape.
* The batched reset (sfkv_rebase_positions_many) against one
  sfkv_rebase_positions call per cache (bytes and state identical) and against
  the oracle, over caches of several configurations, more than one launch's
  worth of caches, zero deltas and empty caches.
* Graph capture: a chain of write + attend calls captured once and replayed,
  and the 240-call step of the benchmark captured and replayed, each replay
  checked against the oracle (chained calls under graph capture are how the
  Runway Characters post says its kernels were tested, "What Broke in
  Production").
* The range contract of the bf16 storage: values just inside the documented
  saturation bound are used exactly; values past it act as if clamped there.
"""
import numpy as np
import pytest
import torch

from oracle.cache import RingCache as OracleCache, softmax_attention
from oracle import bf16 as obf16
from streaming_fp8_kv_amd import workloads as W
from tests.gpu_helpers import (A_MAX, B_MEAN, Mirror, attention_error, say,
                               spread_rows)

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


@pytest.mark.parametrize("storage", ["fp8", "bf16"])
def test_attend_after_rebase_without_write_tiny(sfkv, storage):
    """Tiny session: after each write, a partial rebase then attend, and at reset
    steps a reset to position 0 then attend, both on the last write's queries;
    every output checked in full against the oracle."""
    spec = W.TINY
    say(f"case attend after rebase, tiny, {storage}")
    m = Mirror(sfkv, rope_for(sfkv, spec.shape), spec, storage=storage)
    fs = W.FrameStream(spec)
    for step in range(spec.steps):
        q, k, v = fs.frame()
        if step == 0:
            m.calibrate(k, v)
        m.write(k, v)
        m.check_attend(q, tag=f"step {step} after write")
        if step % 2 == 1 and m.ora.next_pos > 3:
            m.rebase(3)                                # positions stay >= 0 or just below
            m.check_cache(f"step {step} after rebase 3")
            m.check_attend(q, tag=f"step {step} rebase 3, no write")
        if step % 3 == 2:
            m.rebase(m.ora.next_pos)                   # reset: the queries now sit at -16 .. -1
            assert m.ora.last_pos0 < 0
            m.check_cache(f"step {step} after reset")
            m.check_attend(q, tag=f"step {step} reset, no write")


@pytest.mark.parametrize("storage", ["fp8", "bf16"])
def test_attend_after_rebase_without_write_production(sfkv, storage):
    """Production shape (24 x 128, 757 tokens, 5,788 slots, wrapped): reset to
    position 0 after the 9th frame, then attend with that frame's queries at
    positions -757 .. -1; then the next write and attend as usual."""
    spec = W.PROD
    heads = [0, 7, 23]
    say(f"case attend after rebase, production, {storage}")
    m = Mirror(sfkv, rope_for(sfkv, spec.shape), spec, heads=heads, storage=storage)
    fs = W.FrameStream(spec)
    for step in range(spec.steps):
        q, k, v = fs.frame()
        if step == 0:
            m.calibrate(k, v)
        m.write(k, v)
    rows = spread_rows(757, 64)
    m.check_attend(q, rows=rows, tag="before reset")
    m.rebase(m.ora.next_pos)
    assert m.ora.last_pos0 == -757
    m.check_cache("after reset")
    m.check_attend(q, rows=rows, tag="reset, no write")
    q, k, v = fs.frame()
    m.write(k, v)
    m.check_cache("write after reset")
    m.check_attend(q, rows=rows, tag="write after reset")


def _session(sfkv, rope, cfg, storage, lens, seed):
    """A GPU cache and its oracle twin after writes of the given lengths."""
    heads, d, cap, max_new = cfg
    code = sfkv.STORE_BF16 if storage == "bf16" else sfkv.STORE_E4M3
    c = sfkv.RingCache(rope, heads, cap, max_new, storage=code)
    o = OracleCache(heads, d, cap, max_new, rope.base, rope.max_position, mode=storage)
    spec = W.WorkloadSpec(name="rb", shape=W.CacheShape(heads, d, cap, max_new, max_position=rope.max_position),
                          seed=seed, dtype=torch.float32, dist="normal", sigma_q=(0.5, 2.0),
                          sigma_kv=(0.5, 2.0), steps=len(lens))
    fs = W.FrameStream(spec)
    for i, n in enumerate(lens):
        q, k, v = fs.frame(n)
        if i == 0:
            c.calibrate_scales(k.cuda(), v.cuda())
            o.calibrate(k.numpy(), v.numpy())
        c.cache_write(k.cuda(), v.cuda())
        o.write(k.numpy(), v.numpy())
    return c, o


def test_rebase_many_equals_single_calls_and_oracle(sfkv):
    """Three configurations (one split over two launches), zero deltas, a cache
    with no tokens; the batched call leaves every buffer and state exactly as
    one sfkv_rebase_positions per cache does, and as the oracle's rebase."""
    say("case rebase_positions_many against single calls and the oracle")
    rope64 = sfkv.Rope(64, 4096)
    rope128 = sfkv.Rope(128, 4096)
    rope128b = sfkv.Rope(128, 2048)
    rng = np.random.default_rng(7)
    plans = []
    for i in range(133):                       # more than one launch (128 per launch)
        plans.append(((1, 64, 64, 16), "fp8", rope64, [16] * int(rng.integers(1, 7))))
    for i in range(4):
        plans.append(((3, 128, 333, 100), "bf16", rope128, [100, 37, 100, 100][: 1 + i]))
    for i in range(3):
        plans.append(((2, 128, 200, 200), "fp8", rope128b, [200, 13, 57][: 1 + i]))
    a_side, b_side, oracles, deltas = [], [], [], []
    for j, (cfg, storage, rope, lens) in enumerate(plans):
        ca, o = _session(sfkv, rope, cfg, storage, lens, 100 + j)
        cb, _ = _session(sfkv, rope, cfg, storage, lens, 100 + j)
        nxt = o.next_pos
        dl = 0 if j % 17 == 5 else int(rng.integers(0, nxt + 1))
        if j % 29 == 3:
            dl = nxt                            # a full reset
        a_side.append(ca)
        b_side.append(cb)
        oracles.append(o)
        deltas.append(dl)
    # an empty cache: nothing written, only delta 0 is allowed
    code = sfkv.STORE_E4M3
    empty_a = sfkv.RingCache(rope64, 1, 64, 16, storage=code)
    empty_b = sfkv.RingCache(rope64, 1, 64, 16, storage=code)
    a_side.append(empty_a)
    b_side.append(empty_b)
    deltas.append(0)
    oracles.append(None)
    torch.cuda.synchronize()

    # errors first: nothing changes
    before = [c.state() for c in a_side]
    with pytest.raises(sfkv.SfkvError) as e:
        sfkv.rebase_positions_many([a_side[0].handle, a_side[1].handle, a_side[0].handle], [0, 0, 0])
    assert e.value.status == sfkv.EINVAL
    with pytest.raises(sfkv.SfkvError) as e:
        sfkv.rebase_positions_many([a_side[0].handle, a_side[1].handle],
                                   [0, a_side[1].state()["next_pos"] + 1])
    assert e.value.status == sfkv.ERANGE
    with pytest.raises(sfkv.SfkvError) as e:
        sfkv.rebase_positions_many([a_side[0].handle], [-1])
    assert e.value.status == sfkv.ERANGE
    assert [c.state() for c in a_side] == before

    order = list(rng.permutation(len(a_side)))     # groups interleaved in the list
    sfkv.rebase_positions_many([a_side[i].handle for i in order], [deltas[i] for i in order])
    for c, dl in zip(b_side, deltas):
        c.rebase_positions(dl)
    torch.cuda.synchronize()
    for j, (ca, cb, o, dl) in enumerate(zip(a_side, b_side, oracles, deltas)):
        assert ca.state() == cb.state(), f"cache {j}: state differs"
        assert torch.equal(ca.buf, cb.buf), f"cache {j}: buffer differs from the single call's"
        if o is None:
            continue
        o.rebase(dl)
        nv = o.n_valid
        k = ca.k_codes().cpu().numpy()
        if o.mode == "bf16":
            k = k.view(np.uint16)
        assert np.array_equal(k[:, :nv], o.k[:, :nv]), f"cache {j}: K differs from the oracle"
        assert np.array_equal(ca.positions().cpu().numpy()[:nv], o.pos[:nv]), f"cache {j}: positions"
        assert ca.state()["next_pos"] == o.next_pos
    say(f"  {len(a_side)} caches identical")


def test_rebase_many_production_then_attend(sfkv):
    """Three production caches (24 x 128, 5,788 slots, wrapped) reset together
    by one batched call; codes and positions checked on three heads against
    the oracle, then attention on the last queries (negative positions)."""
    spec = W.PROD
    heads = [0, 12, 23]
    say("case rebase_positions_many production")
    rope = rope_for(sfkv, spec.shape)
    mirrors, lastq = [], []
    for i in range(3):
        m = Mirror(sfkv, rope, spec, heads=heads)
        fs = W.FrameStream(spec, seed=spec.seed * 100 + i)
        for step in range(spec.prefill_frames + 1):
            q, k, v = fs.frame()
            if step == 0:
                m.calibrate(k, v)
            m.write(k, v)
        mirrors.append(m)
        lastq.append(q)
    sfkv.rebase_positions_many([m.gpu.handle for m in mirrors], [m.ora.next_pos for m in mirrors])
    for m in mirrors:
        m.ora.rebase(m.ora.next_pos)
    for i, (m, q) in enumerate(zip(mirrors, lastq)):
        m.check_cache(f"cache {i} after batched reset")
        m.check_attend(q, rows=spread_rows(757, 48), tag=f"cache {i} reset, no write")


@pytest.mark.parametrize("fused", [False, True])
def test_graph_replay_against_oracle(sfkv, fused):
    """write -> attend chained four times, captured once and replayed three
    times with eager work in between; after every replay the ring matches the
    oracle's bit for bit and every captured output meets the parity bar against
    the oracle's attention at that point of the chain."""
    say(f"case graph replay against the oracle (fused={fused})")
    spec = W.PROD
    s = spec.shape
    heads = [0, 5, 17, 23]
    rope = rope_for(sfkv, s)
    m = Mirror(sfkv, rope, spec, heads=heads)
    fs = W.FrameStream(spec, seed=88)
    frames = [fs.frame() for _ in range(7)]
    m.calibrate(frames[0][1], frames[0][2])
    for q, k, v in frames[:3]:
        m.write(k, v)
    ws = torch.empty(m.gpu.workspace_bytes(), dtype=torch.uint8, device="cuda")
    dev = [tuple(t.cuda() for t in f) for f in frames[3:]]
    outs = [torch.empty(757, s.heads, s.head_dim, device="cuda") for _ in dev]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for (q, k, v), o in zip(dev, outs):
                if fused:
                    m.gpu.write_attend(k, v, q, out=o, workspace=ws)
                else:
                    m.gpu.cache_write(k, v)
                    m.gpu.attend(q, out=o, workspace=ws)
    torch.cuda.synchronize()
    # the oracle runs the chain once; the replays write the same frames at the
    # same slots and positions, so the expected state is the same after each
    refs = []
    rows = spread_rows(757, 40)
    for q, k, v in frames[3:]:
        m.ora.write(m._sub(k), m._sub(v))
        refs.append(m.ora.attend(m._sub(q), rows=rows))
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda").sum()
        graph.replay()
        torch.cuda.synchronize()
        m.check_cache(f"replay {rep}")
        for i, (o, ref) in enumerate(zip(outs, refs)):
            got = o[torch.as_tensor(rows)][:, heads].cpu().numpy()
            assert np.isfinite(got).all(), f"replay {rep}: output {i} not written"
            a, b = attention_error(got, ref)
            say(f"  replay {rep} call {i}: A={a:.2e} B={b:.2e}")
            assert a <= A_MAX and b <= B_MEAN
        del junk


def test_sweep_captured_step_and_batched_reset(sfkv):
    """The benchmark's 240-call step: one eager step, then the step captured as a
    graph and replayed twice, then the batched reset of all 240 caches and an
    attend on each of three mirrored caches with its last queries; caches 0, 119
    and 239 are checked against the oracle after every stage."""
    from streaming_fp8_kv_amd.sweep import Sweep
    say("case step_240x captured step and batched reset")
    sw = Sweep(sfkv, n_caches=W.CALLS_PER_STEP, keep_frames_of=(0, 119, 239))
    sw.prefill()
    mirrors = {}
    for ci in (0, 119, 239):
        m = Mirror(sfkv, sw.rope, W.SWEEP, heads=[0, 9, 23])
        m.gpu = sw.caches[ci]
        for step, (q, k, v) in enumerate(sw.kept[ci]):
            if step == 0:
                m.ora.calibrate(m._sub(k), m._sub(v))
            if step < len(sw.kept[ci]) - 1:
                m.ora.write(m._sub(k), m._sub(v))     # the last kept frame is the step frame
        mirrors[ci] = m
    rows = spread_rows(757, 32)

    def check(stage, write):
        torch.cuda.synchronize()
        for ci, m in mirrors.items():
            q, k, v = sw.kept[ci][-1]
            if write:
                m.ora.write(m._sub(k), m._sub(v))
            m.check_cache(f"{stage}, cache {ci}")
            got = sw.outs[ci][torch.as_tensor(rows)][:, m.heads].cpu().numpy()
            ref = m.ora.attend(m._sub(q), rows=rows)
            a, b = attention_error(got, ref)
            say(f"  {stage}, cache {ci}: A={a:.2e} B={b:.2e}")
            assert a <= A_MAX and b <= B_MEAN

    sw.step()
    check("eager step", True)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            sw.step()
    torch.cuda.synchronize()
    for rep in range(2):
        for ci in mirrors:
            sw.outs[ci].fill_(float("nan"))
        graph.replay()
        check(f"replay {rep}", rep == 0)
    del graph
    sw.reset_all()
    for ci, m in mirrors.items():
        m.ora.rebase(m.ora.next_pos)
        sfkv.attend(sw.caches[ci].handle, sw.frames[ci][0], sw.outs[ci], sw.workspace)
    check("batched reset, attend without write", False)


def _bound_case(sfkv, factor):
    """bf16 storage, 4 heads: calibrate on a normal frame, then write a frame
    whose values reach `factor` times the head's saturation bound 65504 * 2^e_v."""
    shape = W.CacheShape(4, 128, 512, 128, max_position=4096)
    spec = W.WorkloadSpec(name="bf16_bound", shape=shape, seed=23, dtype=torch.float32, dist="normal",
                          sigma_q=(0.5, 2.0), sigma_kv=(0.5, 2.0), steps=2)
    m = Mirror(sfkv, rope_for(sfkv, shape), spec, storage="bf16")
    fs = W.FrameStream(spec)
    q, k, v = fs.frame()
    m.calibrate(k, v)
    m.write(k, v)
    q, k, v = fs.frame()
    bound = 65504.0 * m.factors[2].astype(np.float64)          # per head
    vmax = v.abs().amax(dim=(0, 2)).double().numpy()
    v = (v.double() * torch.from_numpy(factor * bound / vmax)[None, :, None]).float()
    m.write(k, v)
    m.check_cache("large frame")
    return m, q, bound


def test_bf16_values_just_inside_the_bound(sfkv):
    say("case bf16 values at 0.99 of the saturation bound")
    m, q, bound = _bound_case(sfkv, 0.99)
    vv = obf16.decode(m.codes("v", m.ora.n_valid)).astype(np.float64)
    assert np.all(np.abs(vv).max(axis=(1, 2)) <= bound)          # the stored values stay inside
    assert np.all(np.abs(vv).max(axis=(1, 2)) >= 0.98 * bound)
    m.check_attend(q, tag="inside the bound")


def test_bf16_values_past_the_bound_saturate_there(sfkv):
    """Values 4x the bound: the output equals the oracle's attention over the
    stored values clamped at +-65504 * 2^e_v (the documented contract), and is
    far from the unclamped one."""
    say("case bf16 values at 4x the saturation bound")
    m, q, bound = _bound_case(sfkv, 4.0)
    out = m.gpu.attend(q.cuda())
    torch.cuda.synchronize()
    nv = m.ora.n_valid
    kk = obf16.decode(m.codes("k", nv)).astype(np.float64)
    vv = obf16.decode(m.codes("v", nv)).astype(np.float64)
    qr = m.ora.rotated_queries(m._sub(q))
    clamped = softmax_attention(qr, kk, np.clip(vv, -bound[:, None, None], bound[:, None, None]))
    plain = softmax_attention(qr, kk, vv)
    got = out.cpu().numpy()
    a, b = attention_error(got, clamped)
    a2, b2 = attention_error(got, plain)
    say(f"  against clamped: A={a:.2e} B={b:.2e}; against unclamped: A={a2:.2e} B={b2:.2e}")
    assert a <= A_MAX and b <= B_MEAN
    assert b2 > 10 * B_MEAN
