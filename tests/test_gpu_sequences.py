"""Random call sequences against the oracle: every entry point of the ring, in a
seeded random order, on an E4M3 and a bf16 cache side by side. Writes of 1 to
80 tokens into a 200-slot ring (so it wraps at every offset), separate and fused
write + attend, the allocation-free fused call, repeated attends of one frame,
single and batched resets by random deltas (attends straight after a reset put
the frame's queries at negative positions), and a re-calibration. After every
step the stored bytes, positions, scales and ring counters must equal the
oracle's, and every attention output must meet the parity bar against the
oracle fed the GPU's own cache."""
import numpy as np
import pytest
import torch

from streaming_fp8_kv_amd import workloads as W
from tests.gpu_helpers import A_MAX, B_MEAN, Mirror, attention_error, say

pytestmark = pytest.mark.gpu

OPS = ("write_then_attend", "write_attend", "write_attend_noalloc", "write_only", "attend_again",
       "rebase_one", "rebase_both", "recalibrate")


@pytest.fixture(scope="module")
def sfkv():
    from streaming_fp8_kv_amd import sfkv as lib
    return lib


def _check_out(m, out, q, tag):
    torch.cuda.synchronize()
    n = q.shape[0]
    rows = np.arange(n)
    got = out[:, m.heads].cpu().numpy()
    ref = m.reference_from_gpu_cache(q, rows)
    assert np.isfinite(out.cpu().numpy()).all(), f"{tag}: non-finite attention output"
    a, b = attention_error(got, ref)
    assert a <= A_MAX and b <= B_MEAN, f"{tag}: A={a:.3e} (bar {A_MAX}) B={b:.3e} (bar {B_MEAN})"


@pytest.mark.parametrize("seed,d", [(11, 128), (12, 64), (13, 128)])
def test_random_call_sequences(sfkv, seed, d):
    heads, cap, max_new, maxpos, steps = 3, 200, 80, 1200, 48
    shape = W.CacheShape(heads, d, cap, max_new, max_position=maxpos)
    spec = W.WorkloadSpec(name="sequences", shape=shape, seed=seed, dtype=torch.bfloat16, dist="normal",
                          sigma_q=(0.5, 4.0), sigma_kv=(0.5, 4.0), steps=steps)
    rope = sfkv.Rope(d, maxpos)
    mirrors = {st: Mirror(sfkv, rope, spec, storage=st) for st in ("fp8", "bf16")}
    fs = W.FrameStream(spec)
    rng = np.random.default_rng(seed)
    last_q = None
    ran = {o: 0 for o in OPS}
    say(f"case random sequences seed {seed} d {d}")
    first = True
    for step in range(steps):
        if first:
            op = "write_then_attend"
        else:
            op = OPS[rng.integers(len(OPS))]
            if op == "attend_again" and last_q is None:
                op = "write_only"
        n = int(rng.integers(1, max_new + 1))
        room = min(maxpos - m.ora.next_pos for m in mirrors.values())
        forced = (op.startswith("write") or op == "recalibrate") and n > room
        if forced:
            op = "rebase_both"                       # positions would run off the table
        ran[op] += 1
        tag = f"seed {seed} d {d} step {step} {op}"
        if op.startswith("write") or op == "recalibrate":
            q, k, v = fs.frame(n)
        if first:
            for m in mirrors.values():
                m.calibrate(k, v)
            first = False
        for st, m in mirrors.items():
            t = f"{tag} {st}"
            if op == "write_then_attend":
                m.write(k, v)
                m.check_cache(t)
                m.check_attend(q, tag=t)
            elif op == "write_attend":
                out = m.gpu.write_attend(k.cuda(), v.cuda(), q.cuda())
                m.ora.write(m._sub(k), m._sub(v))
                m.check_cache(t)
                _check_out(m, out, q, t)
            elif op == "write_attend_noalloc":
                out = torch.empty(n, heads, d, device="cuda")
                sfkv.write_attend_noalloc(m.gpu.handle, k.cuda(), v.cuda(), q.cuda(), out)
                m.ora.write(m._sub(k), m._sub(v))
                m.check_cache(t)
                _check_out(m, out, q, t)
            elif op == "write_only":
                m.write(k, v)
                m.check_cache(t)
            elif op == "attend_again":
                m.check_attend(last_q, tag=t)
            elif op == "rebase_one":
                delta = int(rng.integers(0, m.ora.next_pos + 1))
                m.rebase(delta)
                m.check_cache(t)
            elif op == "recalibrate":
                m.calibrate(k, v)
                m.check_cache(t)
        if op == "rebase_both":
            ms = list(mirrors.values())
            deltas = [int(rng.integers(0, m.ora.next_pos + 1)) for m in ms]
            if forced or rng.integers(2):
                deltas = [m.ora.next_pos for m in ms]  # a full reset to position 0
            sfkv.rebase_positions_many([m.gpu.handle for m in ms], deltas)
            for m, dl in zip(ms, deltas):
                m.ora.rebase(dl)
                m.check_cache(f"{tag} delta {dl}")
        if op.startswith("write"):
            last_q = q
    for m in mirrors.values():
        assert m.gpu.state()["tokens"] == m.ora.tokens
    assert all(ran.values()), f"operations never drawn: {[o for o, c in ran.items() if not c]}"
