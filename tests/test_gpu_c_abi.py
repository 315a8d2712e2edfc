"""The C ABI driven from plain C (tests/c_abi/session.c, no Python or torch in
that process), checked against the oracle.

The test writes seeded frames to a file, runs the C program as a child process
on the GPU, and compares what it wrote back: the final cache contents bit for
bit with the oracle's, and every frame's attention output against the oracle's
fp64 attention over the oracle's own cache (bit-identical to the GPU's, as the
final comparison and the per-step parity tests establish), to the same bar as
the other GPU tests.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

from streaming_fp8_kv_amd import workloads as W
from tests.gpu_helpers import A_MAX, B_MEAN, attention_error, bf16_staging_factors, say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_abi", "session")


@pytest.mark.parametrize("storage", ["fp8", "bf16"])
def test_c_session_matches_oracle(tmp_path, storage):
    from oracle.cache import RingCache as OracleCache, softmax_attention
    if not os.path.exists(EXE):
        pytest.skip("tests/c_abi/session is not built (streaming_fp8_kv_amd.build builds it with the library)")
    spec = W.TINY
    s = spec.shape
    frames, reset_before = 7, 4
    say(f"case c_abi session {storage}: {s.heads} x {s.head_dim}, {s.capacity} slots, {frames} frames")
    fs = W.FrameStream(spec)
    data = [fs.frame() for _ in range(frames)]
    inp, outp = tmp_path / "in.bin", tmp_path / "out.bin"
    hdr = np.array([s.heads, s.head_dim, s.capacity, s.new_tokens, frames, 1 if storage == "bf16" else 0,
                    reset_before, s.max_position], dtype=np.int32)
    with open(inp, "wb") as f:
        f.write(hdr.tobytes())
        for q, k, v in data:
            f.write(np.array([q.shape[0]], dtype=np.int32).tobytes())
            for t in (q, k, v):
                f.write(np.ascontiguousarray(t.float().numpy()).tobytes())
    sys.stdout.flush()
    r = subprocess.run([EXE, str(inp), str(outp)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, f"session failed: {r.stderr}"

    ora = OracleCache(s.heads, s.head_dim, s.capacity, s.new_tokens, s.rope_base, s.max_position, mode=storage)
    raw = open(outp, "rb").read()
    off = 0
    for i, (q, k, v) in enumerate(data):
        kn, vn = k.float().numpy(), v.float().numpy()
        if i == 0:
            ora.calibrate(kn, vn)
        if i == reset_before:
            ora.rebase(ora.next_pos)
        ora.write(kn, vn)
        n = q.shape[0]
        got = np.frombuffer(raw, dtype=np.float32, count=n * s.heads * s.head_dim, offset=off)
        got = got.reshape(n, s.heads, s.head_dim)
        off += got.nbytes
        kk, vv = ora.dequantized()
        ref = softmax_attention(ora.rotated_queries(q.float().numpy()), kk, vv)
        a, b = attention_error(got, ref)
        say(f"  frame {i}: A={a:.2e} B={b:.2e}")
        assert a <= A_MAX and b <= B_MEAN, f"frame {i}: A={a:.3e} B={b:.3e}"
    code = np.uint16 if storage == "bf16" else np.uint8
    plane = s.heads * s.capacity * s.head_dim
    k_plane = np.frombuffer(raw, dtype=code, count=plane, offset=off).reshape(s.heads, s.capacity, s.head_dim)
    off += k_plane.nbytes
    v_plane = np.frombuffer(raw, dtype=code, count=plane, offset=off).reshape(s.heads, s.capacity, s.head_dim)
    off += v_plane.nbytes
    pos = np.frombuffer(raw, dtype=np.int32, count=s.capacity, offset=off)
    off += pos.nbytes
    scales = np.frombuffer(raw, dtype=np.float32, count=4 * s.heads, offset=off).reshape(4, s.heads)
    off += scales.nbytes
    assert off == len(raw)
    nv = ora.n_valid
    assert np.array_equal(k_plane[:, :nv], ora.k[:, :nv])
    assert np.array_equal(v_plane[:, :nv], ora.v[:, :nv])
    assert np.array_equal(pos[:nv], ora.pos[:nv])
    if storage == "bf16":
        want = bf16_staging_factors(data[0][1].float().numpy(), data[0][2].float().numpy(), 0, s.rope_base)
    else:
        want = ora.scales()
    assert np.array_equal(scales, want)
