"""CPU oracle for the streaming FP8 ring KV cache -- TEST INFRASTRUCTURE ONLY.

This package is the slow, plain reference the HIP path is checked against.
Only the test suite, the smoke check of the entry module and the CPU-baseline
leg of the benchmark may import it; the product path never does, and it shares
no code, tables or helpers with the HIP library (each side builds its own RoPE
table and its own FP8 codec from the definitions).

What it computes follows the Runway Characters post, "Do It Once, at Write
Time" (RoPE and per-head FP8 quantisation applied once, as each frame enters a
ring; a single delta rotation at each position reset; positions in time order
once the ring wraps) and "Where the Time Went" (the launch software's
per-call re-rotation, re-quantisation and copy-shift of a linear window, kept
here as the plain semantics the ring must reproduce).

Modules:
  e4m3       OCP E4M3FN encode (clamp, round-to-nearest-even) and decode
  bf16       bfloat16 encode (round-to-nearest-even) and decode, for the
             non-FP8 ring variant
  rope       RoPE table (fp64 libm, rounded to fp32) and pair rotation
  cache      the ring cache: calibrate, write, attend, rebase
  reference  plain definitions the ring is pinned against: direct softmax
             attention, the linear read-time-RoPE cache, slot-order positions

Parity status of each function is stated in its own docstring.
"""
