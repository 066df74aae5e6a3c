"""CPU fp64 reference for the gated delta-rule hot path.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or run
anything in this package: only the test suite, the smoke check of the package
entry point and the CPU-baseline leg of the benchmark use it. It shares no code
with the HIP library; it takes plain numpy arrays and returns numpy arrays.

Every function is written from the two pages that define the method:

* "LeapQuant: an 8-bit recurrent state that stops rounding every token"
  (ai.satyajit.si) -- the delta-rule and Gated DeltaNet updates (section "The
  state, from the update rule up", eq. 1 and eq. 3), per-token rounding (section
  "Rounding every token", eq. 2), the window leap (section "Fix one: leap over a
  window", eq. 4 and eq. 10), compensator tokens (section "Fix two", eq. 5) and
  row smoothing (section "Fix three", eq. 7), and the stored layout (section
  "What 1.19 bytes buys").
* "ZeCO: Zero Communication Overhead Sequence Parallelism for Linear Attention"
  (paper summary) -- gated linear attention per token and per chunk (section
  "Gated Linear Attention (GLA) Formulation"), and the decomposition of a shard
  around its incoming state (section "Global State Update Formula", eq. 6).

Orientation: every state is ``[d_v][d_k]`` (rows are value channels). The pages
write ``d_k x d_v``; their formulas are used transposed.

Every function here is pinned by a test under tests/test_oracle_*.py against
what the pages and the mathematics fix (exact rationals, closed forms, special
cases, identities between separately written forms). What stays "parity
unpinned" are not functions but trend statements about the method's error (the
error-ordering tests and the GPU error study), whose page numbers come from a
simulator the page does not fully specify.
"""
from . import gdn, gla, kda, kda_leapq, leapq  # noqa: F401
