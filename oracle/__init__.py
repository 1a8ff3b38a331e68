"""Plain CPU oracle for the packed variable-length causal attention path.

TEST INFRASTRUCTURE.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import, call or link anything in this
package.  The GPU library never uses it, and the two share no code, header,
table or constant generator; only the seeded input generators in
``workloads`` feed both.

Contents (each function cites the passage it follows):
  pack        cu_seqlens, segment ids, positions, shifted labels, loss mask,
              target count, max_seqlen, cu validation bits
  rope        per-segment rotary embedding, fp64 with one bf16 rounding
  attention   fp64 block-diagonal causal attention (C loop, explicit mask,
              and per-segment unpacked forms)
  accounting  slot, waste and pair counts used for useful-FLOP figures
  loss        packed cross-entropy: loss sum, target count, per-segment sums,
              token / sample averages, gradient of the loss sum

Every function here is pinned by tests that do not restate its own formula
(worked examples printed on the pages, closed forms, invariants, library
routines on special cases, brute force on tiny inputs).
"""

from . import accounting, attention, loss, pack, rope  # noqa: F401
