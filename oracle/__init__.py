"""CPU oracle for one DWDP rank's MoE block.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only the test suite, the
package smoke check and the benchmark's CPU-baseline leg may import it.  The
GPU path never calls into it and shares no code with it: this package holds
its own number codecs, routing, permutation, FFN and combine, written plainly
in numpy (fp64 unless a precision is fixed) so that each step can be checked
against its definition by eye.

What it computes (DWDP paper summary, §2 and §4.2): DWDP changes where the
expert weights live and when they are copied, not what the layer computes, so
the oracle is the textbook MoE layer -- a softmax top-k gate, per-expert SwiGLU
FFNs and a weighted sum, plus an always-on shared expert -- together with the
chunked round-robin copy plan of the prefetch (§4.3.2).

Modules
  codecs    bf16 and OCP FP8 E4M3 rounding, written from the format definitions
  moe       routing, permutation, expert FFN, combine, fp8 block / group quantisation
  prefetch  round-robin chunk plan of the layer-ahead expert prefetch

Every function is pinned by the oracle self-tests (closed forms, brute force,
library routines, invariants); none is "parity unpinned".
"""
