"""CPU oracle for the one-pass block-diffusion draft + lossless verify path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only the tests, the smoke check and the benchmark's CPU-baseline leg do.  It
shares no code with the HIP library; both sides receive their inputs from the
seeded generators in ``synth``.

The oracle is the plain definition of each step, in float64, with bfloat16
rounding only at the points where the library stores bfloat16 (weights, fused
features, KV cache, norm outputs fed to a projection, attention output, the
SiLU-times-up product, the final hidden state).  Sources, by page:

* DFlash review (block diffusion for flash speculative decoding),
  "Method / Inference": feature fusion H_t = RMSNorm(W_c [H^l1; ...; H^l5]);
  KV injection Q_i = W_i^Q H_d, K_i = [W_i^K H_t; W_i^K H_d],
  V_i = [W_i^V H_t; W_i^V H_d]; one parallel pass over the masked block;
  "Preliminary": tau in [1, gamma+1] counts the bonus token,
  L = (T_draft + T_verify) / tau.
* DStill, "Setup and notation": block of B positions, anchor at 0, masks at
  1..B-1, bidirectional inside the block, context strictly before the anchor;
  factorised per-position proposal; "Inference": greedy = top-1 per position,
  rejection-sampling verification with correction / bonus token.
* SPOT, "Method": D draft copies behind a shared prefix, each copy attending
  the prefix and itself; a shared Gumbel table couples the draws.
* D-Loop, section 2 Eq. (1): the factorised proposal q = prod_k q_k.

Parity pins for each function live in ``tests/test_oracle_*.py``.  Parity
unpinned: the numeric drafter outputs at full 8B-like sizes on random weights
(no page prints a worked example); they are bounded only by the pinned
properties of each step and by agreement between the two implementations.
"""
