"""Plain fp64 CPU oracle for the vocab-wide softmax reductions.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
library and imports nothing from ``vocab_wide_softmax_amd``.

What it computes (the pages are DeepSpeed PR #8838 "Add Triton kernels for
vocab-parallel logprobs, entropy and KL" and RL-Kernel PR #208 "Add TP Fused
linear logp Triton"):

* ``reductions``  -- per-row log-softmax, per-token log-probabilities, entropy
  H = -sum p log p and KL(A||B) = sum p_A (log p_A - log p_B), forward and
  backward, written as the plain two-pass definitions (max, then sums) in
  float64. The single-read identities H = log S - W/S and
  KL = W/S_A - log S_A + log S_B (PR #8838, second commit message and the
  review comment proposing a single read) are evaluated separately by
  ``single_read_identities`` as a self-check, never as the answer.
* ``topk``        -- multi-id (top-k) log-probabilities: K ids per row, ignored
  slots, duplicate ids whose upstream gradients add (the PR #8838 test list).
* ``jsd``         -- the generalized Jensen-Shannon divergence of the JSD pull
  request pasted into PR #8838 (mixture weight beta on the teacher; beta = 0
  and 1 are the forward and reverse KL branches), with gradients to both inputs.
* ``linear_logp`` -- the fused linear-logp variant of RL-Kernel PR #208
  (PR body, "Implementation"): logits z = h W^T in float64, then the same
  log-probability and its gradients dh, dW by the chain rule.
* ``compare``     -- the element-wise acceptance rule used by the parity tests
  (relative bound plus a conditioning-scaled bound, identical NaN/inf
  placement) and the bf16 round-to-nearest-even helpers it needs.

Every function that has no independent pin would say "parity unpinned"; all
functions here are pinned by tests/test_oracle_pins*.py (brute force at 50
digits with mpmath, torch.log_softmax and autograd in float64, closed forms,
identities, finite differences and the extreme-range cases the pages describe).
"""

from . import reductions, topk, jsd, linear_logp, compare  # noqa: F401
