"""CPU oracle for the one-shot Lamport-mailbox gather of vocab-parallel logits.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or run anything in this
package. The product path (``tp_vocab_logits_amd``) never imports it, and this
package imports nothing from the product path: the two share no code.

Sources (cited by page title and section, never by line):

* API page -- the vLLM API documentation page
  ``vllm.models.kimi_k3.nvidia.specialized_decode.runtime.logits_gather``
  (module description, ``HeadGather`` class description, the printed sources of
  ``HeadGather.__init__``, ``HeadGather.__call__``, ``_install_gather`` and
  ``install_logits_gather``).
* PR 55021 -- vLLM pull request "[Perf][Kimi-K3] Use the one-shot custom
  all-gather for TP logits" (sections Purpose, Test Plan, Test Result).

Contents:

* :mod:`oracle.gather` -- the plain definition of the gathered result, a
  step-by-step simulator of the two-parity mailbox protocol (push with sentinel
  rewrite, poll, copy, re-arm, parity flip, declines, split push/collect), and
  the construction rules.
* :mod:`oracle.gemm` -- the vocab-parallel lm_head shard product in float64
  and a float -> BF16 round-to-nearest-even written from the IEEE-754 format.

Pins (``tests/oracle_pins.py``, run by ``tests/test_oracle_pins.py``; each
planted mistake of ``tests/test_oracle_mutants.py`` trips at least one):

* the gather definition, the protocol simulator, the vocabulary slice and the
  construction rules: torch's BF16 memory layout, numpy's stack/transpose for
  the NCCL layout, a hand-worked golden gather, an exhaustive 4^8 tiny case,
  value equivalence and an XOR invariant, randomised call sequences;
* ``lm_head_shard`` / ``lm_head_entry``: a hand-worked golden product, one-hot
  and closed-form inputs, torch's float64 matmul;
* ``round_to_bf16`` / ``bf16_to_f64``: torch's float32 -> BF16 conversion over
  every class of float32 input;
* ``relative_frobenius_error``: hand-worked norm ratios
  (``tests/golden/rel_frobenius_error.txt``).
"""

from . import gather, gemm  # noqa: F401
