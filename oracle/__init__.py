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

Every function here is pinned by ``tests/test_oracle_*.py`` against facts the
pages or mathematics fix; none is "parity unpinned".
"""

from . import gather, gemm  # noqa: F401
