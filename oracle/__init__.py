"""CPU oracle for the Markov draft loop and rejection verification.

TEST INFRASTRUCTURE ONLY. Nothing in the product path (the HIP library and
its Python binding) may import, call or link anything in this package; only
the tests, the smoke check and the benchmark's CPU-baseline leg use it.

It is a plain, slow, obviously correct NumPy implementation of what the hot
path computes, in float64 except where a decision (an argmax, an accept test)
is taken in the kernel's float32, as the pages fix fp32 Gumbel noise by
default. Every function cites the passage of the pages it follows:

* "DSparkSpeculator" API page (vllm.v1.worker.gpu.spec_decode.dspark.speculator),
  methods ``_sample_markov_chain``, ``_sample_sequential`` and ``_sample_logits``;
* vLLM PR #65007 "vocab-parallel DSpark Markov sampling / vocab-sharded
  verification", sections Overview, Part 1, Part 2 and Tests;
* vLLM PR #63554 "batch-sharded draft logits cache", section Notes.

Parity status per function:

* ``philox4x32_10``     pinned (known-answer values from an independent library build)
* ``uniform24`` / ``gumbel`` pinned (exhaustive/closed-form checks, high-precision decimal logs)
* ``argmax_rule``       pinned (NumPy argmax semantics, blockwise composition)
* ``bf16_rne``          pinned (torch's bf16 conversion)
* ``draft_loop``        pinned (special cases, Gumbel-max law, Markov chain law by chi-square)
* ``verify``            pinned (rejection-sampling law, special cases, greedy textbook rule)
* ``top_p_keep``        pinned (brute-force threshold formulation on the pages' row families)
* ``topk_columns``      pinned (torch.topk on distinct values; order invariants with ties, NaN, signed zeros)
* ``draft_loop(topk=)`` pinned (k = V equals the dense loop; the dense loop on the masked base; k = 1; the law)
* ``draft_logits``      pinned (exact fsum dot products on small shapes; unit hidden vectors pick lm_head columns)
"""
from .philox import philox4x32_10, PHILOX_M0, PHILOX_M1, PHILOX_W0, PHILOX_W1  # noqa: F401
from .noise import (SALT_ACCEPT, SALT_DRAFT, SALT_RESAMPLE, noise_words, uniform24, gumbel,  # noqa: F401
                    gumbel_row, accept_uniform)
from .core import argmax_rule, bf16_rne, bf16_to_f64, top_two_margin, topk_columns  # noqa: F401
from .draft import draft_loop  # noqa: F401
from .verify import verify, top_p_keep  # noqa: F401
from .lm_head import draft_logits  # noqa: F401
