"""Float64 CPU oracle for the POET-X layer hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (``orthogonal_reparameterized_poetx_amd``) never imports it, and
this package imports nothing from the product path: the two share no code.

The oracle is written from these pages (cited by title and section):

* [P3] "POET-X: Memory-efficient LLM Training by Scaling Orthogonal
  Transformation" (gist.science summary of arXiv 2603.05500), section
  "Technische samenvatting" > "Methodologie", items 1-5.  The authority on
  what POET-X computes; item 5 also names POET-XQ (base weights stored
  quantized, e.g. INT8, and dequantized on the fly): ``quantize_rows`` /
  ``dequantize_rows``.
* [P1] "POET-X：基于正交变换缩放的内存高效LLM训练方法" (ai-stack.site review),
  最佳实践 实践 2 (Cayley transform, autodiff to the generator),
  实践 4 (recompute, det = 1), 实践 5 (fp32 accumulation).
* [P2] "POET方法：重塑大型语言模型训练新篇章" (showapi.com), section 1.2
  (spectral invariance of orthogonal equivalence transforms).

Every function is pinned by ``tests/test_oracle_*.py`` against closed forms,
invariants, dense brute force and finite differences.  No function here is
"parity unpinned".
"""

from .poetx import (  # noqa: F401
    GOLDEN_GAMMA,
    adam_step,
    backward,
    block_count,
    cayley,
    cayley_neumann,
    chain_rule,
    cnp_error_bound,
    dense_orthogonal,
    dequantize_rows,
    forward,
    make_permutation,
    merge,
    mix64,
    pack,
    quantize_rows,
    round_bf16,
    triu_pairs,
    unpack,
    unpack_skew,
)
