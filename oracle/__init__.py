"""Plain fp64 CPU oracle for the weight-only low-bit decode GEMV hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path (the
C++ packer and HIP kernels in ``memory_bound_decode_amd``) shares no code with it
and never calls it.

Sources (cited by page title and section throughout):

* [Bonsai2]   "Ternary Bonsai 2" hands-on walkthrough (27B model squeezed to 6 GB),
              §1.2 (the ``block_ternary`` absmean quantizer), §3.4 and §5.5
              (all-zero blocks get scale 1 and a zero flag).
* [GPT54-INT4] "GPT-5.4 small-model compression in practice: INT4 quantization +
              channel pruning + distillation + attention-head sparsity", §3.2
              (group-128 symmetric INT4: scale = max|w| / 7, codes in [-7, 7]).
* [Cassandra] review of "Cassandra: Enabling Reasoning LLMs at Edge via
              Self-Speculative Decoding", §3.1 (bf16 fields and the 0.15625 worked
              example), §3.2 (Wanda value pruning with a keep bitmap, mantissa
              truncation, the speculation + verification = original invariant,
              draft zero-fill), §3.3 (frequency-ranked unary exponent code; MX
              shared exponent), §3.5 (per-chunk parallel unary decoding).
* [Bolt]      "Nemotron 3.5 Bolt teardown", background section: decode is bound
              by weight bandwidth, which is why only weights are compressed.

Modules: ``bits`` (bf16 / fp16 fields and rounding), ``ternary``, ``int4``,
``cassandra`` (pruning, split, codebook, unary stream, tiles, spec decode,
restore), ``mx`` (MX-32 variant), ``gemv`` (fp64 products, MoE, error metric).

Parity status: every function is pinned by ``tests/test_oracle_*.py`` against the
pages' worked example and printed codewords, closed forms, invariants, library
routines or exact ``fractions.Fraction`` brute force, except where a function's
docstring says "parity unpinned" (the bit layouts the pages leave open, and the
MX-32 layout beyond its invariants).
"""
from . import bits, ternary, int4, cassandra, mx, gemv  # noqa: F401
