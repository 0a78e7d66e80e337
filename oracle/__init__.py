"""CPU oracle for the CSA2 hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(the C-ABI library and its Python binding) never imports, calls or links it, and
this package shares no code with it: the only common module is ``synth``, which
draws the seeded inputs and holds none of the method's arithmetic.

The oracle is plain numpy, slow and literal.  Each function cites the passage of
the pages it follows:

* the model card "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache
  Compression" (Hugging Face), section Introduction, paragraph "Compressed
  Sparse Attention 2 (CSA2)";
* the aiwiki article "DeepSeek V4.1-Flash", sections "Compressed Sparse
  Attention 2" and "KV-cache formats and bounded replay";
* the thinkplainai post "DeepSeek-V4.1-Flash: a 1M-context multimodal MoE built
  for agent work", table "Key specs".

Where the pages leave a step open the function states the reading it takes.
Floating point is fp64 except where a decision (a quantised code, a Top-K
membership) is taken: there the oracle computes in the precision the reading
fixes (fp32 canonical index scores), so both sides decide on the same numbers.

Parity pins: every function is pinned by ``tests/test_oracle_*.py`` against
closed forms, brute force or textbook routines.  The fp32 rounding sequence of
``index_scores`` is a reading (the plain left-to-right order); it is pinned by
hand-derived results on cancelling inputs, by exact rational evaluation of that
order with one rounding per step, by exact integer cases and by the fp32 error
bound against the exact dot product; see its docstring.
"""
from .formats import (  # noqa: F401
    E2M1_MAGNITUDES, e2m1_value, e4m3_value, e4m3_encode_ratio, e4m3_encode,
    e2m1_encode, bf16_value, fma_f32,
)
from .csa2 import (  # noqa: F401
    OracleCache, quantize_rows, pack_nibbles, unpack_nibbles, index_scores,
    topk_select, build_pool, index_topk, sparse_attention, query_index_values,
    run_layers,
)
