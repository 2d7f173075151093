"""Plain fp64 CPU oracle for masked paged attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the library (``masked_paged_attention_amd``)
imports, links or calls anything in this package; only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use it.
It shares no code, constant or helper with the HIP path.

Every function is written from the definitions on the source pages:

* the attention formula A = softmax(QK^T/sqrt(d) + M), O = A V and the rule that a
  masked key carries zero probability -- nalar.dev article "Padding mask tidak
  menghapus komputasi padding pada dense attention", section "Masking mengubah
  kelayakan relasi attention";
* the operator parameters (paged key/value, blockTables, host seqLen/kvSeqLen,
  slopes, maskType 3/4/5/9, headNum/kvHeadNum, qkScale) -- Ascend ATB page
  "PrefixEncoder", parameter table;
* the compressed causal / ALiBi masks -- Ascend ATB page "压缩mask" (compressed
  mask), section "约束说明" (constraints);
* the MLA operator (qNope 512 + qRope 64, ctKV 512 latent = V, contextLens,
  qseqlen, SPEC mask, LSE) -- Ascend ATB page "MLA", parameter table.

Where the pages are silent or garbled the module docstrings state the reading
taken.  Parity of every function here is pinned by the CPU tests in
``tests/test_oracle_*.py`` (brute force, closed forms, invariants).
"""

from .attention import (  # noqa: F401
    MASK_NONE,
    MASK_ALIBI,
    MASK_ALIBI_SQRT,
    MASK_ALIBI_LEFT,
    MASK_CAUSAL,
    MASK_CHUNKED_CAUSAL,
    MLA_MASK_UNDEFINED,
    MLA_MASK_SPEC,
    MLA_CALC_UNDEFINED,
    MLA_CALC_SPEC,
    MLA_CALC_PREFILL,
    prefix_encoder,
    prefix_encoder_rows,
    mla,
    mla_rows,
    lse_merge,
    attend,
)
from . import masks  # noqa: F401
