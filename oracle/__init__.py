"""CPU oracle for exact tiled attention -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, the package smoke check and the benchmark's CPU-baseline
leg may import anything from here.  The product path (the HIP library and its
Python binding) never imports, links or calls this package, and this package
imports nothing from the product path.

Sources cited in this package (web pages; sections named as headed there):

[FUSED07]  "Модуль 07: Fused-операторы и FlashAttention" -- course
           *LLM Inference Systems*, hermes-agent.ru.
[LESSON]   "FlashAttention: внимание без матрицы n×n" -- lesson 5.7.2,
           ai.flicky.cc.
[NOTE]     "Atencja od strony jądra: FlashAttention, softmax online i
           połączona dekwantyzacja" -- trefon.com notes.
[BOOK5]    "Глава 5. Операторы и среда выполнения" -- AI infra book,
           bojieli.github.io.
"""
from .attention import (  # noqa: F401
    as_f64,
    softmax_attention,
    softmax_attention_rows,
    online_fold_attention,
    attention_backward,
    decode_attention,
    decode_attention_fp8,
    decode_attention_int8,
    e4m3_to_f64,
    int8_to_f64,
    fp8_attention_inputs,
    decode_split_merge,
    online_normalizer,
    online_weighted_sum,
    causal_block_pairs,
    causal_offset,
)
