"""Plain fp64 CPU oracle for the HySparse2 hybrid-block decode path and the
KV-Bridging projection.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The
product path (``long_context_kv_hs2_amd``) never imports, links or runs it,
and this package imports nothing from the product path.

Sources cited in the docstrings (the pages are news reports of arXiv
2609.26368; none prints an equation, table, figure or code):

* [zh]  readaitime.com news of 2026-09-24 (Traditional Chinese), no headings;
        paragraphs are named by their subject.
* [en]  "Luo Fuli Teases Xiaomi MiMo-V3 Architecture: HySparse2 Enables Early
        Prefill Exit" (ai.synthepulse.app story 13379).
* [pt]  lt.allworld.media article 189823470 (Portuguese), no headings.
* [fr]  toolnavs.com article 2080 (French), sections "Ce que fait HySparse2",
        "Le Prefill s'arrete a mi-chemin", "Les chiffres mesures".
* [ko]  toolnavs.com article 2080 (Korean), sections "HySparse2가 한 일",
        "Prefill은 절반에서 끝난다", "실측 수치".

Every function of ``hs2_oracle`` has a pin in ``tests/test_oracle.py`` or
``tests/test_codecs.py`` (closed forms, brute force on tiny inputs, the
library routine ``scaled_dot_product_attention`` in float64, and values from
the OCP 8-bit floating-point specification).  No function is "parity
unpinned".
"""

from .hs2_oracle import (  # noqa: F401
    HEAD_DIM,
    N_Q_HEADS,
    WINDOW,
    TOP_K,
    BAND_REL,
    bf16_bits_to_f64,
    f64_to_bf16_bits,
    e4m3_value_table,
    e4m3_bytes_to_f64,
    f64_to_e4m3,
    quantize_rows_e4m3,
    SWA_WINDOW,
    swa_ring_slots,
    swa_attention,
    decode_kv,
    full_attention,
    token_scores,
    select_tokens,
    sparse_attention,
    decode_sequence,
    decode_block,
    bridge_kv,
    bridge_kv_fp8,
)
