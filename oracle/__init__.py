"""CPU oracle for the MoE FFN layer forward (test infrastructure).

A plain, slow, fp64 numpy restatement of what the layer computes, written from
the article texts that define the method.  It is test infrastructure only:
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it; the product path (``fp8_grouped_gemm_amd``) never
does, and this package imports nothing from it.

Sources (cited by page title / host and section):
  * MegaMoE + DeepGEMM walkthrough (discosf.com), sec. 2.1 (top-k weighted sum),
    sec. 2.2 (softmax with per-expert bias), sec. 3.2 (grouped GEMM, group sizes),
    sec. 3.3 (e4m3 clamp-and-round quantisation, fp32 accumulation, RNE to bf16).
  * Dense GEMM to TP-MoE (cf-1.com), sec. 3.1 (gate normalisation choices),
    sec. 4.2 (grouped GEMM = loop of per-expert GEMMs).
  * DeepSeek-V4 lecture 4 (tqpw.cn), sec. 2.2 (hash routing), sec. 2.3 (fp32
    softmax), sec. 3.1 (block-wise 4-bit weights with max-abs scale).
  * DeepSeek MoE architecture (mooersco.com), ch. 1 (top-k then softmax variant),
    sec. 2.5 (expert capacity and silent overflow drop).
  * DeepSeek open-source week (qidao123.com), day 3 (fine-grained scaling,
    two-level accumulation).

Functions whose result no test pins to an independent fact say "parity
unpinned" in their docstring.
"""
from .codecs import (E4M3_MAX, bf16_round, e4m3_decode, e4m3_decode_table, e4m3_encode,
                     int4_dequant, int4_dequant_exact, int4_quant_rows, quant_fp8_act,
                     quant_fp8_weight,
                     dequant_fp8_act, dequant_fp8_weight)
from .moe import (capacity, combine, dispatch, dispatch_masked, grouped_gemm, grouped_gemm_w4a8, grouped_gemm_fp8, hash_route,
                  layer_forward, router_logits, rows_bound, silu, swiglu, topk_route)

__all__ = [
    "E4M3_MAX", "bf16_round", "e4m3_decode", "e4m3_decode_table", "e4m3_encode",
    "int4_dequant", "int4_dequant_exact", "int4_quant_rows", "quant_fp8_act", "quant_fp8_weight",
    "dequant_fp8_act", "dequant_fp8_weight", "capacity", "combine", "dispatch", "dispatch_masked",
    "grouped_gemm", "grouped_gemm_fp8", "grouped_gemm_w4a8", "hash_route", "layer_forward", "router_logits",
    "rows_bound", "silu", "swiglu", "topk_route",
]
