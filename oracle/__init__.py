"""CPU oracle for the routed-MoE layer over a bounded, all-layer-shared expert cache.

TEST INFRASTRUCTURE ONLY.  Only tests, the smoke check and the benchmark's CPU
baseline may import this package.  It shares no code with the GPU library: it
is a plain, slow, fp64 restatement of what the method computes, so that a
reader can check each function against the pages by eye.

Sources (cited by page title and section in each function):
  [FT-KR]  "FreeToken: ... Edge-Serving에 대한 연구" -- FreeToken paper summary
           (discuss.pytorch.kr).  Sections used: "FreeToken의 설계" (design,
           Figure 2 prose), "전층 이중 버퍼링" (full-layer double buffering),
           "라우터를 따라 움직이는 LRU 캐시" (router-following LRU cache),
           "측정된 대역폭이 분할을 결정합니다" (measured bandwidths decide the
           split: B_R, T_fill, T_cpu, q*), "탄력적 메모리 관리" (elastic memory),
           "CUDA Graph와 공존하는 LRU 캐시" (graph-compatible LRU cache),
           "전문가 뱅크와 FTW 포맷" (expert banks), "실험 환경" (Table 1).
  [FT-CN]  "论文精读 · FreeToken: 边缘原生的 MoE 服务系统" -- reading notes
           (qqtang-code.github.io).  Sections: 04 Design (Figure 2 caption,
           mechanisms 1-3 and the displayed equations), 05 Implementation.
  [SPARK]  "Luce Spark" forum post (molayo1419.me): bounded async slot ring;
           full residency is bit-identical to all-GPU execution.

Parity status of each function is stated in its docstring; readings of points
the pages leave open are listed in the repository's design notes.
"""
from .formats import bf16_to_f64, e2m1_decode, dequant_fp4, e8m0_decode, dequant_mxfp4, expert_weights_f64
from .router import router_logits, topk_order, route
from .qstar import MODE_FUSED, MODE_OFFLOAD, MODE_CPU, MODE_HYBRID, qstar_split, qstar_real
from .cache import (ExpertCache, NaiveListCache, LookupResult, KIND_HIT, KIND_FILL, KIND_CPU, KIND_BUF)
from .ffn import silu, expert_ffn, moe_combine, moe_layer_dense
from .layer import OracleMoE
from .mx import e4m3_decode, mxfp8_quantize, mxfp8_dequant, mxfp8_round, expert_ffn_mx
from .placement import (POLICY_LRU, POLICY_PREFILL, POLICY_STATIC, POLICY_PINNED_RING, replay as placement_replay,
                        routing_counts, top_keys, static_resident)

__all__ = [
    "bf16_to_f64", "e2m1_decode", "dequant_fp4", "e8m0_decode", "dequant_mxfp4", "expert_weights_f64",
    "router_logits", "topk_order", "route",
    "MODE_FUSED", "MODE_OFFLOAD", "MODE_CPU", "MODE_HYBRID", "qstar_split", "qstar_real",
    "ExpertCache", "NaiveListCache", "LookupResult", "KIND_HIT", "KIND_FILL", "KIND_CPU", "KIND_BUF",
    "silu", "expert_ffn", "moe_combine", "moe_layer_dense", "OracleMoE",
    "e4m3_decode", "mxfp8_quantize", "mxfp8_dequant", "mxfp8_round", "expert_ffn_mx",
    "POLICY_LRU", "POLICY_PREFILL", "POLICY_STATIC", "POLICY_PINNED_RING", "placement_replay",
    "routing_counts", "top_keys", "static_resident",
]
