"""Plain, slow, fp64 CPU oracle for the hybrid gated-SWA / global causal GQA attention layer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this package: only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call it. It shares no code with the HIP library (no kernels, headers, helpers,
tables or constants) and never imports it.

Sources (cited by page title and section; the pages are the authority on what is computed):

* "ZGCM-1-7B 完全解説 ... 全公開基盤モデル" (gotosocial.chinng-lab-srv.dev), section
  "アーキテクチャ — スライディングウィンドウとグローバル注意のハイブリッド設計": layer
  schedule, the GatedSWA formula, QK-RMSNorm and partial RoPE with rotary ratio 0.33, the
  KV-cache footprint.
* "ZGCM-1: A Fully Open and Extremely Efficient Foundation Model for Math and Agentic
  Search" (jaehun.me review), sections "1) 구조·시스템 공동 설계", "게이트형 SWA의 동작"
  (worked window/gate example) and "KV 캐시가 6.4배 줄어드는 이유" (per-token KV bytes).
* hyper.ai summary of arXiv 2609.13356, section "方法" (the GatedSWA display equation).

Parity status per function is listed in ``oracle/attn.py``'s header.
"""

from .attn import (  # noqa: F401
    rotary_dim_for,
    rmsnorm,
    partial_rope,
    sigmoid,
    visible_mask,
    prefill,
    prefill_rows,
    decode_global,
    decode_swa,
    layer_kinds,
    kv_bytes_per_token,
)
