"""CPU oracle for jagged (variable-length) multi-head attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute anything in this package: only the test suite, the smoke check of the
package entry module and the CPU-baseline leg of the benchmark use it.

It is a plain, slow, obviously correct fp64 NumPy implementation of what the
HIP path computes, written from the pages that describe the method:

* [GEM-MFU, Detailed notes: jagged input] -- web page piletech.kr/articles/112134
  (Meta's GEM ads model training efficiency write-up), section "상세 정리"
  (Detailed notes), item on the jagged-input problem: per-request sequences
  have different lengths; padding wastes compute; attention patterns include
  self attention and cross attention with asymmetric Q/KV lengths.
* [GEM-MFU, Detailed notes: JFA] -- same page and section, item on Jagged
  Flash Attention: attention computed directly on variable-length tensors,
  masking done by subtraction rather than a -inf fill, an atomic-free
  backward.  Flash attention is an exact reformulation of attention, so the
  oracle writes out the plain definition.
* [GEM-MFU, Detailed notes: GDPA] -- same page and section, item on
  Generalized Dot-Product Attention: a non-softmax activation in place of
  softmax.
* [GEM infra, Training infrastructure] -- web page aicasebook.dev/setup/21
  ("Meta의 광고 추천 파운데이션 모델 GEM -- 아키텍처, 학습 인프라"), section
  "학습 인프라" (Training infrastructure): in-house kernels plus computation
  fusion for jagged user sequences.

Modules:
  attention -- jagged forward / backward, softmax and SiLU (GDPA)
  schedule  -- the integer work-list enumeration of the tile scheduler
  rope      -- rotary position embedding of BlockAttention
               ([GEM-MFU, Detailed notes: BlockAttention item])
  pooled    -- pooled multi-head attention (shared seed queries per sequence)
               ([GEM-MFU, Detailed notes: jagged input])
  bbs       -- Base Batch Shuffling, the batch former ahead of the path
               ([GEM-MFU, Detailed notes: Base Batch Shuffling item])
  mx        -- MXFP8 attention forward: OCP Microscaling E4M3 operands and
               the online quantisation of the softmax numerator
               ([GEM-MFU, Key points: MXFP8], [GEM-MFU, Detailed notes:
               MXFP8 item])

Every function is pinned by tests marked "not gpu" against an independent
brute-force implementation, library special cases, closed forms, invariants
and finite differences.
"""

from .attention import attention_fwd, attention_bwd, visible_mask  # noqa: F401
from .bbs import bbs_plan, merged_loads  # noqa: F401
from .mx import mx_attention_bwd, mx_attention_fwd, mx_quantize_keys, mx_quantize_rows  # noqa: F401
from .pooled import pooled_bwd, pooled_fwd  # noqa: F401
from .rope import rope, sequence_positions  # noqa: F401
from .schedule import (  # noqa: F401
    fwd_tile_costs,
    kv_tile_costs,
    worklist,
)
