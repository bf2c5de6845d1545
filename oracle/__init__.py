"""CPU oracle for the hybrid H/R/T masked-attention backbone.

TEST INFRASTRUCTURE ONLY.  Plain, slow, float64 numpy code that states what the
method computes, written from the pages' equations and rules.  Only the test
suite, the smoke check and the CPU-baseline leg of the benchmark may import it.
It shares no code with the HIP library or its Python binding, and the product
path never calls it.

Pages cited (their titles; sections as numbered on each page):
  [explainer] "美团推荐大模型 MTFM (Meituan Foundation Model) 深度硬核解析：跨场景推荐的
              终极答案？" (dingyadong.top)
  [blog]      "MTFM：美团统一推荐基座大模型在外卖多业务场景的落地实践" (Meituan tech
              blog, mirrored on dujian.net)
  [digest]    "外卖几条业务线共用一套精排骨干：美团 MTFM 免掉跨业务特征对齐，推理成本降 24%"
              (neodrop.ai)

Modules:
  mask   - the dynamic visibility mask by literal rule enumeration, and the
           per-row / per-tile metadata derived from it by brute force.
  model  - group LayerNorm, the full-attention layer, the target-attention
           layer and the hybrid backbone (forward).
  grad   - hand-derived backward of both layer types.
  v2     - the V2 target side (AutoSplit, per-sub-token SwiGLU FFN, token
           mixing, mean pooling).
  sparse - 2:4 structured pruning of the projection weights.

Parity status: every function here is pinned by the not-gpu tests (worked
example from [explainer] §8.2, brute force, closed forms, invariants, library
special cases, finite differences).  Absolute activation values are printed
nowhere on the pages, so they are pinned only through those properties.
"""
from . import mask, model, grad, v2, sparse  # noqa: F401
