"""CPU oracle for the expert-parallel MoE layer (route, layout, dispatch,
grouped SwiGLU FFN, combine).

TEST INFRASTRUCTURE.  This package is a plain, slow, obviously correct numpy
statement of what the layer computes, written from the pages' description of
the method.  It shares no code with the HIP path and is never imported by the
product package; only the tests, the package smoke check and the bench's
CPU-baseline leg use it.

Sources (cited by title and section in each function):
  * "Anatomy of a high-performance EP kernel" (euno.news, Korean) and its
    Chinese translation (66bd.net) -- the problem statement and the worked
    router rows;
  * Moreh, "21K output tokens/s DeepSeek inference on AMD Instinct MI300X
    GPUs with Expert Parallelism" -- expert placement and load balancing;
  * SGLang documentation, "Expert Parallelism" -- the stage pipeline.

Parity status of each function (what pins it, in tests/test_oracle_*.py):
  route          pinned: worked rows, closed-form two-way gates, full softmax
                 at K = E, brute-force top-K over {-1,0,1}^E.
  route_shared   pinned: the layer with a shared expert equals the routed
                 layer plus a dense SwiGLU of the shared weights per token.
  layout         pinned: brute-force construction, sum of counts, bijection.
  layout_masked  pinned: agrees with the contiguous layout (a different
                 construction) shifted to fixed row blocks; overflow keeps the
                 first cap_e slots of an expert in (t, k) order.
  dispatch/combine pinned: identity-expert round trip returns x * sum(gates).
  eplb           expert placement (Moreh report, load balancing between GPUs):
                 pinned by a hand-worked case, a perfect split, exhaustive
                 optima of small instances, and the report's outcome (2x ->
                 within 5%) on the EP-share workload's routing.
  expert_ffn     pinned: dense SwiGLU via torch CPU, pure-Python brute force.
  numerics       pinned: exhaustive bf16 / e4m3 casts against torch.
  fp8 block geometry and scale rule: parity unpinned by the pages (a reading
  both sides implement); its properties are checked.
"""
from . import eplb, numerics
from .moe import (route, route_shared, layout, layout_masked, dispatch, silu, expert_ffn, grouped_ffn,
                  grouped_ffn_masked, combine, layer)

__all__ = ["eplb", "numerics", "route", "route_shared", "layout", "layout_masked", "dispatch", "silu", "expert_ffn",
           "grouped_ffn", "grouped_ffn_masked", "combine", "layer"]
