"""CPU oracle of one MoE layer (forward and backward) and of its MXFP8 format.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import or run anything here.  The GPU
library (``mixture_experts_layer_offsets_amd``) shares no code with it and
never calls it: the oracle exists to check that library.

Modules:
  numerics  bf16 / fp32 rounding points
  mx        E4M3 + E8M0 block quantiser (OCP Microscaling conversion)
  layer     router, top-k, layout, dispatch, SwiGLU experts, combine, backward,
            plus a per-token brute-force evaluator and a sampled weight-gradient
            evaluator for sizes the full oracle cannot finish

Parity status: every function is pinned by ``tests/test_oracle_*.py`` against
something other than itself (hand-computed fixtures, closed forms, library
routines, brute force, finite differences, an independent autograd
formulation, weights exactly representable along one axis only for the MX
quantisation axes), except the choice of the MX recipe of the backward pass
(which tensors the backward quantises): "parity unpinned" for that choice,
since the pages do not say; its arithmetic is pinned through the quantiser,
the weight axes and the bf16 path.
"""
from . import layer, mx, numerics  # noqa: F401
from .layer import (ExpertWeights, TokenEvaluator, backward, combine,  # noqa: F401
                    dispatch, expert_weight_grad_columns, forward, layout,
                    router_backward, router_logits, topk_softmax)
