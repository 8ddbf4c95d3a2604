"""CPU oracle for varlen grouped-query attention — TEST INFRASTRUCTURE ONLY.

This package is the slow, plain, fp64 statement of what the library computes.
It exists to check the HIP path; nothing in the product path may import, call
or execute it. Only the test suite, the smoke check and the benchmark's CPU
baseline leg use it. It shares no code with the HIP path (no kernels, headers,
helpers or constants) and imports nothing from the product package.

Sources (web pages), cited in the modules by the short tags below:

  [FROST#552]  cudnn-frontend issue #552, "frost(sdpa): THD execute host
               round-trip — D2H sync, per-total recompile, and CUDA-graph
               capture" (sections: Context; How the other backends avoid this;
               Proposal to evaluate).
  [SPLITK]     magik.net blog, "The Orchestrator's Moment: Wiring Split-K
               Dispatch into a Custom CUDA Attention Kernel" (sections: The
               Context: Why Split-K Matters; The Thinking Process; Assumptions
               and Their Validity; Output Knowledge Created).
  [KERNBENCH]  kernbench2 commit page docs/adr-proposed (commits "GQA via
               M-fold" finding, and the reframe onto the greenlet tl API with
               tree reduction of running (m, l, O)).
  [TE#24]      TransformerEngine PR #24, "[PyTorch] Build the attention padding
               mask without host syncs" (sections: Description; Changes;
               Equivalence).
  [ASTRAI]     AstrAI commit log for csrc/kernels/gqa_decode_attn.cu (commits:
               split-KV with (O, m, l) partials and combine kernel; decode MMA
               with cp.async / XOR swizzle / pre-scaled Q; HEAD_DIM=32 case;
               MMA decode header, dispatch_decode, prefill tiling).

Modules:
  attention  fp64 varlen GQA attention, split partials and the LSE merge,
             attention over gathered (index-listed) keys
  backward   fp64 gradients dq, dk, dv of the same attention (chain rule
             through the softmax)
  brute      scalar pure-Python triple loops (tiny inputs only; a pin)
  mask       padding mask: vectorised formula and the per-sequence loop form
  chooser    plan-time split-count / grid rule
  bf16       exact round-to-nearest-even of fp64 to bfloat16

Every function here is pinned by the CPU tests (tests/test_oracle_*.py)
against something other than itself: brute force, a library routine, closed
forms, invariants, or the case counts the pages print.
"""
