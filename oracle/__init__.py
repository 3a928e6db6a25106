"""CPU oracle for one block-diffusion denoising step.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports this package: only
the tests, the smoke check and the benchmark's CPU-baseline leg do. It is a plain,
slow, float64 NumPy statement of what the step computes, written from the pages
and sharing no code with the HIP kernels.

Pages cited in this package (by title and section):
  [P1] "DiffusionGemma: vLLM에서 네이티브로 처음 지원되는 첫 번째 Diffusion LLM"
       (agentlenshq.com blog summary of the vLLM integration)
  [P2] "DiffusionGemma 개발자 가이드" (molayo1419.me retelling of the developer guide)
  [P3] "DiffusionGemma u vLLM: prvi diskretni difuzijski model od 26 milijardi
       parametara integriran u produkcijsko okruženje" (24-ai.news)

Every function is pinned by a CPU test against something other than itself
(closed forms, library routines, brute force on tiny inputs, invariants);
the pins are listed in tests/test_oracle_*.py.
"""
from .attn import attn_mixed, key_range, CAUSAL, BIDIR  # noqa: F401
from .kvcache import attn_mixed_paged, kv_write, gather_rows, pool_row  # noqa: F401
from .philox import philox4x64_10, uniform24, renoise_token  # noqa: F401
from .sampler import (row_stats, candidate, select, convergence, sampler_step,  # noqa: F401
                      CONF_NEG_ENTROPY, CONF_MAX_PROB, CONV_AND, CONV_OR, FIXED_SHIFT)
from .selfcond import selfcond_embed, softmax_rows  # noqa: F401
from .inject import selfcond_inject, gelu_tanh  # noqa: F401
from .fp8 import (e4m3_value, e4m3_decode, e4m3_encode, quantize, dequantize, attn_mixed_fp8,  # noqa: F401
                  attn_mixed_paged_fp8, kv_write_fp8, E4M3_MAX)
