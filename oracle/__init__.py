"""CPU oracle of the melded FP8 LoRA linear step (FALQON).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
CPU-baseline leg of bench.py, never by the HIP library or its binding.  It
shares no code with fp8_quantized_lora_amd/.
"""
from . import baselines, e2m1, e4m3, e5m2
from .melded import (fp8_quantize, dequantize, melded_linear_fwd, melded_linear_bwd,
                     fp4_quantize, melded_linear_fwd_fp4,
                     melded_linear_fwd_frozen_a,
                     melded_linear_bwd_frozen_a, fp8_dequantize, adapter_step, adapter_step_adamw, adamw_scalars, adamw_update,
                     rowwise_proxy_update, row_scores, select_rows,
                     rowwise_proxy_update_topk_rank, component_scores, select_components,
                     rank_delta, num_threads, set_num_threads)

__all__ = ["baselines", "e2m1", "e4m3", "e5m2", "fp8_quantize", "dequantize", "melded_linear_fwd", "melded_linear_bwd",
           "fp4_quantize", "melded_linear_fwd_fp4",
           "melded_linear_fwd_frozen_a", "melded_linear_bwd_frozen_a", "fp8_dequantize",
           "adapter_step", "adapter_step_adamw", "adamw_scalars", "adamw_update",
           "rowwise_proxy_update", "row_scores", "select_rows",
           "rowwise_proxy_update_topk_rank", "component_scores", "select_components",
           "rank_delta", "num_threads", "set_num_threads"]
