"""MI355X (gfx950) quantized-linear library for mixed-precision video DiTs.

The method is 6Bit-Diffusion's inference-time NVFP4/INT8 mixed precision
(abstract; Fig. 2 and Fig. 3 captions) with the Temporal Delta Cache
(abstract; Fig. 4 caption).  All work runs in the HIP kernels of
``libqact.so``; this package only binds its C ABI (``include/qact.h``) and
allocates buffers with torch.
"""
from ._lib import (AMAX_GIVEN, BLK_RUN0, BLK_RUN1, BLK_SKIP0, BLK_SKIP1, EPI_GELU_TANH,
                   EPI_NONE, EXPORTS, INT8, LIB_PATH, NOALLOC_SCRATCH_BYTES, NVFP4, OUT_BF16, OUT_F32, ROUTE_INT8,
                   ROUTE_NVFP4, TSCALE_GIVEN, QactError, act_quant, act_quant_routed, act_quant_workspace,
                   block_gamma, build_info, cosine_from_sums, decide_step, delta_cosine,
                   dmpq_fit, dmpq_mask, gamma_from_sums, gate, int8_weight_planes,
                   int8_weight_planes_bytes, int8_weight_planes_count, lib, qlinear,
                   qlinear_int8, qlinear_int8_acc, qlinear_int8_noalloc,
                   qlinear_int8_amax, qlinear_int8_q, qlinear_layer_workspace, qlinear_nvfp4,
                   qlinear_nvfp4_amax, qlinear_nvfp4_q, qlinear_routed, qlinear_routed_workspace,
                   qlinear_workspace, reduce_workspace,
                   rel_err, rel_err_from_sums, rel_l2_from_sums, set_gate, set_gemm_events,
                   strerror, tdc_apply, tdc_apply_amax, tdc_apply_ring, tdc_decide, tdc_decide_cos,
                   tdc_update, tdc_update_ring)
from .buffers import (empty_int8_act, empty_int8_planes, empty_nvfp4, workspace)

__all__ = [n for n in dir() if not n.startswith("_")]
