"""invariant_numerics_amd: batch-invariant, fixed-reduction-order token log-probabilities on
AMD Instinct MI355X (gfx950).

The computation runs in libinvnum.so (hand-written HIP kernels behind a C ABI, declared in
include/invnum.h).  ``binding`` is a thin ctypes layer with the same entry-point names;
``decoder`` assembles a Llama-shaped decoder from those calls.  PyTorch provides device
memory and streams only.
"""
from . import binding  # noqa: F401  (fails loudly if libinvnum.so is missing)
from .binding import (  # noqa: F401
    InvError, inv_add, inv_attention_decode, inv_attention_decode_noalloc,
    inv_attention_decode_noalloc_max_bytes, inv_gemm_backward, inv_gemm_backward_workspace_bytes, inv_attention_decode_workspace_bytes,
    inv_attention_prefill, inv_attention_prefill_workspace_bytes, inv_embed, inv_eval_numerics, inv_fixed_order_gemm, inv_gated_gemm,
    inv_get_constants, inv_kernel_route,
    inv_lmhead_logit_grad, inv_lmhead_logit_grad_workspace_bytes, inv_lmhead_logprob_top2, inv_lmhead_workspace_bytes, inv_mfma_f32_check, inv_mfma32_f32_check,
    inv_mfma_bf16_check, inv_mfma_rate_probe, inv_read_stream_probe, inv_qkv_rope_kv_append, inv_rmsnorm, inv_rmsnorm_gemm,
    inv_rmsnorm_qkv_rope_kv_append, inv_rope_kv_append,
    inv_round_activations, inv_status_string, inv_swiglu,
)
