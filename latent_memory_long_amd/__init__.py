"""MI355X (gfx950) implementation of Memory Sparse Attention's routing + sparse-attention
hot path: chunk-mean pooling with document-wise RoPE, the cosine router scan, top-k
document selection, and sparse GQA attention over the selected memory plus the local
context.  The kernels live in csrc/ and are reached through the C ABI of include/msa.h;
``binding`` exposes the same entry points to Python.
"""
from .binding import (  # noqa: F401
    MSA_BF16, MSA_F32, MSA_ROPE_K, MSA_ROPE_KR, MSA_ROPE_V, LIB_PATH, MsaError,
    msa_chunk_offsets, msa_last_error, msa_pool, msa_route_scan, msa_route_topk,
    msa_route_topk_workspace, msa_topk, msa_topk_workspace,
    msa_sparse_attn, msa_sparse_attn_workspace, msa_status_string, msa_version,
    msa_sparse_attn_backward, msa_sparse_attn_backward_workspace,
    msa_route_backward, msa_route_backward_workspace,
    MSA_AUX_BCE, MSA_AUX_INFONCE, msa_route_aux_loss,
    MSA_ERR_IO, msa_bank_save, msa_bank_read_info, msa_bank_load,
    MSA_OK, MSA_ERR_INVALID_ARG, MSA_ERR_UNSUPPORTED, MSA_ERR_WORKSPACE, MSA_ERR_HIP,
    RouteKeys, msa_krbar_elems, msa_krbar_pack, msa_krbar_unpack,
    msa_route_topk_noalloc, MSA_ROUTE_TOPK_NOALLOC_SCRATCH_BYTES,
)
