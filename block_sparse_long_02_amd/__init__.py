"""MiniMax Sparse Attention (MSA) forward path for MI355X (gfx950).

The computation lives in libmsa.so (hand-written HIP kernels behind the C ABI
of include/msa.h); `binding` marshals torch tensors into it and `inputs`
draws the seeded synthetic workloads.  Importing the package does not load
the library; the first call does, and fails loudly if it is not built.
"""
from .binding import (MSA_CHECK_LENS, MSA_DENSE, MSA_FORCE_SINK, MSA_GIVEN_INDICES, MSA_OP_BACKWARD, MSA_OP_DECODE,  # noqa: F401
                      MSA_ONE_PASS_INDEX, MSA_OP_INDEX_TOPK,
                      MSA_OP_PREFILL, MSAError, load_library, make_dims, msa_abi_version,
                      msa_decode, msa_decode_noalloc, msa_dims, msa_index_scores, msa_index_topk, msa_indexer_kl, msa_prefill,
                      msa_prefill_backward,
                      msa_status_string,
                      msa_profile_begin, msa_profile_end, msa_stage_name, msa_workspace_bytes,
                      scores_row_stride)
