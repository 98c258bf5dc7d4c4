"""MI355X (gfx950) MiniMax Sparse Attention hot path.

The index branch (block max-pool, q.blockmax scores, causal top-K) and the
sparse branch (GQA over the selected blocks, KV outer / gather Q, with a
log-sum-exp merge) run as HIP kernels behind the C ABI of ``include/msa.h``;
``ops`` binds each entry point under its own name and ``pipeline`` chains them
for a whole prefill or decode step.
"""
from .ops import (MsaError, load, msa_index_pool, msa_index_topk,  # noqa: F401
                  msa_index_topk_decode, msa_invert_selection,
                  msa_sparse_gqa_decode, msa_sparse_gqa_prefill)
