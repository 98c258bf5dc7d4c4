"""Host-side checks of the Python binding (no GPU): the bindings pass sizes,
not shapes, to the C calls, so each compares the tensors' layouts with the
sizes it hands over and raises ValueError on a mismatch."""
import pytest


def test_bindings_refuse_mismatched_layouts():
    """The bindings pass sizes, not shapes, to the C calls, so each checks
    the tensors' layouts first (before any device check: CPU tensors reach
    the shape test here) -- pages of another block size, caches of another
    head dimension, tables of another sequence count are refused."""
    import torch
    from block_sparse_attention_index_amd import ops
    bf = torch.bfloat16
    q = torch.zeros(2, 8, 64, dtype=bf)
    sel = torch.zeros(2, 4, dtype=torch.int32)
    seq = torch.zeros(2, dtype=torch.int64)
    with pytest.raises(ValueError, match="k_pages"):     # pages of block 128, block 64 stated
        ops.msa_sparse_gqa_decode_paged(q, torch.zeros(6, 2, 128, 64, dtype=bf),
                                        torch.zeros(6, 2, 128, 64, dtype=bf),
                                        torch.zeros(2, 3, dtype=torch.int32), seq, sel, 64)
    with pytest.raises(ValueError, match="block_table"):  # table rows != sequences
        ops.msa_sparse_gqa_decode_paged(q, torch.zeros(6, 2, 64, 64, dtype=bf),
                                        torch.zeros(6, 2, 64, 64, dtype=bf),
                                        torch.zeros(3, 3, dtype=torch.int32), seq, sel, 64)
    with pytest.raises(ValueError, match="k_cache"):      # head dimension 32, q has 64
        ops.msa_sparse_gqa_decode(q, torch.zeros(2, 2, 256, 32, dtype=bf),
                                  torch.zeros(2, 2, 256, 32, dtype=bf), seq, sel, 64)
    with pytest.raises(ValueError, match="^v has"):       # v differs from k
        ops.msa_sparse_gqa_prefill(q, torch.zeros(2, 16, 64, dtype=bf),
                                   torch.zeros(2, 8, 64, dtype=bf), sel,
                                   torch.zeros(2, dtype=torch.int32),
                                   torch.zeros(8, dtype=torch.int32), sel, 8)
    with pytest.raises(ValueError, match="k_pages"):      # paged prefill, wrong block
        ops.msa_sparse_gqa_prefill_paged(q, torch.zeros(6, 2, 32, 64, dtype=bf),
                                         torch.zeros(6, 2, 32, 64, dtype=bf),
                                         torch.zeros(4, dtype=torch.int32), sel,
                                         torch.zeros(5, dtype=torch.int32),
                                         torch.zeros(8, dtype=torch.int32), sel, 64)
    kn = torch.zeros(2, 2, 64, dtype=bf)
    iq = torch.zeros(2, 16)
    with pytest.raises(ValueError, match="kmax"):          # summaries of another d_idx
        ops.msa_decode_step(q, kn, kn, iq, iq, torch.zeros(2, 2, 256, 64, dtype=bf),
                            torch.zeros(2, 2, 256, 64, dtype=bf), torch.zeros(2, 4, 8), seq,
                            64, 4)
    with pytest.raises(ValueError, match="k_pages"):       # paged step, pages of other heads
        ops.msa_decode_step_paged(q, kn, kn, iq, iq, torch.zeros(6, 4, 64, 64, dtype=bf),
                                  torch.zeros(6, 4, 64, 64, dtype=bf),
                                  torch.zeros(2, 3, dtype=torch.int32), torch.zeros(2, 4, 16),
                                  seq, 64, 4, 192)
