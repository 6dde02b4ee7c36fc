"""Plain fp64 CPU oracle for block-sparse attention with NABLA / sliding-tile masks.

TEST INFRASTRUCTURE ONLY. The product path (the HIP library and its Python
binding) never imports, calls or links anything here; only the tests, the smoke
check and the benchmark's CPU-baseline leg do. Nothing here is blocked, fused or
reordered beyond the definitions it cites, so each step can be checked against the
pages by eye:

  nabla.py      adaptive block mask: block pooling, reduced map, row softmax,
                descending sort, exclusive cumulative mass, threshold at 1 - thr;
                the Top-k alternative (fixed count per row) on the same map
  sta.py        static sliding-tile block mask (tile window, clipped at borders)
  attention.py  softmax attention restricted to the kept N x N blocks
  attention_bwd.py  its gradients dQ, dK, dV (plain derivative of the same definition)
  csr.py        union of masks and the per-query-block kv index lists
  fp8.py        e4m3fn encoding and per-block fp8 quantisation of Q and K (optionally after
                the randomised Hadamard rotation of incoherent processing)
  reorder.py    token orders (tile-major / fractal flattening, spatial-major) and reordering

Pins: every function is checked by `tests/test_oracle_*.py` against closed forms,
brute force, textbook identities or library routines (see those files).
"""
from .nabla import block_pool, reduced_map, row_softmax, cdf_select, nabla_mask, nabla_masks, topk_select, topk_mask
from .sta import sta_block_mask, sta_token_mask
from .attention import block_sparse_attention
from .attention_bwd import block_sparse_attention_bwd
from .csr import mask_or, mask_to_csr, longest_first_order
from .fp8 import decode_e4m3fn, encode_e4m3fn, fwht_rows, quantize_blocks, quantize_blocks_rotated
from .reorder import order_coords, reorder_tokens

__all__ = ["block_pool", "reduced_map", "row_softmax", "cdf_select", "nabla_mask", "topk_select", "topk_mask",
           "nabla_masks", "sta_block_mask", "sta_token_mask", "block_sparse_attention",
           "block_sparse_attention_bwd",
           "mask_or", "mask_to_csr", "longest_first_order", "decode_e4m3fn", "encode_e4m3fn",
           "quantize_blocks", "order_coords", "reorder_tokens"]
