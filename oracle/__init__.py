"""CPU oracle for the NUMA-aware attention and the CAC-scheduled GEMM (test
infrastructure).

Only tests/, ``__graft_entry__.smoke()`` and bench.py's cpu_baseline leg may
import this package.  It shares no code with the HIP path.
"""
from .sdpa import attention, attention_head_rows, attention_sampled, kv_head
from .split import causal_offset, merge, partial_attention, partial_head_rows
from .backward import (attention_backward, backward_key_rows, backward_query_rows,
                       backward_zero_keys)
from .gemm import cac_tile_table, gemm
from .remap import (NBF, NHF, SBF, SHF, LONGEST_FIRST, BALANCED_SPLIT, MODE_NAMES,
                     acc_is_split, chiplet_swizzle, folded, num_workgroups, row_blocks,
                     slice_starts, wg_map, wg_table, xcd_of)

__all__ = [
    "attention", "attention_head_rows", "attention_sampled", "kv_head",
    "causal_offset", "merge", "partial_attention", "partial_head_rows",
    "attention_backward", "backward_key_rows", "backward_query_rows", "backward_zero_keys",
    "cac_tile_table", "gemm",
    "NBF", "NHF", "SBF", "SHF", "LONGEST_FIRST", "BALANCED_SPLIT", "MODE_NAMES",
    "acc_is_split", "chiplet_swizzle", "folded", "num_workgroups", "row_blocks",
    "slice_starts", "wg_map", "wg_table", "xcd_of",
]
