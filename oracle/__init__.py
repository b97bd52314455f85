"""CPU oracle for paged decode attention and its cache operations.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import, call or execute anything under
oracle/.  The product library never routes through it, and it imports nothing
from the product package: the two share no code.
"""
from .attention import attend, decode_attention, gather_logical, widen
from .block_manager import BlockManagerModel, OutOfBlocks
from .cache_ops import copy_blocks, reshape_and_cache, slot_address, swap_blocks

__all__ = ["attend", "decode_attention", "gather_logical", "widen",
           "BlockManagerModel", "OutOfBlocks", "copy_blocks",
           "reshape_and_cache", "slot_address", "swap_blocks"]
