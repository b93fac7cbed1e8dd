"""MI355X-native paged-KV decode: Python binding of libpagedkv.so.

* :class:`BlockManager` -- host block manager (``pa_bm_*``);
* :class:`Scheduler` -- continuous-batching scheduler (``pa_sched_*``);
* :func:`pa_write_kv`, :func:`pa_copy_blocks`, :func:`pa_swap_out`,
  :func:`pa_swap_in`, :func:`pa_decode`, :func:`pa_write_decode`,
  :func:`pa_decode_workspace_bytes`,
  :func:`pa_decode_shared`, :func:`pa_write_decode_shared`,
  :func:`pa_decode_shared_workspace_bytes`, :func:`pa_prefill`, :func:`pa_decode_noalloc`
  -- the device calls, on torch tensors;
* :func:`pa_shared_plan` -- host planner of shared-prefix groups for
  :func:`pa_decode_shared`;
* :func:`pa_stream_read` -- measurement helper: a streaming read of one
  buffer, the HBM read rate the decode bandwidth is reported beside.

The C ABI is declared in ``include/pagedkv.h``.  Importing this package
loads the library and fails if it has not been built
(``python paged_kv_cache_136_amd/build.py``).
"""

from ._lib import LIB_PATH, OutOfBlocks, PagedKVError, lib
from .block_manager import BlockManager
from .scheduler import Scheduler
from .ops import (pa_copy_blocks, pa_decode, pa_decode_noalloc, pa_decode_noalloc_max_bytes,
                  pa_decode_shared, pa_decode_shared_workspace_bytes,
                  pa_decode_workspace_bytes, pa_prefill, pa_shared_plan,
                  pa_stream_read, pa_swap_in, pa_swap_out, pa_write_decode,
                  pa_write_decode_shared, pa_write_kv, swap_record_bytes)

lib()  # load now: a missing library is an import error, never a fallback

__all__ = ["BlockManager", "Scheduler", "OutOfBlocks", "PagedKVError", "pa_write_kv", "pa_copy_blocks",
           "pa_swap_out", "pa_swap_in", "swap_record_bytes", "pa_decode", "pa_write_decode", "pa_prefill",
           "pa_decode_workspace_bytes", "pa_decode_shared", "pa_decode_shared_workspace_bytes",
           "pa_shared_plan", "pa_write_decode_shared",
           "pa_decode_noalloc", "pa_decode_noalloc_max_bytes", "pa_stream_read", "LIB_PATH"]
