"""CPU oracle for attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
definition that the HIP kernels are checked against.  Only the tests, the
smoke check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may
import it; the library itself never does, and nothing here imports the
library.

Arithmetic is float64 on the exact float values of the bfloat16 inputs.
Every function is pinned by ``tests/test_oracle.py`` (closed forms, brute
force on tiny inputs, a library attention routine, permutation invariance and
the pages' worked examples); there is no "parity unpinned" function here.
"""
from .block_manager import BlockManager, block_hash, fnv1a64  # noqa: F401
from .fp8 import (  # noqa: F401
    E4M3_MAX,
    dequantize,
    e4m3_decode,
    e4m3_encode,
    kvcache_store_fp8,
    paged_decode_fp8,
    paged_prefill_fp8,
    quantize,
)
from .paged_attention import (  # noqa: F401
    bf16_to_f64,
    kv_head_for,
    kvcache_store,
    paged_decode,
    paged_prefill,
    softmax_attention,
    unpage,
    visible,
)
