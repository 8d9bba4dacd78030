"""Python binding of libpagedattn: paged-KV attention for MI355X (gfx950).

Argument marshalling only.  Every operation runs in the library's HIP
kernels; PyTorch supplies device memory and the current stream.  Tensors must
be contiguous HIP tensors (bf16 data, int32 indices); nothing is cast or
copied behind the caller's back, and nothing here synchronizes.

If ``libpagedattn.so`` has not been built, every call raises: there is no
fallback path.  Build it with ``python -m paged_kv_cache_86_amd.build``.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpagedattn.so")

PA_OK = 0
PA_BF16 = 0
PA_F32 = 1
PA_ERR_SCRATCH = -8
#: Bytes of the fixed scratch array pa_paged_decode_append_noalloc uses on each GPU.
DECODE_SCRATCH_BYTES = 64 << 20

#: Every symbol ``include/pagedattn.h`` declares.
EXPORTED_SYMBOLS = (
    "pa_status_string",
    "pa_kvcache_store",
    "pa_paged_decode_workspace_bytes",
    "pa_paged_decode",
    "pa_paged_prefill",
    "pa_paged_prefill_fp8",
    "pa_paged_gather",
    "pa_stream_read",
    "pa_decode_time_next_launch",
    "pa_kvcache_store_fp8",
    "pa_paged_decode_fp8_workspace_bytes",
    "pa_paged_decode_fp8",
    "pa_paged_decode_append",
    "pa_paged_decode_append_fp8",
    "pa_paged_decode_append_noalloc",
    "pa_decode_graph_create",
    "pa_decode_graph_buffers",
    "pa_decode_graph_bucket",
    "pa_decode_graph_run",
    "pa_decode_graph_destroy",
    "pa_paged_attention_mixed",
    "pa_bm_create",
    "pa_bm_destroy",
    "pa_bm_num_free",
    "pa_bm_can_allocate",
    "pa_bm_allocate",
    "pa_bm_can_append",
    "pa_bm_append",
    "pa_bm_deallocate",
    "pa_bm_seq_info",
    "pa_bm_block_table",
    "pa_bm_free_list",
    "pa_bm_ref_count",
    "pa_bm_prepare_decode",
    "pa_bm_prepare_prefill",
)

_lib = None


class PagedAttnError(RuntimeError):
    """A libpagedattn call returned a non-zero status."""

    def __init__(self, func: str, status: int, message: str):
        super().__init__(f"{func} failed with status {status}: {message}")
        self.status = status


def load_library() -> ctypes.CDLL:
    """Load ``libpagedattn.so`` (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m paged_kv_cache_86_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.pa_status_string.argtypes = [I]
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_kvcache_store.argtypes = [P, P, P, I, P, P, I, I, I, I, P]
    lib.pa_kvcache_store.restype = I
    lib.pa_paged_decode_workspace_bytes.argtypes = [I, I, I, I, I, I]
    lib.pa_paged_decode_workspace_bytes.restype = Z
    lib.pa_paged_decode.argtypes = [P, P, P, P, I, P, I, I, I, I, I, I, F, P, I, P, Z, P]
    lib.pa_paged_decode.restype = I
    lib.pa_paged_prefill.argtypes = [P, P, P, P, I, I, I, P, P, P, I, P, I, I, I, I, I, F, P, I, P]
    lib.pa_paged_prefill.restype = I
    lib.pa_paged_prefill_fp8.argtypes = [P, P, I, I, I, P, P, P, I, P, I, I, I, I, I, F, F, F, P, I,
                                         P]
    lib.pa_paged_prefill_fp8.restype = I
    lib.pa_paged_gather.argtypes = [P, P, I, P, P, I, I, I, I, I, I, P, P]
    lib.pa_paged_gather.restype = I
    lib.pa_stream_read.argtypes = [P, Z, P, P]
    lib.pa_stream_read.restype = I
    lib.pa_decode_time_next_launch.argtypes = [P, P]
    lib.pa_decode_time_next_launch.restype = I
    lib.pa_kvcache_store_fp8.argtypes = [P, P, P, I, P, P, I, I, I, I, F, F, P]
    lib.pa_kvcache_store_fp8.restype = I
    lib.pa_paged_decode_fp8_workspace_bytes.argtypes = [I, I, I, I, I, I]
    lib.pa_paged_decode_fp8_workspace_bytes.restype = Z
    lib.pa_paged_decode_fp8.argtypes = [P, P, P, P, I, P, I, I, I, I, I, I, F, F, F, P, I, P, Z,
                                        P]
    lib.pa_paged_decode_fp8.restype = I
    lib.pa_paged_decode_append.argtypes = [P, P, P, P, P, P, P, I, P, I, I, I, I, I, I, F, P, I,
                                           P, Z, P]
    lib.pa_paged_decode_append.restype = I
    lib.pa_paged_decode_append_fp8.argtypes = [P, P, P, P, P, P, P, I, P, I, I, I, I, I, I, F,
                                               F, F, P, I, P, Z, P]
    lib.pa_paged_decode_append_fp8.restype = I
    lib.pa_paged_decode_append_noalloc.argtypes = [P, P, P, P, P, P, P, I, P, I, I, I, I, I, I, F,
                                                   P, I, P]
    lib.pa_paged_decode_append_noalloc.restype = I
    PP = ctypes.POINTER(ctypes.c_void_p)
    lib.pa_decode_graph_create.argtypes = [I, I, I, I, I, I, I, I, F, F, F, P, P, I, PP]
    lib.pa_decode_graph_create.restype = I
    lib.pa_decode_graph_buffers.argtypes = [P, PP, PP, PP, PP]
    lib.pa_decode_graph_buffers.restype = I
    lib.pa_decode_graph_bucket.argtypes = [P, I]
    lib.pa_decode_graph_bucket.restype = I
    lib.pa_decode_graph_run.argtypes = [P, I, P, P, P, P, P, I, P, P, P]
    lib.pa_decode_graph_run.restype = I
    lib.pa_decode_graph_destroy.argtypes = [P]
    lib.pa_decode_graph_destroy.restype = I
    lib.pa_paged_attention_mixed.argtypes = [P, P, P, P, P, I, I, I, I, P, P, P, I, P, I, I, I, I,
                                             I, F, P, I, P, Z, P, P]
    lib.pa_paged_attention_mixed.restype = I
    L, IP = ctypes.c_int64, ctypes.POINTER(ctypes.c_int)
    bm_sigs = {
        "pa_bm_create": [I, I, I, PP], "pa_bm_destroy": [P], "pa_bm_num_free": [P],
        "pa_bm_can_allocate": [P, I], "pa_bm_allocate": [P, L, P, I, IP],
        "pa_bm_can_append": [P, L], "pa_bm_append": [P, L, ctypes.c_int32],
        "pa_bm_deallocate": [P, L], "pa_bm_seq_info": [P, L, IP, IP, IP],
        "pa_bm_block_table": [P, L, P, I], "pa_bm_free_list": [P, P, I],
        "pa_bm_ref_count": [P, I], "pa_bm_prepare_decode": [P, P, I, I, P, P, P],
        "pa_bm_prepare_prefill": [P, P, I, I, P, P, P, P, I, IP, IP],
    }
    for name, args in bm_sigs.items():
        getattr(lib, name).argtypes = args
        getattr(lib, name).restype = I
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().pa_status_string(int(status)).decode()


def _raise_on(func: str, status: int) -> None:
    if status != PA_OK:
        raise PagedAttnError(func, status, status_string(status))


def _torch():
    import torch
    return torch


def _check(t, dtype, name: str, ndim: int):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device (HIP) tensor, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(_torch().cuda.current_stream(device).cuda_stream)


def _out_dtype(out) -> int:
    torch = _torch()
    if out.dtype == torch.bfloat16:
        return PA_BF16
    if out.dtype == torch.float32:
        return PA_F32
    raise TypeError(f"out must be bfloat16 or float32, got {out.dtype}")


def _cache_geometry(k_cache, v_cache, dtype=None):
    torch = _torch()
    dtype = torch.bfloat16 if dtype is None else dtype
    _check(k_cache, dtype, "k_cache", 4)
    _check(v_cache, dtype, "v_cache", 4)
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must have the same shape")
    return tuple(int(x) for x in k_cache.shape)  # NB, BS, Hkv, D


def kvcache_store(k, v, slot_mapping, k_cache, v_cache) -> None:
    """Write row t of k/v into cache slot ``slot_mapping[t]`` (negative = skip)."""
    torch = _torch()
    NB, BS, Hkv, D = _cache_geometry(k_cache, v_cache)
    _check(k, torch.bfloat16, "k", 3)
    _check(v, torch.bfloat16, "v", 3)
    _check(slot_mapping, torch.int32, "slot_mapping", 1)
    T = int(k.shape[0])
    if tuple(k.shape) != (T, Hkv, D) or tuple(v.shape) != (T, Hkv, D):
        raise ValueError(f"k and v must be [T, {Hkv}, {D}]")
    if slot_mapping.shape[0] != T:
        raise ValueError("slot_mapping must have one entry per token")
    rc = load_library().pa_kvcache_store(_ptr(k), _ptr(v), _ptr(slot_mapping), T, _ptr(k_cache),
                                         _ptr(v_cache), NB, BS, Hkv, D, _stream(k.device))
    _raise_on("pa_kvcache_store", rc)


def decode_workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                           block_size: int, max_blocks_per_seq: int) -> int:
    return int(load_library().pa_paged_decode_workspace_bytes(
        num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq))


_workspaces = {}


def decode_workspace(nbytes: int, device):
    """A byte buffer of at least ``nbytes`` for decode partials and arrival counters, kept per
    device and reused (zeroed when allocated; every decode call leaves its counters at zero)."""
    torch = _torch()
    dev = torch.device(device)
    key = dev.index if dev.index is not None else torch.cuda.current_device()
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=dev)
        _workspaces[key] = ws
    return ws


def _decode_shapes(q, block_tables, context_lens, out, D):
    torch = _torch()
    _check(q, torch.bfloat16, "q", 3)
    _check(block_tables, torch.int32, "block_tables", 2)
    _check(context_lens, torch.int32, "context_lens", 1)
    B, Hq, Dq = (int(x) for x in q.shape)
    if Dq != D:
        raise ValueError("q head_dim differs from the cache's")
    if block_tables.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("block_tables and context_lens need one row per sequence")
    _check(out, out.dtype, "out", 3)
    if tuple(out.shape) != (B, Hq, D):
        raise ValueError(f"out must be [{B}, {Hq}, {D}]")
    return B, Hq, int(block_tables.shape[1])


def _workspace_for(workspace, need, device):
    if workspace is None:
        return decode_workspace(need, device)
    _check(workspace, _torch().uint8, "workspace", 1)
    return workspace


def paged_decode(q, k_cache, v_cache, block_tables, context_lens, scale: Optional[float], out,
                 workspace=None) -> None:
    """out[i, h] = softmax(scale * q[i, h] . K_i^T) V_i over the paged context of sequence i."""
    NB, BS, Hkv, D = _cache_geometry(k_cache, v_cache)
    B, Hq, MBS = _decode_shapes(q, block_tables, context_lens, out, D)
    need = decode_workspace_bytes(B, Hq, Hkv, D, BS, MBS) if B > 0 else 0
    workspace = _workspace_for(workspace, need, q.device)
    sc = float(scale) if scale is not None else 0.0
    rc = load_library().pa_paged_decode(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), MBS, _ptr(context_lens), B, Hq,
        Hkv, D, BS, NB, sc, _ptr(out), _out_dtype(out), _ptr(workspace), int(workspace.numel()),
        _stream(q.device))
    _raise_on("pa_paged_decode", rc)


def _new_tokens(k_new, v_new, slot_mapping, B, Hkv, D):
    torch = _torch()
    _check(k_new, torch.bfloat16, "k_new", 3)
    _check(v_new, torch.bfloat16, "v_new", 3)
    _check(slot_mapping, torch.int32, "slot_mapping", 1)
    if tuple(k_new.shape) != (B, Hkv, D) or tuple(v_new.shape) != (B, Hkv, D):
        raise ValueError(f"k_new and v_new must be [{B}, {Hkv}, {D}]")
    if slot_mapping.shape[0] != B:
        raise ValueError("slot_mapping must have one entry per sequence")


def paged_decode_append(q, k_new, v_new, slot_mapping, k_cache, v_cache, block_tables,
                        context_lens, scale: Optional[float], out, workspace=None) -> None:
    """kvcache_store of each sequence's new token followed by paged_decode, in one call."""
    NB, BS, Hkv, D = _cache_geometry(k_cache, v_cache)
    B, Hq, MBS = _decode_shapes(q, block_tables, context_lens, out, D)
    _new_tokens(k_new, v_new, slot_mapping, B, Hkv, D)
    need = decode_workspace_bytes(B, Hq, Hkv, D, BS, MBS) if B > 0 else 0
    workspace = _workspace_for(workspace, need, q.device)
    sc = float(scale) if scale is not None else 0.0
    rc = load_library().pa_paged_decode_append(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), _ptr(k_cache), _ptr(v_cache),
        _ptr(block_tables), MBS, _ptr(context_lens), B, Hq, Hkv, D, BS, NB, sc, _ptr(out),
        _out_dtype(out), _ptr(workspace), int(workspace.numel()), _stream(q.device))
    _raise_on("pa_paged_decode_append", rc)


def paged_decode_append_noalloc(q, k_new, v_new, slot_mapping, k_cache, v_cache, block_tables,
                                context_lens, scale: Optional[float], out) -> None:
    """paged_decode_append with the library's fixed per-GPU scratch instead of a workspace: no
    device memory is allocated by this call or by the library behind it."""
    NB, BS, Hkv, D = _cache_geometry(k_cache, v_cache)
    B, Hq, MBS = _decode_shapes(q, block_tables, context_lens, out, D)
    _new_tokens(k_new, v_new, slot_mapping, B, Hkv, D)
    sc = float(scale) if scale is not None else 0.0
    rc = load_library().pa_paged_decode_append_noalloc(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), _ptr(k_cache), _ptr(v_cache),
        _ptr(block_tables), MBS, _ptr(context_lens), B, Hq, Hkv, D, BS, NB, sc, _ptr(out),
        _out_dtype(out), _stream(q.device))
    _raise_on("pa_paged_decode_append_noalloc", rc)


def kvcache_store_fp8(k, v, slot_mapping, k_cache, v_cache, k_scale: float,
                      v_scale: float) -> None:
    """Quantize row t of k/v to E4M3 codes (x / scale) into uint8 cache slot ``slot_mapping[t]``."""
    torch = _torch()
    NB, BS, Hkv, D = _cache_geometry(k_cache, v_cache, torch.uint8)
    _check(k, torch.bfloat16, "k", 3)
    _check(v, torch.bfloat16, "v", 3)
    _check(slot_mapping, torch.int32, "slot_mapping", 1)
    T = int(k.shape[0])
    if tuple(k.shape) != (T, Hkv, D) or tuple(v.shape) != (T, Hkv, D):
        raise ValueError(f"k and v must be [T, {Hkv}, {D}]")
    if slot_mapping.shape[0] != T:
        raise ValueError("slot_mapping must have one entry per token")
    rc = load_library().pa_kvcache_store_fp8(
        _ptr(k), _ptr(v), _ptr(slot_mapping), T, _ptr(k_cache), _ptr(v_cache), NB, BS, Hkv, D,
        float(k_scale), float(v_scale), _stream(k.device))
    _raise_on("pa_kvcache_store_fp8", rc)


def decode_fp8_workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int,
                               head_dim: int, block_size: int, max_blocks_per_seq: int) -> int:
    return int(load_library().pa_paged_decode_fp8_workspace_bytes(
        num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq))


def paged_decode_fp8(q, k_cache, v_cache, block_tables, context_lens, scale: Optional[float],
                     k_scale: float, v_scale: float, out, workspace=None) -> None:
    """Decode over uint8 E4M3 pools: keys code * k_scale, values code * v_scale."""
    torch = _torch()
    NB, BS, Hkv, D = _cache_geometry(k_cache, v_cache, torch.uint8)
    B, Hq, MBS = _decode_shapes(q, block_tables, context_lens, out, D)
    need = decode_fp8_workspace_bytes(B, Hq, Hkv, D, BS, MBS) if B > 0 else 0
    workspace = _workspace_for(workspace, need, q.device)
    sc = float(scale) if scale is not None else 0.0
    rc = load_library().pa_paged_decode_fp8(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), MBS, _ptr(context_lens), B, Hq,
        Hkv, D, BS, NB, sc, float(k_scale), float(v_scale), _ptr(out), _out_dtype(out),
        _ptr(workspace), int(workspace.numel()), _stream(q.device))
    _raise_on("pa_paged_decode_fp8", rc)


def paged_prefill(q, k_new, v_new, cu_seqlens_q, block_tables, context_lens, out, *, k_cache,
                  v_cache, scale: Optional[float] = None, max_q_len: Optional[int] = None) -> None:
    """Prefix-hit prefill over the flattened chunk ``q`` delimited by ``cu_seqlens_q``.

    ``max_q_len`` is a host-side upper bound of the per-sequence chunk length;
    when omitted the total token count is used (correct, with a larger grid).
    """
    torch = _torch()
    NB, BS, Hkv, D = _cache_geometry(k_cache, v_cache)
    _check(q, torch.bfloat16, "q", 3)
    _check(k_new, torch.bfloat16, "k_new", 3)
    _check(v_new, torch.bfloat16, "v_new", 3)
    _check(cu_seqlens_q, torch.int32, "cu_seqlens_q", 1)
    _check(block_tables, torch.int32, "block_tables", 2)
    _check(context_lens, torch.int32, "context_lens", 1)
    Tq, Hq, Dq = (int(x) for x in q.shape)
    if Dq != D or tuple(k_new.shape) != (Tq, Hkv, D) or tuple(v_new.shape) != (Tq, Hkv, D):
        raise ValueError("q / k_new / v_new shapes disagree with the cache")
    B = int(context_lens.shape[0])
    if cu_seqlens_q.shape[0] != B + 1 or block_tables.shape[0] != B:
        raise ValueError("cu_seqlens_q must be [B+1] and block_tables [B, MBS]")
    _check(out, out.dtype, "out", 3)
    if tuple(out.shape) != (Tq, Hq, D):
        raise ValueError(f"out must be [{Tq}, {Hq}, {D}]")
    mq = Tq if max_q_len is None else int(max_q_len)
    sc = float(scale) if scale is not None else 0.0
    rc = load_library().pa_paged_prefill(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(cu_seqlens_q), B, Tq, mq, _ptr(k_cache),
        _ptr(v_cache), _ptr(block_tables), int(block_tables.shape[1]), _ptr(context_lens), Hq, Hkv,
        D, BS, NB, sc, _ptr(out), _out_dtype(out), _stream(q.device))
    _raise_on("pa_paged_prefill", rc)


def paged_prefill_fp8(q, cu_seqlens_q, block_tables, context_lens, out, *, k_cache, v_cache,
                      scale: Optional[float], k_scale: float, v_scale: float,
                      max_q_len: Optional[int] = None) -> None:
    """Prefix-hit prefill over uint8 E4M3 pools that already hold the chunk's own tokens:
    every key 0 .. ctx-1 is read through the block table (keys code * k_scale, values
    code * v_scale)."""
    torch = _torch()
    NB, BS, Hkv, D = _cache_geometry(k_cache, v_cache, torch.uint8)
    _check(q, torch.bfloat16, "q", 3)
    _check(cu_seqlens_q, torch.int32, "cu_seqlens_q", 1)
    _check(block_tables, torch.int32, "block_tables", 2)
    _check(context_lens, torch.int32, "context_lens", 1)
    Tq, Hq, Dq = (int(x) for x in q.shape)
    if Dq != D:
        raise ValueError("q's head_dim disagrees with the cache")
    B = int(context_lens.shape[0])
    if cu_seqlens_q.shape[0] != B + 1 or block_tables.shape[0] != B:
        raise ValueError("cu_seqlens_q must be [B+1] and block_tables [B, MBS]")
    _check(out, out.dtype, "out", 3)
    if tuple(out.shape) != (Tq, Hq, D):
        raise ValueError(f"out must be [{Tq}, {Hq}, {D}]")
    mq = Tq if max_q_len is None else int(max_q_len)
    sc = float(scale) if scale is not None else 0.0
    rc = load_library().pa_paged_prefill_fp8(
        _ptr(q), _ptr(cu_seqlens_q), B, Tq, mq, _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        int(block_tables.shape[1]), _ptr(context_lens), Hq, Hkv, D, BS, NB, sc, float(k_scale),
        float(v_scale), _ptr(out), _out_dtype(out), _stream(q.device))
    _raise_on("pa_paged_prefill_fp8", rc)


def paged_attention_mixed(q, k_new, v_new, slot_mapping, cu_seqlens_q, block_tables,
                          context_lens, out, *, k_cache, v_cache, num_prefill_seqs: int,
                          prefill_tokens: int, max_prefill_q_len: Optional[int] = None,
                          scale: Optional[float] = None, workspace=None,
                          decode_stream=None) -> None:
    """Store every new token, then attend: chunks (sequences 0..num_prefill_seqs-1, rows
    0..prefill_tokens-1) and one-token decode rows (the remaining sequences, one row each)."""
    torch = _torch()
    NB, BS, Hkv, D = _cache_geometry(k_cache, v_cache)
    _check(q, torch.bfloat16, "q", 3)
    _check(k_new, torch.bfloat16, "k_new", 3)
    _check(v_new, torch.bfloat16, "v_new", 3)
    _check(slot_mapping, torch.int32, "slot_mapping", 1)
    _check(cu_seqlens_q, torch.int32, "cu_seqlens_q", 1)
    _check(block_tables, torch.int32, "block_tables", 2)
    _check(context_lens, torch.int32, "context_lens", 1)
    T, Hq, Dq = (int(x) for x in q.shape)
    B = int(context_lens.shape[0])
    P = int(num_prefill_seqs)
    nd = B - P
    if Dq != D or tuple(k_new.shape) != (T, Hkv, D) or tuple(v_new.shape) != (T, Hkv, D):
        raise ValueError("q / k_new / v_new shapes disagree with the cache")
    if T != int(prefill_tokens) + nd or slot_mapping.shape[0] != T:
        raise ValueError("rows must be prefill_tokens + one per decode sequence")
    if block_tables.shape[0] != B or cu_seqlens_q.shape[0] < P + 1:
        raise ValueError("block_tables [B, MBS] and cu_seqlens_q [>= num_prefill_seqs+1] expected")
    _check(out, out.dtype, "out", 3)
    if tuple(out.shape) != (T, Hq, D):
        raise ValueError(f"out must be [{T}, {Hq}, {D}]")
    MBS = int(block_tables.shape[1])
    need = decode_workspace_bytes(nd, Hq, Hkv, D, BS, MBS) if nd > 0 else 0
    workspace = _workspace_for(workspace, need, q.device)
    sc = float(scale) if scale is not None else 0.0
    mq = int(prefill_tokens) if max_prefill_q_len is None else int(max_prefill_q_len)
    ds = ctypes.c_void_p(decode_stream.cuda_stream) if decode_stream is not None else None
    rc = load_library().pa_paged_attention_mixed(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), _ptr(cu_seqlens_q), P, nd,
        int(prefill_tokens), mq, _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), MBS,
        _ptr(context_lens), Hq, Hkv, D, BS, NB, sc, _ptr(out), _out_dtype(out), _ptr(workspace),
        int(workspace.numel()), _stream(q.device), ds)
    _raise_on("pa_paged_attention_mixed", rc)


def paged_gather(cache, block_tables, context_lens, cu_seqlens_k, max_context_len: int, out) -> None:
    """Test aid: out[cu_seqlens_k[i] + j] = row of logical token j of sequence i."""
    torch = _torch()
    _check(cache, torch.bfloat16, "cache", 4)
    NB, BS, Hkv, D = (int(x) for x in cache.shape)
    _check(block_tables, torch.int32, "block_tables", 2)
    _check(context_lens, torch.int32, "context_lens", 1)
    _check(cu_seqlens_k, torch.int32, "cu_seqlens_k", 1)
    _check(out, torch.bfloat16, "out", 3)
    B = int(context_lens.shape[0])
    rc = load_library().pa_paged_gather(
        _ptr(cache), _ptr(block_tables), int(block_tables.shape[1]), _ptr(context_lens),
        _ptr(cu_seqlens_k), B, int(max_context_len), Hkv, D, BS, NB, _ptr(out),
        _stream(cache.device))
    _raise_on("pa_paged_gather", rc)


def stream_read(src, sink) -> None:
    """Measurement aid: read every byte of `src` once (see pa_stream_read); `sink` is a
    device tensor of at least 4 bytes that the kernel may overwrite."""
    if not (src.is_cuda and src.is_contiguous() and sink.is_cuda and sink.is_contiguous()):
        raise ValueError("stream_read: src and sink must be contiguous device tensors")
    if sink.numel() * sink.element_size() < 4:
        raise ValueError("stream_read: sink must hold at least 4 bytes")
    rc = load_library().pa_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                                       _stream(src.device))
    _raise_on("pa_stream_read", rc)


def decode_time_next_launch(start_event, end_event) -> None:
    """Measurement aid: the next decode call of this thread records the two torch.cuda.Event
    objects (recorded once before, so that they exist) around its main split kernel."""
    rc = load_library().pa_decode_time_next_launch(ctypes.c_void_p(start_event.cuda_event),
                                                   ctypes.c_void_p(end_event.cuda_event))
    _raise_on("pa_decode_time_next_launch", rc)


def default_scale(head_dim: int) -> float:
    """1/sqrt(head_dim) rounded to float32, the value the kernels use for scale <= 0."""
    import struct
    return struct.unpack("f", struct.pack("f", 1.0 / math.sqrt(head_dim)))[0]


def paged_decode_append_fp8(q, k_new, v_new, slot_mapping, k_cache, v_cache, block_tables,
                            context_lens, scale: Optional[float], k_scale: float, v_scale: float,
                            out, workspace=None) -> None:
    """kvcache_store_fp8 of each sequence's new token followed by paged_decode_fp8, in one call."""
    torch = _torch()
    NB, BS, Hkv, D = _cache_geometry(k_cache, v_cache, torch.uint8)
    B, Hq, MBS = _decode_shapes(q, block_tables, context_lens, out, D)
    _new_tokens(k_new, v_new, slot_mapping, B, Hkv, D)
    need = decode_fp8_workspace_bytes(B, Hq, Hkv, D, BS, MBS) if B > 0 else 0
    workspace = _workspace_for(workspace, need, q.device)
    sc = float(scale) if scale is not None else 0.0
    rc = load_library().pa_paged_decode_append_fp8(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), _ptr(k_cache), _ptr(v_cache),
        _ptr(block_tables), MBS, _ptr(context_lens), B, Hq, Hkv, D, BS, NB, sc, float(k_scale),
        float(v_scale), _ptr(out), _out_dtype(out), _ptr(workspace), int(workspace.numel()),
        _stream(q.device))
    _raise_on("pa_paged_decode_append_fp8", rc)


class DecodeGraph:
    """Graph-captured fused store + decode steps over fixed caches, one graph per batch bucket.

    ``run`` takes the step's q / k_new / v_new as device tensors (or None when they were
    written into :attr:`q`, :attr:`k_new`, :attr:`v_new` in place) and the index arrays as
    host (CPU) int32 tensors or arrays; rows past the batch are padded with sentinels.
    """

    def __init__(self, k_cache, v_cache, max_batch: int, num_q_heads: int,
                 max_blocks_per_seq: int, scale: Optional[float] = None, *,
                 k_scale: Optional[float] = None, v_scale: Optional[float] = None,
                 out_dtype=None):
        torch = _torch()
        fp8 = k_cache.dtype == torch.uint8
        if fp8 and (k_scale is None or v_scale is None):
            raise ValueError("an FP8 cache needs k_scale and v_scale")
        NB, BS, Hkv, D = _cache_geometry(k_cache, v_cache, k_cache.dtype if fp8 else None)
        out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
        self._lib = load_library()
        self._caches = (k_cache, v_cache)  # keep the pools alive
        self.device = k_cache.device
        self.max_batch, self.num_q_heads, self.num_kv_heads, self.head_dim = (
            int(max_batch), int(num_q_heads), Hkv, D)
        self.out_dtype = out_dtype
        handle = ctypes.c_void_p()
        with torch.cuda.device(self.device):
            rc = self._lib.pa_decode_graph_create(
                int(max_batch), int(num_q_heads), Hkv, D, BS, NB, int(max_blocks_per_seq),
                1 if fp8 else 0, float(scale) if scale is not None else 0.0,
                float(k_scale) if fp8 else 1.0, float(v_scale) if fp8 else 1.0,
                _ptr(k_cache), _ptr(v_cache), PA_F32 if out_dtype == torch.float32 else PA_BF16,
                ctypes.byref(handle))
        _raise_on("pa_decode_graph_create", rc)
        self._h = handle
        ptrs = [ctypes.c_void_p() for _ in range(4)]
        _raise_on("pa_decode_graph_buffers", self._lib.pa_decode_graph_buffers(
            self._h, *[ctypes.byref(p) for p in ptrs]))
        self._buf_ptrs = [p.value for p in ptrs]

    def bucket(self, batch: int) -> int:
        return int(self._lib.pa_decode_graph_bucket(self._h, int(batch)))

    def buffer_ptrs(self):
        """Device addresses of the static q, k_new, v_new and out buffers."""
        return tuple(self._buf_ptrs)

    def run(self, batch: int, q, k_new, v_new, slot_mapping, block_tables, context_lens,
            out=None) -> None:
        import numpy as np
        torch = _torch()

        def host_i32(a, name, ndim):
            a = a.numpy() if isinstance(a, torch.Tensor) else a
            a = np.ascontiguousarray(a, dtype=np.int32)
            if a.ndim != ndim:
                raise ValueError(f"{name} must have {ndim} dims")
            return a

        B = int(batch)
        sl = host_i32(slot_mapping, "slot_mapping", 1)
        bt = host_i32(block_tables, "block_tables", 2)
        cl = host_i32(context_lens, "context_lens", 1)
        if sl.shape[0] < B or cl.shape[0] < B or bt.shape[0] < B:
            raise ValueError("index arrays need one row per sequence")
        for t, name, rows, heads in ((q, "q", B, self.num_q_heads), (k_new, "k_new", B, self.num_kv_heads),
                                     (v_new, "v_new", B, self.num_kv_heads)):
            if t is not None:
                _check(t, torch.bfloat16, name, 3)
                if tuple(t.shape) != (rows, heads, self.head_dim):
                    raise ValueError(f"{name} must be [{rows}, {heads}, {self.head_dim}]")
        if out is not None:
            _check(out, self.out_dtype, "out", 3)
            if tuple(out.shape) != (B, self.num_q_heads, self.head_dim):
                raise ValueError("out shape")

        def p(t):
            return ctypes.c_void_p(t.data_ptr()) if t is not None else None

        rc = self._lib.pa_decode_graph_run(
            self._h, B, p(q), p(k_new), p(v_new), sl.ctypes.data_as(ctypes.c_void_p),
            bt.ctypes.data_as(ctypes.c_void_p), int(bt.shape[1]), cl.ctypes.data_as(ctypes.c_void_p),
            p(out), _stream(self.device))
        _raise_on("pa_decode_graph_run", rc)

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            self._lib.pa_decode_graph_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class BlockManager:
    """Host block manager with prefix caching (the library's C++ implementation).

    Sequences are named by integer ids.  Methods raise :class:`PagedAttnError` on errors
    (``status`` PA_ERR_OUT_OF_BLOCKS = -6, PA_ERR_SEQUENCE = -7, ...); nothing touches the GPU.
    """

    def __init__(self, num_blocks: int, block_size: int, hash_bits: int = 64):
        self._lib = load_library()
        h = ctypes.c_void_p()
        _raise_on("pa_bm_create", self._lib.pa_bm_create(int(num_blocks), int(block_size),
                                                         int(hash_bits), ctypes.byref(h)))
        self._h = h
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)

    def _status(self, name, rc):
        if rc < 0:
            _raise_on(name, rc)
        return rc

    @property
    def num_free(self) -> int:
        return self._status("pa_bm_num_free", self._lib.pa_bm_num_free(self._h))

    def can_allocate(self, num_tokens: int) -> bool:
        return bool(self._status("pa_bm_can_allocate",
                                 self._lib.pa_bm_can_allocate(self._h, int(num_tokens))))

    def allocate(self, seq_id: int, tokens) -> int:
        import numpy as np
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        cached = ctypes.c_int(0)
        self._status("pa_bm_allocate", self._lib.pa_bm_allocate(
            self._h, int(seq_id), t.ctypes.data_as(ctypes.c_void_p), int(t.size),
            ctypes.byref(cached)))
        return cached.value

    def can_append(self, seq_id: int) -> bool:
        return bool(self._status("pa_bm_can_append", self._lib.pa_bm_can_append(self._h, int(seq_id))))

    def append(self, seq_id: int, token: int) -> None:
        self._status("pa_bm_append", self._lib.pa_bm_append(self._h, int(seq_id), int(token)))

    def deallocate(self, seq_id: int) -> None:
        self._status("pa_bm_deallocate", self._lib.pa_bm_deallocate(self._h, int(seq_id)))

    def seq_info(self, seq_id: int):
        """(num_tokens, num_cached_tokens, num_blocks) of a live sequence."""
        a, b, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
        self._status("pa_bm_seq_info", self._lib.pa_bm_seq_info(
            self._h, int(seq_id), ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
        return a.value, b.value, c.value

    def block_table(self, seq_id: int):
        import numpy as np
        n = self._status("pa_bm_block_table", self._lib.pa_bm_block_table(self._h, int(seq_id), None, 0))
        out = np.empty(n, dtype=np.int32)
        self._lib.pa_bm_block_table(self._h, int(seq_id), out.ctypes.data_as(ctypes.c_void_p), n)
        return out.tolist()

    def free_list(self):
        import numpy as np
        n = self._status("pa_bm_free_list", self._lib.pa_bm_free_list(self._h, None, 0))
        out = np.empty(n, dtype=np.int32)
        self._lib.pa_bm_free_list(self._h, out.ctypes.data_as(ctypes.c_void_p), n)
        return out.tolist()

    def ref_count(self, block_id: int) -> int:
        return self._status("pa_bm_ref_count", self._lib.pa_bm_ref_count(self._h, int(block_id)))

    def prepare_decode(self, seq_ids, max_blocks_per_seq: int):
        """(slot_mapping [B], context_lens [B], block_tables [B, MBS]) int32 arrays."""
        import numpy as np
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        B = int(ids.size)
        slots = np.empty(B, np.int32)
        lens = np.empty(B, np.int32)
        tables = np.empty((B, int(max_blocks_per_seq)), np.int32)
        vp = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
        self._status("pa_bm_prepare_decode", self._lib.pa_bm_prepare_decode(
            self._h, vp(ids), B, int(max_blocks_per_seq), vp(slots), vp(lens), vp(tables)))
        return slots, lens, tables

    def prepare_prefill(self, seq_ids, max_blocks_per_seq: int):
        """dict of cu_seqlens_q, context_lens, block_tables, slot_mapping, total_q, max_q_len."""
        import numpy as np
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        B = int(ids.size)
        cap = sum(self.seq_info(i)[0] - self.seq_info(i)[1] for i in ids.tolist())
        cu = np.empty(B + 1, np.int32)
        lens = np.empty(B, np.int32)
        tables = np.empty((B, int(max_blocks_per_seq)), np.int32)
        slots = np.empty(max(cap, 1), np.int32)
        tq, mq = ctypes.c_int(), ctypes.c_int()
        vp = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
        self._status("pa_bm_prepare_prefill", self._lib.pa_bm_prepare_prefill(
            self._h, vp(ids), B, int(max_blocks_per_seq), vp(cu), vp(lens), vp(tables), vp(slots),
            int(cap), ctypes.byref(tq), ctypes.byref(mq)))
        return {"cu_seqlens_q": cu, "context_lens": lens, "block_tables": tables,
                "slot_mapping": slots[:tq.value], "total_q": tq.value, "max_q_len": mq.value}

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            self._lib.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
