"""ctypes binding of libmqa_indexer.so (include/mqa_indexer.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, then their device pointers and the current HIP stream are handed to
the C ABI.  Every step of the op runs in the library's HIP kernels; there is no
other implementation behind these functions, and a missing library raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmqa_indexer.so")

MQA_OK = 0
MQA_ERR_INVALID_ARG = -1
MQA_ERR_UNSUPPORTED = -2
MQA_ERR_LAUNCH = -3
MQA_ERR_DEVICE = -4

EXPORTED = ("mqa_is_supported", "mqa_logits_prefill", "paged_mqa_logits_decode",
            "mqa_topk_indices", "mqa_topk_indices_ws", "mqa_topk_workspace_size",
            "paged_mqa_topk_decode", "paged_mqa_topk_decode_noalloc",
            "paged_mqa_topk_workspace_size", "mqa_kcache_quantize_insert", "mqa_last_error")
# bytes of the library's static scratch (MQA_NOALLOC_SCRATCH_BYTES in the header)
NOALLOC_SCRATCH_BYTES = 128 << 20
MQA_DTYPE_FP32 = 0
MQA_DTYPE_BF16 = 1
MQA_KV_SLOT_MAJOR = 0
MQA_KV_PRESHUFFLED = 1


class MQAError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class Tunables(ctypes.Structure):
    """mqa_tunables: 0 in a field means the host heuristic chooses."""
    _fields_ = [("block_m", ctypes.c_int), ("split_n", ctypes.c_int),
                ("num_warps", ctypes.c_int), ("reverse_rows", ctypes.c_int),
                ("rows_per_block", ctypes.c_int), ("split_kv", ctypes.c_int),
                ("ring_depth", ctypes.c_int)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load the HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise MQAError(MQA_ERR_DEVICE, f"{path} is missing: build it with "
                       "`python -m sparse_attention_indexer_scaled_amd.build`")
    lib = ctypes.CDLL(path)
    P, I = ctypes.c_void_p, ctypes.c_int
    lib.mqa_is_supported.restype = I
    lib.mqa_is_supported.argtypes = [I, I, I]
    lib.mqa_last_error.restype = ctypes.c_char_p
    lib.mqa_last_error.argtypes = []
    lib.mqa_logits_prefill.restype = I
    lib.mqa_logits_prefill.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, P, P]
    lib.paged_mqa_logits_decode.restype = I
    lib.paged_mqa_logits_decode.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, I, P, P]
    lib.mqa_topk_indices.restype = I
    lib.mqa_topk_indices.argtypes = [P, I, I, I, P, P]
    lib.mqa_topk_indices_ws.restype = I
    lib.mqa_topk_indices_ws.argtypes = [P, I, I, I, P, P, ctypes.c_size_t, P]
    lib.mqa_topk_workspace_size.restype = ctypes.c_size_t
    lib.mqa_topk_workspace_size.argtypes = [I, I]
    lib.paged_mqa_topk_decode.restype = I
    lib.paged_mqa_topk_decode.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, I, P,
                                          ctypes.c_size_t, P, P]
    lib.paged_mqa_topk_decode_noalloc.restype = I
    lib.paged_mqa_topk_decode_noalloc.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, I,
                                                  P, P]
    lib.paged_mqa_topk_workspace_size.restype = ctypes.c_size_t
    lib.paged_mqa_topk_workspace_size.argtypes = [I, I, I]
    lib.mqa_kcache_quantize_insert.restype = I
    lib.mqa_kcache_quantize_insert.argtypes = [P, I, P, P, I, I, I, I, I, P]
    _lib = lib
    return lib


def last_error() -> str:
    return load_library().mqa_last_error().decode()


def _check(rc: int):
    if rc != MQA_OK:
        raise MQAError(rc, last_error())


def is_supported(num_heads: int, head_dim: int, kv_block_size: int = 0) -> bool:
    return bool(load_library().mqa_is_supported(int(num_heads), int(head_dim), int(kv_block_size)))


def _bytes(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    if t.dtype != torch.uint8:
        raise TypeError(f"{name} must be float8_e4m3fn or uint8 bytes, got {t.dtype}")
    return t


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(getattr(stream, "cuda_stream", stream))


def _layout(preshuffle: bool) -> int:
    return MQA_KV_PRESHUFFLED if preshuffle else MQA_KV_SLOT_MAJOR


def _tun(tunables: Optional[Tunables]):
    return ctypes.byref(tunables) if tunables is not None else None


def mqa_logits_prefill(q_fp8: torch.Tensor, k_fp8: torch.Tensor, kv_scale: torch.Tensor,
                       weights: torch.Tensor, cu_seqlen_ks: torch.Tensor,
                       cu_seqlen_ke: torch.Tensor, logits: Optional[torch.Tensor] = None,
                       clean_logits: bool = True, tunables: Optional[Tunables] = None,
                       stream=None) -> torch.Tensor:
    """q_fp8 [M,H,D], k_fp8 [N,D] (fp8 e4m3fn), kv_scale [N] f32, weights [M,H] f32,
    cu_seqlen_ks/ke [M] int32 -> logits [M,N] f32 (allocated if not given)."""
    q = _bytes(q_fp8, "q_fp8")
    k = _bytes(k_fp8, "k_fp8")
    M, H, D = q.shape
    N = k.shape[0]
    if k.shape != (N, D) or kv_scale.shape != (N,) or weights.shape != (M, H):
        raise ValueError("shape mismatch")
    if cu_seqlen_ks.shape != (M,) or cu_seqlen_ke.shape != (M,):
        raise ValueError("cu_seqlen_ks/ke must be [M]")
    if logits is None:
        logits = torch.empty((M, N), dtype=torch.float32, device=q.device)
    if logits.shape != (M, N):
        raise ValueError("logits must be [M, N]")
    rc = load_library().mqa_logits_prefill(
        _dev(q, "q_fp8"), _dev(k, "k_fp8"), _dev(kv_scale, "kv_scale", torch.float32),
        _dev(weights, "weights", torch.float32), _dev(cu_seqlen_ks, "cu_seqlen_ks", torch.int32),
        _dev(cu_seqlen_ke, "cu_seqlen_ke", torch.int32), _dev(logits, "logits", torch.float32),
        M, N, H, D, int(bool(clean_logits)), _tun(tunables), _stream(stream, q.device))
    _check(rc)
    return logits


def paged_mqa_logits_decode(q_fp8: torch.Tensor, kv_cache: torch.Tensor, weights: torch.Tensor,
                            context_lens: torch.Tensor, block_tables: torch.Tensor,
                            max_model_len: int, kv_block_size: int = 64,
                            logits: Optional[torch.Tensor] = None, clean_logits: bool = True,
                            tunables: Optional[Tunables] = None, stream=None,
                            preshuffle: bool = False) -> torch.Tensor:
    """q_fp8 [B,next_n,H,D] fp8, kv_cache [num_blocks, bs*(D+4)] bytes, weights
    [B*next_n,H] f32, context_lens [B] int32, block_tables [B,max_blocks] int32
    -> logits [B*next_n, max_model_len] f32 (allocated if not given).
    preshuffle: the cache's K rows are in the preshuffled (16,16) order."""
    q = _bytes(q_fp8, "q_fp8")
    cache = _bytes(kv_cache, "kv_cache")
    B, next_n, H, D = q.shape
    num_blocks = cache.shape[0]
    if cache.dim() != 2 or cache.shape[1] != kv_block_size * (D + 4):
        raise ValueError("kv_cache must be [num_blocks, kv_block_size*(head_dim+4)] bytes")
    if weights.shape != (B * next_n, H) or context_lens.shape != (B,):
        raise ValueError("shape mismatch")
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [B, max_blocks_per_seq]")
    rows = B * next_n
    if logits is None:
        logits = torch.empty((rows, max_model_len), dtype=torch.float32, device=q.device)
    if logits.shape != (rows, max_model_len):
        raise ValueError("logits must be [B*next_n, max_model_len]")
    rc = load_library().paged_mqa_logits_decode(
        _dev(q, "q_fp8"), _dev(cache, "kv_cache"), _dev(weights, "weights", torch.float32),
        _dev(context_lens, "context_lens", torch.int32),
        _dev(block_tables, "block_tables", torch.int32), _dev(logits, "logits", torch.float32),
        B, next_n, H, D, int(kv_block_size), _layout(preshuffle), num_blocks, block_tables.shape[1],
        int(max_model_len), int(bool(clean_logits)), _tun(tunables), _stream(stream, q.device))
    _check(rc)
    return logits


def topk_indices(logits: torch.Tensor, k: int, indices: Optional[torch.Tensor] = None,
                 stream=None) -> torch.Tensor:
    """logits [rows, cols] f32 -> indices [rows, k] int32: columns by decreasing
    value (ties: smaller column first), -inf/NaN never listed, -1 padding."""
    if logits.dim() != 2:
        raise ValueError("logits must be [rows, cols]")
    rows, cols = logits.shape
    if indices is None:
        indices = torch.empty((rows, k), dtype=torch.int32, device=logits.device)
    if indices.shape != (rows, k):
        raise ValueError("indices must be [rows, k]")
    rc = load_library().mqa_topk_indices(
        _dev(logits, "logits", torch.float32), rows, cols, int(k),
        _dev(indices, "indices", torch.int32), _stream(stream, logits.device))
    _check(rc)
    return indices


def topk_workspace_size(rows: int, cols: int) -> int:
    return int(load_library().mqa_topk_workspace_size(int(rows), int(cols)))


def topk_indices_ws(logits: torch.Tensor, k: int, indices: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """topk_indices with a workspace (mqa_topk_indices_ws): the same indices;
    long rows are split over several workgroups.  workspace: a uint8 device
    tensor of at least topk_workspace_size(rows, cols) bytes (allocated from
    torch's caching allocator when not given)."""
    if logits.dim() != 2:
        raise ValueError("logits must be [rows, cols]")
    rows, cols = logits.shape
    if indices is None:
        indices = torch.empty((rows, k), dtype=torch.int32, device=logits.device)
    if indices.shape != (rows, k):
        raise ValueError("indices must be [rows, k]")
    if workspace is None:
        workspace = torch.empty(max(topk_workspace_size(rows, cols), 1), dtype=torch.uint8,
                                device=logits.device)
    ws = _bytes(workspace, "workspace")
    rc = load_library().mqa_topk_indices_ws(
        _dev(logits, "logits", torch.float32), rows, cols, int(k),
        _dev(indices, "indices", torch.int32), _dev(ws, "workspace"), ws.numel(),
        _stream(stream, logits.device))
    _check(rc)
    return indices


def paged_mqa_topk_workspace_size(batch: int, next_n: int, max_model_len: int) -> int:
    return int(load_library().paged_mqa_topk_workspace_size(int(batch), int(next_n),
                                                              int(max_model_len)))


def paged_mqa_topk_decode(q_fp8: torch.Tensor, kv_cache: torch.Tensor, weights: torch.Tensor,
                          context_lens: torch.Tensor, block_tables: torch.Tensor,
                          max_model_len: int, k: int, kv_block_size: int = 64,
                          indices: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None,
                          tunables: Optional[Tunables] = None, stream=None,
                          preshuffle: bool = False) -> torch.Tensor:
    """The top-k indices [B*next_n, k] int32 of the decode logits (as
    topk_indices(paged_mqa_logits_decode(...), k)), without writing the logits.
    workspace: a uint8 device tensor of at least paged_mqa_topk_workspace_size
    bytes (allocated from torch's caching allocator when not given)."""
    q = _bytes(q_fp8, "q_fp8")
    cache = _bytes(kv_cache, "kv_cache")
    B, next_n, H, D = q.shape
    if cache.dim() != 2 or cache.shape[1] != kv_block_size * (D + 4):
        raise ValueError("kv_cache must be [num_blocks, kv_block_size*(head_dim+4)] bytes")
    if weights.shape != (B * next_n, H) or context_lens.shape != (B,):
        raise ValueError("shape mismatch")
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [B, max_blocks_per_seq]")
    rows = B * next_n
    if indices is None:
        indices = torch.empty((rows, k), dtype=torch.int32, device=q.device)
    if indices.shape != (rows, k):
        raise ValueError("indices must be [B*next_n, k]")
    if workspace is None:
        need = paged_mqa_topk_workspace_size(B, next_n, max_model_len)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ws = _bytes(workspace, "workspace")
    rc = load_library().paged_mqa_topk_decode(
        _dev(q, "q_fp8"), _dev(cache, "kv_cache"), _dev(weights, "weights", torch.float32),
        _dev(context_lens, "context_lens", torch.int32),
        _dev(block_tables, "block_tables", torch.int32), _dev(indices, "indices", torch.int32),
        B, next_n, H, D, int(kv_block_size), _layout(preshuffle), cache.shape[0],
        block_tables.shape[1], int(max_model_len), int(k), _dev(ws, "workspace"), ws.numel(),
        _tun(tunables), _stream(stream, q.device))
    _check(rc)
    return indices


def paged_mqa_topk_decode_noalloc(q_fp8: torch.Tensor, kv_cache: torch.Tensor,
                                  weights: torch.Tensor, context_lens: torch.Tensor,
                                  block_tables: torch.Tensor, max_model_len: int, k: int,
                                  indices: torch.Tensor, kv_block_size: int = 64,
                                  tunables: Optional[Tunables] = None, stream=None,
                                  preshuffle: bool = False) -> torch.Tensor:
    """paged_mqa_topk_decode with the library's static scratch as its
    workspace: no device allocation in the call (the caller passes
    `indices`, [B*next_n, k] int32).  Calls that overlap on one device race."""
    q = _bytes(q_fp8, "q_fp8")
    cache = _bytes(kv_cache, "kv_cache")
    B, next_n, H, D = q.shape
    if cache.dim() != 2 or cache.shape[1] != kv_block_size * (D + 4):
        raise ValueError("kv_cache must be [num_blocks, kv_block_size*(head_dim+4)] bytes")
    if weights.shape != (B * next_n, H) or context_lens.shape != (B,):
        raise ValueError("shape mismatch")
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [B, max_blocks_per_seq]")
    if indices.shape != (B * next_n, k):
        raise ValueError("indices must be [B*next_n, k]")
    rc = load_library().paged_mqa_topk_decode_noalloc(
        _dev(q, "q_fp8"), _dev(cache, "kv_cache"), _dev(weights, "weights", torch.float32),
        _dev(context_lens, "context_lens", torch.int32),
        _dev(block_tables, "block_tables", torch.int32), _dev(indices, "indices", torch.int32),
        B, next_n, H, D, int(kv_block_size), _layout(preshuffle), cache.shape[0],
        block_tables.shape[1], int(max_model_len), int(k), _tun(tunables),
        _stream(stream, q.device))
    _check(rc)
    return indices


def kcache_quantize_insert(k: torch.Tensor, slot_mapping: torch.Tensor, kv_cache: torch.Tensor,
                           kv_block_size: int = 64, stream=None,
                           preshuffle: bool = False) -> torch.Tensor:
    """k [T, 128] float32 or bfloat16, slot_mapping [T] int64 (negative = skip),
    kv_cache [num_blocks, kv_block_size * 132] uint8 (updated in place; K rows
    in the preshuffled (16,16) order when preshuffle is set)."""
    if k.dim() != 2:
        raise ValueError("k must be [num_tokens, head_dim]")
    T, D = k.shape
    dtype = {torch.float32: MQA_DTYPE_FP32, torch.bfloat16: MQA_DTYPE_BF16}.get(k.dtype)
    if dtype is None:
        raise TypeError("k must be float32 or bfloat16, got %s" % k.dtype)
    cache = _bytes(kv_cache, "kv_cache")
    if cache.dim() != 2 or cache.shape[1] != kv_block_size * (D + 4):
        raise ValueError("kv_cache must be [num_blocks, kv_block_size*(head_dim+4)] bytes")
    if slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be [num_tokens]")
    rc = load_library().mqa_kcache_quantize_insert(
        _dev(k, "k"), dtype, _dev(slot_mapping, "slot_mapping", torch.int64), _dev(cache, "kv_cache"),
        T, D, int(kv_block_size), _layout(preshuffle), cache.shape[0], _stream(stream, k.device))
    _check(rc)
    return kv_cache
