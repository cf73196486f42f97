"""ctypes binding of libmla (argument marshalling only).

Every step of the path runs in the HIP kernels of ``libmla.so``; this module
checks tensor dtypes, shapes and devices, passes raw device pointers and the
current HIP stream, and raises on a non-zero status.  There is no fallback:
if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libmla.so"
LATENT, ROPE, NOPE, VDIM, PAGE = 512, 64, 128, 128, 64
FP8_ROW_BYTES = 656  # FP8 cache row (see include/mla.h)

_lib = None


class MLAError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: status {status} ({status_string(status)})")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("heads", ctypes.c_int32), ("kv_lora", ctypes.c_int32), ("rope", ctypes.c_int32),
                ("qk_nope", ctypes.c_int32), ("v_dim", ctypes.c_int32), ("page", ctypes.c_int32)]


def lib_path() -> str:
    """libmla.so next to this file, or the file MLA_LIB names (the sanitizer
    build of the same sources, for the ABI tests)."""
    return os.environ.get("MLA_LIB") or os.path.join(PKG, LIB_NAME)


def load() -> ctypes.CDLL:
    """Load libmla.so (built by ``mla_latent_kv_07_amd/build.py``)."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python mla_latent_kv_07_amd/build.py`"
                           " (the HIP library is required; there is no fallback)")
    lib = ctypes.CDLL(path)
    P, I32, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    DP = ctypes.POINTER(Dims)
    lib.mla_cache_insert.argtypes = [DP, P, P, F, F, P, I32, P, I32, I32, P, I32, P]
    lib.mla_cache_insert.restype = ctypes.c_int
    lib.mla_decode_workspace_bytes.argtypes = [DP, I32, I32, I32, I32]
    lib.mla_decode_workspace_bytes.restype = SZ
    lib.mla_decode.argtypes = [DP, P, P, P, I32, P, I32, P, I32, I32, I32, F, P, P, SZ, I32, P]
    lib.mla_decode.restype = ctypes.c_int
    lib.mla_cache_insert_fp8.argtypes = lib.mla_cache_insert.argtypes
    lib.mla_cache_insert_fp8.restype = ctypes.c_int
    lib.mla_decode_fp8.argtypes = lib.mla_decode.argtypes
    lib.mla_decode_fp8.restype = ctypes.c_int
    lib.mla_prefill_workspace_bytes.argtypes = [DP, I32, I32]
    lib.mla_prefill_workspace_bytes.restype = SZ
    lib.mla_prefill.argtypes = [DP, P, P, P, I32, P, I32, P, I32, I32, I32, F, P, P, SZ, P]
    lib.mla_prefill.restype = ctypes.c_int
    lib.mla_decode_step.argtypes = [DP, P, P, P, F, F, P, P, I32, P, I32, P, I32, I32, I32, F, P,
                                    P, SZ, I32, P]
    lib.mla_decode_step.restype = ctypes.c_int
    lib.mla_decode_step_fp8.argtypes = lib.mla_decode_step.argtypes
    lib.mla_decode_step_fp8.restype = ctypes.c_int
    lib.mla_dsa_select.argtypes = [I32, P, P, P, P, P, I32, P, I32, I32, I32, P, I32, P, P, P]
    lib.mla_dsa_select.restype = ctypes.c_int
    lib.mla_dsa_workspace_bytes.argtypes = [DP, I32, I32, I32, I32]
    lib.mla_dsa_workspace_bytes.restype = SZ
    lib.mla_dsa_decode.argtypes = [DP, P, P, P, I32, P, I32, P, I32, I32, I32, P, P, P, P, I32, F,
                                   P, P, P, SZ, I32, P]
    lib.mla_dsa_decode.restype = ctypes.c_int
    lib.mla_dsa_decode_fp8.argtypes = lib.mla_dsa_decode.argtypes
    lib.mla_dsa_decode_fp8.restype = ctypes.c_int
    lib.mla_profile_collect_calls.argtypes = [ctypes.POINTER(ctypes.c_double), I32,
                                              ctypes.POINTER(I32)]
    lib.mla_profile_collect_calls.restype = ctypes.c_int
    lib.mla_status_string.argtypes = [ctypes.c_int]
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_profile_enable.argtypes = [I32]
    lib.mla_profile_enable.restype = ctypes.c_int
    lib.mla_profile_collect.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I32)]
    lib.mla_profile_collect.restype = ctypes.c_int
    lib.mla_abi_version.argtypes = []
    lib.mla_abi_version.restype = ctypes.c_int
    lib.mla_debug_checks.argtypes = [I32]
    lib.mla_debug_checks.restype = ctypes.c_int
    lib.mla_decode_noalloc.argtypes = [DP, P, P, P, I32, P, I32, P, I32, I32, I32, F, P, I32, P]
    lib.mla_decode_noalloc.restype = ctypes.c_int
    lib.mla_noalloc_scratch_bytes.argtypes = []
    lib.mla_noalloc_scratch_bytes.restype = SZ
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().mla_status_string(int(status)).decode()


def abi_version() -> int:
    return int(load().mla_abi_version())


def debug_checks(enable: int = -1) -> int:
    """mla_debug_checks: enable (1) or disable (0) the host-side checks of
    block tables and lengths; -1 only queries.  Returns the previous setting."""
    return int(load().mla_debug_checks(int(enable)))


def dims(heads: int) -> Dims:
    return Dims(heads, LATENT, ROPE, NOPE, VDIM, PAGE)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(t, name, dtype, shape=None, device=None):
    import torch
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a GPU tensor")
    return t


def _check_cache(cache, fp8: bool, dev):
    import torch
    if fp8:
        return _check(cache, "cache", torch.uint8, (cache.shape[0], PAGE, FP8_ROW_BYTES), dev)
    return _check(cache, "cache", torch.bfloat16, (cache.shape[0], PAGE, LATENT + ROPE), dev)


def cache_insert(kv_a, rms_w, block_table, seq_lens, cache, *, eps: float = 1e-6,
                 rope_base: float = 10000.0, heads: int = 16, stream=None,
                 fp8: bool = False) -> None:
    """mla_cache_insert (fp8=False: cache bf16 [num_blocks, 64, 576]) or
    mla_cache_insert_fp8 (fp8=True: cache uint8 [num_blocks, 64, 656]):
    kv_a bf16 [B, q_len, 576], rms_w bf16 [512], block_table int32
    [B, max_blocks], seq_lens int32 [B] (post-insert lengths); the cache is
    updated in place."""
    import torch
    bsz, q_len = kv_a.shape[0], kv_a.shape[1]
    dev = cache.device
    _check(kv_a, "kv_a", torch.bfloat16, (bsz, q_len, LATENT + ROPE), dev)
    _check(rms_w, "rms_w", torch.bfloat16, (LATENT,), dev)
    _check(block_table, "block_table", torch.int32, None, dev)
    _check(seq_lens, "seq_lens", torch.int32, (bsz,), dev)
    _check_cache(cache, fp8, dev)
    d = dims(heads)
    fn = load().mla_cache_insert_fp8 if fp8 else load().mla_cache_insert
    st = fn(ctypes.byref(d), _ptr(kv_a), _ptr(rms_w), eps, rope_base, _ptr(block_table),
            block_table.shape[1], _ptr(seq_lens), bsz, q_len, _ptr(cache), cache.shape[0],
            _stream(stream))
    if st != 0:
        raise MLAError(st, "mla_cache_insert_fp8" if fp8 else "mla_cache_insert")


def decode_workspace_bytes(heads: int, batch: int, q_len: int, max_seq_len: int,
                           num_splits_hint: int = 0) -> int:
    d = dims(heads)
    return int(load().mla_decode_workspace_bytes(ctypes.byref(d), batch, q_len, max_seq_len,
                                                 num_splits_hint))


def decode(q, kv_b, cache, block_table, seq_lens, max_seq_len: int, *,
           softmax_scale: float | None = None, out=None, workspace=None,
           num_splits_hint: int = 0, stream=None, fp8: bool = False):
    """mla_decode (fp8=False: cache bf16 [num_blocks, 64, 576]) or
    mla_decode_fp8 (fp8=True: cache uint8 [num_blocks, 64, 656]):
    q bf16 [B, q_len, H, 192], kv_b bf16 [H*256, 512]; returns out bf16
    [B, q_len, H, 128]."""
    import torch
    bsz, q_len, heads = q.shape[0], q.shape[1], q.shape[2]
    dev = cache.device
    _check(q, "q", torch.bfloat16, (bsz, q_len, heads, NOPE + ROPE), dev)
    _check(kv_b, "kv_b", torch.bfloat16, (heads * (NOPE + VDIM), LATENT), dev)
    _check_cache(cache, fp8, dev)
    _check(block_table, "block_table", torch.int32, None, dev)
    _check(seq_lens, "seq_lens", torch.int32, (bsz,), dev)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(NOPE + ROPE)
    if out is None:
        out = torch.empty((bsz, q_len, heads, VDIM), dtype=torch.bfloat16, device=dev)
    _check(out, "out", torch.bfloat16, (bsz, q_len, heads, VDIM), dev)
    need = decode_workspace_bytes(heads, bsz, q_len, max_seq_len, num_splits_hint)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(workspace, "workspace", torch.uint8, None, dev)
    d = dims(heads)
    fn = load().mla_decode_fp8 if fp8 else load().mla_decode
    st = fn(ctypes.byref(d), _ptr(q), _ptr(kv_b), _ptr(cache), cache.shape[0], _ptr(block_table),
            block_table.shape[1], _ptr(seq_lens), bsz, q_len, max_seq_len, softmax_scale,
            _ptr(out), _ptr(workspace), workspace.numel(), num_splits_hint, _stream(stream))
    if st != 0:
        raise MLAError(st, "mla_decode_fp8" if fp8 else "mla_decode")
    return out


def decode_step(q, kv_a, rms_w, kv_b, cache, block_table, seq_lens, max_seq_len: int, *,
                eps: float = 1e-6, rope_base: float = 10000.0,
                softmax_scale: float | None = None, out=None, workspace=None,
                num_splits_hint: int = 0, stream=None, fp8: bool = False):
    """mla_decode_step (fp8=False) or mla_decode_step_fp8 (fp8=True): the
    insert of kv_a bf16 [B, q_len, 576] into the cache, RoPE on q's q_pe (q
    bf16 [B, q_len, H, 192], q_pe NOT rotated) and the decode, in three
    launches; returns out bf16 [B, q_len, H, 128].  The cache is updated in
    place."""
    import torch
    bsz, q_len, heads = q.shape[0], q.shape[1], q.shape[2]
    dev = cache.device
    _check(q, "q", torch.bfloat16, (bsz, q_len, heads, NOPE + ROPE), dev)
    _check(kv_a, "kv_a", torch.bfloat16, (bsz, q_len, LATENT + ROPE), dev)
    _check(rms_w, "rms_w", torch.bfloat16, (LATENT,), dev)
    _check(kv_b, "kv_b", torch.bfloat16, (heads * (NOPE + VDIM), LATENT), dev)
    _check_cache(cache, fp8, dev)
    _check(block_table, "block_table", torch.int32, None, dev)
    _check(seq_lens, "seq_lens", torch.int32, (bsz,), dev)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(NOPE + ROPE)
    if out is None:
        out = torch.empty((bsz, q_len, heads, VDIM), dtype=torch.bfloat16, device=dev)
    _check(out, "out", torch.bfloat16, (bsz, q_len, heads, VDIM), dev)
    need = decode_workspace_bytes(heads, bsz, q_len, max_seq_len, num_splits_hint)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(workspace, "workspace", torch.uint8, None, dev)
    d = dims(heads)
    fn = load().mla_decode_step_fp8 if fp8 else load().mla_decode_step
    st = fn(ctypes.byref(d), _ptr(q), _ptr(kv_a), _ptr(rms_w), eps, rope_base, _ptr(kv_b),
            _ptr(cache), cache.shape[0], _ptr(block_table), block_table.shape[1], _ptr(seq_lens),
            bsz, q_len, max_seq_len, softmax_scale, _ptr(out), _ptr(workspace), workspace.numel(),
            num_splits_hint, _stream(stream))
    if st != 0:
        raise MLAError(st, "mla_decode_step_fp8" if fp8 else "mla_decode_step")
    return out


def prefill_workspace_bytes(heads: int, batch: int, max_seq_len: int) -> int:
    d = dims(heads)
    return int(load().mla_prefill_workspace_bytes(ctypes.byref(d), batch, max_seq_len))


def prefill(q, kv_b, cache, block_table, seq_lens, max_seq_len: int, *,
            softmax_scale: float | None = None, out=None, workspace=None, stream=None):
    """mla_prefill: q bf16 [B, S, H, 192] (q_pe rotated), kv_b bf16
    [H*256, 512], cache bf16 [num_blocks, 64, 576] already holding the S new
    tokens; returns out bf16 [B, S, H, 128]."""
    import torch
    bsz, q_len, heads = q.shape[0], q.shape[1], q.shape[2]
    dev = cache.device
    _check(q, "q", torch.bfloat16, (bsz, q_len, heads, NOPE + ROPE), dev)
    _check(kv_b, "kv_b", torch.bfloat16, (heads * (NOPE + VDIM), LATENT), dev)
    _check_cache(cache, False, dev)
    _check(block_table, "block_table", torch.int32, None, dev)
    _check(seq_lens, "seq_lens", torch.int32, (bsz,), dev)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(NOPE + ROPE)
    if out is None:
        out = torch.empty((bsz, q_len, heads, VDIM), dtype=torch.bfloat16, device=dev)
    _check(out, "out", torch.bfloat16, (bsz, q_len, heads, VDIM), dev)
    need = prefill_workspace_bytes(heads, bsz, max_seq_len)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(workspace, "workspace", torch.uint8, None, dev)
    d = dims(heads)
    st = load().mla_prefill(ctypes.byref(d), _ptr(q), _ptr(kv_b), _ptr(cache), cache.shape[0],
                            _ptr(block_table), block_table.shape[1], _ptr(seq_lens), bsz, q_len,
                            max_seq_len, softmax_scale, _ptr(out), _ptr(workspace),
                            workspace.numel(), _stream(stream))
    if st != 0:
        raise MLAError(st, "mla_prefill")
    return out


IDX_DIM = 128  # index query / key width of the sparse-attention indexer


def _check_index(index_q, index_w, index_k, index_k_scale, bsz, num_blocks, dev):
    import torch
    hi = index_q.shape[1]
    _check(index_q, "index_q", torch.uint8, (bsz, hi, IDX_DIM), dev)
    _check(index_w, "index_w", torch.float32, (bsz, hi), dev)
    _check(index_k, "index_k", torch.uint8, (num_blocks, PAGE, IDX_DIM), dev)
    _check(index_k_scale, "index_k_scale", torch.float32, (num_blocks, PAGE), dev)
    return hi


def dsa_select(index_q, index_w, index_k, index_k_scale, block_table, seq_lens,
               max_seq_len: int, top_k: int, *, scores=None, indices=None, counts=None,
               stream=None):
    """mla_dsa_select: index scores of the cached positions and the top-k
    selection.  index_q uint8 [B, Hi, 128] (E4M3), index_w fp32 [B, Hi],
    index_k uint8 [num_blocks, 64, 128] (E4M3), index_k_scale fp32
    [num_blocks, 64].  Returns (scores fp32 [B, max_seq_len], indices int32
    [B, top_k] ascending with -1 padding, counts int32 [B])."""
    import torch
    bsz = index_q.shape[0]
    dev = index_q.device
    hi = _check_index(index_q, index_w, index_k, index_k_scale, bsz, index_k.shape[0], dev)
    _check(block_table, "block_table", torch.int32, None, dev)
    _check(seq_lens, "seq_lens", torch.int32, (bsz,), dev)
    if scores is None:
        scores = torch.empty((bsz, max_seq_len), dtype=torch.float32, device=dev)
    if indices is None:
        indices = torch.empty((bsz, top_k), dtype=torch.int32, device=dev)
    if counts is None:
        counts = torch.empty((bsz,), dtype=torch.int32, device=dev)
    _check(scores, "scores", torch.float32, None, dev)
    if scores.dim() != 2 or scores.shape[0] != bsz:
        raise ValueError("scores: expected [B, stride]")
    _check(indices, "indices", torch.int32, (bsz, top_k), dev)
    _check(counts, "counts", torch.int32, (bsz,), dev)
    st = load().mla_dsa_select(hi, _ptr(index_q), _ptr(index_w), _ptr(index_k),
                               _ptr(index_k_scale), _ptr(block_table), block_table.shape[1],
                               _ptr(seq_lens), bsz, max_seq_len, top_k, _ptr(scores),
                               scores.shape[1], _ptr(indices), _ptr(counts), _stream(stream))
    if st != 0:
        raise MLAError(st, "mla_dsa_select")
    return scores, indices, counts


def dsa_workspace_bytes(heads: int, batch: int, max_seq_len: int, top_k: int,
                        num_splits_hint: int = 0) -> int:
    d = dims(heads)
    return int(load().mla_dsa_workspace_bytes(ctypes.byref(d), batch, max_seq_len, top_k,
                                              num_splits_hint))


def noalloc_scratch_bytes() -> int:
    """Size of the device scratch mla_decode_noalloc works in."""
    return int(load().mla_noalloc_scratch_bytes())


def decode_noalloc(q, kv_b, cache, block_table, seq_lens, max_seq_len: int, *,
                   softmax_scale: float | None = None, out=None, num_splits_hint: int = 0,
                   stream=None):
    """mla_decode_noalloc: mla_decode (bf16 cache) working in the library's
    own device scratch instead of a caller workspace; ``out`` must be given
    by a caller that cannot allocate."""
    import torch
    bsz, q_len, heads = q.shape[0], q.shape[1], q.shape[2]
    dev = cache.device
    _check(q, "q", torch.bfloat16, (bsz, q_len, heads, NOPE + ROPE), dev)
    _check(kv_b, "kv_b", torch.bfloat16, (heads * (NOPE + VDIM), LATENT), dev)
    _check_cache(cache, False, dev)
    _check(block_table, "block_table", torch.int32, None, dev)
    _check(seq_lens, "seq_lens", torch.int32, (bsz,), dev)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(NOPE + ROPE)
    if out is None:
        out = torch.empty((bsz, q_len, heads, VDIM), dtype=torch.bfloat16, device=dev)
    _check(out, "out", torch.bfloat16, (bsz, q_len, heads, VDIM), dev)
    d = dims(heads)
    st = load().mla_decode_noalloc(ctypes.byref(d), _ptr(q), _ptr(kv_b), _ptr(cache),
                                   cache.shape[0], _ptr(block_table), block_table.shape[1],
                                   _ptr(seq_lens), bsz, q_len, max_seq_len, softmax_scale,
                                   _ptr(out), num_splits_hint, _stream(stream))
    if st != 0:
        raise MLAError(st, "mla_decode_noalloc")
    return out


def dsa_decode(q, kv_b, cache, block_table, seq_lens, max_seq_len: int, index_q, index_w,
               index_k, index_k_scale, top_k: int, *, softmax_scale: float | None = None,
               out=None, indices_out=None, workspace=None, num_splits_hint: int = 0,
               stream=None, fp8: bool = False):
    """mla_dsa_decode (fp8=False: cache bf16 [num_blocks, 64, 576]) or
    mla_dsa_decode_fp8 (fp8=True: cache uint8 [num_blocks, 64, 656]): top-k
    selection by the index scores, then the MLA decode of one new token per
    sequence (q bf16 [B, 1, H, 192], q_pe rotated) over the kept positions.  Returns out bf16
    [B, 1, H, 128]; ``indices_out`` (int32 [B, top_k]), when given, receives
    the kept positions."""
    import torch
    bsz, q_len, heads = q.shape[0], q.shape[1], q.shape[2]
    dev = cache.device
    if q_len != 1:
        raise ValueError("dsa_decode: one new token per sequence (q_len 1)")
    _check(q, "q", torch.bfloat16, (bsz, 1, heads, NOPE + ROPE), dev)
    _check(kv_b, "kv_b", torch.bfloat16, (heads * (NOPE + VDIM), LATENT), dev)
    _check_cache(cache, fp8, dev)
    _check(block_table, "block_table", torch.int32, None, dev)
    _check(seq_lens, "seq_lens", torch.int32, (bsz,), dev)
    hi = _check_index(index_q, index_w, index_k, index_k_scale, bsz, cache.shape[0], dev)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(NOPE + ROPE)
    if out is None:
        out = torch.empty((bsz, 1, heads, VDIM), dtype=torch.bfloat16, device=dev)
    _check(out, "out", torch.bfloat16, (bsz, 1, heads, VDIM), dev)
    if indices_out is not None:
        _check(indices_out, "indices_out", torch.int32, (bsz, top_k), dev)
    need = dsa_workspace_bytes(heads, bsz, max_seq_len, top_k, num_splits_hint)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(workspace, "workspace", torch.uint8, None, dev)
    d = dims(heads)
    fn = load().mla_dsa_decode_fp8 if fp8 else load().mla_dsa_decode
    st = fn(ctypes.byref(d), _ptr(q), _ptr(kv_b), _ptr(cache), cache.shape[0], _ptr(block_table),
            block_table.shape[1], _ptr(seq_lens), bsz, max_seq_len, hi, _ptr(index_q),
            _ptr(index_w), _ptr(index_k), _ptr(index_k_scale), top_k, softmax_scale, _ptr(out),
            _ptr(indices_out), _ptr(workspace), workspace.numel(), num_splits_hint,
            _stream(stream))
    if st != 0:
        raise MLAError(st, "mla_dsa_decode_fp8" if fp8 else "mla_dsa_decode")
    return out


STAGES = ("prep", "decode", "combine")


def profile_enable(max_calls: int) -> None:
    """Record HIP events around each stage of the next ``max_calls`` decodes."""
    st = load().mla_profile_enable(int(max_calls))
    if st != 0:
        raise MLAError(st, "mla_profile_enable")


def profile_collect() -> tuple[dict, int]:
    """Summed milliseconds per stage over the timed decode calls, and their count."""
    ms = (ctypes.c_double * len(STAGES))()
    calls = ctypes.c_int32()
    st = load().mla_profile_collect(ms, ctypes.byref(calls))
    if st != 0:
        raise MLAError(st, "mla_profile_collect")
    return {k: ms[i] for i, k in enumerate(STAGES)}, int(calls.value)


def profile_collect_calls(max_calls: int) -> list[tuple[float, float, float]]:
    """Each timed call's three stage times in milliseconds, in call order."""
    ms = (ctypes.c_double * (3 * max(int(max_calls), 1)))()
    calls = ctypes.c_int32()
    st = load().mla_profile_collect_calls(ms, int(max_calls), ctypes.byref(calls))
    if st != 0:
        raise MLAError(st, "mla_profile_collect_calls")
    return [(ms[3 * c], ms[3 * c + 1], ms[3 * c + 2]) for c in range(int(calls.value))]
