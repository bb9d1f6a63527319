"""Python binding of libpf (PackForcing partition attention on MI355X).

Argument marshalling only: every function passes device pointers, sizes and
the current HIP stream to the C ABI declared in include/pf.h, and every step
runs in libpf's HIP kernels. torch supplies device memory and streams.

Tensors are torch CUDA tensors laid out [rows][heads][128], dtype bfloat16
(or int16 holding bfloat16 bits); index arrays are int32. If libpf.so has not
been built, importing this package raises ImportError: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
# PF_LIBRARY may name another build of the same library (the host-sanitizer
# build, libpf_asan.so, for the sanitized host-side tests)
LIB_PATH = os.environ.get("PF_LIBRARY") or os.path.join(_HERE, "libpf.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m bounded_kv_cache_pf_amd.build` "
                      "(or __graft_entry__.build()); the package has no CPU fallback")

lib = ctypes.CDLL(LIB_PATH)

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int
_sz = ctypes.c_size_t

_SIGNATURES = {
    "pf_abi_version": ([], ctypes.c_int),
    "pf_status_name": ([_i32], ctypes.c_char_p),
    "pf_last_error_message": ([], ctypes.c_char_p),
    "pf_score_select_workspace_bytes": ([_i64, _i32, _i32, _i32], _sz),
    "pf_score_select": ([_p, _i64, _i32, _p, _i32, _i32, _i32, _p, _p, _p, _sz, _p], _i32),
    "pf_selection_deltas": ([_p, _i32, _p, _i32, ctypes.c_int32, ctypes.c_int32, _p, _p], _i32),
    "pf_rope_shift": ([_p, _i32, _i64, _i64, _p, _p, _i32, ctypes.c_double, _p], _i32),
    "pf_score_select_batched_workspace_bytes": ([_i64, _i32, _i32, _i32, _i32], _sz),
    "pf_score_select_sub_workspace_bytes": ([_i64, _i32, _i32, _i32, _i32, _i32], _sz),
    "pf_score_select_sub": ([_p, _i64, _i32, _i32, _i32, _p, _i32, _i32, _i32, _p, _p, _p, _sz, _p], _i32),
    "pf_score_select_batched": ([_p, _i64, _i64, _i32, _p, _i64, _i32, _i32, _i32, _i32, _p, _p, _p, _sz, _p],
                                _i32),
    "pf_selection_deltas_batched": ([_p, _i32, _p, _i32, ctypes.c_int32, ctypes.c_int32, _i32, _p, _p], _i32),
    "pf_rope_shift_batched": ([_p, _i64, _i32, _i64, _i64, _p, _p, _i32, _i32, ctypes.c_double, _p], _i32),
    "pf_rollin": ([_p, _p, _p, _i32, _i32, _i32, _p, _p, ctypes.c_int32, _p], _i32),
    "pf_rollin_batched": ([_p, _p, _i64, _p, _i32, _i32, _i32, _i32, _p, _p, _i64, ctypes.c_int32, _i32, _p], _i32),
    "pf_select_place": ([_p, _i64, _i32, _p, _i32, _i32, _i32, _p, ctypes.c_int32, ctypes.c_int32, _p, _p, _p, _p,
                         _sz, _p], _i32),
    "pf_select_place_batched": ([_p, _i64, _i64, _i32, _p, _i64, _i32, _i32, _i32, _p, ctypes.c_int32,
                                 ctypes.c_int32, _i32, _p, _p, _p, _p, _sz, _p], _i32),
    "pf_select_random": ([_i32, _i32, ctypes.c_uint64, ctypes.c_uint64, _i32, _p, _p], _i32),
    "pf_hr_conv_workspace_bytes": ([_i32] * 9, _sz),
    "pf_hr_conv": ([_p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _p, _p, _i32, _i32, _p, _p, _sz, _p], _i32),
    "pf_hr_branch_workspace_bytes": ([_i32, _i32, _i32, _i32, _i32, _p, _i32], _sz),
    "pf_hr_branch_out_tokens": ([_i32, _i32, _i32], _i64),
    "pf_hr_branch": ([_p, _i32, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _p, _i32, _p, _p, _sz, _p], _i32),
    "pf_partition_attn_workspace_bytes": ([_i64, _i32, _i64], _sz),
    "pf_partition_attn": ([_p, _i64, _i32,
                           _p, _p, _i64,
                           _p, _p, _i32, _i32, _p, _i32,
                           _p, _p, _i64,
                           _p, _p, _i64,
                           ctypes.c_float, _p, _p, _p, _sz, _p], _i32),
    "pf_partition_attn_noalloc": ([_p, _i64, _i32,
                                   _p, _p, _i64,
                                   _p, _p, _i32, _i32, _p, _i32,
                                   _p, _p, _i64,
                                   _p, _p, _i64,
                                   ctypes.c_float, _p, _p, _p], _i32),
}
for _name, (_args, _ret) in _SIGNATURES.items():
    _fn = getattr(lib, _name)
    _fn.argtypes = _args
    _fn.restype = _ret

PF_OK = 0
HEAD_DIM = 128


class PFError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        name = lib.pf_status_name(status).decode()
        msg = lib.pf_last_error_message().decode()
        super().__init__(f"{where}: {name}: {msg}")
        self.name = name


def _check(status: int, where: str) -> None:
    if status != PF_OK:
        raise PFError(status, where)


def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream_obj(stream):
    torch = _torch()
    return torch.cuda.current_stream() if stream is None else stream


def _stream(stream) -> Optional[int]:
    return _stream_obj(stream).cuda_stream


def _new(shape, dtype, device, stream):
    """A tensor the binding allocates for a call launched on `stream`.

    torch allocates it on the current stream. When the call runs on another
    stream, the tensor is also recorded on that one, so the caching allocator
    does not hand its memory to a later allocation before the kernels queued
    there have finished with it (the binding drops its workspace on return)."""
    torch = _torch()
    t = torch.empty(shape, dtype=dtype, device=device)
    if stream is not None:
        t.record_stream(stream)
    return t


def _same_device(t, device, what: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{what} must be a CUDA tensor")
    if t.device != device:
        raise ValueError(f"{what} is on {t.device}, the call's inputs on {device}")


def _kv_rows(t, heads: int, what: str) -> int:
    torch = _torch()
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError(f"{what} must be a CUDA tensor")
    if t.dtype not in (torch.bfloat16, torch.int16):
        raise TypeError(f"{what} must be bfloat16 (or int16 bf16 bits), got {t.dtype}")
    if t.dim() != 3 or t.shape[1] != heads or t.shape[2] != HEAD_DIM or not t.is_contiguous():
        raise ValueError(f"{what} must be a contiguous [rows][{heads}][128] tensor, got {tuple(t.shape)}")
    return int(t.shape[0])


def _i32_vec(t, what: str) -> None:
    torch = _torch()
    if t is None:
        return
    if not t.is_cuda or t.dtype != torch.int32 or not t.is_contiguous():
        raise TypeError(f"{what} must be a contiguous int32 CUDA tensor")


def _out_i32(t, shape, device, stream, what: str):
    """An int32 output the kernels write numel(shape) entries of: allocated
    when None, otherwise checked (CUDA, same device, int32, contiguous, large
    enough) so that a short or host buffer never reaches a kernel."""
    torch = _torch()
    n = 1
    for d in (shape if isinstance(shape, tuple) else (shape,)):
        n *= int(d)
    if t is None:
        return _new(shape, torch.int32, device, stream)
    _i32_vec(t, what)
    _same_device(t, device, what)
    if t.numel() < n:
        raise ValueError(f"{what} holds {t.numel()} entries, the call writes {n}")
    return t


def _out_f32(t, shape, device, stream, what: str):
    """A float32 output with the same rules as _out_i32."""
    torch = _torch()
    n = 1
    for d in (shape if isinstance(shape, tuple) else (shape,)):
        n *= int(d)
    if t is None:
        return _new(shape, torch.float32, device, stream)
    if not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous():
        raise TypeError(f"{what} must be a contiguous float32 CUDA tensor")
    _same_device(t, device, what)
    if t.numel() < n:
        raise ValueError(f"{what} holds {t.numel()} entries, the call writes {n}")
    return t


def _workspace(ws, need: int, device, stream):
    """(tensor, bytes) of the call's workspace: a new one of `need` bytes
    (at least 1) when None, else the caller's, which must be a contiguous CUDA
    tensor on the inputs' device; its size is checked by the library."""
    torch = _torch()
    if ws is None:
        n = max(int(need), 1)
        return _new(n, torch.uint8, device, stream), n
    if not ws.is_cuda or not ws.is_contiguous():
        raise TypeError("workspace must be a contiguous CUDA tensor")
    _same_device(ws, device, "workspace")
    return ws, ws.numel() * ws.element_size()


def _check_inputs(device, **tensors) -> None:
    for what, t in tensors.items():
        if t is not None:
            _same_device(t, device, what)


def pf_score_select_workspace_bytes(n_q: int, n_heads: int, n_blocks: int, n_c: int) -> int:
    return int(lib.pf_score_select_workspace_bytes(n_q, n_heads, n_blocks, n_c))


def _pool_blocks(pool_k, heads: int, n_c: int) -> int:
    rows = _kv_rows(pool_k, heads, "pool_k")
    if n_c <= 0 or rows % n_c:
        raise ValueError("pool rows must be a multiple of n_c")
    return rows // n_c


def pf_score_select(q, pool_k, n_c: int, top_k: int, ids_out=None, scores_out=None, workspace=None,
                    stream=None) -> Tuple[object, object]:
    """Top-k pool blocks by pooled query-key affinity. Returns (ids int32[top_k], scores f32[n_blocks])."""
    heads = int(q.shape[1])
    n_q = _kv_rows(q, heads, "q")
    n_blocks = _pool_blocks(pool_k, heads, n_c)
    _check_inputs(q.device, pool_k=pool_k)
    ids_out = _out_i32(ids_out, top_k, q.device, stream, "ids_out")
    scores_out = _out_f32(scores_out, n_blocks, q.device, stream, "scores_out")
    ws, have = _workspace(workspace, pf_score_select_workspace_bytes(n_q, heads, n_blocks, n_c), q.device, stream)
    _check(lib.pf_score_select(_ptr(q), n_q, heads, _ptr(pool_k), n_blocks, n_c, top_k, _ptr(ids_out),
                               _ptr(scores_out), _ptr(ws), have, _stream(stream)), "pf_score_select")
    return ids_out, scores_out


def pf_select_place(q, pool_k, n_c: int, top_k: int, pos_tags, recent_first_frame: int, block_frames: int,
                    ids_out=None, deltas_out=None, scores_out=None, workspace=None, stream=None):
    """Selection and placement in one call: the same ids, scores, deltas and tag
    updates as pf_score_select then pf_selection_deltas. Returns (ids, deltas, scores)."""
    heads = int(q.shape[1])
    n_q = _kv_rows(q, heads, "q")
    n_blocks = _pool_blocks(pool_k, heads, n_c)
    _i32_vec(pos_tags, "pos_tags")
    if pos_tags is None or pos_tags.numel() != n_blocks:
        raise ValueError(f"pos_tags must hold {n_blocks} int32 tags")
    _check_inputs(q.device, pool_k=pool_k, pos_tags=pos_tags)
    ids_out = _out_i32(ids_out, top_k, q.device, stream, "ids_out")
    deltas_out = _out_i32(deltas_out, top_k, q.device, stream, "deltas_out")
    scores_out = _out_f32(scores_out, n_blocks, q.device, stream, "scores_out")
    ws, have = _workspace(workspace, pf_score_select_workspace_bytes(n_q, heads, n_blocks, n_c), q.device, stream)
    _check(lib.pf_select_place(_ptr(q), n_q, heads, _ptr(pool_k), n_blocks, n_c, top_k, _ptr(pos_tags),
                               recent_first_frame, block_frames, _ptr(ids_out), _ptr(deltas_out), _ptr(scores_out),
                               _ptr(ws), have, _stream(stream)), "pf_select_place")
    return ids_out, deltas_out, scores_out


def pf_score_select_sub_workspace_bytes(n_q: int, n_heads: int, q_step: int, head_step: int, n_blocks: int,
                                        n_c: int) -> int:
    return int(lib.pf_score_select_sub_workspace_bytes(n_q, n_heads, q_step, head_step, n_blocks, n_c))


def pf_score_select_sub(q, pool_k, n_c: int, top_k: int, q_step: int, head_step: int, ids_out=None,
                        scores_out=None, workspace=None, stream=None) -> Tuple[object, object]:
    """Top-k scored from query rows 0, q_step, ... and heads 0, head_step, ... only."""
    heads = int(q.shape[1])
    n_q = _kv_rows(q, heads, "q")
    n_blocks = _pool_blocks(pool_k, heads, n_c)
    _check_inputs(q.device, pool_k=pool_k)
    ids_out = _out_i32(ids_out, top_k, q.device, stream, "ids_out")
    scores_out = _out_f32(scores_out, n_blocks, q.device, stream, "scores_out")
    need = pf_score_select_sub_workspace_bytes(n_q, heads, q_step, head_step, n_blocks, n_c)
    ws, have = _workspace(workspace, need, q.device, stream)
    _check(lib.pf_score_select_sub(_ptr(q), n_q, heads, q_step, head_step, _ptr(pool_k), n_blocks, n_c, top_k,
                                   _ptr(ids_out), _ptr(scores_out), _ptr(ws), have, _stream(stream)),
           "pf_score_select_sub")
    return ids_out, scores_out


def pf_select_random(n_blocks: int, top_k: int, seed: int, counter: int, n_batch: int = 1, ids_out=None,
                     device="cuda", stream=None):
    """The random-selection baseline: top_k distinct blocks of n_blocks per cache,
    ascending, from stream (seed, counter + b). Returns int32 [n_batch][top_k]
    (or [top_k] when n_batch == 1 and ids_out is None)."""
    torch = _torch()
    dev = torch.device(device) if ids_out is None else ids_out.device
    shape = (n_batch, top_k) if n_batch > 1 else top_k
    ids_out = _out_i32(ids_out, shape, dev, stream, "ids_out")
    _check(lib.pf_select_random(n_blocks, top_k, seed & (2 ** 64 - 1), counter & (2 ** 64 - 1), n_batch,
                                _ptr(ids_out), _stream(stream)), "pf_select_random")
    return ids_out


def pf_selection_deltas(ids, pos_tags, recent_first_frame: int, block_frames: int, deltas_out=None,
                        stream=None):
    """Per-block temporal shift placing the selected blocks before the recent block; updates pos_tags."""
    _i32_vec(ids, "ids")
    _i32_vec(pos_tags, "pos_tags")
    if ids is None or pos_tags is None:
        raise TypeError("ids and pos_tags are required")
    _check_inputs(ids.device, pos_tags=pos_tags)
    deltas_out = _out_i32(deltas_out, ids.numel(), ids.device, stream, "deltas_out")
    _check(lib.pf_selection_deltas(_ptr(ids), ids.numel(), _ptr(pos_tags), pos_tags.numel(),
                                   recent_first_frame, block_frames, _ptr(deltas_out), _stream(stream)),
           "pf_selection_deltas")
    return deltas_out


def pf_rope_shift(k, rows_per_block: int, deltas, block_ids=None, rope_base: float = 10000.0, stream=None):
    """Rotate the temporal dims of the listed blocks of k in place by their deltas."""
    heads = int(k.shape[1])
    rows = _kv_rows(k, heads, "k")
    if rows_per_block <= 0 or rows % rows_per_block:
        raise ValueError("k rows must be a multiple of rows_per_block")
    _i32_vec(deltas, "deltas")
    _i32_vec(block_ids, "block_ids")
    if deltas is None:
        raise TypeError("deltas is required")
    _check_inputs(k.device, deltas=deltas, block_ids=block_ids)
    n_shift = deltas.numel()
    if block_ids is not None and block_ids.numel() != n_shift:
        raise ValueError("block_ids and deltas differ in length")
    _check(lib.pf_rope_shift(_ptr(k), heads, rows_per_block, rows // rows_per_block, _ptr(block_ids),
                             _ptr(deltas), n_shift, rope_base, _stream(stream)), "pf_rope_shift")
    return k


def _batched_rows(t, what: str) -> Tuple[int, int, int, int]:
    """(batch, rows, heads, batch stride in elements) of a [batch][rows][heads][128]
    bf16 tensor whose caches are each contiguous (the batch stride may be larger
    than one cache, e.g. a view of the first rows of bigger slabs)."""
    torch = _torch()
    if not t.is_cuda:
        raise ValueError(f"{what} must be a CUDA tensor")
    if t.dtype not in (torch.bfloat16, torch.int16):
        raise TypeError(f"{what} must be bfloat16 (or int16 bf16 bits), got {t.dtype}")
    if t.dim() != 4 or t.shape[3] != HEAD_DIM or not t[0].is_contiguous() or \
            t.stride()[1:] != (t.shape[2] * HEAD_DIM, HEAD_DIM, 1):
        raise ValueError(f"{what} must be [batch][rows][heads][128] with contiguous caches, got {tuple(t.shape)}")
    return int(t.shape[0]), int(t.shape[1]), int(t.shape[2]), int(t.stride(0))


def pf_score_select_batched_workspace_bytes(n_q: int, n_heads: int, n_blocks: int, n_c: int, n_batch: int) -> int:
    return int(lib.pf_score_select_batched_workspace_bytes(n_q, n_heads, n_blocks, n_c, n_batch))


def _batched_pool(q, pool_k, n_c: int):
    nb, n_q, heads, q_stride = _batched_rows(q, "q")
    nb2, rows, heads2, p_stride = _batched_rows(pool_k, "pool_k")
    if nb2 != nb or heads2 != heads:
        raise ValueError("q and pool_k differ in batch or heads")
    if n_c <= 0 or rows % n_c:
        raise ValueError("pool rows must be a multiple of n_c")
    _check_inputs(q.device, pool_k=pool_k)
    return nb, n_q, heads, q_stride, p_stride, rows // n_c


def pf_score_select_batched(q, pool_k, n_c: int, top_k: int, ids_out=None, scores_out=None, workspace=None,
                            stream=None):
    """Selection over a batch of caches: q [B][n_q][H][128], pool_k [B][M*n_c][H][128].
    Returns (ids int32[B][top_k], scores f32[B][M])."""
    nb, n_q, heads, q_stride, p_stride, n_blocks = _batched_pool(q, pool_k, n_c)
    ids_out = _out_i32(ids_out, (nb, top_k), q.device, stream, "ids_out")
    scores_out = _out_f32(scores_out, (nb, n_blocks), q.device, stream, "scores_out")
    need = pf_score_select_batched_workspace_bytes(n_q, heads, n_blocks, n_c, nb)
    ws, have = _workspace(workspace, need, q.device, stream)
    _check(lib.pf_score_select_batched(_ptr(q), q_stride, n_q, heads, _ptr(pool_k), p_stride, n_blocks, n_c,
                                       top_k, nb, _ptr(ids_out), _ptr(scores_out), _ptr(ws), have,
                                       _stream(stream)), "pf_score_select_batched")
    return ids_out, scores_out


def pf_select_place_batched(q, pool_k, n_c: int, top_k: int, pos_tags, recent_first_frame: int,
                            block_frames: int, ids_out=None, deltas_out=None, scores_out=None, workspace=None,
                            stream=None):
    """pf_select_place over a batch of caches: q [B][n_q][H][128], pool_k [B][M*n_c][H][128],
    pos_tags int32 [B][M]. Returns (ids [B][top_k], deltas [B][top_k], scores [B][M])."""
    nb, n_q, heads, q_stride, p_stride, n_blocks = _batched_pool(q, pool_k, n_c)
    _i32_vec(pos_tags, "pos_tags")
    if pos_tags is None or pos_tags.numel() != nb * n_blocks:
        raise ValueError(f"pos_tags must hold {nb} x {n_blocks} int32 tags")
    _check_inputs(q.device, pos_tags=pos_tags)
    ids_out = _out_i32(ids_out, (nb, top_k), q.device, stream, "ids_out")
    deltas_out = _out_i32(deltas_out, (nb, top_k), q.device, stream, "deltas_out")
    scores_out = _out_f32(scores_out, (nb, n_blocks), q.device, stream, "scores_out")
    need = pf_score_select_batched_workspace_bytes(n_q, heads, n_blocks, n_c, nb)
    ws, have = _workspace(workspace, need, q.device, stream)
    _check(lib.pf_select_place_batched(_ptr(q), q_stride, n_q, heads, _ptr(pool_k), p_stride, n_blocks, n_c, top_k,
                                       _ptr(pos_tags), recent_first_frame, block_frames, nb, _ptr(ids_out),
                                       _ptr(deltas_out), _ptr(scores_out), _ptr(ws), have,
                                       _stream(stream)), "pf_select_place_batched")
    return ids_out, deltas_out, scores_out


def pf_selection_deltas_batched(ids, pos_tags, recent_first_frame: int, block_frames: int, deltas_out=None,
                                stream=None):
    """Placement for a batch: ids int32[B][top_k], pos_tags int32[B][n_blocks] (updated)."""
    _i32_vec(ids, "ids")
    _i32_vec(pos_tags, "pos_tags")
    if ids is None or pos_tags is None:
        raise TypeError("ids and pos_tags are required")
    if ids.dim() != 2 or pos_tags.dim() != 2 or ids.shape[0] != pos_tags.shape[0]:
        raise ValueError("ids and pos_tags must be [batch][top_k] and [batch][n_blocks]")
    _check_inputs(ids.device, pos_tags=pos_tags)
    deltas_out = _out_i32(deltas_out, tuple(ids.shape), ids.device, stream, "deltas_out")
    _check(lib.pf_selection_deltas_batched(_ptr(ids), int(ids.shape[1]), _ptr(pos_tags), int(pos_tags.shape[1]),
                                           recent_first_frame, block_frames, int(ids.shape[0]), _ptr(deltas_out),
                                           _stream(stream)), "pf_selection_deltas_batched")
    return deltas_out


def pf_rope_shift_batched(k, rows_per_block: int, deltas, block_ids=None, rope_base: float = 10000.0,
                          stream=None):
    """In-place temporal shift over a batch: k [B][rows][H][128], deltas int32[B][n_shift]."""
    nb, rows, heads, k_stride = _batched_rows(k, "k")
    if rows_per_block <= 0 or rows % rows_per_block:
        raise ValueError("k rows must be a multiple of rows_per_block")
    _i32_vec(deltas, "deltas")
    _i32_vec(block_ids, "block_ids")
    if deltas is None or deltas.dim() != 2 or deltas.shape[0] != nb:
        raise ValueError("deltas must be [batch][n_shift]")
    _check_inputs(k.device, deltas=deltas, block_ids=block_ids)
    n_shift = int(deltas.shape[1])
    if block_ids is not None and tuple(block_ids.shape) != tuple(deltas.shape):
        raise ValueError("block_ids and deltas differ in shape")
    _check(lib.pf_rope_shift_batched(_ptr(k), k_stride, heads, rows_per_block, rows // rows_per_block,
                                     _ptr(block_ids), _ptr(deltas), n_shift, nb, rope_base, _stream(stream)),
           "pf_rope_shift_batched")
    return k


def pf_rollin(pool_k, pool_v, pos_tags, slot: int, block_k, block_v, first_frame: int, stream=None):
    """Copy one compressed block into pool slot `slot` and set its position tag."""
    heads = int(pool_k.shape[1])
    n_c = _kv_rows(block_k, heads, "block_k")
    if _kv_rows(block_v, heads, "block_v") != n_c:
        raise ValueError("block_k and block_v differ in rows")
    rows = _kv_rows(pool_k, heads, "pool_k")
    if _kv_rows(pool_v, heads, "pool_v") != rows or (slot + 1) * n_c > rows:
        raise ValueError("pool_k/pool_v must match and hold the slot")
    _i32_vec(pos_tags, "pos_tags")
    if pos_tags is not None and pos_tags.numel() <= slot:
        raise ValueError("pos_tags has no entry for the slot")
    _check_inputs(pool_k.device, pool_v=pool_v, block_k=block_k, block_v=block_v, pos_tags=pos_tags)
    _check(lib.pf_rollin(_ptr(pool_k), _ptr(pool_v), _ptr(pos_tags), heads, n_c, slot, _ptr(block_k), _ptr(block_v),
                         first_frame, _stream(stream)), "pf_rollin")


def pf_rollin_batched(pool_k, pool_v, pos_tags, slot: int, block_k, block_v, first_frame: int, stream=None):
    """Roll-in over a batch: pool_k/v [B][rows][H][128] (caches contiguous), pos_tags int32[B][cap],
    block_k/v [B][n_c][H][128]."""
    nb, rows, heads, p_stride = _batched_rows(pool_k, "pool_k")
    nb2, rows2, _, _ = _batched_rows(pool_v, "pool_v")
    nb3, n_c, _, b_stride = _batched_rows(block_k, "block_k")
    _batched_rows(block_v, "block_v")
    if nb2 != nb or nb3 != nb or rows2 != rows or (slot + 1) * n_c > rows:
        raise ValueError("pool and block batches must match and the pool must hold the slot")
    if pool_v.stride(0) != p_stride or block_v.stride(0) != b_stride or tuple(block_v.shape) != tuple(block_k.shape):
        raise ValueError("K and V tensors must have the same shapes and batch strides")
    _i32_vec(pos_tags, "pos_tags")
    t_stride = 0
    if pos_tags is not None:
        if pos_tags.dim() != 2 or pos_tags.shape[0] != nb or pos_tags.shape[1] <= slot:
            raise ValueError("pos_tags must be [batch][capacity] with room for the slot")
        t_stride = int(pos_tags.stride(0))
    _check_inputs(pool_k.device, pool_v=pool_v, block_k=block_k, block_v=block_v, pos_tags=pos_tags)
    _check(lib.pf_rollin_batched(_ptr(pool_k), _ptr(pool_v), p_stride, _ptr(pos_tags), t_stride, heads, n_c, slot,
                                 _ptr(block_k), _ptr(block_v), b_stride, first_frame, nb, _stream(stream)),
           "pf_rollin_batched")


def pf_partition_attn_workspace_bytes(n_q: int, n_heads: int, n_keys: int) -> int:
    return int(lib.pf_partition_attn_workspace_bytes(n_q, n_heads, n_keys))


def _attn_shapes(q, sink_k, sink_v, pool_k, pool_v, n_c, mid_ids, recent_k, recent_v, cur_k, cur_v):
    """Row counts of the partitions (and pool blocks), checked against each other."""
    heads = int(q.shape[1])
    n_q = _kv_rows(q, heads, "q")
    n_sink = _kv_rows(sink_k, heads, "sink_k")
    if _kv_rows(sink_v, heads, "sink_v") != n_sink:
        raise ValueError("sink_k and sink_v differ in rows")
    n_rec = _kv_rows(recent_k, heads, "recent_k")
    if _kv_rows(recent_v, heads, "recent_v") != n_rec:
        raise ValueError("recent_k and recent_v differ in rows")
    n_cur = _kv_rows(cur_k, heads, "cur_k")
    if _kv_rows(cur_v, heads, "cur_v") != n_cur:
        raise ValueError("cur_k and cur_v differ in rows")
    n_sel = 0 if mid_ids is None else mid_ids.numel()
    n_blocks = 0
    if n_sel:
        _i32_vec(mid_ids, "mid_ids")
        rows = _kv_rows(pool_k, heads, "pool_k")
        if _kv_rows(pool_v, heads, "pool_v") != rows or n_c <= 0 or rows % n_c:
            raise ValueError("pool_k/pool_v rows must match and be a multiple of n_c")
        n_blocks = rows // n_c
    _check_inputs(q.device, sink_k=sink_k, sink_v=sink_v, recent_k=recent_k, recent_v=recent_v, cur_k=cur_k,
                  cur_v=cur_v, **({"pool_k": pool_k, "pool_v": pool_v, "mid_ids": mid_ids} if n_sel else {}))
    return heads, n_q, n_sink, n_sel, n_blocks, n_rec, n_cur


def _attn_out(o, lse, want_lse, q, heads, n_q, stream):
    torch = _torch()
    if o is None:
        o = _new(tuple(q.shape), q.dtype, q.device, stream)
    else:
        _same_device(o, q.device, "o")
        if o.dtype not in (torch.bfloat16, torch.int16) or not o.is_contiguous():
            raise TypeError("o must be a contiguous bfloat16 (or int16) CUDA tensor")
        if tuple(o.shape) != tuple(q.shape):
            raise ValueError(f"o must have q's shape {tuple(q.shape)}, got {tuple(o.shape)}")
    if lse is None and want_lse:
        lse = _new((heads, n_q), torch.float32, q.device, stream)
    elif lse is not None:
        if not lse.is_cuda or lse.dtype != torch.float32 or not lse.is_contiguous():
            raise TypeError("lse must be a contiguous float32 CUDA tensor")
        _same_device(lse, q.device, "lse")
        if lse.numel() != heads * n_q:
            raise ValueError(f"lse must hold {heads} x {n_q} values, got {lse.numel()}")
    return o, lse


def pf_partition_attn(q, sink_k, sink_v, pool_k, pool_v, n_c: int, mid_ids, recent_k, recent_v, cur_k, cur_v,
                      scale: float = 0.0, o=None, lse=None, want_lse: bool = False, workspace=None, stream=None):
    """softmax(scale Q K^T) V over sink || pool[mid_ids] || recent || cur. Returns (o, lse or None)."""
    heads, n_q, n_sink, n_sel, n_blocks, n_rec, n_cur = _attn_shapes(
        q, sink_k, sink_v, pool_k, pool_v, n_c, mid_ids, recent_k, recent_v, cur_k, cur_v)
    o, lse = _attn_out(o, lse, want_lse, q, heads, n_q, stream)
    need = int(lib.pf_partition_attn_workspace_bytes(n_q, heads, n_sink + n_sel * n_c + n_rec + n_cur))
    if workspace is None and need == 0:
        ws, have = None, 0
    else:
        ws, have = _workspace(workspace, need, q.device, stream)
    _check(lib.pf_partition_attn(_ptr(q), n_q, heads,
                                 _ptr(sink_k), _ptr(sink_v), n_sink,
                                 _ptr(pool_k) if n_sel else None, _ptr(pool_v) if n_sel else None, n_blocks,
                                 n_c, _ptr(mid_ids) if n_sel else None, n_sel,
                                 _ptr(recent_k), _ptr(recent_v), n_rec,
                                 _ptr(cur_k), _ptr(cur_v), n_cur,
                                 float(scale), _ptr(o), _ptr(lse), _ptr(ws), have, _stream(stream)),
           "pf_partition_attn")
    return o, lse


def pf_partition_attn_noalloc(q, sink_k, sink_v, pool_k, pool_v, n_c: int, mid_ids, recent_k, recent_v, cur_k,
                              cur_v, o, lse=None, scale: float = 0.0, stream=None):
    """pf_partition_attn with the library's fixed device scratch array in place of a
    workspace: the caller passes every buffer, including o (and lse if wanted),
    and the call allocates nothing. Calls overlapping on one GPU race."""
    heads, n_q, n_sink, n_sel, n_blocks, n_rec, n_cur = _attn_shapes(
        q, sink_k, sink_v, pool_k, pool_v, n_c, mid_ids, recent_k, recent_v, cur_k, cur_v)
    if o is None:
        raise TypeError("o is required: pf_partition_attn_noalloc allocates nothing")
    o, lse = _attn_out(o, lse, False, q, heads, n_q, None)
    _check(lib.pf_partition_attn_noalloc(_ptr(q), n_q, heads,
                                         _ptr(sink_k), _ptr(sink_v), n_sink,
                                         _ptr(pool_k) if n_sel else None, _ptr(pool_v) if n_sel else None,
                                         n_blocks, n_c, _ptr(mid_ids) if n_sel else None, n_sel,
                                         _ptr(recent_k), _ptr(recent_v), n_rec,
                                         _ptr(cur_k), _ptr(cur_v), n_cur,
                                         float(scale), _ptr(o), _ptr(lse), _stream(stream)),
           "pf_partition_attn_noalloc")
    return o, lse


# ---------------------------------------------------------------------------
# HR branch of the compressor
# ---------------------------------------------------------------------------

HR_STAGES = 4


def _act5(t, what: str) -> Tuple[int, int, int, int, int]:
    """A contiguous channels-last bf16 activation [B][T][H][W][C] on the GPU."""
    torch = _torch()
    if not t.is_cuda:
        raise ValueError(f"{what} must be a CUDA tensor")
    if t.dtype not in (torch.bfloat16, torch.int16):
        raise TypeError(f"{what} must be bfloat16 (or int16 bf16 bits), got {t.dtype}")
    if t.dim() != 5 or not t.is_contiguous():
        raise ValueError(f"{what} must be a contiguous [B][T][H][W][C] tensor, got {tuple(t.shape)}")
    return tuple(int(v) for v in t.shape)


def _f32_vec(t, n: int, what: str) -> None:
    torch = _torch()
    if t is None:
        return
    if not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != n:
        raise TypeError(f"{what} must be a contiguous float32 CUDA tensor of {n} values")


def pf_hr_conv_workspace_bytes(n_batch: int, T: int, H: int, W: int, c_in: int, kernel, c_out: int) -> int:
    kt, kh, kw = kernel
    return int(lib.pf_hr_conv_workspace_bytes(n_batch, T, H, W, c_in, kt, kh, kw, c_out))


def _bf16_out(t, shape, like, stream, what: str):
    torch = _torch()
    if t is None:
        return _new(shape, like.dtype, like.device, stream)
    if not t.is_cuda or t.dtype not in (torch.bfloat16, torch.int16) or not t.is_contiguous():
        raise TypeError(f"{what} must be a contiguous bfloat16 (or int16) CUDA tensor")
    _same_device(t, like.device, what)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} must be a contiguous {tuple(shape)} tensor, got {tuple(t.shape)}")
    return t


def pf_hr_conv(x, w, bias, kernel, act: bool = True, y=None, workspace=None, stream=None):
    """One strided 3D convolution (kernel = stride) plus bias and SiLU.
    x [B][T][H][W][C_in], w [C_out][kt][kh][kw][C_in] (bf16 bits), bias fp32 [C_out] or None."""
    B, T, H, W, c_in = _act5(x, "x")
    kt, kh, kw = kernel
    c_out = int(w.shape[0])
    if tuple(w.shape) != (c_out, kt, kh, kw, c_in) or not w.is_contiguous() or not w.is_cuda:
        raise ValueError(f"w must be a contiguous [{c_out}][{kt}][{kh}][{kw}][{c_in}] CUDA tensor")
    _f32_vec(bias, c_out, "bias")
    _check_inputs(x.device, w=w, bias=bias)
    y = _bf16_out(y, (B, T // kt, H // kh, W // kw, c_out), x, stream, "y")
    need = pf_hr_conv_workspace_bytes(B, T, H, W, c_in, kernel, c_out)
    if workspace is None and need == 0:
        ws, have = None, 0
    else:
        ws, have = _workspace(workspace, need, x.device, stream)
    _check(lib.pf_hr_conv(_ptr(x), B, T, H, W, c_in, kt, kh, kw, _ptr(w), _ptr(bias), c_out, 1 if act else 0,
                          _ptr(y), _ptr(ws), have, _stream(stream)), "pf_hr_conv")
    return y


def pf_hr_branch_workspace_bytes(n_batch: int, T: int, H: int, W: int, c_in: int, widths, hidden: int) -> int:
    wa = (ctypes.c_int * HR_STAGES)(*widths)
    return int(lib.pf_hr_branch_workspace_bytes(n_batch, T, H, W, c_in, wa, hidden))


def pf_hr_branch(z, stages, proj, out=None, workspace=None, stream=None):
    """The HR branch on a latent block z [B][T][H][W][C]: stages is a list of
    four (w, bias) pairs (kernels 2x1x1 then 1x2x2 three times, SiLU after
    each), proj is (w [hidden][C_last], bias). Returns [B][N_c][hidden]."""
    B, T, H, W, c_in = _act5(z, "z")
    if len(stages) != HR_STAGES:
        raise ValueError(f"stages must hold {HR_STAGES} (weight, bias) pairs")
    widths = [int(w.shape[0]) for w, _ in stages]
    for s, (w, b) in enumerate(stages):
        if not w.is_cuda or not w.is_contiguous() or w.dim() != 5:
            raise ValueError(f"stage {s} weight must be a contiguous [C_out][kt][kh][kw][C_in] CUDA tensor")
        _f32_vec(b, widths[s], f"stage {s} bias")
        _check_inputs(z.device, **{f"stage {s} weight": w, f"stage {s} bias": b})
    wp, bp = proj
    hidden = int(wp.shape[0])
    if not wp.is_cuda or not wp.is_contiguous() or wp.dim() != 2 or int(wp.shape[1]) != widths[-1]:
        raise ValueError(f"proj weight must be a contiguous [hidden][{widths[-1]}] CUDA tensor")
    _f32_vec(bp, hidden, "proj bias")
    _check_inputs(z.device, proj_weight=wp, proj_bias=bp)
    n_c = int(lib.pf_hr_branch_out_tokens(T, H, W))
    if n_c <= 0:
        raise ValueError(f"the latent block must be at least 2 x 8 x 8, got {T} x {H} x {W}")
    out = _bf16_out(out, (B, n_c, hidden), z, stream, "out")
    ws, have = _workspace(workspace, pf_hr_branch_workspace_bytes(B, T, H, W, c_in, widths, hidden), z.device,
                          stream)
    ws_arr = (ctypes.c_void_p * HR_STAGES)(*[w.data_ptr() for w, _ in stages])
    bs_arr = (ctypes.c_void_p * HR_STAGES)(*[None if b is None else b.data_ptr() for _, b in stages])
    wd_arr = (ctypes.c_int * HR_STAGES)(*widths)
    _check(lib.pf_hr_branch(_ptr(z), B, T, H, W, c_in, ws_arr, bs_arr, wd_arr, _ptr(wp), _ptr(bp), hidden,
                            _ptr(out), _ptr(ws), have, _stream(stream)), "pf_hr_branch")
    return out
