"""Python binding of libfp8ts.so: FP8-e4m3 top-k sparse attention on MI355X.

Argument marshalling only.  Every step runs in the HIP library; torch is used
for device memory and the current stream.  If the library cannot be loaded
the calls raise: there is no CPU fallback.

Functions (same names as the C ABI in ``include/fp8ts.h``):

* :func:`fp8_quantize`     bf16/fp16 tensor -> e4m3 bytes (per-tensor scale).
* :func:`indexer_topk`     lightning-indexer ascending top-k block ids.
* :func:`sparse_attn_fwd`  sparse attention forward (token or block mode).
* :func:`fp8_cache_store`  quantize new K / V / index-K rows into a paged e4m3 cache.
* :func:`fp8_rope_quantize` RoPE fused with e4m3 quantization of Q or K.
* :func:`fp8_qknorm_rope_quantize` per-head RMS norm + RoPE + e4m3 of the index
  query / key, into fp8 rows and/or the paged index-K cache.

fp8 tensors are exchanged as ``torch.uint8`` holding e4m3fn bytes
(``torch.float8_e4m3fn`` inputs are accepted and viewed as bytes).
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8ts.so")

BF16, FP16 = 0, 1
TOKEN_MODE, BLOCK_MODE = 0, 1
_ST_OK, _ST_EINVAL, _ST_EUNSUP, _ST_EHIP = 0, 1, 2, 3

_lib = None

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_fp = ctypes.POINTER(ctypes.c_float)
_sz = ctypes.c_size_t

_SIGNATURES = {
    "fp8ts_last_error": ([], ctypes.c_char_p),
    "fp8ts_abi_version": ([], ctypes.c_int),
    "fp8_quantize": ([_vp, _i32, _i64, _i64, _i64, _vp, _i64, _fp, _vp], ctypes.c_int),
    "fp8_quantize_pair": ([_vp, _vp, _i64, _fp, _vp, _vp, _i64, _fp, _i32, _vp], ctypes.c_int),
    "indexer_topk_workspace_size": ([_i32, _i32, _i32], _sz),
    "indexer_topk": ([_vp, _vp, _i64, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                      _fp, _fp, _i32, _vp, _vp, _sz, _vp], ctypes.c_int),
    "fp8_cache_store": ([_vp, _vp, _i32, _i64, _i32, _i32, _i32, _i64, _i64, _i64, _i64, _vp, _vp, _i64, _i32,
                         _fp, _vp], ctypes.c_int),
    "fp8_rope_quantize": ([_vp, _vp, _i32, _i64, _i32, _i32, _i32, _i64, _i64, _i64, _i64, _vp, _i64, _vp, _i32,
                           _vp, _i64, _i64, _fp, _vp], ctypes.c_int),
    "fp8_qknorm_rope_quantize": ([_vp, _i32, _i64, _i32, _i32, _i32, _i64, _i64, _vp, _f32, _vp, _i64, _vp,
                                  _i32, _vp, _i64, _i64, _vp, _vp, _i64, _i32, _fp, _vp], ctypes.c_int),
    "sparse_attn_workspace_size": ([_i32] * 10, _sz),
    "sparse_attn_fwd": ([_i32, _vp, _vp, _vp, _i64, _vp, _i32, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32,
                         _i32, _i32, _i32, _i32, _i32, _i32, _f32, _fp, _fp, _fp, _vp, _vp, _vp, _vp, _vp,
                         _sz, _vp], ctypes.c_int),
    "sparse_attn_fwd_noalloc": ([_i32, _vp, _vp, _vp, _i64, _vp, _i32, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32,
                                 _i32, _i32, _i32, _i32, _i32, _i32, _f32, _fp, _fp, _fp, _vp, _vp, _vp, _vp,
                                 _vp], ctypes.c_int),
    "sparse_attn_noalloc_scratch_bytes": ([], _sz),
}

EXPORTED = tuple(_SIGNATURES)


class Fp8tsError(RuntimeError):
    """A HIP runtime failure reported by the library."""


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libfp8ts.so (once).  Raises if it is missing: no fallback exists.

    ``FP8TS_LIB`` in the environment selects another build of the same library.
    """
    global _lib
    if _lib is not None:
        return _lib
    path = path or os.environ.get("FP8TS_LIB") or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m fp8_top_sparse_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (args, res) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status == _ST_OK:
        return
    msg = _lib.fp8ts_last_error().decode()
    if status in (_ST_EINVAL, _ST_EUNSUP):
        raise ValueError(msg)
    raise Fp8tsError(msg)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _scale(s: Optional[float]):
    return None if s is None else ctypes.byref(ctypes.c_float(float(s)))


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _bytes(t: torch.Tensor) -> torch.Tensor:
    if t.dtype == torch.uint8:
        return t
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8)
    raise ValueError(f"expected e4m3 bytes (uint8 or float8_e4m3fn), got {t.dtype}")


def _i32t(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype != torch.int32 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 tensor")
    return t


def flatten_to_2d(x: torch.Tensor):
    """(rows, cols, row_stride) of ``x`` seen as rows of its last dim.

    The quantize entry takes any tensor whose last dim is contiguous and whose
    leading dims collapse onto one row stride, as the fp8 quantize wrapper on
    the sglang PR 25460 digest does by flattening to 2-D (code excerpt of
    fp8_quantize.py).  The leading dims are merged from the innermost one
    outward: each must step by the row stride times the rows merged so far;
    a dim of size 1 adds no rows and its stride does not matter.  Raises
    ValueError when the last dim is not contiguous or no single row stride
    describes the leading dims.
    """
    if x.dim() == 0:
        return 1, 1, 1
    cols = x.shape[-1]
    if x.numel() == 0:
        return 0, cols, cols
    if cols > 1 and x.stride(-1) != 1:
        raise ValueError(f"last dim must be contiguous (stride {x.stride(-1)})")
    rows, row_stride = 1, None
    for d in range(x.dim() - 2, -1, -1):
        n, step = x.shape[d], x.stride(d)
        if n == 1:
            continue
        if row_stride is None:
            row_stride = step
        elif step != row_stride * rows:
            raise ValueError(f"cannot flatten dim {d}: stride {step} != {row_stride * rows}")
        rows *= n
    return rows, cols, cols if row_stride is None else row_stride


def _same_device(what: str, dev: torch.device, *tensors) -> None:
    """Every given tensor must be a CUDA tensor on ``dev`` (the library takes raw device pointers)."""
    for t in tensors:
        if t is not None and (t.device.type != "cuda" or t.device != dev):
            raise ValueError(f"{what}: every tensor must be on {dev} (got one on {t.device})")


def _check_out(t: torch.Tensor, name: str, dtype, shape) -> None:
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} "
                         f"(got {t.dtype} {tuple(t.shape)})")


def fp8_quantize(x: torch.Tensor, scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                 stream=None) -> torch.Tensor:
    """e4m3 bytes of ``x / scale`` (``scale=None``: no scaling), same shape as x."""
    lib = load()
    if x.dtype == torch.bfloat16:
        dt = BF16
    elif x.dtype == torch.float16:
        dt = FP16
    else:
        raise ValueError(f"x must be bf16 or fp16, got {x.dtype}")
    rows, cols, xs = flatten_to_2d(x)
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    out = _bytes(out)
    if tuple(out.shape) != tuple(x.shape):
        raise ValueError(f"out shape {tuple(out.shape)} != x shape {tuple(x.shape)}")
    orows, _, os_ = flatten_to_2d(out)
    if orows != rows:
        raise ValueError("out does not flatten like x")
    _check(lib.fp8_quantize(_ptr(x), dt, rows, cols, xs, _ptr(out), os_, _scale(scale), _stream(stream)))
    return out


def fp8_quantize_pair(x0: torch.Tensor, scale0: Optional[float], x1: torch.Tensor, scale1: Optional[float], *,
                      out0: Optional[torch.Tensor] = None, out1: Optional[torch.Tensor] = None,
                      stream=None):
    """``(fp8_quantize(x0, scale0), fp8_quantize(x1, scale1))`` in one launch.

    Both tensors contiguous, of one dtype (bf16 or fp16), with element counts
    that are multiples of 8.  Returns ``(out0, out1)``, shaped like the inputs.
    """
    lib = load()
    if x0.dtype != x1.dtype or x0.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError(f"x0 and x1 must share a bf16 or fp16 dtype, got {x0.dtype} and {x1.dtype}")
    dt = BF16 if x0.dtype == torch.bfloat16 else FP16
    if not x0.is_contiguous() or not x1.is_contiguous():
        raise ValueError("x0 and x1 must be contiguous")
    outs = []
    for x, o in ((x0, out0), (x1, out1)):
        if o is None:
            o = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
        ob = _bytes(o)
        if tuple(ob.shape) != tuple(x.shape) or not ob.is_contiguous():
            raise ValueError(f"out shape {tuple(ob.shape)} != x shape {tuple(x.shape)}, or not contiguous")
        outs.append((o, ob))
    _check(lib.fp8_quantize_pair(_ptr(x0), _ptr(outs[0][1]), x0.numel(), _scale(scale0), _ptr(x1),
                                 _ptr(outs[1][1]), x1.numel(), _scale(scale1), dt, _stream(stream)))
    return outs[0][0], outs[1][0]


def indexer_topk(idx_q: torch.Tensor, idx_k: torch.Tensor, block_table: torch.Tensor,
                 cu_seqlens_q: torch.Tensor, seq_lens: torch.Tensor, *, max_q_len: int, sm_scale: float,
                 topk: int, idx_q_scale: Optional[float] = None, idx_k_scale: Optional[float] = None,
                 out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                 stream=None) -> torch.Tensor:
    """Top-k block ids ``[H, total_q, topk]`` int32, strictly ascending, -1 padded.

    idx_q ``[total_q, H, 128]`` e4m3; idx_k ``[num_pages, 128, 128]`` e4m3;
    block_table ``[batch, max_blocks]``; cu_seqlens_q ``[batch+1]``; seq_lens ``[batch]``.
    """
    lib = load()
    q = _bytes(idx_q)
    k = _bytes(idx_k)
    if q.dim() != 3 or k.dim() != 3 or not q.is_contiguous() or not k.is_contiguous():
        raise ValueError("idx_q must be [T, H, D] and idx_k [pages, page, D], contiguous")
    T, H, D = q.shape
    pages, page, Dk = k.shape
    if Dk != D:
        raise ValueError(f"idx_k head dim {Dk} != idx_q head dim {D}")
    bt = _i32t(block_table, "block_table")
    cu = _i32t(cu_seqlens_q, "cu_seqlens_q")
    sl = _i32t(seq_lens, "seq_lens")
    if bt.dim() != 2:
        raise ValueError("block_table must be [batch, max_blocks]")
    B, max_blocks = bt.shape
    if cu.numel() != B + 1 or sl.numel() != B:
        raise ValueError(f"cu_seqlens_q needs batch + 1 = {B + 1} entries and seq_lens {B} "
                         f"(got {cu.numel()} and {sl.numel()})")
    if out is None:
        out = torch.empty((H, T, topk), dtype=torch.int32, device=q.device)
    _check_out(out, "out", torch.int32, (H, T, topk))
    need = lib.indexer_topk_workspace_size(T, H, max_blocks)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _same_device("indexer_topk", q.device, q, k, bt, cu, sl, out, workspace)
    _check(lib.indexer_topk(_ptr(q), _ptr(k), pages, _ptr(bt), max_blocks, _ptr(cu), _ptr(sl), B, T,
                            int(max_q_len), H, D, page, float(sm_scale), _scale(idx_q_scale),
                            _scale(idx_k_scale), int(topk), _ptr(out), _ptr(workspace), wsz,
                            _stream(stream)))
    return out


def _attention(noalloc: bool, q: torch.Tensor, k: torch.Tensor, indices: torch.Tensor, *, sm_scale: float,
               mode: str = "token", v: Optional[torch.Tensor] = None, d_v: Optional[int] = None,
               topk_length: Optional[torch.Tensor] = None, block_table: Optional[torch.Tensor] = None,
               cu_seqlens_q: Optional[torch.Tensor] = None, seq_lens: Optional[torch.Tensor] = None,
               max_q_len: int = 0, q_scale: Optional[float] = None, k_scale: Optional[float] = None,
               v_scale: Optional[float] = None, attn_sink: Optional[torch.Tensor] = None,
               out: Optional[torch.Tensor] = None, max_logits: Optional[torch.Tensor] = None,
               lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
               stream=None):
    """Argument marshalling shared by sparse_attn_fwd and sparse_attn_fwd_noalloc.

    mode "token": q ``[T, Hq, 576]``, k ``[S, 576]`` (V = first d_v=512 columns
    unless ``v [S, 512]`` is given), indices ``[T, topk]`` token ids.
    mode "block": q ``[T, Hq, 128]``, k/v ``[pages, Hkv, 128, 128]`` paged caches,
    indices ``[Hidx, T, topk]`` block ids, plus block_table / cu_seqlens_q /
    seq_lens / max_q_len as for :func:`indexer_topk`.
    """
    lib = load()
    qb = _bytes(q)
    kb = _bytes(k)
    vb = None if v is None else _bytes(v)
    if qb.dim() != 3 or not qb.is_contiguous():
        raise ValueError("q must be a contiguous [T, Hq, Dqk] tensor")
    T, Hq, Dqk = qb.shape
    idx = _i32t(indices, "indices")
    for t in (kb, vb):
        if t is not None and not t.is_contiguous():
            raise ValueError("k / v must be contiguous")
    if mode == "token":
        m = TOKEN_MODE
        if kb.dim() != 2:
            raise ValueError("token mode: k must be [S, Dqk]")
        num_kv, Hkv, Hidx = kb.shape[0], 1, 1
        Dv = d_v if d_v is not None else (vb.shape[-1] if vb is not None else 512)
        if kb.shape[1] != Dqk:
            raise ValueError(f"token mode: k rows hold {kb.shape[1]} bytes, q rows {Dqk}")
        if vb is not None and (vb.dim() != 2 or tuple(vb.shape) != (num_kv, Dv)):
            raise ValueError(f"token mode: v must be [{num_kv}, {Dv}] (got {tuple(vb.shape)})")
        if vb is None and Dv > Dqk:
            raise ValueError(f"token mode: V = the first {Dv} columns of k needs rows of at least {Dv} bytes")
        if idx.dim() != 2 or idx.shape[0] != T:
            raise ValueError("token mode: indices must be [T, topk]")
        topk = idx.shape[1]
        page, max_blocks, B = 0, 0, 0
        bt = cu = sl = None
    elif mode == "block":
        m = BLOCK_MODE
        if kb.dim() != 4 or vb is None or vb.dim() != 4:
            raise ValueError("block mode: k and v must be [pages, Hkv, page, D]")
        num_kv, Hkv, page, kd = kb.shape
        Dv = vb.shape[-1] if d_v is None else d_v
        if kd != Dqk:
            raise ValueError(f"block mode: k rows hold {kd} bytes, q rows {Dqk}")
        if tuple(vb.shape) != (num_kv, Hkv, page, Dv):
            raise ValueError(f"block mode: v must be [{num_kv}, {Hkv}, {page}, {Dv}] like k (got {tuple(vb.shape)})")
        if idx.dim() != 3 or idx.shape[1] != T:
            raise ValueError("block mode: indices must be [Hidx, T, topk]")
        Hidx, topk = idx.shape[0], idx.shape[2]
        bt = _i32t(block_table, "block_table")
        cu = _i32t(cu_seqlens_q, "cu_seqlens_q")
        sl = _i32t(seq_lens, "seq_lens")
        if bt.dim() != 2:
            raise ValueError("block_table must be [batch, max_blocks]")
        B, max_blocks = bt.shape
        if cu.numel() != B + 1 or sl.numel() != B:
            raise ValueError(f"cu_seqlens_q needs batch + 1 = {B + 1} entries and seq_lens {B} "
                             f"(got {cu.numel()} and {sl.numel()})")
    else:
        raise ValueError(f"mode must be 'token' or 'block', got {mode!r}")
    tl = None if topk_length is None else _i32t(topk_length, "topk_length")
    if tl is not None and tl.numel() != T:
        raise ValueError(f"topk_length needs one entry per query token ({T}, got {tl.numel()})")
    sink = None
    if attn_sink is not None:
        if attn_sink.dtype != torch.float32 or attn_sink.numel() != Hq:
            raise ValueError("attn_sink must be float32 [Hq]")
        sink = attn_sink.contiguous()
    dev = qb.device
    if out is None:
        out = torch.empty((T, Hq, Dv), dtype=torch.bfloat16, device=dev)
    if max_logits is None:
        max_logits = torch.empty((T, Hq), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=dev)
    _check_out(out, "out", torch.bfloat16, (T, Hq, Dv))
    _check_out(max_logits, "max_logits", torch.float32, (T, Hq))
    _check_out(lse, "lse", torch.float32, (T, Hq))
    args = (m, _ptr(qb), _ptr(kb), _ptr(vb), num_kv, _ptr(idx), topk, _ptr(tl), _ptr(bt), max_blocks, _ptr(cu),
            _ptr(sl), B, T, int(max_q_len), Hq, Hkv, Hidx, Dqk, Dv, page, float(sm_scale), _scale(q_scale),
            _scale(k_scale), _scale(v_scale), _ptr(sink), _ptr(out), _ptr(max_logits), _ptr(lse))
    if noalloc:
        _same_device("sparse_attn_fwd_noalloc", dev, qb, kb, vb, idx, tl, bt, cu, sl, sink, out, max_logits, lse)
        _check(lib.sparse_attn_fwd_noalloc(*args, _stream(stream)))
        return out, max_logits, lse
    need = lib.sparse_attn_workspace_size(m, B, T, int(max_q_len), Hq, Hkv, Hidx, Dv, topk, max_blocks)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _same_device("sparse_attn_fwd", dev, qb, kb, vb, idx, tl, bt, cu, sl, sink, out, max_logits, lse, workspace)
    _check(lib.sparse_attn_fwd(*args, _ptr(workspace), wsz, _stream(stream)))
    return out, max_logits, lse


def sparse_attn_fwd(q: torch.Tensor, k: torch.Tensor, indices: torch.Tensor, *, sm_scale: float,
                    mode: str = "token", v: Optional[torch.Tensor] = None, d_v: Optional[int] = None,
                    topk_length: Optional[torch.Tensor] = None, block_table: Optional[torch.Tensor] = None,
                    cu_seqlens_q: Optional[torch.Tensor] = None, seq_lens: Optional[torch.Tensor] = None,
                    max_q_len: int = 0, q_scale: Optional[float] = None, k_scale: Optional[float] = None,
                    v_scale: Optional[float] = None, attn_sink: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None, max_logits: Optional[torch.Tensor] = None,
                    lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                    stream=None):
    """Sparse attention forward.  Returns ``(out bf16, max_logits fp32, lse fp32)``.

    mode "token": q ``[T, Hq, 576]``, k ``[S, 576]`` (V = first d_v=512 columns
    unless ``v [S, 512]`` is given), indices ``[T, topk]`` token ids.
    mode "block": q ``[T, Hq, 128]``, k/v ``[pages, Hkv, 128, 128]`` paged caches,
    indices ``[Hidx, T, topk]`` block ids, plus block_table / cu_seqlens_q /
    seq_lens / max_q_len as for :func:`indexer_topk`.  ``workspace`` (uint8,
    at least sparse_attn_workspace_size bytes) is allocated when not given.
    """
    return _attention(False, q, k, indices, sm_scale=sm_scale, mode=mode, v=v, d_v=d_v, topk_length=topk_length,
                      block_table=block_table, cu_seqlens_q=cu_seqlens_q, seq_lens=seq_lens, max_q_len=max_q_len,
                      q_scale=q_scale, k_scale=k_scale, v_scale=v_scale, attn_sink=attn_sink, out=out,
                      max_logits=max_logits, lse=lse, workspace=workspace, stream=stream)


def sparse_attn_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, indices: torch.Tensor, *, sm_scale: float,
                            mode: str = "token", v: Optional[torch.Tensor] = None, d_v: Optional[int] = None,
                            topk_length: Optional[torch.Tensor] = None, block_table: Optional[torch.Tensor] = None,
                            cu_seqlens_q: Optional[torch.Tensor] = None, seq_lens: Optional[torch.Tensor] = None,
                            max_q_len: int = 0, q_scale: Optional[float] = None, k_scale: Optional[float] = None,
                            v_scale: Optional[float] = None, attn_sink: Optional[torch.Tensor] = None,
                            out: Optional[torch.Tensor] = None, max_logits: Optional[torch.Tensor] = None,
                            lse: Optional[torch.Tensor] = None, stream=None):
    """:func:`sparse_attn_fwd` on the library's own per-device scratch (no
    workspace argument, no device allocation inside the library call).  The
    library allocates nothing; to keep the whole call allocation-free pass
    ``out``, ``max_logits`` and ``lse``.  Calls needing more scratch than
    ``sparse_attn_noalloc_scratch_bytes()`` raise ValueError."""
    return _attention(True, q, k, indices, sm_scale=sm_scale, mode=mode, v=v, d_v=d_v, topk_length=topk_length,
                      block_table=block_table, cu_seqlens_q=cu_seqlens_q, seq_lens=seq_lens, max_q_len=max_q_len,
                      q_scale=q_scale, k_scale=k_scale, v_scale=v_scale, attn_sink=attn_sink, out=out,
                      max_logits=max_logits, lse=lse, stream=stream)


def sparse_attn_noalloc_scratch_bytes() -> int:
    """Bytes of the per-device scratch behind :func:`sparse_attn_fwd_noalloc`."""
    return int(load().sparse_attn_noalloc_scratch_bytes())


def _token_head_view(x: torch.Tensor, name: str):
    """(N, H, D, token_stride, head_stride) of a [N, D] or [N, H, D] source."""
    if x.dim() == 2:
        x = x.unsqueeze(1)
    if x.dim() != 3:
        raise ValueError(f"{name} must be [N, D] or [N, H, D]")
    if x.shape[-1] > 1 and x.stride(-1) != 1:
        raise ValueError(f"{name}: last dim must be contiguous")
    n, h, d = x.shape
    return n, h, d, x.stride(0), x.stride(1)


def fp8_cache_store(x: torch.Tensor, slot_mapping: torch.Tensor, cache: torch.Tensor, *,
                    scale: Optional[float] = None, x2: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """Quantize ``x`` (and ``x2``) and write token n into slot ``slot_mapping[n]`` of ``cache``.

    x ``[N, H, D]`` or ``[N, D]`` bf16/fp16 (any token / head strides);
    slot_mapping int64 ``[N]`` (negative = skip); cache e4m3 bytes
    ``[pages, H, page_size, D + D2]``, ``[pages, page_size, D + D2]`` (one head)
    or ``[S, D + D2]`` (flat rows, page_size 1).  Returns ``cache`` (written in place).
    """
    lib = load()
    if x.dtype == torch.bfloat16:
        dt = BF16
    elif x.dtype == torch.float16:
        dt = FP16
    else:
        raise ValueError(f"x must be bf16 or fp16, got {x.dtype}")
    n, h, d, xts, xhs = _token_head_view(x, "x")
    d2, x2ts, x2hs = 0, 0, 0
    if x2 is not None:
        if x2.dtype != x.dtype:
            raise ValueError("x2 must have the dtype of x")
        n2, h2, d2, x2ts, x2hs = _token_head_view(x2, "x2")
        if (n2, h2) != (n, h):
            raise ValueError("x2 must have the token and head counts of x")
    if slot_mapping.dtype != torch.int64 or not slot_mapping.is_contiguous() or slot_mapping.numel() != n:
        raise ValueError("slot_mapping must be a contiguous int64 tensor with one slot per token")
    cb = _bytes(cache)
    if not cb.is_contiguous():
        raise ValueError("cache must be contiguous")
    if cb.dim() == 4:
        pages, ch, page, row = cb.shape
    elif cb.dim() == 3:
        (pages, page, row), ch = cb.shape, 1
    elif cb.dim() == 2:
        (pages, row), ch, page = cb.shape, 1, 1
    else:
        raise ValueError("cache must be [pages, H, page, row], [pages, page, row] or [S, row]")
    if ch != h or row != d + d2:
        raise ValueError(f"cache heads/row ({ch}, {row}) do not match the sources ({h}, {d} + {d2})")
    _check(lib.fp8_cache_store(_ptr(x), _ptr(x2), dt, n, h, d, d2, xts, xhs, x2ts, x2hs, _ptr(slot_mapping),
                               _ptr(cb), pages, page, _scale(scale), _stream(stream)))
    return cache


def fp8_rope_quantize(x_pe: torch.Tensor, cos_sin_cache: torch.Tensor, positions: torch.Tensor, *,
                      x_nope: Optional[torch.Tensor] = None, is_neox: bool = True,
                      scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    """e4m3 rows ``[N, H, nope + rope]`` = quantize(x_nope) ++ quantize(rope(x_pe)).

    x_pe ``[N, H, R]``, ``[N, 1, R]`` or ``[N, R]`` (the last two: one rope head
    shared by all heads); x_nope ``[N, H, nope]`` or None; cos_sin_cache fp32
    ``[max_position, R]`` (cosines then sines); positions int64 ``[N]``.
    """
    lib = load()
    if x_pe.dtype == torch.bfloat16:
        dt = BF16
    elif x_pe.dtype == torch.float16:
        dt = FP16
    else:
        raise ValueError(f"x_pe must be bf16 or fp16, got {x_pe.dtype}")
    n, hp, r, pts, phs = _token_head_view(x_pe, "x_pe")
    nope, nts, nhs, h = 0, 0, 0, hp
    if x_nope is not None:
        if x_nope.dtype != x_pe.dtype:
            raise ValueError("x_nope must have the dtype of x_pe")
        n2, h, nope, nts, nhs = _token_head_view(x_nope, "x_nope")
        if n2 != n or hp not in (1, h):
            raise ValueError("x_nope and x_pe disagree on tokens / heads")
    if hp == 1:
        phs = 0                                   # one rope head, broadcast
    if cos_sin_cache.dtype != torch.float32 or cos_sin_cache.dim() != 2 or not cos_sin_cache.is_contiguous() \
            or cos_sin_cache.shape[1] != r:
        raise ValueError("cos_sin_cache must be a contiguous float32 [max_position, rope_dim] tensor")
    if positions.dtype != torch.int64 or not positions.is_contiguous() or positions.numel() != n:
        raise ValueError("positions must be a contiguous int64 tensor with one position per token")
    if out is None:
        out = torch.empty((n, h, nope + r), dtype=torch.uint8, device=x_pe.device)
    ob = _bytes(out)
    if ob.dim() != 3 or tuple(ob.shape) != (n, h, nope + r) or ob.stride(-1) != 1:
        raise ValueError(f"out must be [N, H, {nope + r}] with a contiguous last dim")
    _check(lib.fp8_rope_quantize(_ptr(x_nope), _ptr(x_pe), dt, n, h, nope, r, nts, nhs, pts, phs,
                                 _ptr(cos_sin_cache), cos_sin_cache.shape[0], _ptr(positions), int(bool(is_neox)),
                                 _ptr(ob), ob.stride(0), ob.stride(1), _scale(scale), _stream(stream)))
    return out


def fp8_qknorm_rope_quantize(x: torch.Tensor, norm_weight: torch.Tensor, eps: float, *, rope_dim: int = 0,
                             cos_sin_cache: Optional[torch.Tensor] = None,
                             positions: Optional[torch.Tensor] = None, is_neox: bool = True,
                             scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                             write_out: bool = True, slot_mapping: Optional[torch.Tensor] = None,
                             cache: Optional[torch.Tensor] = None, stream=None) -> Optional[torch.Tensor]:
    """e4m3 rows ``[N, H, D]`` of quantize(rope_last_R(rms_norm(x) * w)).

    x ``[N, H, D]`` or ``[N, D]`` bf16/fp16; norm_weight fp32 ``[D]``; the last
    ``rope_dim`` dims are rotated (cos_sin_cache fp32 ``[max_position,
    rope_dim]``, positions int64 ``[N]``).  With ``slot_mapping`` (int64 ``[N]``)
    the rows are also stored into ``cache`` (e4m3 bytes ``[pages, H, page, D]``
    or ``[pages, page, D]`` for one head).  ``write_out=False`` skips the
    returned rows (store only); then None is returned.
    """
    lib = load()
    if x.dtype == torch.bfloat16:
        dt = BF16
    elif x.dtype == torch.float16:
        dt = FP16
    else:
        raise ValueError(f"x must be bf16 or fp16, got {x.dtype}")
    n, h, d, xts, xhs = _token_head_view(x, "x")
    if norm_weight.dtype != torch.float32 or not norm_weight.is_contiguous() or norm_weight.numel() != d:
        raise ValueError(f"norm_weight must be a contiguous float32 tensor of {d} values")
    r = int(rope_dim)
    if r > 0:
        if cos_sin_cache is None or positions is None:
            raise ValueError("rope_dim > 0 needs cos_sin_cache and positions")
        if cos_sin_cache.dtype != torch.float32 or cos_sin_cache.dim() != 2 or \
                not cos_sin_cache.is_contiguous() or cos_sin_cache.shape[1] != r:
            raise ValueError("cos_sin_cache must be a contiguous float32 [max_position, rope_dim] tensor")
        if positions.dtype != torch.int64 or not positions.is_contiguous() or positions.numel() != n:
            raise ValueError("positions must be a contiguous int64 tensor with one position per token")
    max_pos = cos_sin_cache.shape[0] if (r > 0 and cos_sin_cache is not None) else 0
    ob = None
    if write_out:
        if out is None:
            out = torch.empty((n, h, d), dtype=torch.uint8, device=x.device)
        ob = _bytes(out)
        if ob.dim() != 3 or tuple(ob.shape) != (n, h, d) or ob.stride(-1) != 1:
            raise ValueError(f"out must be [N, H, {d}] with a contiguous last dim")
    pages, page, cb = 0, 1, None
    if slot_mapping is not None:
        if slot_mapping.dtype != torch.int64 or not slot_mapping.is_contiguous() or slot_mapping.numel() != n:
            raise ValueError("slot_mapping must be a contiguous int64 tensor with one slot per token")
        if cache is None:
            raise ValueError("slot_mapping needs a cache")
        cb = _bytes(cache)
        if not cb.is_contiguous():
            raise ValueError("cache must be contiguous")
        if cb.dim() == 4:
            pages, ch, page, row = cb.shape
        elif cb.dim() == 3:
            (pages, page, row), ch = cb.shape, 1
        else:
            raise ValueError("cache must be [pages, H, page, D] or [pages, page, D]")
        if ch != h or row != d:
            raise ValueError(f"cache heads/row ({ch}, {row}) do not match x ({h}, {d})")
    _check(lib.fp8_qknorm_rope_quantize(_ptr(x), dt, n, h, d, r, xts, xhs, _ptr(norm_weight), float(eps),
                                        _ptr(cos_sin_cache) if r > 0 else None, max_pos,
                                        _ptr(positions) if r > 0 else None, int(bool(is_neox)), _ptr(ob),
                                        ob.stride(0) if ob is not None else 0,
                                        ob.stride(1) if ob is not None else 0, _ptr(slot_mapping), _ptr(cb),
                                        pages, page, _scale(scale), _stream(stream)))
    return out if write_out else None


__all__ = ["fp8_quantize", "fp8_quantize_pair", "indexer_topk", "sparse_attn_fwd", "sparse_attn_fwd_noalloc",
           "sparse_attn_noalloc_scratch_bytes", "fp8_cache_store", "fp8_rope_quantize",
           "fp8_qknorm_rope_quantize", "load", "flatten_to_2d", "EXPORTED",
           "Fp8tsError", "BF16", "FP16", "TOKEN_MODE", "BLOCK_MODE"]
