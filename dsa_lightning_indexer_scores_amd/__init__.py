"""IndexCache over DSA lightning-indexer scores, native on AMD MI355X (gfx950).

Thin Python binding of the C ABI in include/indexcache.h (libindexcache.so,
built in-tree by ``python -m dsa_lightning_indexer_scores_amd.build_lib``).
This module only marshals arguments: torch supplies device memory and the
current HIP stream, and every step of the computation runs in the library's
HIP kernels.  There is no fallback: if the library is missing, every call
raises.

Functions mirror the C entry points (without the ``ic_`` prefix):
  indexer_topk(q_I, w, k_I, k)          -> idx [B, Lq, k] int32
  indexer_scores(q_I, w, k_I)           -> scores [B, Lq, row_stride] fp32
  topk_rows(scores, first_len, k)       -> idx [rows, k] int32
  topk_rows_seq(scores, seq_len, k)     -> idx [rows, k] int32 (few long rows: segmented)
  sparse_attn(q, kv, idx)               -> out [B, Lq, H, d] bf16
  run_stack(pattern, layers, k)         -> (outs, idx_cache, stats)
  run_stack_varlen(pattern, layers, k, q_len, pos0) -> (outs, idx_cache, stats)
  run_stack_dynamic(pattern, layers, k, probe_stride, tau)
                                        -> (outs, idx_cache, stats, refreshed, recall)
  decode_step(pattern, layers, seq_len, k) -> (outs, idx_cache, stats)
  decode_step_static(pattern, layers, seq_len, k) -> (outs, idx_cache, stats), no workspace
  decode_indexer_scores(q_I, w, k_I, seq_len) -> scores [B, row_stride] fp32 (one decode F layer)
  decode_attn(q, kv, idx)               -> out [B, 1, H, d] bf16 (one decode layer)
  index_overlap(idx_a, idx_b)           -> (inter, jaccard, recall, means)
  overlap_matrix(idx_list)              -> (J [n, n], R [n, n]) mean Jaccard / recall of every pair
  distill_kl(q_I, w, k_I, idx, qs, kvs) -> (kl [B, Lq], mean)
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libindexcache.so")

IC_OK, IC_ERR_ARG, IC_ERR_SHAPE, IC_ERR_DTYPE, IC_ERR_PATTERN = 0, 1, 2, 3, 4
IC_ERR_NO_CACHED_INDICES, IC_ERR_WORKSPACE, IC_ERR_HIP = 5, 6, 7
IC_BF16, IC_FP8_E4M3 = 0, 1
IC_OP_INDEXER_TOPK, IC_OP_SPARSE_ATTN, IC_OP_RUN_STACK, IC_OP_DECODE_STEP, IC_OP_INDEXER_SCORES = 0, 1, 2, 3, 4
IC_OP_RUN_STACK_VARLEN = 5
IC_OP_DISTILL_KL = 6
IC_OP_DECODE_ATTN = 7


class Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "Lq", "Lk", "pos0", "H_I", "d_I", "k", "H", "d", "idx_dtype", "chunk")]


class Layer(ctypes.Structure):
    _fields_ = [("q_I", ctypes.c_void_p), ("w", ctypes.c_void_p), ("k_I", ctypes.c_void_p),
                ("q", ctypes.c_void_p), ("kv", ctypes.c_void_p), ("out", ctypes.c_void_p)]


class Stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("layers", "indexer_calls", "attn_calls", "score_tiles")]

    def as_dict(self) -> Dict[str, int]:
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


class ICError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"ic status {status}: {msg}")
        self.status = status


class NoCachedIndices(ICError):
    """An S layer came before any F layer, so there are no cached indices to reuse."""


_lib = None


def lib() -> ctypes.CDLL:
    """Load libindexcache.so (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m dsa_lightning_indexer_scores_amd.build_lib`")
    L = ctypes.CDLL(LIB_PATH, mode=ctypes.RTLD_GLOBAL)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    P = ctypes.POINTER
    L.ic_workspace_size.argtypes = [P(Shape), ctypes.c_int]
    L.ic_workspace_size.restype = sz
    L.ic_indexer_topk.argtypes = [P(Shape), vp, vp, vp, vp, vp, sz, vp]
    L.ic_indexer_scores.argtypes = [P(Shape), vp, vp, vp, vp, i64, vp]
    L.ic_topk_rows.argtypes = [vp, i64, i32, i32, i32, vp, vp]
    L.ic_topk_rows_seq.argtypes = [vp, i64, i32, vp, i32, i32, vp, vp, sz, vp]
    L.ic_topk_rows_seq_ws.argtypes = [i32, i32, i32]
    L.ic_topk_rows_seq_ws.restype = sz
    L.ic_index_overlap.argtypes = [vp, vp, i64, i32, vp, vp, vp, vp, vp]
    L.ic_run_stack_varlen.argtypes = [ctypes.c_char_p, i32, P(Layer), P(Shape), P(ctypes.c_int32), P(ctypes.c_int32),
                                      vp, vp, sz, P(Stats), vp]
    L.ic_sparse_attn.argtypes = [P(Shape), vp, vp, vp, vp, vp, sz, vp]
    L.ic_distill_kl.argtypes = [P(Shape), vp, vp, vp, vp, i32, P(vp), P(vp), vp, vp, vp, sz, vp]
    L.ic_run_stack_dynamic.argtypes = [ctypes.c_char_p, i32, P(Layer), P(Shape), i32, ctypes.c_double, vp, vp, vp,
                                       vp, sz, P(Stats), vp]
    L.ic_run_stack_dynamic_ws.argtypes = [P(Shape), i32]
    L.ic_run_stack_dynamic_ws.restype = sz
    L.ic_run_stack.argtypes = [ctypes.c_char_p, i32, P(Layer), P(Shape), vp, vp, sz, P(Stats), vp]
    L.ic_decode_step.argtypes = [ctypes.c_char_p, i32, P(Layer), P(Shape), vp, vp, vp, sz, P(Stats), vp]
    L.ic_decode_step_static.argtypes = [ctypes.c_char_p, i32, P(Layer), P(Shape), vp, vp, P(Stats), vp]
    L.ic_decode_indexer_scores.argtypes = [P(Shape), vp, vp, vp, vp, vp, i64, vp]
    L.ic_decode_attn.argtypes = [P(Shape), vp, vp, vp, vp, vp, sz, vp]
    L.ic_get_stats.argtypes = [P(Stats)]
    L.ic_last_error.restype = ctypes.c_char_p
    L.ic_version.restype = i32
    for fn in ("ic_indexer_topk", "ic_indexer_scores", "ic_topk_rows", "ic_topk_rows_seq", "ic_index_overlap",
               "ic_sparse_attn", "ic_run_stack", "ic_run_stack_varlen", "ic_distill_kl", "ic_run_stack_dynamic",
               "ic_decode_step", "ic_decode_step_static", "ic_decode_indexer_scores", "ic_decode_attn",
               "ic_get_stats"):
        getattr(L, fn).restype = ctypes.c_int
    _lib = L
    return L


def last_error() -> str:
    return lib().ic_last_error().decode()


def version() -> int:
    return int(lib().ic_version())


def _check(status: int):
    if status != IC_OK:
        msg = last_error()
        if status == IC_ERR_NO_CACHED_INDICES:
            raise NoCachedIndices(status, msg)
        raise ICError(status, msg)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t: torch.Tensor, name: str, dtypes, ndim: int, gpu: bool = True):
    """dtype, rank and layout of one tensor argument; gpu=False leaves the device to a
    later check (the stack calls check every layer's shapes first)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if gpu and not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")


def _on_gpu(named, device):
    """Every (name, tensor) pair must live on the one GPU `device`."""
    for name, t in named:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")


_IDX_DTYPES = (torch.bfloat16, torch.uint8, torch.float8_e4m3fn)


def _idx_dtype(t: torch.Tensor) -> int:
    return IC_BF16 if t.dtype == torch.bfloat16 else IC_FP8_E4M3


def make_shape(B, Lq, Lk, k, H=1, d=64, H_I=1, d_I=32, idx_dtype=IC_BF16, pos0=0, chunk=0) -> Shape:
    return Shape(B, Lq, Lk, pos0, H_I, d_I, k, H, d, idx_dtype, chunk)


def workspace_size(shape: Shape, op: int) -> int:
    return int(lib().ic_workspace_size(ctypes.byref(shape), op))


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return ws
    if ws is not None and ws.numel() >= nbytes and ws.data_ptr() % 256 == 0:
        return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _indexer_shape(q_I, w, k_I, k, pos0, chunk, H=1, d=64, gpu=True) -> Shape:
    _need(q_I, "q_I", _IDX_DTYPES, 4, gpu)
    _need(w, "w", (torch.float32,), 3, gpu)
    _need(k_I, "k_I", _IDX_DTYPES, 3, gpu)
    if k_I.dtype != q_I.dtype:
        raise TypeError("q_I and k_I must have the same dtype")
    B, Lq, H_I, d_I = q_I.shape
    if tuple(w.shape) != (B, Lq, H_I) or k_I.shape[0] != B or k_I.shape[2] != d_I:
        raise ValueError(f"inconsistent shapes q_I {tuple(q_I.shape)}, w {tuple(w.shape)}, k_I {tuple(k_I.shape)}")
    return make_shape(B, Lq, k_I.shape[1], k, H, d, H_I, d_I, _idx_dtype(q_I), pos0, chunk)


def indexer_topk(q_I, w, k_I, k: int, pos0: int = 0, chunk: int = 0, idx=None, ws=None, stream=None):
    """Lightning-indexer scores + per-query top-k of one F layer -> idx [B, Lq, k] int32."""
    s = _indexer_shape(q_I, w, k_I, k, pos0, chunk)
    if idx is None:
        idx = torch.empty((s.B, s.Lq, k), dtype=torch.int32, device=q_I.device)
    ws = _workspace(workspace_size(s, IC_OP_INDEXER_TOPK), q_I.device, ws)
    _check(lib().ic_indexer_topk(ctypes.byref(s), _ptr(q_I), _ptr(w), _ptr(k_I), _ptr(idx), _ptr(ws),
                                 0 if ws is None else ws.numel(), _stream(stream)))
    return idx


def indexer_scores(q_I, w, k_I, pos0: int = 0, row_stride: Optional[int] = None, scores=None, stream=None):
    """Raw fp32 indexer scores [B, Lq, row_stride]; row t is valid for keys 0..pos0+t."""
    s = _indexer_shape(q_I, w, k_I, 1, pos0, 0)
    row_stride = s.pos0 + s.Lq if row_stride is None else row_stride
    if scores is None:
        scores = torch.full((s.B, s.Lq, row_stride), float("nan"), dtype=torch.float32, device=q_I.device)
    _check(lib().ic_indexer_scores(ctypes.byref(s), _ptr(q_I), _ptr(w), _ptr(k_I), _ptr(scores),
                                   row_stride, _stream(stream)))
    return scores


def topk_rows(scores, first_len: int, k: int, idx=None, stream=None):
    """Top-k of score rows [rows, row_stride]; row r has first_len + r visible entries."""
    _need(scores, "scores", (torch.float32,), 2)
    rows, stride = scores.shape
    if idx is None:
        idx = torch.empty((rows, k), dtype=torch.int32, device=scores.device)
    _check(lib().ic_topk_rows(_ptr(scores), stride, rows, first_len, k, _ptr(idx), _stream(stream)))
    return idx


def topk_rows_seq_ws(rows: int, max_len: int, k: int) -> int:
    return int(lib().ic_topk_rows_seq_ws(rows, max_len, k))


def topk_rows_seq(scores, seq_len, k: int, max_len: Optional[int] = None, idx=None, ws=None,
                  segmented: bool = True, stream=None):
    """Top-k of score rows [rows, row_stride]; row r has seq_len[r] (device int32) visible
    entries, at most max_len (default row_stride).  segmented=False forces the
    one-workgroup-per-row path for long rows."""
    _need(scores, "scores", (torch.float32,), 2)
    _need(seq_len, "seq_len", (torch.int32,), 1)
    rows, stride = scores.shape
    max_len = stride if max_len is None else max_len
    if idx is None:
        idx = torch.empty((rows, k), dtype=torch.int32, device=scores.device)
    if segmented:
        ws = _workspace(topk_rows_seq_ws(rows, max_len, k), scores.device, ws)
    else:
        ws = None
    _check(lib().ic_topk_rows_seq(_ptr(scores), stride, rows, _ptr(seq_len), max_len, k, _ptr(idx), _ptr(ws),
                                  0 if ws is None else ws.numel(), _stream(stream)))
    return idx


def index_overlap(idx_a, idx_b, stream=None):
    """Per-row overlap of two index caches [..., k] int32 (rows ascending, -1 padded).
    Returns (inter int32 [...], jaccard fp32 [...], recall fp32 [...], means fp32 [2] =
    (mean Jaccard, mean recall)), all on the GPU."""
    for t, name in ((idx_a, "idx_a"), (idx_b, "idx_b")):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous int32 GPU tensor")
    if idx_a.shape != idx_b.shape:
        raise ValueError(f"idx_a {tuple(idx_a.shape)} and idx_b {tuple(idx_b.shape)} differ")
    k = idx_a.shape[-1]
    lead = idx_a.shape[:-1]
    rows = idx_a.numel() // k
    dev = idx_a.device
    inter = torch.empty(lead, dtype=torch.int32, device=dev)
    jac = torch.empty(lead, dtype=torch.float32, device=dev)
    rec = torch.empty(lead, dtype=torch.float32, device=dev)
    means = torch.empty(2, dtype=torch.float32, device=dev)
    _check(lib().ic_index_overlap(_ptr(idx_a), _ptr(idx_b), rows, k, _ptr(inter), _ptr(jac), _ptr(rec), _ptr(means),
                                  _stream(stream)))
    return inter, jac, rec, means


def overlap_matrix(idx_list, stream=None):
    """Cross-layer overlap heatmap (the skill page's Step 1 over every pair of layers):
    for index caches idx_list[a] [..., k] int32 (rows ascending, -1 padded, all of one
    shape), returns two [n, n] float64 numpy arrays, J[a, b] = mean over rows of the
    Jaccard of idx_a and idx_b and R[a, b] = mean over rows of |A & B| / |B|, each entry
    from one ic_index_overlap call (the diagonal too).  Synchronises the stream."""
    n = len(idx_list)
    J = np.zeros((n, n))
    R = np.zeros((n, n))
    pending = []
    for a in range(n):
        for b in range(n):
            pending.append((a, b, index_overlap(idx_list[a], idx_list[b], stream=stream)[3]))
    for a, b, means in pending:
        m = means.cpu().numpy()
        J[a, b], R[a, b] = float(m[0]), float(m[1])
    return J, R


def format_heatmap(M, labels=None, fmt="{:5.2f}") -> str:
    """A plain-text rendering of a square matrix such as overlap_matrix's J."""
    n = M.shape[0]
    labels = labels or [str(i) for i in range(n)]
    w = max(len(fmt.format(1.0)), max(len(x) for x in labels))
    head = " " * w + " " + " ".join(x.rjust(w) for x in labels)
    rows = [labels[i].rjust(w) + " " + " ".join(fmt.format(M[i, j]).rjust(w) for j in range(n)) for i in range(n)]
    return "\n".join([head] + rows)


def _attn_shape(q, kv, k, pos0=0, gpu=True) -> Shape:
    _need(q, "q", (torch.bfloat16,), 4, gpu)
    _need(kv, "kv", (torch.bfloat16,), 4, gpu)
    B, Lq, H, d = q.shape
    if kv.shape[0] != B or kv.shape[2] != 2 or kv.shape[3] != d:
        raise ValueError(f"kv must be [B, Lk, 2, d]; got {tuple(kv.shape)} for q {tuple(q.shape)}")
    return make_shape(B, Lq, kv.shape[1], k, H, d, pos0=pos0)


def sparse_attn(q, kv, idx, out=None, stream=None):
    """Sparse attention over the selected rows -> out [B, Lq, H, d] bf16."""
    _need(idx, "idx", (torch.int32,), 3)
    s = _attn_shape(q, kv, idx.shape[2], pos0=max(0, kv.shape[1] - q.shape[1]))
    if tuple(idx.shape[:2]) != (s.B, s.Lq):
        raise ValueError("idx must be [B, Lq, k]")
    if out is None:
        out = torch.empty_like(q)
    _check(lib().ic_sparse_attn(ctypes.byref(s), _ptr(q), _ptr(kv), _ptr(idx), _ptr(out), None, 0, _stream(stream)))
    return out


def distill_kl(q_I, w, k_I, idx, qs: Sequence[torch.Tensor], kvs: Sequence[torch.Tensor], pos0: int = 0,
               chunk: int = 0, kl=None, mean=None, ws=None, stream=None):
    """Multi-layer distillation loss (forward) of one F layer and the layers it serves.

    q_I, w, k_I: the F layer's indexer inputs; idx [B, Lq, k] int32: the entries the
    loss is taken over; qs[j] [B, Lq, H, d] and kvs[j] [B, Lk, 2, d] bf16: the served
    layers, the F layer first.  Returns (kl [B, Lq] fp32 in nats, mean [1] fp32)."""
    if len(qs) != len(kvs) or not 1 <= len(qs) <= 16:
        raise ValueError("qs and kvs must list the same 1..16 served layers")
    _need(idx, "idx", (torch.int32,), 3)
    B, Lq = q_I.shape[:2]
    H, d = qs[0].shape[2], qs[0].shape[3]
    for q, kv in zip(qs, kvs):
        _need(q, "q", (torch.bfloat16,), 4)
        _need(kv, "kv", (torch.bfloat16,), 4)
        if tuple(q.shape) != (B, Lq, H, d) or tuple(kv.shape) != (B, k_I.shape[1], 2, d):
            raise ValueError(f"served layer shapes q {tuple(q.shape)}, kv {tuple(kv.shape)} do not match")
    s = _indexer_shape(q_I, w, k_I, idx.shape[2], pos0, chunk, H=H, d=d)
    if tuple(idx.shape[:2]) != (B, Lq):
        raise ValueError("idx must be [B, Lq, k]")
    dev = q_I.device
    if kl is None:
        kl = torch.empty((B, Lq), dtype=torch.float32, device=dev)
    if mean is None:
        mean = torch.empty(1, dtype=torch.float32, device=dev)
    ws = _workspace(workspace_size(s, IC_OP_DISTILL_KL), dev, ws)
    qa = (ctypes.c_void_p * len(qs))(*[q.data_ptr() for q in qs])
    kva = (ctypes.c_void_p * len(kvs))(*[kv.data_ptr() for kv in kvs])
    _check(lib().ic_distill_kl(ctypes.byref(s), _ptr(q_I), _ptr(w), _ptr(k_I), _ptr(idx), len(qs), qa, kva,
                               _ptr(kl), _ptr(mean), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))
    return kl, mean


def _layers_struct(pattern: str, layers: Sequence[Dict[str, torch.Tensor]], outs: List[torch.Tensor]):
    arr = (Layer * len(layers))()
    for i, lay in enumerate(layers):
        arr[i] = Layer(_ptr(lay.get("q_I")), _ptr(lay.get("w")), _ptr(lay.get("k_I")), _ptr(lay["q"]),
                       _ptr(lay["kv"]), _ptr(outs[i]))
    return arr


def _check_like(t, name: str, dtype, shape):
    """t must be a contiguous tensor of exactly this dtype and shape (the device is
    checked afterwards, once every shape is known to be right)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_indexer_layers(pattern, layers, ref_shapes, dtype, optional_on_s: bool):
    """Every F layer (and, with optional_on_s, every S layer that brings them) must carry
    q_I, w, k_I of the reference shapes and dtype: the kernels read them at those sizes."""
    q_shape, w_shape, k_shape = ref_shapes
    for l, (c, lay) in enumerate(zip(pattern, layers)):
        have = [lay.get(name) is not None for name in ("q_I", "w", "k_I")]
        if c in "F1":
            if not all(have):
                raise ValueError(f"F layer {l} needs q_I, w and k_I")
        elif not optional_on_s or not any(have):
            continue
        elif not all(have):
            raise ValueError(f"layer {l}: q_I, w and k_I must be all present or all absent")
        _check_like(lay["q_I"], f"layers[{l}].q_I", dtype, q_shape)
        _check_like(lay["w"], f"layers[{l}].w", torch.float32, w_shape)
        _check_like(lay["k_I"], f"layers[{l}].k_I", dtype, k_shape)


def _stack_outputs(layers, outs, idx_cache, idx_shape, extra=()):
    """Shape-check caller outputs, then put every tensor of the call on one GPU, then
    allocate the outputs the caller did not pass.  Returns (outs, idx_cache)."""
    q = layers[0]["q"]
    if outs is not None:
        if len(outs) != len(layers):
            raise ValueError(f"outs must list {len(layers)} tensors, got {len(outs)}")
        for l, o in enumerate(outs):
            _check_like(o, f"outs[{l}]", torch.bfloat16, q.shape)
    if idx_cache is not None:
        _check_like(idx_cache, "idx_cache", torch.int32, idx_shape)
    named = [(f"layers[{l}].{key}", lay.get(key)) for l, lay in enumerate(layers)
             for key in ("q_I", "w", "k_I", "q", "kv")]
    named += [(f"outs[{l}]", o) for l, o in enumerate(outs or [])]
    named += [("idx_cache", idx_cache)] + list(extra)
    _on_gpu(named, q.device)
    if outs is None:
        outs = [torch.empty_like(lay["q"]) for lay in layers]
    if idx_cache is None:
        idx_cache = torch.empty(idx_shape, dtype=torch.int32, device=q.device)
    return outs, idx_cache


def _check_pattern(pattern: str, n_layers: int):
    """The library's pattern rules, checked before any tensor: length, the F/S/1/0
    alphabet, and no S layer before the first F layer (nothing cached to reuse)."""
    if len(pattern) != n_layers:
        raise ValueError(f"pattern length {len(pattern)} != {n_layers} layers")
    bad = [c for c in pattern if c not in "FS10"]
    if bad:
        raise ICError(IC_ERR_PATTERN, f"pattern char {bad[0]!r} is not one of F, S, 1, 0")
    first_f = next((i for i, c in enumerate(pattern) if c in "F1"), len(pattern))
    if first_f > 0:
        raise NoCachedIndices(IC_ERR_NO_CACHED_INDICES,
                              "no cached indices: layer 0 is S and no F layer precedes it")


def _stack_shape(pattern, layers, k, chunk, pos0, optional_on_s: bool = False):
    """Shape of a prefill or decode stack call, after checking the pattern and the dtype,
    shape and layout of every layer's tensors (not yet their device: see _stack_outputs)."""
    _check_pattern(pattern, len(layers))
    q, kv = layers[0]["q"], layers[0]["kv"]
    s = _attn_shape(q, kv, k, pos0, gpu=False)
    for l, lay in enumerate(layers):
        _check_like(lay["q"], f"layers[{l}].q", torch.bfloat16, q.shape)
        _check_like(lay["kv"], f"layers[{l}].kv", torch.bfloat16, kv.shape)
    src = next((l for c, l in zip(pattern, layers) if c in "F1" and l.get("q_I") is not None), None)
    if src is None and optional_on_s:
        src = next((l for l in layers if l.get("q_I") is not None), None)
    if src is None:
        _check_indexer_layers(pattern, layers, (None, None, None), None, optional_on_s)
        return s
    si = _indexer_shape(src["q_I"], src["w"], src["k_I"], k, pos0, chunk, gpu=False)
    s.H_I, s.d_I, s.idx_dtype, s.chunk = si.H_I, si.d_I, si.idx_dtype, si.chunk
    if si.Lk != s.Lk:
        raise ValueError("k_I and kv must have the same row capacity")
    if si.B != s.B or si.Lq != s.Lq:
        raise ValueError("q_I and q must have the same batch and query count")
    _check_indexer_layers(pattern, layers, (src["q_I"].shape, src["w"].shape, src["k_I"].shape),
                          src["q_I"].dtype, optional_on_s)
    return s


def run_stack(pattern: str, layers: Sequence[Dict[str, torch.Tensor]], k: int, chunk: int = 0, pos0: int = 0,
              outs: Optional[List[torch.Tensor]] = None, idx_cache=None, ws=None, stream=None):
    """Prefill an F/S stack.  layers[l]: q, kv (+ q_I, w, k_I on F layers)."""
    s = _stack_shape(pattern, layers, k, chunk, pos0)
    outs, idx_cache = _stack_outputs(layers, outs, idx_cache, (s.B, s.Lq, k))
    dev = layers[0]["q"].device
    # a caller's workspace of one score tile is enough (top-k then stays on the stream);
    # otherwise allocate the recommended two tiles
    if ws is None or ws.numel() < workspace_size(s, IC_OP_INDEXER_TOPK) or ws.data_ptr() % 256:
        ws = _workspace(workspace_size(s, IC_OP_RUN_STACK), dev, None)
    arr = _layers_struct(pattern, layers, outs)
    st = Stats()
    _check(lib().ic_run_stack(pattern.encode(), len(layers), arr, ctypes.byref(s), _ptr(idx_cache), _ptr(ws),
                              0 if ws is None else ws.numel(), ctypes.byref(st), _stream(stream)))
    return outs, idx_cache, st.as_dict()


def run_stack_dynamic(pattern: str, layers: Sequence[Dict[str, torch.Tensor]], k: int, probe_stride: int,
                      tau: float, chunk: int = 0, pos0: int = 0, outs: Optional[List[torch.Tensor]] = None,
                      idx_cache=None, ws=None, stream=None):
    """Prefill an F/S stack whose S layers that bring q_I, w, k_I probe the index cache and
    re-index when the pooled recall of their own top-k in it is below tau.
    Returns (outs, idx_cache, stats, refreshed [n_layers, B] int32 (-1: no probe),
    recall [n_layers, B] fp32 (nan: no probe)), all tensors on the GPU."""
    s = _stack_shape(pattern, layers, k, chunk, pos0, optional_on_s=True)
    outs, idx_cache = _stack_outputs(layers, outs, idx_cache, (s.B, s.Lq, k))
    dev = layers[0]["q"].device
    refreshed = torch.full((len(layers), s.B), -1, dtype=torch.int32, device=dev)
    recall = torch.full((len(layers), s.B), float("nan"), dtype=torch.float32, device=dev)
    ws = _workspace(int(lib().ic_run_stack_dynamic_ws(ctypes.byref(s), probe_stride)), dev, ws)
    arr = _layers_struct(pattern, layers, outs)
    st = Stats()
    _check(lib().ic_run_stack_dynamic(pattern.encode(), len(layers), arr, ctypes.byref(s), probe_stride, float(tau),
                                      _ptr(idx_cache), _ptr(refreshed), _ptr(recall), _ptr(ws),
                                      0 if ws is None else ws.numel(), ctypes.byref(st), _stream(stream)))
    return outs, idx_cache, st.as_dict(), refreshed, recall


def run_stack_varlen(pattern: str, layers: Sequence[Dict[str, torch.Tensor]], k: int, q_len: Sequence[int],
                     pos0: Sequence[int], chunk: int = 0, outs: Optional[List[torch.Tensor]] = None, idx_cache=None,
                     ws=None, stream=None):
    """Ragged batched prefill: sequence b brings q_len[b] queries at positions pos0[b].. of its own
    cache.  layers[l]: packed q [T, H, d] (+ q_I [T, H_I, d_I], w [T, H_I] on F layers) with
    T = sum(q_len), and per-sequence caches kv [B, Lk, 2, d] (+ k_I [B, Lk, d_I])."""
    B, T = len(q_len), int(sum(q_len))
    if len(pos0) != B:
        raise ValueError("q_len and pos0 must have one entry per sequence")
    _check_pattern(pattern, len(layers))
    q0, kv0 = layers[0]["q"], layers[0]["kv"]
    _need(q0, "q", (torch.bfloat16,), 3, gpu=False)
    _need(kv0, "kv", (torch.bfloat16,), 4, gpu=False)
    if q0.shape[0] != T or kv0.shape[0] != B or kv0.shape[2] != 2 or kv0.shape[3] != q0.shape[2]:
        raise ValueError(f"q {tuple(q0.shape)} / kv {tuple(kv0.shape)} do not match q_len (B={B}, T={T})")
    s = make_shape(B, T, kv0.shape[1], k, q0.shape[1], q0.shape[2], chunk=chunk)
    for l, lay in enumerate(layers):
        _check_like(lay["q"], f"layers[{l}].q", torch.bfloat16, q0.shape)
        _check_like(lay["kv"], f"layers[{l}].kv", torch.bfloat16, kv0.shape)
    first_f = next((l for c, l in zip(pattern, layers) if c in "F1" and l.get("q_I") is not None), None)
    if first_f is not None:
        _need(first_f["q_I"], "q_I", _IDX_DTYPES, 3, gpu=False)
        s.H_I, s.d_I = first_f["q_I"].shape[1], first_f["q_I"].shape[2]
        s.idx_dtype = _idx_dtype(first_f["q_I"])
        _check_indexer_layers(pattern, layers, ((T, s.H_I, s.d_I), (T, s.H_I), (B, s.Lk, s.d_I)),
                              first_f["q_I"].dtype, False)
    else:
        _check_indexer_layers(pattern, layers, (None, None, None), None, False)
    outs, idx_cache = _stack_outputs(layers, outs, idx_cache, (T, k))
    ws = _workspace(workspace_size(s, IC_OP_RUN_STACK_VARLEN), q0.device, ws)
    arr = _layers_struct(pattern, layers, outs)
    st = Stats()
    ql = (ctypes.c_int32 * B)(*[int(x) for x in q_len])
    p0 = (ctypes.c_int32 * B)(*[int(x) for x in pos0])
    _check(lib().ic_run_stack_varlen(pattern.encode(), len(layers), arr, ctypes.byref(s), ql, p0, _ptr(idx_cache),
                                     _ptr(ws), 0 if ws is None else ws.numel(), ctypes.byref(st), _stream(stream)))
    return outs, idx_cache, st.as_dict()


def decode_step(pattern: str, layers: Sequence[Dict[str, torch.Tensor]], seq_len: torch.Tensor, k: int,
                outs: Optional[List[torch.Tensor]] = None, idx_cache=None, ws=None, stream=None):
    """One decode step.  layers[l]: q [B,1,H,d], kv [B,cap,2,d] (+ q_I [B,1,H_I,d_I], w [B,1,H_I], k_I [B,cap,d_I])."""
    s = _stack_shape(pattern, layers, k, 0, 0)
    s.pos0 = 0
    if s.Lq != 1:
        raise ValueError(f"decode takes one query per sequence; q has {s.Lq}")
    _check_like(seq_len, "seq_len", torch.int32, (s.B,))
    outs, idx_cache = _stack_outputs(layers, outs, idx_cache, (s.B, 1, k), extra=[("seq_len", seq_len)])
    ws = _workspace(workspace_size(s, IC_OP_DECODE_STEP), layers[0]["q"].device, ws)
    arr = _layers_struct(pattern, layers, outs)
    st = Stats()
    _check(lib().ic_decode_step(pattern.encode(), len(layers), arr, ctypes.byref(s), _ptr(seq_len), _ptr(idx_cache),
                                _ptr(ws), 0 if ws is None else ws.numel(), ctypes.byref(st), _stream(stream)))
    return outs, idx_cache, st.as_dict()


def decode_step_static(pattern: str, layers: Sequence[Dict[str, torch.Tensor]], seq_len: torch.Tensor, k: int,
                       outs: Optional[List[torch.Tensor]] = None, idx_cache=None, stream=None):
    """decode_step without a workspace: the library's fixed per-GPU scratch array serves
    (IC_DECODE_STATIC_SCRATCH_BYTES); nothing is allocated when outs and idx_cache are
    given.  Calls that overlap on one GPU race on that array."""
    s = _stack_shape(pattern, layers, k, 0, 0)
    s.pos0 = 0
    if s.Lq != 1:
        raise ValueError(f"decode takes one query per sequence; q has {s.Lq}")
    _check_like(seq_len, "seq_len", torch.int32, (s.B,))
    outs, idx_cache = _stack_outputs(layers, outs, idx_cache, (s.B, 1, k), extra=[("seq_len", seq_len)])
    arr = _layers_struct(pattern, layers, outs)
    st = Stats()
    _check(lib().ic_decode_step_static(pattern.encode(), len(layers), arr, ctypes.byref(s), _ptr(seq_len),
                                       _ptr(idx_cache), ctypes.byref(st), _stream(stream)))
    return outs, idx_cache, st.as_dict()


def decode_indexer_scores(q_I, w, k_I, seq_len, row_stride: Optional[int] = None, scores=None, stream=None):
    """Indexer scores of one decode step's F layer: q_I [B,1,H_I,d_I], w [B,1,H_I] against
    keys 0..seq_len[b]-1 of k_I [B,Lk,d_I] -> scores [B, row_stride] fp32 (row b valid for
    its first seq_len[b] entries)."""
    s = _indexer_shape(q_I, w, k_I, 1, 0, 0)
    if s.Lq != 1:
        raise ValueError(f"decode takes one query per sequence; q_I has {s.Lq}")
    _need(seq_len, "seq_len", (torch.int32,), 1)
    if seq_len.shape[0] != s.B:
        raise ValueError(f"seq_len has {seq_len.shape[0]} entries for B = {s.B}")
    row_stride = (s.Lk + 3) // 4 * 4 if row_stride is None else row_stride
    if scores is None:
        scores = torch.full((s.B, row_stride), float("nan"), dtype=torch.float32, device=q_I.device)
    _check_like(scores, "scores", torch.float32, (s.B, row_stride))
    _check(lib().ic_decode_indexer_scores(ctypes.byref(s), _ptr(q_I), _ptr(w), _ptr(k_I), _ptr(seq_len), _ptr(scores),
                                          row_stride, _stream(stream)))
    return scores


def decode_attn(q, kv, idx, out=None, ws=None, stream=None):
    """Sparse attention of one decode layer: q [B,1,H,d], kv [B,Lk,2,d], idx [B,1,k] -> out [B,1,H,d]."""
    _need(idx, "idx", (torch.int32,), 3)
    s = _attn_shape(q, kv, idx.shape[2])
    if s.Lq != 1 or tuple(idx.shape[:2]) != (s.B, 1):
        raise ValueError("decode attention takes q [B,1,H,d] and idx [B,1,k]")
    if out is None:
        out = torch.empty_like(q)
    _check_like(out, "out", torch.bfloat16, q.shape)
    ws = _workspace(workspace_size(s, IC_OP_DECODE_ATTN), q.device, ws)
    _check(lib().ic_decode_attn(ctypes.byref(s), _ptr(q), _ptr(kv), _ptr(idx), _ptr(out), _ptr(ws),
                                0 if ws is None else ws.numel(), _stream(stream)))
    return out


def get_stats() -> Dict[str, int]:
    st = Stats()
    _check(lib().ic_get_stats(ctypes.byref(st)))
    return st.as_dict()
