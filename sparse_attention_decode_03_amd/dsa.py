"""Thin ctypes binding of libdsa.so (include/dsa.h).

Argument marshalling only: shapes are packed into `dsa_shape`, torch tensors
are passed as device pointers together with the current HIP stream, and a
non-zero return code becomes a `DsaError` carrying `dsa_last_error()`. Every
step of the path runs in the library's HIP kernels; there is no fallback. If
the library is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdsa.so")

DSA_OK = 0
DSA_EINVAL = -1
DSA_EUNSUPPORTED = -2
DSA_ERANGE = -3
DSA_EWORKSPACE = -4
DSA_ELAUNCH = -5
DSA_EMETADATA = -6
DSA_META_DEVICE = 0
DSA_META_HOST = 1
NOALLOC_SCRATCH_BYTES = 64 << 20
SELECT_DIRECT_MAX = 24576  # DSA_SELECT_DIRECT_MAX: one-kernel selection up to this max_len

# Every symbol include/dsa.h declares.
EXPORTS = (
    "dsa_workspace_bytes",
    "dsa_index_scores",
    "dsa_topk_select",
    "dsa_mla_decode",
    "dsa_decode_k",
    "dsa_decode_k_noalloc",
    "dsa_decode_k_timed",
    "dsa_cache_write",
    "dsa_topk_select_pooled",
    "dsa_pooled_workspace_bytes",
    "dsa_pool_score_stride",
    "dsa_score_stride",
    "dsa_bt_entries_needed",
    "dsa_check_metadata",
    "dsa_last_error",
)


class DsaError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"dsa error {code}: {message}")
        self.code = code
        self.message = message


class Shape(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("rows_per_seq", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("latent_dim", ctypes.c_int32),
        ("index_heads", ctypes.c_int32),
        ("index_dim", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_len", ctypes.c_int32),
        ("k_capacity", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
    ]

    @property
    def num_rows(self) -> int:
        return self.num_seqs * self.rows_per_seq

    def __repr__(self) -> str:
        return "Shape(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


def shape_of(inputs: dict, **over) -> Shape:
    """dsa_shape for a dict produced by workloads.make_inputs."""
    f = dict(
        num_seqs=inputs["num_seqs"], rows_per_seq=inputs["rows_per_seq"],
        num_heads=inputs["num_heads"], latent_dim=inputs["latent_dim"],
        index_heads=inputs["index_heads"], index_dim=inputs["index_dim"],
        top_k=inputs["top_k"], page_size=inputs["page_size"], max_len=inputs["max_len"],
        k_capacity=inputs["k_capacity"], max_blocks_per_seq=inputs["max_blocks"],
        num_pages=inputs["num_pages"],
    )
    f.update(over)
    return Shape(**f)


_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdsa.so (raises if it is absent: there is no other path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is missing: build it with `python -m sparse_attention_decode_03_amd.build`")
    lib = ctypes.CDLL(path)
    P, S = ctypes.c_void_p, ctypes.POINTER(Shape)
    i32, f32, sz = ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.dsa_workspace_bytes.argtypes = [S]
    lib.dsa_workspace_bytes.restype = sz
    lib.dsa_index_scores.argtypes = [S, P, P, P, P, P, P]
    lib.dsa_index_scores.restype = i32
    lib.dsa_topk_select.argtypes = [S, P, P, P, P, sz, P]
    lib.dsa_topk_select.restype = i32
    lib.dsa_mla_decode.argtypes = [S, P, P, P, P, P, f32, f32, P, P, sz, P]
    lib.dsa_mla_decode.restype = i32
    lib.dsa_decode_k.argtypes = [S, P, P, P, P, P, P, P, f32, f32, P, P, P, P, sz, P]
    lib.dsa_decode_k.restype = i32
    lib.dsa_decode_k_timed.argtypes = [S, P, P, P, P, P, P, P, f32, f32, P, P, P, P, sz, P,
                                       ctypes.POINTER(ctypes.c_void_p)]
    lib.dsa_decode_k_timed.restype = i32
    lib.dsa_decode_k_noalloc.argtypes = [S, P, P, P, P, P, P, P, f32, f32, P, P, P, P]
    lib.dsa_decode_k_noalloc.restype = i32
    lib.dsa_cache_write.argtypes = [S, P, P, P, P, P, P, P, f32, f32, P, P, P, P]
    lib.dsa_cache_write.restype = i32
    lib.dsa_score_stride.argtypes = [S]
    lib.dsa_score_stride.restype = sz
    lib.dsa_pooled_workspace_bytes.argtypes = [S, i32]
    lib.dsa_pooled_workspace_bytes.restype = sz
    lib.dsa_pool_score_stride.argtypes = [S, i32]
    lib.dsa_pool_score_stride.restype = sz
    lib.dsa_topk_select_pooled.argtypes = [S, i32, P, P, P, P, P, sz, P]
    lib.dsa_topk_select_pooled.restype = i32
    lib.dsa_bt_entries_needed.argtypes = [sz, sz, sz]
    lib.dsa_bt_entries_needed.restype = sz
    lib.dsa_check_metadata.argtypes = [S, P, P, P, i32, P]
    lib.dsa_check_metadata.restype = i32
    lib.dsa_last_error.argtypes = []
    lib.dsa_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def last_error() -> str:
    return load().dsa_last_error().decode()


def _check(rc: int) -> None:
    if rc != DSA_OK:
        raise DsaError(rc, last_error())


def _ptr(t) -> Optional[int]:
    """Device pointer of a tensor (None -> NULL; ints pass through)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def workspace_bytes(shape: Shape) -> int:
    return int(load().dsa_workspace_bytes(ctypes.byref(shape)))


def score_stride(shape: Shape) -> int:
    """Row stride (floats) of a scores buffer for `shape`."""
    return int(load().dsa_score_stride(ctypes.byref(shape)))


def bt_entries_needed(seq_len: int, k: int, block_size: int) -> int:
    return int(load().dsa_bt_entries_needed(seq_len, k, block_size))


def index_scores(shape: Shape, q_idx, w, k_normed, seq_lens, scores, stream=None) -> None:
    _check(load().dsa_index_scores(ctypes.byref(shape), _ptr(q_idx), _ptr(w), _ptr(k_normed),
                                   _ptr(seq_lens), _ptr(scores), _stream(stream)))


def topk_select(shape: Shape, scores, seq_lens, sel, ws, ws_bytes: Optional[int] = None,
                stream=None) -> None:
    nb = ws_bytes if ws_bytes is not None else ws.numel() * ws.element_size()
    _check(load().dsa_topk_select(ctypes.byref(shape), _ptr(scores), _ptr(seq_lens), _ptr(sel),
                                  _ptr(ws), nb, _stream(stream)))


def pooled_workspace_bytes(shape: Shape, kp: int) -> int:
    return int(load().dsa_pooled_workspace_bytes(ctypes.byref(shape), kp))


def pool_score_stride(shape: Shape, kp: int) -> int:
    """Row stride (floats) of a pool-scores buffer for `shape` and pools of kp tokens."""
    return int(load().dsa_pool_score_stride(ctypes.byref(shape), kp))


def topk_select_pooled(shape: Shape, kp: int, pool_scores, seq_lens, sel, ws,
                       ws_bytes: Optional[int] = None, stream=None, pool_valid=None) -> None:
    """dsa_topk_select_pooled; pool_valid ([S, pool stride] uint8, or None)
    gates candidacy."""
    nb = ws_bytes if ws_bytes is not None else ws.numel() * ws.element_size()
    _check(load().dsa_topk_select_pooled(ctypes.byref(shape), kp, _ptr(pool_scores),
                                         _ptr(pool_valid), _ptr(seq_lens), _ptr(sel), _ptr(ws),
                                         nb, _stream(stream)))


def mla_decode(shape: Shape, q, kv_cache, block_tables, seq_lens, sel, kv_scale: float,
               sm_scale: float, out, ws, ws_bytes: Optional[int] = None, stream=None) -> None:
    nb = ws_bytes if ws_bytes is not None else ws.numel() * ws.element_size()
    _check(load().dsa_mla_decode(ctypes.byref(shape), _ptr(q), _ptr(kv_cache), _ptr(block_tables),
                                 _ptr(seq_lens), _ptr(sel), kv_scale, sm_scale, _ptr(out), _ptr(ws),
                                 nb, _stream(stream)))


def decode_k(shape: Shape, q_idx, w, k_normed, q, kv_cache, block_tables, seq_lens,
             kv_scale: float, sm_scale: float, scores, sel, out, ws,
             ws_bytes: Optional[int] = None, stream=None) -> None:
    nb = ws_bytes if ws_bytes is not None else ws.numel() * ws.element_size()
    _check(load().dsa_decode_k(ctypes.byref(shape), _ptr(q_idx), _ptr(w), _ptr(k_normed), _ptr(q),
                               _ptr(kv_cache), _ptr(block_tables), _ptr(seq_lens), kv_scale,
                               sm_scale, _ptr(scores), _ptr(sel), _ptr(out), _ptr(ws), nb,
                               _stream(stream)))


def check_metadata(shape: Shape, seq_lens, block_tables, sel=None, stream=None) -> None:
    """Raises DsaError (DSA_EMETADATA) if the lengths, the reachable
    block-table entries or the selection are out of contract. Torch CUDA
    tensors are checked in stream order (a synchronising call); numpy arrays
    are checked on the host."""
    import numpy as np
    if isinstance(seq_lens, np.ndarray):
        arrs = [np.ascontiguousarray(a, dtype=np.int32) if a is not None else None
                for a in (seq_lens, block_tables, sel)]
        ptrs = [a.ctypes.data if a is not None else None for a in arrs]
        _check(load().dsa_check_metadata(ctypes.byref(shape), *ptrs, DSA_META_HOST, None))
        return
    _check(load().dsa_check_metadata(ctypes.byref(shape), _ptr(seq_lens), _ptr(block_tables),
                                     _ptr(sel), DSA_META_DEVICE, _stream(stream)))


def decode_k_timed(shape: Shape, q_idx, w, k_normed, q, kv_cache, block_tables, seq_lens,
                   kv_scale: float, sm_scale: float, scores, sel, out, ws, events,
                   ws_bytes: Optional[int] = None, stream=None) -> None:
    """dsa_decode_k with ten torch.cuda.Events (timing enabled, each already
    recorded once so that it exists) bound in start/stop pairs to the index,
    filter, finish, attention and merge kernels."""
    if len(events) != 10:
        raise ValueError("decode_k_timed takes 10 events")
    nb = ws_bytes if ws_bytes is not None else ws.numel() * ws.element_size()
    handles = (ctypes.c_void_p * 10)(*[e.cuda_event for e in events])
    _check(load().dsa_decode_k_timed(ctypes.byref(shape), _ptr(q_idx), _ptr(w), _ptr(k_normed),
                                     _ptr(q), _ptr(kv_cache), _ptr(block_tables), _ptr(seq_lens),
                                     kv_scale, sm_scale, _ptr(scores), _ptr(sel), _ptr(out),
                                     _ptr(ws), nb, _stream(stream), handles))


def decode_k_noalloc(shape: Shape, q_idx, w, k_normed, q, kv_cache, block_tables, seq_lens,
                     kv_scale: float, sm_scale: float, scores, sel, out, stream=None) -> None:
    """dsa_decode_k with the library's per-device scratch array as workspace."""
    _check(load().dsa_decode_k_noalloc(ctypes.byref(shape), _ptr(q_idx), _ptr(w), _ptr(k_normed),
                                       _ptr(q), _ptr(kv_cache), _ptr(block_tables),
                                       _ptr(seq_lens), kv_scale, sm_scale, _ptr(scores),
                                       _ptr(sel), _ptr(out), _stream(stream)))


def cache_write(shape: Shape, kv_a, latent_w, k_proj, k_w, k_b, seq_lens, block_tables,
                eps: float, kv_scale: float, kv_cache, k_normed, valid=None, stream=None) -> None:
    """dsa_cache_write; valid ([S, k_capacity] uint8, or None) receives the
    validity marks."""
    _check(load().dsa_cache_write(ctypes.byref(shape), _ptr(kv_a), _ptr(latent_w), _ptr(k_proj),
                                  _ptr(k_w), _ptr(k_b), _ptr(seq_lens), _ptr(block_tables), eps,
                                  kv_scale, _ptr(kv_cache), _ptr(k_normed),
                                  None if valid is None else _ptr(valid), _stream(stream)))


class DeviceStep:
    """Device-resident buffers of one decode step (inputs from
    workloads.make_inputs copied to the GPU once; outputs and workspace
    allocated once). Plumbing for tests and the benchmark."""

    def __init__(self, inputs: dict, device: str = "cuda", **shape_over):
        import torch
        self.inputs = inputs
        self.shape = shape_of(inputs, **shape_over)
        sh = self.shape
        dev = torch.device(device)

        import numpy as np
        self.q_idx = torch.from_numpy(inputs["q_idx"].view(np.int16)).to(dev)
        self.w = torch.from_numpy(inputs["w"]).to(dev)
        self.k_normed = torch.from_numpy(inputs["k_normed"].view(np.int16)).to(dev)
        self.q = torch.from_numpy(inputs["q"].view(np.int16)).to(dev)
        self.kv_cache = torch.from_numpy(inputs["kv_cache"]).to(dev)
        self.block_tables = torch.from_numpy(inputs["block_tables"]).to(dev)
        self.seq_lens = torch.from_numpy(inputs["seq_lens"]).to(dev)
        R = sh.num_rows
        self.scores = torch.empty((R, score_stride(sh)), dtype=torch.float32, device=dev)
        self.sel = torch.empty((R, sh.top_k), dtype=torch.int32, device=dev)
        self.out = torch.empty((R, sh.num_heads, sh.latent_dim), dtype=torch.int16, device=dev)
        nb = workspace_bytes(sh)
        if nb == 0:
            raise DsaError(DSA_EINVAL, last_error())
        self.ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        self.kv_scale = float(inputs["kv_scale"])
        self.sm_scale = float(inputs["sm_scale"])

    def decode_k(self, stream=None) -> None:
        decode_k(self.shape, self.q_idx, self.w, self.k_normed, self.q, self.kv_cache,
                 self.block_tables, self.seq_lens, self.kv_scale, self.sm_scale, self.scores,
                 self.sel, self.out, self.ws, stream=stream)

    def index_scores(self, stream=None) -> None:
        index_scores(self.shape, self.q_idx, self.w, self.k_normed, self.seq_lens, self.scores,
                     stream=stream)

    def topk_select(self, stream=None) -> None:
        topk_select(self.shape, self.scores, self.seq_lens, self.sel, self.ws, stream=stream)

    def mla_decode(self, stream=None) -> None:
        mla_decode(self.shape, self.q, self.kv_cache, self.block_tables, self.seq_lens, self.sel,
                   self.kv_scale, self.sm_scale, self.out, self.ws, stream=stream)
