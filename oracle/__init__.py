"""CPU oracle for the DSA decode path (test infrastructure only).

Only the tests, `__graft_entry__.smoke()` and the `cpu_baseline` leg of
`bench.py` may import this package. The product path (the HIP library and its
Python binding) never imports, links or calls it.

The arithmetic lives in plain C (`dsa_oracle.c`, IEEE double precision); this
module only marshals numpy arrays through ctypes. `build()` compiles the C file
with gcc into `liboracle.so` next to it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "dsa_oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")

_lib: Optional[ctypes.CDLL] = None


def build() -> str:
    """Compile the oracle with gcc (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
           SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def _load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build()
    lib = ctypes.CDLL(LIB)
    P = ctypes.c_void_p
    i32, i64, dbl = ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f64.restype = dbl
    lib.oracle_e4m3fn_to_f64.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3fn_to_f64.restype = dbl
    lib.oracle_index_scores.argtypes = [i32, i32, i32, i32, P, P, P, i64, P, i64, P]
    lib.oracle_index_scores.restype = i32
    lib.oracle_topk_row.argtypes = [i64, i64, P, P]
    lib.oracle_topk_row.restype = i32
    lib.oracle_topk.argtypes = [i32, i64, i64, P, P, P]
    lib.oracle_topk.restype = i32
    lib.oracle_mla_decode.argtypes = [i32, i32, i32, i32, P, P, i64, i32, P, i64, P, P, i64,
                                      dbl, dbl, P]
    lib.oracle_mla_decode.restype = i32
    lib.oracle_mla_decode_abs.argtypes = [i32, i32, i32, i32, P, P, i64, i32, P, i64, P, P,
                                          i64, dbl, dbl, P]
    lib.oracle_mla_decode_abs.restype = i32
    lib.oracle_softmax_weights.argtypes = [i32, i32, i32, i32, i32, P, P, i64, i32, P, i64, P,
                                           P, i64, dbl, dbl, P]
    lib.oracle_softmax_weights.restype = i32
    lib.oracle_e4m3fn_encode.argtypes = [ctypes.c_double]
    lib.oracle_e4m3fn_encode.restype = ctypes.c_uint8
    lib.oracle_bf16_encode.argtypes = [ctypes.c_double]
    lib.oracle_bf16_encode.restype = ctypes.c_uint16
    lib.oracle_latent_row.argtypes = [i32, P, P, ctypes.c_double, ctypes.c_double, P, P]
    lib.oracle_latent_row.restype = i32
    lib.oracle_layernorm_row.argtypes = [i32, P, P, P, ctypes.c_double, P, P]
    lib.oracle_layernorm_row.restype = i32
    lib.oracle_cache_write.argtypes = [i32, i32, i32, i32, P, P, P, P, P, P, P, i64, i64, i64,
                                       i64, ctypes.c_double, ctypes.c_double, P, P, P]
    lib.oracle_cache_write.restype = i32
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = i32
    _lib = lib
    return lib


class OracleError(RuntimeError):
    pass


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a: np.ndarray) -> ctypes.c_void_p:
    return ctypes.c_void_p(a.ctypes.data)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise OracleError(f"{what} failed with code {rc}")


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def bf16_to_f64(code: int) -> float:
    return float(_load().oracle_bf16_to_f64(int(code)))


def e4m3_to_f64(code: int) -> float:
    return float(_load().oracle_e4m3fn_to_f64(int(code)))


def index_scores(q_idx, w, k_normed, seq_lens, rows_per_seq: int = 1,
                 max_len: Optional[int] = None) -> np.ndarray:
    """scores [R, max_len] float64; q_idx [R,Hi,D] bf16 codes, w [R,Hi] f32,
    k_normed [S,cap,D] bf16 codes, seq_lens [R]."""
    q_idx = _c(q_idx, np.uint16)
    w = _c(w, np.float32)
    k_normed = _c(k_normed, np.uint16)
    seq_lens = _c(seq_lens, np.int32)
    R, Hi, D = q_idx.shape
    cap = k_normed.shape[1]
    if max_len is None:
        max_len = int(seq_lens.max()) if R else 0
    out = np.zeros((R, max_len), dtype=np.float64)
    rc = _load().oracle_index_scores(R, rows_per_seq, Hi, D, _p(q_idx), _p(w), _p(k_normed),
                                     cap, _p(seq_lens), max_len, _p(out))
    _check(rc, "oracle_index_scores")
    return out


def topk_row(scores_row, L: int, top_k: int) -> np.ndarray:
    s = _c(scores_row, np.float64)
    assert s.shape[0] >= L
    sel = np.empty(top_k, dtype=np.int32)
    _check(_load().oracle_topk_row(L, top_k, _p(s), _p(sel)), "oracle_topk_row")
    return sel


def topk(scores, seq_lens, top_k: int) -> np.ndarray:
    """sel [R, top_k] int32: ascending selected ids, -1 padded. `scores` may be
    float32 (the GPU's) or float64; float32 widens to float64 exactly."""
    s = _c(scores, np.float64)
    seq_lens = _c(seq_lens, np.int32)
    R, max_len = s.shape
    sel = np.empty((R, top_k), dtype=np.int32)
    _check(_load().oracle_topk(R, max_len, top_k, _p(s), _p(seq_lens), _p(sel)), "oracle_topk")
    return sel


def pooled_select(pool_scores, seq_lens, kp: int, select_k: int, pool_valid=None,
                  rows_per_seq: int = 1) -> np.ndarray:
    """Pooled selection and its expansion to tokens: sel [R, select_k*kp + kp - 1]
    int32, -1 padded.

    Follows the doc of the prefill row-group selector on the glm5next_dsa
    layer.rs source page: pool p (tokens p*kp .. p*kp + kp - 1) is a candidate
    of a row only when it is complete (pool_valid[p]) and its last token is
    visible to the row's query, i.e. p < (q_pos + 1) / kp = L // kp; the row
    expands row_select_k = min(select_k, L // kp) pool places (the per-row
    correction of the expansion), filled by its top candidates under the
    total order (score descending, pool index ascending); the selected pools
    expand to their kp tokens each, and the row's visible tail (tokens
    L // kp * kp .. L - 1, the incomplete pool) is written from slot
    row_select_k * kp on.
    Readings: pools expand in ascending pool order (as the per-token ids are
    ascending); the pool scores are an input (how the pages form them from
    the gate and the positional term is not on the pages); pool_valid
    [S, >= max pools] (None: every visible pool complete) belongs to the
    sequence, row r to sequence r // rows_per_seq; a non-candidate is never
    taken, so a row with fewer candidates than row_select_k leaves the rest
    of its pool places -1 and its tail where its position puts it."""
    seq_lens = _c(seq_lens, np.int32)
    R = seq_lens.shape[0]
    width = select_k * kp + kp - 1
    out = np.full((R, width), -1, dtype=np.int32)
    for r in range(R):
        L = int(seq_lens[r])
        pvis = L // kp
        rsk = min(select_k, pvis)
        cand = [p for p in range(pvis)
                if pool_valid is None or pool_valid[r // rows_per_seq][p]]
        tokens = []
        if cand:
            sc = np.asarray(pool_scores[r], dtype=np.float64)[cand]
            order = topk_row(sc, len(cand), select_k)[:min(rsk, len(cand))]
            pools = sorted(cand[int(i)] for i in order)
            tokens = [int(p) * kp + i for p in pools for i in range(kp)]
        out[r, :len(tokens)] = tokens
        tail = list(range(pvis * kp, L))
        out[r, rsk * kp:rsk * kp + len(tail)] = tail
    return out


def mla_decode(q, kv_cache, block_tables, seq_lens, sel, kv_scale: float, sm_scale: float,
               rows_per_seq: int = 1) -> np.ndarray:
    """out [R, H, Dl] float64."""
    q = _c(q, np.uint16)
    kv_cache = _c(kv_cache, np.uint8)
    block_tables = _c(block_tables, np.int32)
    seq_lens = _c(seq_lens, np.int32)
    sel = _c(sel, np.int32)
    R, H, Dl = q.shape
    num_pages, ps, Dl2 = kv_cache.shape
    assert Dl2 == Dl
    top_k = sel.shape[1]
    out = np.zeros((R, H, Dl), dtype=np.float64)
    rc = _load().oracle_mla_decode(R, rows_per_seq, H, Dl, _p(q), _p(kv_cache), num_pages, ps,
                                   _p(block_tables), block_tables.shape[1], _p(seq_lens),
                                   _p(sel), top_k, float(kv_scale), float(sm_scale), _p(out))
    _check(rc, "oracle_mla_decode")
    return out


def mla_decode_abs(q, kv_cache, block_tables, seq_lens, sel, kv_scale: float, sm_scale: float,
                   rows_per_seq: int = 1) -> np.ndarray:
    """Error scale [R, H, Dl] float64: sum_j p_j |c_j| with mla_decode's weights
    and rows (a relative rounding u of every weight or partial sum moves the
    output by at most u times this)."""
    q = _c(q, np.uint16)
    kv_cache = _c(kv_cache, np.uint8)
    block_tables = _c(block_tables, np.int32)
    seq_lens = _c(seq_lens, np.int32)
    sel = _c(sel, np.int32)
    R, H, Dl = q.shape
    num_pages, ps, _ = kv_cache.shape
    top_k = sel.shape[1]
    out = np.zeros((R, H, Dl), dtype=np.float64)
    rc = _load().oracle_mla_decode_abs(R, rows_per_seq, H, Dl, _p(q), _p(kv_cache), num_pages, ps,
                                       _p(block_tables), block_tables.shape[1], _p(seq_lens),
                                       _p(sel), top_k, float(kv_scale), float(sm_scale), _p(out))
    _check(rc, "oracle_mla_decode_abs")
    return out


def softmax_weights(q, kv_cache, block_tables, seq_lens, sel, kv_scale: float,
                    sm_scale: float, r: int, h: int, rows_per_seq: int = 1) -> np.ndarray:
    q = _c(q, np.uint16)
    kv_cache = _c(kv_cache, np.uint8)
    block_tables = _c(block_tables, np.int32)
    seq_lens = _c(seq_lens, np.int32)
    sel = _c(sel, np.int32)
    R, H, Dl = q.shape
    num_pages, ps, _ = kv_cache.shape
    top_k = sel.shape[1]
    n = min(top_k, int(seq_lens[r]))
    p = np.zeros(max(n, 1), dtype=np.float64)
    rc = _load().oracle_softmax_weights(rows_per_seq, H, Dl, r, h, _p(q), _p(kv_cache),
                                        num_pages, ps, _p(block_tables), block_tables.shape[1],
                                        _p(seq_lens), _p(sel), top_k, float(kv_scale),
                                        float(sm_scale), _p(p))
    _check(rc, "oracle_softmax_weights")
    return p[:n]


def e4m3_encode(y: float) -> int:
    return int(_load().oracle_e4m3fn_encode(float(y)))


def bf16_encode(y: float) -> int:
    return int(_load().oracle_bf16_encode(float(y)))


def _bf16_values(a) -> np.ndarray:
    """bf16 codes (uint16) to float64 by the definition (the upper half of an fp32)."""
    a = np.asarray(a, dtype=np.uint16)
    f = (a.astype(np.uint32) << 16).view(np.float32)
    return f.astype(np.float64)


def latent_row(x, w, eps: float, kv_scale: float):
    """(y float64 [n], codes uint8 [n]) of one latent row; x, w real values."""
    x = _c(x, np.float64)
    w = _c(w, np.float64)
    y = np.empty_like(x)
    code = np.empty(x.shape[0], dtype=np.uint8)
    _check(_load().oracle_latent_row(x.shape[0], _p(x), _p(w), eps, 1.0 / kv_scale, _p(y),
                                     _p(code)), "oracle_latent_row")
    return y, code


def layernorm_row(x, w, b, eps: float):
    """(y float64 [n], bf16 codes uint16 [n]) of one indexer key row."""
    x = _c(x, np.float64)
    w = _c(w, np.float64)
    b = _c(b, np.float64)
    y = np.empty_like(x)
    code = np.empty(x.shape[0], dtype=np.uint16)
    _check(_load().oracle_layernorm_row(x.shape[0], _p(x), _p(w), _p(b), eps, _p(y), _p(code)),
           "oracle_layernorm_row")
    return y, code


def cache_write(kv_a, latent_w, k_proj, k_w, k_b, seq_lens, block_tables, rows_per_seq: int,
                page_size: int, eps: float, kv_scale: float, kv_cache, k_normed, valid=None):
    """The cache-write step on copies of the caches. kv_a [R,Dl], latent_w [Dl],
    k_proj [R,D], k_w [D], k_b [D] are bf16 codes; kv_cache [pages,ps,Dl] uint8;
    k_normed [S,cap,D] bf16 codes; valid [S,cap] uint8 marks or None. Returns
    (kv_cache', k_normed'), and valid' third when valid is given."""
    kv = _c(_bf16_values(kv_a), np.float64)
    lw = _c(_bf16_values(latent_w), np.float64)
    kp = _c(_bf16_values(k_proj), np.float64)
    kw = _c(_bf16_values(k_w), np.float64)
    kb = _c(_bf16_values(k_b), np.float64)
    seq_lens = _c(seq_lens, np.int32)
    bt = _c(block_tables, np.int32)
    cache = np.array(kv_cache, dtype=np.uint8, copy=True, order="C")
    keys = np.array(k_normed, dtype=np.uint16, copy=True, order="C")
    marks = None if valid is None else np.array(valid, dtype=np.uint8, copy=True, order="C")
    if marks is not None and marks.shape != keys.shape[:2]:
        raise ValueError("valid must be [S, k_capacity]")
    R, Dl = kv.shape
    D = kp.shape[1]
    rc = _load().oracle_cache_write(R, rows_per_seq, Dl, D, _p(kv), _p(lw), _p(kp), _p(kw),
                                    _p(kb), _p(seq_lens), _p(bt), bt.shape[1], page_size,
                                    cache.shape[0], keys.shape[1], eps, kv_scale, _p(cache),
                                    _p(keys), None if marks is None else _p(marks))
    _check(rc, "oracle_cache_write")
    return (cache, keys) if marks is None else (cache, keys, marks)


def decode(inputs: dict, rows=None):
    """End to end on the oracle alone: its own scores, its own selection, its
    own attention. `rows` restricts the work to a subset of rows (all of a
    row's inputs are sliced; sequences are looked up through r // K)."""
    K = inputs["rows_per_seq"]
    R = inputs["seq_lens"].shape[0]
    rows = list(range(R)) if rows is None else list(rows)
    out_scores, out_sel, out_att = [], [], []
    for r in rows:
        s = r // K
        sl = inputs["seq_lens"][r:r + 1]
        sc = index_scores(inputs["q_idx"][r:r + 1], inputs["w"][r:r + 1],
                          inputs["k_normed"][s:s + 1], sl, 1, int(sl[0]))
        se = topk(sc, sl, inputs["top_k"])
        at = mla_decode(inputs["q"][r:r + 1], inputs["kv_cache"],
                        inputs["block_tables"][s:s + 1], sl, se,
                        inputs["kv_scale"], inputs["sm_scale"], 1)
        out_scores.append(sc[0])
        out_sel.append(se[0])
        out_att.append(at[0])
    return out_scores, np.stack(out_sel), np.stack(out_att)
