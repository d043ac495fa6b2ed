"""CPU oracle for MoE expert-parallel dispatch/combine -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it.

The arithmetic lives in ``ep_oracle.c`` (plain single-threaded C, IEEE fp32
in the written order, no fast-math); this module only marshals numpy arrays
to it.  ``page_sim`` restates the DeepEP page's routing simulation in numpy.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ep_oracle.c")
_LIB = os.path.join(_HERE, "libep_oracle.so")

ERR_BAD_INDEX = 1
ERR_DUP_INDEX = 2


def build() -> str:
    """Compile the oracle with gcc (no fast-math, no fp contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-Wall", "-shared",
           "-fPIC", _SRC, "-o", _LIB + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    """The oracle library; EP_ORACLE_LIB names another build of ep_oracle.c
    (the pin tests' mutation check loads deliberately broken copies)."""
    global _lib
    if _lib is None:
        path = os.environ.get("EP_ORACLE_LIB")
        if not path:
            path = _LIB
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
        _lib = ctypes.CDLL(path)
        _declare(_lib)
    return _lib


_P = ctypes.c_void_p
_I = ctypes.c_int
_L = ctypes.c_int64


def _declare(l):
    l.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
    l.orc_bf16_to_f32.restype = ctypes.c_float
    l.orc_f32_to_bf16.argtypes = [ctypes.c_float]
    l.orc_f32_to_bf16.restype = ctypes.c_uint16
    l.orc_e4m3_value.argtypes = [_I]
    l.orc_e4m3_value.restype = ctypes.c_double
    l.orc_e4m3_encode.argtypes = [ctypes.c_float]
    l.orc_e4m3_encode.restype = ctypes.c_uint8
    l.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
    l.orc_e4m3_decode.restype = ctypes.c_float
    l.orc_route.argtypes = [_P, _L, _I, _I, _I, _I, _P]
    l.orc_route.restype = _I
    l.orc_layout_ll.argtypes = [_P, _I, _I, _I, _I, _I, _P, _P, _P]
    l.orc_layout_ll.restype = _I
    l.orc_layout_ht.argtypes = [_P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P]
    l.orc_layout_ht.restype = _I
    l.orc_quantize_row.argtypes = [_P, _I, _P, _P]
    l.orc_quantize_row.restype = None
    l.orc_token_row.argtypes = [_P, _I, _I, _P]
    l.orc_token_row.restype = None
    l.orc_pack_ll.argtypes = [_P, _L, _I, _I, _I, _I, _P, _L, _P]
    l.orc_pack_ll.restype = None
    l.orc_pack_ht.argtypes = [_P, _P, _P, _L, _L, _I, _I, _I, _I, _I, _P, _P,
                              _P, _P, _P, _P, _P, _P, _P, _P, _P]
    l.orc_pack_ht.restype = None
    l.orc_dequant_rows.argtypes = [_P, _L, _L, _I, _I, _P]
    l.orc_dequant_rows.restype = None
    l.orc_combine.argtypes = [_P, _L, _P, _P, _I, _I, _P, _L, _P]
    l.orc_combine.restype = None
    l.orc_combine_backward.argtypes = [_P, _P, _L, _P, _P, _L, _I, _I, _P, _P, _P]
    l.orc_combine_backward.restype = None
    l.orc_layout_ht_rank.argtypes = [_P, _I, _I, _I, _I, _I, _P, _P, _P, _P]
    l.orc_layout_ht_rank.restype = _I
    l.orc_meta_ht_rank.argtypes = [_P, _P, _L, _I, _I, _I, _P, _P, _P]
    l.orc_meta_ht_rank.restype = None
    l.orc_f32_to_bf16_n.argtypes = [_P, _L, _P]
    l.orc_f32_to_bf16_n.restype = None
    l.orc_e4m3_encode_n.argtypes = [_P, _L, _P]
    l.orc_e4m3_encode_n.restype = None


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------------------
# Scalar formats
# ---------------------------------------------------------------------------

def bf16_to_f32(bits: int) -> float:
    return lib().orc_bf16_to_f32(bits)


def f32_to_bf16(x: float) -> int:
    return lib().orc_f32_to_bf16(x)


def f32_to_bf16_array(x: np.ndarray) -> np.ndarray:
    flat = _c(np.ravel(x), np.float32)
    out = np.empty(flat.shape, np.uint16)
    lib().orc_f32_to_bf16_n(_ptr(flat), flat.size, _ptr(out))
    return out.reshape(np.shape(x))


def e4m3_value(code: int) -> float:
    return lib().orc_e4m3_value(code)


def e4m3_encode(x: float) -> int:
    return lib().orc_e4m3_encode(x)


def e4m3_encode_array(x: np.ndarray) -> np.ndarray:
    flat = _c(np.ravel(x), np.float32)
    out = np.empty(flat.shape, np.uint8)
    lib().orc_e4m3_encode_n(_ptr(flat), flat.size, _ptr(out))
    return out.reshape(np.shape(x))


def e4m3_decode(q: int) -> float:
    return lib().orc_e4m3_decode(q)


# ---------------------------------------------------------------------------
# Steps of the path
# ---------------------------------------------------------------------------

def route(scores: np.ndarray, num_nodes: int, top_k: int, max_nodes: int) -> np.ndarray:
    s = _c(scores, np.float32)
    n, e = s.shape
    out = np.empty((n, top_k), dtype=np.int32)
    rc = lib().orc_route(_ptr(s), n, e, num_nodes, top_k, max_nodes, _ptr(out))
    if rc != 0:
        raise ValueError(f"orc_route rejected the configuration (rc={rc})")
    return out


def layout_ll(topk: np.ndarray, num_src: int, num_experts: int, slots: int):
    """-> (counts [E, S], slot_map [S*T, K] (global slot or -1), err bits)."""
    t = _c(topk, np.int32)
    n, k = t.shape
    T = n // num_src
    counts = np.empty((num_experts, num_src), dtype=np.int32)
    slot_map = np.empty((n, k), dtype=np.int32)
    err = np.zeros(1, dtype=np.int32)
    rc = lib().orc_layout_ll(_ptr(t), num_src, T, k, num_experts, slots,
                             _ptr(counts), _ptr(slot_map), _ptr(err))
    if rc != 0:
        raise ValueError(f"orc_layout_ll failed (rc={rc})")
    return counts, slot_map, int(err[0])


def layout_ht(topk: np.ndarray, num_src: int, num_experts: int, num_nodes: int,
              ranks_per_node: int):
    """-> dict(c1, off1, node_row [S*T, N], c2, off2, row2 [S*T, K], err)."""
    t = _c(topk, np.int32)
    n, k = t.shape
    T = n // num_src
    R = num_nodes * ranks_per_node
    c1 = np.empty(R, np.int32); off1 = np.empty(R, np.int32)
    c2 = np.empty(num_experts, np.int32); off2 = np.empty(num_experts, np.int32)
    node_row = np.empty((n, num_nodes), np.int32)
    row2 = np.empty((n, k), np.int32)
    err = np.zeros(1, dtype=np.int32)
    rc = lib().orc_layout_ht(_ptr(t), num_src, T, k, num_experts, num_nodes,
                             ranks_per_node, _ptr(c1), _ptr(off1), _ptr(node_row),
                             _ptr(c2), _ptr(off2), _ptr(row2), _ptr(err))
    if rc != 0:
        raise ValueError(f"orc_layout_ht failed (rc={rc})")
    return dict(c1=c1, off1=off1, node_row=node_row, c2=c2, off2=off2,
                row2=row2, err=int(err[0]))


def quantize_rows(x_bits: np.ndarray):
    """bf16 bits [n, H] -> (codes uint8 [n, H], scales float32 [n, H/128])."""
    x = _c(x_bits, np.uint16)
    n, H = x.shape
    q = np.empty((n, H), np.uint8)
    sc = np.empty((n, H // 128), np.float32)
    f = lib().orc_quantize_row
    for i in range(n):
        f(_ptr(x[i]), H, _ptr(q[i]), _ptr(sc[i]))
    return q, sc


def row_bytes(hidden: int, fp8: bool) -> int:
    return hidden + hidden // 128 * 4 if fp8 else hidden * 2


def token_rows(x_bits: np.ndarray, fp8: bool) -> np.ndarray:
    """The packed row image of each token: uint8 [n, row_bytes]."""
    x = _c(x_bits, np.uint16)
    n, H = x.shape
    out = np.empty((n, row_bytes(H, fp8)), np.uint8)
    f = lib().orc_token_row
    for i in range(n):
        f(_ptr(x[i]), H, int(fp8), _ptr(out[i]))
    return out


def pack_ll(x_bits: np.ndarray, tokens_per_src: int, top_k: int, fp8: bool,
            slot_map: np.ndarray, n_slots_total: int) -> np.ndarray:
    x = _c(x_bits, np.uint16)
    n, H = x.shape
    msg = row_bytes(H, fp8) + 16
    buf = np.zeros((n_slots_total, msg), np.uint8)
    lib().orc_pack_ll(_ptr(x), n, tokens_per_src, H, top_k, int(fp8),
                      _ptr(_c(slot_map, np.int32)), msg, _ptr(buf))
    return buf


def pack_ht(x_bits, topk, weights, tokens_per_src, num_nodes, fp8, node_row, row2,
            rows1, rows2, with_payload=True, out=None, first_token=0):
    """HT stage-1/stage-2 rows and metadata.  With with_payload=False only the
    metadata is produced and x_bits may be any [*, H] array (unused).

    With `out` (a dict as returned by a previous call) the rows of the given
    tokens are written into it, the tokens being tokens first_token ... of
    the batch (x_bits, topk, weights, node_row and row2 hold just those), so
    that disjoint token ranges can be packed into one set of rows."""
    x = _c(x_bits, np.uint16)
    H = x.shape[1]
    n, K = topk.shape
    if with_payload and x.shape[0] != n:
        raise ValueError("x must hold every token when payload rows are produced")
    rb = row_bytes(H, fp8)
    if out is None:
        out = dict(
            stage1=np.zeros((rows1, rb), np.uint8) if with_payload else None,
            meta1_tok=np.zeros(rows1, np.int32), meta1_src=np.zeros(rows1, np.int32),
            meta1_topk=np.zeros((rows1, K), np.int32), meta1_w=np.zeros((rows1, K), np.float32),
            stage2=np.zeros((rows2, rb), np.uint8) if with_payload else None,
            meta2_src=np.zeros(rows2, np.int32), meta2_tok=np.zeros(rows2, np.int32),
            meta2_k=np.zeros(rows2, np.int32))
    w = None if weights is None else _c(weights, np.float32)
    lib().orc_pack_ht(_ptr(x), _ptr(_c(topk, np.int32)), _ptr(w), first_token, n, tokens_per_src,
                      H, K, num_nodes, int(fp8), _ptr(_c(node_row, np.int32)),
                      _ptr(_c(row2, np.int32)), _ptr(out["stage1"]), _ptr(out["meta1_tok"]),
                      _ptr(out["meta1_src"]), _ptr(out["meta1_topk"]), _ptr(out["meta1_w"]),
                      _ptr(out["stage2"]), _ptr(out["meta2_src"]), _ptr(out["meta2_tok"]),
                      _ptr(out["meta2_k"]))
    return out


def dequant_rows(rows: np.ndarray, hidden: int, fp8: bool) -> np.ndarray:
    """Identity expert: packed rows uint8 [n, stride] -> bf16 bits [n, hidden]."""
    r = _c(rows, np.uint8)
    n, stride = r.shape
    y = np.empty((n, hidden), np.uint16)
    lib().orc_dequant_rows(_ptr(r), stride, n, hidden, int(fp8), _ptr(y))
    return y


def combine(Y_bits: np.ndarray, weights: np.ndarray, loc: np.ndarray,
            which: np.ndarray | None = None) -> np.ndarray:
    """bf16 bits Y [rows, H], w [n, K] f32, loc [n, K] -> bf16 bits [len(which) or n, H]."""
    Y = _c(Y_bits, np.uint16)
    H = Y.shape[1]
    w = _c(weights, np.float32)
    lc = _c(loc, np.int32)
    n, K = lc.shape
    wh = None if which is None else _c(which, np.int64)
    n_out = n if wh is None else len(wh)
    out = np.empty((n_out, H), np.uint16)
    lib().orc_combine(_ptr(Y), H, _ptr(w), _ptr(lc), K, H, _ptr(wh), n_out, _ptr(out))
    return out


def combine_backward(g_bits: np.ndarray, weights: np.ndarray, loc: np.ndarray, rows: int,
                     Y_bits: np.ndarray | None = None):
    """Adjoint of combine.  g bf16 bits [n, H], w f32 [n, K], loc [n, K], Y bf16
    bits [rows, H] or None -> (dY bf16 bits [rows, H] (rows no entry points
    at stay 0), dw f64 [n, K] (zeros without Y), sum |g*Y| f64 [n, K])."""
    g = _c(g_bits, np.uint16)
    n, H = g.shape
    w = _c(weights, np.float32)
    lc = _c(loc, np.int32)
    K = lc.shape[1]
    Y = None if Y_bits is None else _c(Y_bits, np.uint16)
    if Y is not None and Y.shape != (rows, H):
        raise ValueError("Y must be [rows, H]")
    dY = np.zeros((rows, H), np.uint16)
    dw = np.zeros((n, K), np.float64)
    da = np.zeros((n, K), np.float64)
    lib().orc_combine_backward(_ptr(g), _ptr(Y), H, _ptr(w), _ptr(lc), n, K, H, _ptr(dY),
                               _ptr(dw), _ptr(da))
    return dY, dw, da


def dispatch_backward(dRows_bits: np.ndarray, loc: np.ndarray) -> np.ndarray:
    """Adjoint of dispatch (straight-through FP8): dx[t] = bf16 of the fp32
    sum over valid k, in k order, of dRows[loc(t,k)] -- combine with unit
    weights."""
    return combine(dRows_bits, np.ones(loc.shape, np.float32), loc)


def layout_ht_rank(topk: np.ndarray, num_src: int, num_experts: int, num_ranks: int):
    """Stage 2 with one row per (token, destination rank) -> dict(c2 [R],
    off2 [R], row2 [S*T, K] (row at the token's first entry on each rank,
    -1 elsewhere), err)."""
    t = _c(topk, np.int32)
    n, k = t.shape
    T = n // num_src
    c2 = np.empty(num_ranks, np.int32)
    off2 = np.empty(num_ranks, np.int32)
    row2 = np.empty((n, k), np.int32)
    err = np.zeros(1, np.int32)
    rc = lib().orc_layout_ht_rank(_ptr(t), num_src, T, k, num_experts, num_ranks, _ptr(c2),
                                  _ptr(off2), _ptr(row2), _ptr(err))
    if rc != 0:
        raise ValueError(f"orc_layout_ht_rank failed (rc={rc})")
    return dict(c2=c2, off2=off2, row2=row2, err=int(err[0]))


def meta_ht_rank(topk: np.ndarray, weights, row2: np.ndarray, num_experts: int, num_ranks: int,
                 rows: int):
    """Per-rank stage-2 received top-k: (local expert ids or -1 [rows, K],
    weights or 0 [rows, K])."""
    t = _c(topk, np.int32)
    n, K = t.shape
    mt = np.full((rows, K), -7, np.int32)
    mw = np.full((rows, K), -7.0, np.float32)
    w = None if weights is None else _c(weights, np.float32)
    lib().orc_meta_ht_rank(_ptr(t), _ptr(w), n, K, num_experts, num_ranks, _ptr(_c(row2, np.int32)),
                           _ptr(mt), _ptr(mw) if w is not None else None)
    return mt, mw

