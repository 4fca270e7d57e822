"""Plain CPU oracle for the fused per-token DiT operators (ctypes over h3oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The GPU library and its Python binding
never import this package.

Arrays are numpy arrays, dense row-major.  bf16 data is carried as ``np.uint16``
bit patterns, fp32 as ``np.float32``.  Every function evaluates its operator in
double and rounds each output element once (see h3oracle.h for the definitions
and the passages they follow).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")
# A test may point the wrapper at a deliberately mutated build of the oracle
# (tests/test_oracle_mutations.py) to prove that the pins catch the mutation.
_LIB_OVERRIDE = os.environ.get("H3_ORACLE_LIB_OVERRIDE")
SRC = os.path.join(HERE, "h3oracle.c")

F32 = 0
BF16 = 1
PAIR_INTERLEAVED = 0
PAIR_HALF_SPLIT = 1

_lib = None


def build(verbose: bool = False) -> str:
    """Compile h3oracle.c with gcc into liboracle.so (always recompiles)."""
    cmd = [
        "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
        "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
        "-o", LIB_PATH + ".tmp", SRC, "-lm",
    ]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        path = _LIB_OVERRIDE or LIB_PATH
        if not _LIB_OVERRIDE and not os.path.exists(LIB_PATH):
            build()
        _lib = ctypes.CDLL(path)
        _declare(_lib)
    return _lib


_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_int = ctypes.c_int
_f = ctypes.c_float
_d = ctypes.c_double


def _declare(L):
    L.oracle_abi_version.restype = _int
    L.oracle_num_threads.restype = _int
    L.oracle_set_num_threads.argtypes = [_int]
    L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
    L.oracle_bf16_to_f32.restype = _f
    L.oracle_f32_to_bf16.argtypes = [_f]
    L.oracle_f32_to_bf16.restype = ctypes.c_uint16
    L.oracle_positions.argtypes = [_p, _i64, _i64, _i32, _i32, _i32, _i32]
    L.oracle_adaln_modulate.argtypes = [_p, _int, _p, _int, _p, _p, _int, _p,
                                        _i64, _i64, _i64, _f]
    L.oracle_adaln_affine_modulate.argtypes = [_p, _int, _p, _int, _p, _p, _p, _p, _int, _p,
                                               _i64, _i64, _i64, _f]
    L.oracle_gated_residual.argtypes = [_p, _int, _p, _int, _p, _p, _i64, _i64, _i64]
    L.oracle_swiglu.argtypes = [_p, _p, _int, _i64, _i64]
    L.oracle_rope_inv_freq.argtypes = [_p, _i32, _i32, _i32, _d]
    L.oracle_qk_rmsnorm_rope3d.argtypes = [_p, _p, _p, _p, _p, _p, _int, _i64,
                                           _i32, _i32, _f, _p, _i32, _i32, _i32,
                                           _d, _int, _int]
    L.oracle_gated_residual_adaln.argtypes = [_p, _int, _p, _int, _p, _p, _int,
                                              _p, _p, _p, _i64, _i64, _i64, _f]
    L.oracle_residual_l1.argtypes = [_p, _p, _p, _int, _i64, _i64]
    L.oracle_subblock_pool.argtypes = [_p, _p, _int, _i64, _i32, _i32, _i32]
    L.oracle_subblock_scores.argtypes = [_p, _p, _p, _i32, _i64, _i64, _i32]
    L.oracle_subblock_keep.argtypes = [_i64, _d, _i32, _i32]
    L.oracle_subblock_keep.restype = _i64
    L.oracle_subblock_select.argtypes = [_p, _p, _i32, _i64, _i64, _i64]


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle arrays are float32 or uint16 (bf16 bits), got {a.dtype}")


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _groups(group, rows):
    if group is None:
        return None
    g = np.ascontiguousarray(group, dtype=np.int64)
    assert g.shape == (rows,)
    return g


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_num_threads(n: int) -> None:
    lib().oracle_set_num_threads(int(n))


# --- conversions -------------------------------------------------------------

def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_scalar(x: float) -> int:
    return int(lib().oracle_f32_to_bf16(ctypes.c_float(x)))


def to_f64(a: np.ndarray) -> np.ndarray:
    """Exact value of a float32 or bf16 array as float64."""
    if a.dtype == np.uint16:
        return bf16_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


# --- operators -----------------------------------------------------------------

def positions(rows: int, T: int, H: int, W: int, n_audio: int,
              token_offset: int = 0) -> np.ndarray:
    out = np.zeros((rows, 3), dtype=np.int32)
    lib().oracle_positions(_ptr(out), rows, token_offset, T, H, W, n_audio)
    return out


def adaln_modulate(x, shift, scale, eps=1e-6, y_dtype=None, group=None,
                   rows_per_group=None):
    """y = LN(x) * (1 + scale[g]) + shift[g]; x [rows, D]; shift/scale [G, D]."""
    x = np.ascontiguousarray(x)
    rows, D = x.shape
    shift = np.ascontiguousarray(shift).reshape(-1, D)
    scale = np.ascontiguousarray(scale).reshape(-1, D)
    assert shift.dtype == scale.dtype
    ydt = x.dtype if y_dtype is None else np.dtype(y_dtype)
    y = np.zeros((rows, D), dtype=ydt)
    g = _groups(group, rows)
    rpg = rows if rows_per_group is None else rows_per_group
    lib().oracle_adaln_modulate(_ptr(y), _dt(y), _ptr(x), _dt(x), _ptr(shift),
                                _ptr(scale), _dt(shift), _ptr(g), max(rpg, 1),
                                rows, D, eps)
    return y


def adaln_affine_modulate(x, gamma, beta, shift, scale, eps=1e-6, y_dtype=None, group=None,
                          rows_per_group=None):
    """y = (LN(x) * gamma + beta) * (1 + scale[g]) + shift[g]; gamma, beta [D]."""
    x = np.ascontiguousarray(x)
    rows, D = x.shape
    gamma = np.ascontiguousarray(gamma).reshape(D)
    beta = np.ascontiguousarray(beta).reshape(D)
    shift = np.ascontiguousarray(shift).reshape(-1, D)
    scale = np.ascontiguousarray(scale).reshape(-1, D)
    for v in (beta, shift, scale):
        assert v.dtype == gamma.dtype
    ydt = x.dtype if y_dtype is None else np.dtype(y_dtype)
    y = np.zeros((rows, D), dtype=ydt)
    g = _groups(group, rows)
    rpg = rows if rows_per_group is None else rows_per_group
    lib().oracle_adaln_affine_modulate(_ptr(y), _dt(y), _ptr(x), _dt(x), _ptr(gamma), _ptr(beta),
                                       _ptr(shift), _ptr(scale), _dt(shift), _ptr(g),
                                       max(rpg, 1), rows, D, eps)
    return y


def gated_residual(x, h, gate, group=None, rows_per_group=None):
    """Returns x + gate[g] * h (new array); gate has x's dtype."""
    x = np.array(x, copy=True, order="C")
    h = np.ascontiguousarray(h)
    rows, D = x.shape
    gate = np.ascontiguousarray(gate).reshape(-1, D)
    assert gate.dtype == x.dtype and h.shape == x.shape
    g = _groups(group, rows)
    rpg = rows if rows_per_group is None else rows_per_group
    lib().oracle_gated_residual(_ptr(x), _dt(x), _ptr(h), _dt(h), _ptr(gate),
                                _ptr(g), max(rpg, 1), rows, D)
    return x


def swiglu(gate_up):
    """gate_up [rows, 2F] -> silu(a) * b, [rows, F]."""
    gu = np.ascontiguousarray(gate_up)
    rows, twoF = gu.shape
    assert twoF % 2 == 0
    out = np.zeros((rows, twoF // 2), dtype=gu.dtype)
    lib().oracle_swiglu(_ptr(out), _ptr(gu), _dt(gu), rows, twoF // 2)
    return out


def rope_inv_freq(d_t, d_h, d_w, theta=10000.0):
    out = np.zeros(((d_t + d_h + d_w) // 2,), dtype=np.float32)
    lib().oracle_rope_inv_freq(_ptr(out), d_t, d_h, d_w, theta)
    return out


def qk_rmsnorm_rope3d(q, k, q_weight, k_weight, pos, split, eps=1e-6,
                      theta=10000.0, angle_mode=0, pairing=PAIR_INTERLEAVED):
    """q, k [rows, heads, Dh]; weights [Dh]; pos [rows, 3] int32; split (d_t, d_h, d_w)."""
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    rows, heads, Dh = q.shape
    assert k.shape == q.shape and k.dtype == q.dtype
    qw = np.ascontiguousarray(q_weight).reshape(Dh)
    kw = np.ascontiguousarray(k_weight).reshape(Dh)
    assert qw.dtype == q.dtype and kw.dtype == q.dtype
    pos = np.ascontiguousarray(pos, dtype=np.int32).reshape(rows, 3)
    d_t, d_h, d_w = split
    assert d_t + d_h + d_w == Dh
    q_out = np.zeros_like(q)
    k_out = np.zeros_like(k)
    lib().oracle_qk_rmsnorm_rope3d(_ptr(q_out), _ptr(k_out), _ptr(q), _ptr(k),
                                   _ptr(qw), _ptr(kw), _dt(q), rows, heads, Dh,
                                   eps, _ptr(pos), d_t, d_h, d_w, theta,
                                   angle_mode, pairing)
    return q_out, k_out


def gated_residual_adaln(x, h, gate, shift, scale, eps=1e-6, y_dtype=None,
                         group=None, rows_per_group=None):
    """Returns (x + gate*h, AdaLN of that); modulation vectors have x's dtype."""
    x = np.array(x, copy=True, order="C")
    h = np.ascontiguousarray(h)
    rows, D = x.shape
    gate = np.ascontiguousarray(gate).reshape(-1, D)
    shift = np.ascontiguousarray(shift).reshape(-1, D)
    scale = np.ascontiguousarray(scale).reshape(-1, D)
    for v in (gate, shift, scale):
        assert v.dtype == x.dtype
    ydt = x.dtype if y_dtype is None else np.dtype(y_dtype)
    y = np.zeros((rows, D), dtype=ydt)
    g = _groups(group, rows)
    rpg = rows if rows_per_group is None else rows_per_group
    lib().oracle_gated_residual_adaln(_ptr(x), _dt(x), _ptr(h), _dt(h),
                                      _ptr(gate), _ptr(y), _dt(y), _ptr(shift),
                                      _ptr(scale), _ptr(g), max(rpg, 1), rows,
                                      D, eps)
    return x, y


def residual_l1(cur, prev):
    """(sum |cur - prev|, sum |prev|) in double."""
    cur = np.ascontiguousarray(cur)
    prev = np.ascontiguousarray(prev)
    assert cur.shape == prev.shape and cur.dtype == prev.dtype
    rows = cur.shape[0]
    hidden = int(np.prod(cur.shape[1:])) if cur.ndim > 1 else 1
    out = np.zeros(2, dtype=np.float64)
    lib().oracle_residual_l1(_ptr(out), _ptr(cur), _ptr(prev), _dt(cur), rows, hidden)
    return float(out[0]), float(out[1])


# --- block-sparse attention router ----------------------------------------------

SUBBLOCK_FIRST_STEP = 10


def subblock_pool(x, block):
    """x [rows, heads, Dh] -> per-block means, float64 [heads, n_blocks, Dh]."""
    x = np.ascontiguousarray(x)
    rows, heads, Dh = x.shape
    nb = (rows + block - 1) // block
    out = np.zeros((heads, nb, Dh), dtype=np.float64)
    lib().oracle_subblock_pool(_ptr(out), _ptr(x), _dt(x), rows, heads, Dh, block)
    return out


def subblock_scores(pq, pk):
    """pq [heads, nbq, Dh], pk [heads, nbk, Dh] (float64) -> [heads, nbq, nbk] float64."""
    pq = np.ascontiguousarray(pq, dtype=np.float64)
    pk = np.ascontiguousarray(pk, dtype=np.float64)
    heads, nbq, Dh = pq.shape
    assert pk.shape[0] == heads and pk.shape[2] == Dh
    nbk = pk.shape[1]
    out = np.zeros((heads, nbq, nbk), dtype=np.float64)
    lib().oracle_subblock_scores(_ptr(out), _ptr(pq), _ptr(pk), heads, nbq, nbk, Dh)
    return out


def subblock_keep(n_blocks, sparsity, step, first_step=SUBBLOCK_FIRST_STEP):
    return int(lib().oracle_subblock_keep(n_blocks, float(sparsity), step, first_step))


def subblock_select(scores, keep):
    """scores [heads, nbq, nbk] -> int32 [heads, nbq, keep] kept key blocks, ascending."""
    scores = np.ascontiguousarray(scores, dtype=np.float64)
    heads, nbq, nbk = scores.shape
    assert 0 <= keep <= nbk
    out = np.zeros((heads, nbq, keep), dtype=np.int32)
    lib().oracle_subblock_select(_ptr(out), _ptr(scores), heads, nbq, nbk, keep)
    return out


def subblock_route(q, k, block, sparsity, step, first_step=SUBBLOCK_FIRST_STEP):
    """Whole router: (kv_blocks int32 [heads, nb, keep], scores float64 [heads, nb, nb])."""
    pq = subblock_pool(q, block)
    pk = subblock_pool(k, block)
    s = subblock_scores(pq, pk)
    keep = subblock_keep(pk.shape[1], sparsity, step, first_step)
    return subblock_select(s, keep), s
