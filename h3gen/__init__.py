"""Seeded counter-based input generator shared by the tests, the oracle checks
and the benchmark (host: h3gen_host.c via gcc; device: h3gen_device.hip via
hipcc).  It holds none of the operators' arithmetic: it only produces the
synthetic inputs, bit-identically on host and device (see h3gen_core.h).

Values are N(mu, sigma)-like (Irwin-Hall of 12 uniforms, bounded at +-6 sigma).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(HERE, "libh3gen_host.so")
DEV_LIB = os.path.join(HERE, "libh3gen_dev.so")

F32 = 0
BF16 = 1

# Fixed tensor ids: the same logical tensor always draws the same stream.
TENSOR_IDS = {
    "x": 1, "shift": 2, "scale": 3, "gate": 4, "h": 5, "gate_up": 6,
    "q": 7, "k": 8, "v": 9, "q_weight": 10, "k_weight": 11,
    "shift2": 12, "scale2": 13, "gate2": 14, "h2": 15, "x_prev": 16,
    "ln_gamma": 17, "ln_beta": 18,
}

# Value distributions of the synthetic workload (mean, standard deviation).
DISTRIBUTIONS = {
    "x": (0.0, 1.0), "h": (0.0, 1.0), "h2": (0.0, 1.0), "gate_up": (0.0, 1.0),
    "q": (0.0, 1.0), "k": (0.0, 1.0), "v": (0.0, 1.0), "x_prev": (0.0, 1.0),
    "shift": (0.0, 0.1), "scale": (0.0, 0.1), "shift2": (0.0, 0.1), "scale2": (0.0, 0.1),
    "gate": (0.0, 0.5), "gate2": (0.0, 0.5),
    "q_weight": (1.0, 0.05), "k_weight": (1.0, 0.05),
    "ln_gamma": (1.0, 0.05), "ln_beta": (0.0, 0.1),
}

_host = None
_dev = None


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)


def build_host(verbose: bool = False) -> str:
    _run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-Wall", "-o", HOST_LIB + ".tmp", os.path.join(HERE, "h3gen_host.c")], verbose)
    os.replace(HOST_LIB + ".tmp", HOST_LIB)
    return HOST_LIB


def build_device(verbose: bool = False, hipcc: str = "/opt/rocm/bin/hipcc") -> str:
    _run([hipcc, "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
          "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-o", DEV_LIB + ".tmp", os.path.join(HERE, "h3gen_device.hip")], verbose)
    os.replace(DEV_LIB + ".tmp", DEV_LIB)
    return DEV_LIB


def host_lib():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            build_host()
        L = ctypes.CDLL(HOST_LIB)
        L.h3gen_fill_host.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                      ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_uint64, ctypes.c_uint64, ctypes.c_float,
                                      ctypes.c_float]
        L.h3gen_fill_rows_host.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                           ctypes.c_int64, ctypes.c_int64, ctypes.c_uint64,
                                           ctypes.c_uint64, ctypes.c_float, ctypes.c_float]
        L.h3gen_fill_cols_host.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                           ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                           ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint64,
                                           ctypes.c_float, ctypes.c_float]
        _host = L
    return _host


def dev_lib():
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_LIB):
            raise RuntimeError(f"device generator not built: {DEV_LIB} (run __graft_entry__.build())")
        L = ctypes.CDLL(DEV_LIB)
        L.h3gen_fill_device.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_uint64, ctypes.c_uint64, ctypes.c_float,
                                        ctypes.c_float, ctypes.c_void_p]
        L.h3gen_fill_device.restype = ctypes.c_int
        _dev = L
    return _dev


def _dist(name, mu, sigma):
    if mu is None or sigma is None:
        m, s = DISTRIBUTIONS[name]
        mu = m if mu is None else mu
        sigma = s if sigma is None else sigma
    return float(mu), float(sigma)


def host_rows(name: str, rows, cols: int, dtype: str = "bf16", seed: int = 0,
              mu=None, sigma=None) -> np.ndarray:
    """Rows of logical tensor `name` ([*, cols]) as a dense numpy array.

    rows: an int n (rows 0..n-1) or a sequence of global row indices.
    dtype 'bf16' -> uint16 bit patterns, 'f32' -> float32.
    """
    mu, sigma = _dist(name, mu, sigma)
    dt = BF16 if dtype == "bf16" else F32
    npdt = np.uint16 if dt == BF16 else np.float32
    tid = TENSOR_IDS[name]
    if isinstance(rows, (int, np.integer)):
        out = np.empty((int(rows), cols), dtype=npdt)
        host_lib().h3gen_fill_host(out.ctypes.data_as(ctypes.c_void_p), dt, 0, int(rows), cols,
                                   cols, seed, tid, mu, sigma)
        return out
    ids = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    out = np.empty((ids.shape[0], cols), dtype=npdt)
    host_lib().h3gen_fill_rows_host(out.ctypes.data_as(ctypes.c_void_p), dt,
                                    ids.ctypes.data_as(ctypes.c_void_p), ids.shape[0], cols,
                                    seed, tid, mu, sigma)
    return out


def host_cols(name: str, rows: int, cols: int, col0: int, ncols: int, dtype: str = "bf16",
              seed: int = 0, mu=None, sigma=None) -> np.ndarray:
    """Columns [col0, col0 + ncols) of rows 0..rows-1 of logical tensor `name`
    ([*, cols]) as a dense [rows, ncols] numpy array."""
    mu, sigma = _dist(name, mu, sigma)
    dt = BF16 if dtype == "bf16" else F32
    out = np.empty((int(rows), int(ncols)), dtype=np.uint16 if dt == BF16 else np.float32)
    host_lib().h3gen_fill_cols_host(out.ctypes.data_as(ctypes.c_void_p), dt, 0, int(rows), cols,
                                    col0, ncols, seed, TENSOR_IDS[name], mu, sigma)
    return out


def fill_device(t, name: str, seed: int = 0, mu=None, sigma=None, row0: int = 0) -> None:
    """Fill a 2-D torch tensor view t ([rows, cols], unit inner stride, any row
    stride) on its device with logical tensor `name` starting at row row0."""
    import torch  # device memory only

    mu, sigma = _dist(name, mu, sigma)
    assert t.dim() == 2 and t.stride(1) == 1, "fill_device wants a 2-D view with unit inner stride"
    if t.dtype == torch.bfloat16:
        dt = BF16
    elif t.dtype == torch.float32:
        dt = F32
    else:
        raise TypeError(t.dtype)
    stream = torch.cuda.current_stream(t.device).cuda_stream
    rc = dev_lib().h3gen_fill_device(ctypes.c_void_p(t.data_ptr()), dt, row0, t.shape[0],
                                     t.shape[1], t.stride(0), seed, TENSOR_IDS[name], mu, sigma,
                                     ctypes.c_void_p(stream))
    if rc != 0:
        raise RuntimeError(f"h3gen_fill_device failed with hip error {rc}")
