"""Helpers for the GPU parity tests: seeded device tensors, their host twins,
and conversions between torch GPU tensors and the oracle's numpy arrays."""
import numpy as np
import torch

import h3gen

DEV = torch.device("cuda:0")


def npdt(dtype):
    return {"bf16": np.uint16, "f32": np.float32}[dtype]


def tdt(dtype):
    return {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]


def dev_tensor(name, rows, cols, dtype, seed=0, row_stride=None, mu=None, sigma=None):
    """[rows, cols] GPU tensor holding logical tensor `name`; with row_stride the
    result is a strided view into a wider buffer (padding filled with NaN)."""
    if row_stride is None or row_stride == cols:
        t = torch.empty(rows, cols, dtype=tdt(dtype), device=DEV)
    else:
        buf = torch.full((rows, row_stride), float("nan"), dtype=tdt(dtype), device=DEV)
        t = buf[:, :cols]
    h3gen.fill_device(t, name, seed=seed, mu=mu, sigma=sigma)
    return t


def host(name, rows, cols, dtype, seed=0, mu=None, sigma=None):
    """Host copy of rows of logical tensor `name` (rows: int or index list)."""
    return h3gen.host_rows(name, rows, cols, dtype, seed=seed, mu=mu, sigma=sigma)


def to_np(t):
    """GPU tensor -> numpy (bf16 as uint16 bit patterns)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    if t.dtype == torch.float32:
        return t.numpy().copy()
    if t.dtype == torch.int32:
        return t.numpy().copy()
    raise TypeError(t.dtype)


def from_np(a, device=DEV):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def rows_of(t, idx):
    """Selected rows of a GPU tensor (any strides) -> numpy."""
    it = torch.as_tensor(np.asarray(idx, dtype=np.int64), device=t.device)
    return to_np(t.index_select(0, it))


def sample_rows(n_rows, n_video=None, every=97, head=64, tail=64):
    """Rows 0..head-1, every `every`-th row, all audio rows, and the last `tail` rows."""
    s = set(range(min(head, n_rows)))
    s.update(range(0, n_rows, every))
    if n_video is not None:
        s.update(range(n_video, n_rows))
    s.update(range(max(0, n_rows - tail), n_rows))
    return np.array(sorted(s), dtype=np.int64)


def kind(dtype):
    return "bf16" if dtype in ("bf16", torch.bfloat16, np.uint16) else "f32"
