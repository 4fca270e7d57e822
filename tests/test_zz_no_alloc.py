"""h3f_residual_l1_noalloc (the entry point for callers that cannot allocate)
against h3f_residual_l1 (caller workspace) and the CPU oracle: the same kernels,
so the two entry points must agree bit for bit; both must match the oracle
within the residual difference's tolerance.  Two calls in a row, the second on
a smaller input, so the second runs on scratch that still holds the first
call's partial sums; then the size limit is checked on the host."""
import ctypes

import numpy as np
import pytest
import torch

import h3gen
import oracle
from gpu_util import DEV, dev_tensor, host

pytestmark = pytest.mark.gpu

h3 = pytest.importorskip("video_diffusion_transformer_h3f_amd")

# fp32 lane sums of 64 terms, a 6-level DPP tree and two fp32 workgroup levels
# before fp64: relative error below ~72 * 2^-24 of the sum of |terms|.
L1_RTOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    h3.lib()
    h3gen.dev_lib()
    yield
    torch.cuda.synchronize()


def _pair(rows, D, dt, pad, seed):
    cur = dev_tensor("x", rows, D, dt, row_stride=D + pad, seed=seed)
    prev = dev_tensor("x_prev", rows, D, dt, row_stride=D + pad, seed=seed)
    return cur, prev


def _check(rows, D, dt, pad, seed):
    print(f"noalloc case rows={rows} D={D} {dt} pad={pad} seed={seed}", flush=True)
    cur, prev = _pair(rows, D, dt, pad, seed)
    ref = torch.full((3,), -1.0, dtype=torch.float64, device=DEV)
    got = torch.full((3,), -2.0, dtype=torch.float64, device=DEV)
    h3.h3f_residual_l1(ref, cur, prev)
    h3.h3f_residual_l1_noalloc(got, cur, prev)
    torch.cuda.synchronize()
    assert torch.equal(got, ref), (got, ref)  # same kernels, same partition: bit-identical
    num, den = oracle.residual_l1(host("x", rows, D, dt, seed=seed),
                                  host("x_prev", rows, D, dt, seed=seed))
    g = got.cpu().numpy()
    assert abs(g[0] - num) <= L1_RTOL * num
    assert abs(g[1] - den) <= L1_RTOL * den
    assert abs(g[2] - num / den) <= 2 * L1_RTOL * (num / den)


@pytest.mark.parametrize("first,second", [
    # the 5 s token shape (39,100 partial pairs), then a ragged smaller one
    ((125120, 5120, "bf16", 0, 0), (1001, 5120, "bf16", 0, 1)),
    # fp32 with padded rows, then a tiny input that fills one partial pair
    ((4099, 1000, "f32", 12, 2), (3, 8, "f32", 0, 3)),
])
def test_noalloc_matches_workspace_entry(first, second):
    _check(*first)
    _check(*second)


def test_noalloc_through_c_abi_and_limit():
    L = h3.lib()
    cap = L.h3f_residual_l1_noalloc_max_bytes()
    assert cap == 4 << 20
    # the largest bf16 hidden-5120 row count that fits, and one beyond it
    rows_fit = 838860
    assert L.h3f_residual_l1_workspace_bytes(rows_fit, 5120, h3.H3F_BF16) <= cap
    assert L.h3f_residual_l1_workspace_bytes(rows_fit + 1, 5120, h3.H3F_BF16) > cap
    # a row count past the scratch is rejected on the host before any launch;
    # the pointers are far-apart addresses that validation never dereferences
    P = ctypes.c_void_p
    st = L.h3f_residual_l1_noalloc(P(0x1000), P(1 << 40), 5120, P(2 << 40), 5120, h3.H3F_BF16,
                                   rows_fit + 1, 5120, None)
    assert h3.STATUS[st] == "H3F_ERR_WORKSPACE"
    out = torch.zeros(3, dtype=torch.float64, device=DEV)
    cur, prev = _pair(64, 5120, "bf16", 0, 4)
    # and the same call at its real size goes through the C ABI on the null stream
    st = L.h3f_residual_l1_noalloc(ctypes.c_void_p(out.data_ptr()),
                                   ctypes.c_void_p(cur.data_ptr()), 5120,
                                   ctypes.c_void_p(prev.data_ptr()), 5120, h3.H3F_BF16, 64,
                                   5120, None)
    assert st == 0
    torch.cuda.synchronize()
    num, den = oracle.residual_l1(host("x", 64, 5120, "bf16", seed=4),
                                  host("x_prev", 64, 5120, "bf16", seed=4))
    g = out.cpu().numpy()
    assert abs(g[0] - num) <= L1_RTOL * num and abs(g[1] - den) <= L1_RTOL * den


def test_noalloc_captured_in_a_graph():
    # the callers this entry point is for: a captured graph replayed with eager work
    # (including another no-allocation call, on the same scratch, ordered on the
    # stream) between the replays; every replay equals the eager result bit for bit
    cur, prev = _pair(30001, 5120, "bf16", 0, 5)
    other_c, other_p = _pair(777, 3072, "bf16", 0, 6)
    want = torch.zeros(3, dtype=torch.float64, device=DEV)
    h3.h3f_residual_l1_noalloc(want, cur, prev)  # eager first: the device address is looked up
    out = torch.zeros(3, dtype=torch.float64, device=DEV)
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        h3.h3f_residual_l1_noalloc(out, cur, prev)
    torch.cuda.synchronize()
    side = torch.zeros(3, dtype=torch.float64, device=DEV)
    side_ref = torch.zeros(3, dtype=torch.float64, device=DEV)
    h3.h3f_residual_l1(side_ref, other_c, other_p)
    for rep in range(4):
        out.fill_(-1.0)
        g.replay()
        h3.h3f_residual_l1_noalloc(side, other_c, other_p)  # same scratch, after the replay
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {rep}"
        assert torch.equal(side, side_ref), f"eager call after replay {rep}"
    # the graph holds pointers: new contents are followed
    prev.mul_(0.5)
    want2 = torch.zeros(3, dtype=torch.float64, device=DEV)
    h3.h3f_residual_l1(want2, cur, prev)
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, want2) and not torch.equal(want2, want)
