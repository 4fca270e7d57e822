"""The benchmark's byte accounting (CPU): algorithmic bytes per call are each
input element read once and each output element written once, with the small
vectors counted once.  Per token at hidden 5120 (bf16 storage): AdaLN reads x
and writes y (2 x 5120 x 2 = 20,480 B), the gated residual reads x and h and
writes x (30,720 B), SwiGLU reads a and b and writes out (3 x 13,824 x 2 =
82,944 B), QK reads q, k and writes q', k' (4 x 40 x 128 x 2 = 40,960 B)."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

C5 = bench.GRIDS["5s"]
N5 = C5["T"] * C5["H"] * C5["W"] + C5["A"]


def test_token_counts():
    assert N5 == 125_120
    c10 = bench.GRIDS["10s"]
    assert c10["T"] * c10["H"] * c10["W"] + c10["A"] == 246_208
    for d in (3072, 4096, 5120, 6144):
        c = bench.GRIDS[f"sweep{d}"]
        assert c["T"] * c["H"] * c["W"] + c["A"] == 32_768
        assert c["heads"] == d // 128 and c["F"] % 128 == 0


@pytest.mark.parametrize("op,per_token,vectors", [
    ("adaln", 20_480, 2 * 5120 * 2),
    ("gated", 30_720, 5120 * 2),
    ("swiglu", 82_944, 0),
    ("qk", 40_960, 2 * 128 * 2),
    ("gated_adaln", 40_960, 3 * 5120 * 2),
])
def test_per_token_bytes_bf16(op, per_token, vectors):
    assert bench.op_bytes(op, N5, C5, 2) == N5 * per_token + vectors
    assert bench.op_bytes(op, 1, C5, 2) == per_token + vectors


def test_fp32_residual_stream_bytes():
    # the chain keeps x in fp32: AdaLN reads 4-byte x, writes bf16 y; the gated
    # residual reads and writes fp32 x and reads bf16 h
    assert bench.op_bytes("adaln", 1, C5, 4) == 5120 * 4 + 5120 * 2 + 2 * 5120 * 4
    assert bench.op_bytes("gated", 1, C5, 4) == 2 * 5120 * 4 + 5120 * 2 + 5120 * 4


def test_step_bytes_match_the_block():
    # one block's six calls at the 5 s shape: 28.3 GB
    step = sum(bench.op_bytes(o, N5, C5, 2)
               for o in ("adaln", "qk", "gated", "adaln", "swiglu", "gated"))
    assert abs(step / 1e9 - 28.32) < 0.01


def test_router_bytes():
    nb, keep = 978, 196
    b = bench.router_bytes(N5, C5, nb, keep)
    assert b == 2 * N5 * 40 * 128 * 2 + 40 * nb * nb * 4 + 40 * nb * keep * 4


def test_more_than_one_gpu_is_refused():
    import subprocess

    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr


@pytest.mark.parametrize("op,per_token,vectors", [
    ("adaln", 2 * 256 * 4, 2 * 256 * 4),
    ("gated", 3 * 256 * 4, 256 * 4),
    ("swiglu", 3 * 512 * 4, 0),
    ("qk", 4 * 4 * 64 * 4, 2 * 64 * 4),
    ("gated_adaln", 4 * 256 * 4, 3 * 256 * 4),
])
def test_per_token_bytes_tiny_fp32(op, per_token, vectors):
    # the tiny configuration: 112 tokens, hidden 256, 4 x 64 heads, SwiGLU inner
    # 512, every tensor fp32
    n = bench.n_tokens(bench.TINY)
    assert n == 2 * 6 * 8 + 16 == 112
    assert bench.op_bytes(op, n, bench.TINY, 4, 4) == n * per_token + vectors
