"""The Python binding rejects arguments the C ABI cannot check for itself -- the
modulation group count against the rows, the modulation and weight dtypes, and
the explicit RoPE positions array -- before it calls into the library.

Runs on the CPU: the device check is replaced by a stub and the library loader
by one that fails, so a check that let the call through would show up as that
failure instead of the expected error."""
import pytest
import torch

import video_diffusion_transformer_h3f_amd as h3


@pytest.fixture
def no_launch(monkeypatch):
    def _fake_dev(*ts):
        return torch.device("cpu")

    def _no_lib():
        raise AssertionError("the library was reached")

    monkeypatch.setattr(h3, "_dev", _fake_dev)
    monkeypatch.setattr(h3, "lib", _no_lib)


R, D = 10, 64
f32, bf16 = torch.float32, torch.bfloat16


def t(*shape, dtype=f32):
    return torch.zeros(*shape, dtype=dtype)


def test_adaln_group_count(no_launch):
    x, y = t(R, D), t(R, D)
    # one group per row needs R groups; the tensors hold one
    with pytest.raises(ValueError, match="modulation groups"):
        h3.h3f_adaln_modulate(y, x, t(D), t(D), rows_per_group=1)
    # 2 groups at 4 rows per group cover 8 of 10 rows
    with pytest.raises(ValueError, match="modulation groups"):
        h3.h3f_adaln_modulate(y, x, t(2, D), t(2, D), rows_per_group=4)
    with pytest.raises(ValueError, match=">= 1"):
        h3.h3f_adaln_modulate(y, x, t(2, D), t(2, D), rows_per_group=0)


def test_adaln_mod_dtype(no_launch):
    # fp32 residual stream with bf16 modulation: the kernel would read fp32 from bf16 buffers
    x, y = t(R, D), t(R, D, dtype=bf16)
    with pytest.raises(TypeError, match="shift"):
        h3.h3f_adaln_modulate(y, x, t(D, dtype=bf16), t(D, dtype=bf16))
    with pytest.raises(TypeError, match="scale"):
        h3.h3f_adaln_modulate(y, x, t(D), t(D, dtype=bf16))


def test_affine_checks(no_launch):
    x, y = t(R, D), t(R, D)
    with pytest.raises(TypeError, match="gamma"):
        h3.h3f_adaln_affine_modulate(y, x, t(D, dtype=bf16), t(D), t(D), t(D))
    with pytest.raises(ValueError, match="modulation groups"):
        h3.h3f_adaln_affine_modulate(y, x, t(D), t(D), t(3, D), t(3, D), rows_per_group=3)


def test_gated_checks(no_launch):
    x, h = t(R, D), t(R, D, dtype=bf16)
    with pytest.raises(TypeError, match="gate"):
        h3.h3f_gated_residual(x, h, t(D, dtype=bf16))
    with pytest.raises(ValueError, match="modulation groups"):
        h3.h3f_gated_residual(x, h, t(D), rows_per_group=5)


def test_gated_adaln_checks(no_launch):
    x, h, y = t(R, D), t(R, D, dtype=bf16), t(R, D, dtype=bf16)
    with pytest.raises(TypeError, match="shift"):
        h3.h3f_gated_residual_adaln(x, h, t(D), t(D, dtype=bf16), t(D), y)
    with pytest.raises(ValueError, match="modulation groups"):
        h3.h3f_gated_residual_adaln(x, h, t(2, D), t(2, D), t(2, D), y, rows_per_group=3)


def test_group_count_accepts_exact_cover(no_launch):
    # 10 rows at 4 per group: 3 groups needed and present -> the call goes through to
    # the (stubbed) library, which is the point where this test stops
    x, y = t(R, D), t(R, D)
    with pytest.raises(AssertionError, match="library was reached"):
        h3.h3f_adaln_modulate(y, x, t(3, D), t(3, D), rows_per_group=4)


def test_rope_positions_validated():
    with pytest.raises(ValueError, match="int32"):
        h3.make_rope(2, 3, 4, 0, (16, 24, 24), positions=torch.zeros(24, 3, dtype=torch.int64))
    with pytest.raises(ValueError, match="int32"):
        h3.make_rope(2, 3, 4, 0, (16, 24, 24), positions=torch.zeros(24, 2, dtype=torch.int32))
    with pytest.raises(ValueError, match="int32"):
        h3.make_rope(2, 3, 4, 0, (16, 24, 24),
                     positions=torch.zeros(3, 24, dtype=torch.int32).t())
    with pytest.raises(ValueError, match="GPU"):
        h3.make_rope(2, 3, 4, 0, (16, 24, 24), positions=torch.zeros(24, 3, dtype=torch.int32))


def test_rope_positions_rows_and_reference(no_launch, monkeypatch):
    # a GPU-less stand-in for a device positions tensor: only the attributes the
    # binding reads
    class FakePos:
        dtype = torch.int32
        shape = (5, 3)
        device = torch.device("cpu")
        is_cuda = True

        def dim(self):
            return 2

        def is_contiguous(self):
            return True

        def data_ptr(self):
            return 0x1000

    pos = FakePos()
    rope = h3.make_rope(2, 3, 4, 0, (16, 24, 24), positions=pos)
    assert rope.positions_tensor is pos  # the struct keeps the array alive
    q = t(R, 2, 64)
    w = t(64)
    with pytest.raises(ValueError, match="5 rows"):
        h3.h3f_qk_rmsnorm_rope3d(t(R, 2, 64), t(R, 2, 64), q, t(R, 2, 64), w, w, rope)
    # a raw pointer set on the struct behind make_rope's back is refused
    bare = h3.make_rope(2, 3, 4, 0, (16, 24, 24))
    bare.positions = 0x2000
    with pytest.raises(ValueError, match="make_rope"):
        h3.h3f_qk_rmsnorm_rope3d(t(R, 2, 64), t(R, 2, 64), q, t(R, 2, 64), w, w, bare)


def test_route_scores_layout():
    # scores rows: dense, or the first nb columns of a [heads, nb, S] buffer; the
    # helper returns the row stride the C call takes
    heads, nb, keep = 3, 33, 7
    kv = torch.zeros(heads, nb, keep, dtype=torch.int32)
    assert h3._route_outputs(kv, t(heads, nb, nb), heads, nb, keep) == nb
    assert h3._route_outputs(kv, t(heads, nb, 64)[:, :, :nb], heads, nb, keep) == 64
    assert h3._route_outputs(kv[:1], t(1, nb, 40)[:, :, :nb], 1, nb, keep) == 40
    with pytest.raises(ValueError, match="evenly spaced"):
        h3._route_outputs(kv, t(heads, nb + 1, nb)[:, 1:], heads, nb, keep)   # head gap
    with pytest.raises(ValueError, match="evenly spaced"):
        h3._route_outputs(kv, t(heads, nb, nb).transpose(1, 2), heads, nb, keep)
    with pytest.raises(ValueError, match="evenly spaced"):
        h3._route_outputs(kv, t(heads, nb, 2 * nb)[:, :, ::2], heads, nb, keep)
    with pytest.raises(ValueError, match=r"\[3, 33, 33\]"):
        h3._route_outputs(kv, t(heads, nb, nb + 1), heads, nb, keep)
    with pytest.raises(TypeError):
        h3._route_outputs(kv, t(heads, nb, nb, dtype=bf16), heads, nb, keep)
    with pytest.raises(ValueError, match="kv_blocks"):
        h3._route_outputs(kv.transpose(0, 1).contiguous().transpose(0, 1), t(heads, nb, nb),
                          heads, nb, keep)
    v = h3.scores_view(heads, nb, "cpu")
    assert v.shape == (heads, nb, nb) and v.stride() == (nb * 64, 64, 1)
