"""QK RMSNorm + 3D RoPE with the router's block pooling fused in
(h3f_qk_rmsnorm_rope3d_pool) and the route finished from its block means
(h3f_subblock_route_pooled), against the plain operator and the CPU oracle.

  - q_out / k_out are bit-identical to h3f_qk_rmsnorm_rope3d's (same per-token
    code);
  - the block means in the workspace match the oracle's pool of the values as
    stored, within the forward-error bound of an fp32 sum of n terms
    (2 gamma_n of the mean of |x|, Higham sec. 3.1) plus one rounding;
  - scores and kept lists of the pooled route meet the same checks as the
    separate route's (tests/test_gpu_router.py): scores within the derived
    bound, kept lists exact on their own scores and valid on the oracle's.
"""
import numpy as np
import pytest
import torch

import h3gen
import oracle
from gpu_util import DEV, dev_tensor, from_np, to_np
from test_gpu_router import (PLAIN_FP32_MIN_BLOCK, assert_scores, block_abs_means,
                             check_selection_on_own_scores, check_selection_valid, gamma,
                             score_tol)

pytestmark = pytest.mark.gpu

h3 = pytest.importorskip("video_diffusion_transformer_h3f_amd")

GRID = dict(T=31, H=48, W=84, A=128, split=(32, 48, 48))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    h3.lib()
    h3gen.dev_lib()
    yield
    torch.cuda.synchronize()


def inputs(rows, heads, packed, seed=0):
    cols = heads * 128
    if packed:
        buf = torch.full((rows, 3, heads, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
        flat = buf.view(rows, 3 * cols)
        h3gen.fill_device(flat[:, :cols], "q", seed=seed)
        h3gen.fill_device(flat[:, cols:2 * cols], "k", seed=seed)
        q, k = buf[:, 0], buf[:, 1]
    else:
        q = dev_tensor("q", rows, cols, "bf16", seed=seed).view(rows, heads, 128)
        k = dev_tensor("k", rows, cols, "bf16", seed=seed).view(rows, heads, 128)
    qw = dev_tensor("q_weight", 1, 128, "bf16").view(128)
    kw = dev_tensor("k_weight", 1, 128, "bf16").view(128)
    return q, k, qw, kw


def run_pool(q, k, qw, kw, rope, block):
    rows, heads, _ = q.shape
    nb, _, need = h3.h3f_subblock_plan(rows, heads, 128, block, 0.8, 10)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)   # NaN-filled floats
    qo = torch.empty(rows, heads, 128, dtype=torch.bfloat16, device=DEV)
    ko = torch.empty_like(qo)
    h3.h3f_qk_rmsnorm_rope3d_pool(qo, ko, q, k, qw, kw, rope, block, ws)
    torch.cuda.synchronize()
    return qo, ko, ws, nb


def host_bits(t):
    return to_np(t.contiguous())


def check_means(ws, nb, qo_h, ko_h, block):
    rows, heads, _ = qo_h.shape
    means = ws.view(torch.float32)[:2 * heads * nb * 128].view(2, heads, nb, 128).cpu().numpy()
    for t, x in enumerate((qo_h, ko_h)):
        ref = oracle.subblock_pool(x, block)                       # [heads, nb, 128] double
        amean = block_abs_means(x, block)
        tol = 2 * gamma(block) * amean + 2.0 ** -24 * np.abs(ref) + 1e-30
        err = np.abs(means[t].astype(np.float64) - ref)
        worst = float((err / tol).max())
        print(f"  {'qk'[t]} block means: max err/tol {worst:.3g}")
        assert worst <= 1.0


CASES = [
    # rows, heads, block, packed, pairing, explicit positions
    (4096 + 77, 3, 128, False, h3.H3F_ROPE_INTERLEAVED, False),
    (4096, 8, 64, True, h3.H3F_ROPE_HALF_SPLIT, False),
    (5000, 2, 1000, False, h3.H3F_ROPE_INTERLEAVED, True),
    (4096 + 3, 5, 4099, False, h3.H3F_ROPE_INTERLEAVED, False),
    (4096, 1, 1, False, h3.H3F_ROPE_INTERLEAVED, False),   # one token per block: chunks half empty
    (4096 + 5, 2, 3, True, h3.H3F_ROPE_HALF_SPLIT, True),  # ragged 3-token blocks, every option
]


@pytest.mark.parametrize("case", CASES, ids=["ragged-3heads", "packed-halfsplit",
                                             "long-blocks-positions", "one-block",
                                             "block1-one-head", "block3-packed-half-positions"])
def test_qk_pool_outputs_and_means(case):
    rows, heads, block, packed, pairing, explicit = case
    print(f"qk pool rows={rows} heads={heads} block={block} packed={packed} pairing={pairing} "
          f"positions={explicit}", flush=True)
    q, k, qw, kw = inputs(rows, heads, packed, seed=7)
    pos = None
    if explicit:
        pos = from_np(oracle.positions(rows, GRID["T"], GRID["H"], GRID["W"], GRID["A"],
                                       token_offset=99_000))
    rope = h3.make_rope(GRID["T"], GRID["H"], GRID["W"], GRID["A"], GRID["split"],
                        token_offset=0 if explicit else 99_000, positions=pos, pairing=pairing)
    qo, ko, ws, nb = run_pool(q, k, qw, kw, rope, block)
    qp, kp = torch.empty_like(qo), torch.empty_like(ko)
    h3.h3f_qk_rmsnorm_rope3d(qp, kp, q, k, qw, kw, rope)
    assert torch.equal(qo, qp) and torch.equal(ko, kp), "fused outputs must equal the plain operator's"
    qo_h, ko_h = host_bits(qo), host_bits(ko)
    check_means(ws, nb, qo_h, ko_h, block)

    # the route finished from the fused means
    for sparsity, step in ((0.8, 10), (0.75, 30)):
        _, keep, _ = h3.h3f_subblock_plan(rows, heads, 128, block, sparsity, step)
        kv = torch.full((heads, nb, keep), -7, dtype=torch.int32, device=DEV)
        sc = torch.full((heads, nb, nb), float("nan"), dtype=torch.float32, device=DEV)
        h3.h3f_subblock_route_pooled(kv, sc, rows, heads, block, sparsity, step, ws)
        kv, sc = to_np(kv), to_np(sc)
        kv_ref, sc_ref = oracle.subblock_route(qo_h, ko_h, block, sparsity, step)
        tol = score_tol(sc_ref, block_abs_means(qo_h, block), block_abs_means(ko_h, block), block)
        assert_scores(sc, sc_ref, tol, f"pooled-route scores s={sparsity}",
                      plain_fp32=block >= PLAIN_FP32_MIN_BLOCK)
        check_selection_on_own_scores(kv, sc)
        check_selection_valid(kv, sc_ref, tol)


def test_route_pooled_dense_step_reads_no_workspace():
    rows, heads, block = 4096 + 5, 2, 128
    nb = 33
    kv = torch.full((heads, nb, nb), -1, dtype=torch.int32, device=DEV)
    sc = torch.full((heads, nb, nb), 5.0, dtype=torch.float32, device=DEV)
    empty = torch.empty(0, dtype=torch.uint8, device=DEV)
    h3.h3f_subblock_route_pooled(kv, sc, rows, heads, block, 0.8, 9, empty)
    torch.cuda.synchronize()
    assert (to_np(kv) == np.arange(nb, dtype=np.int32)).all()
    assert (to_np(sc) == 5.0).all()


def test_qk_pool_full_5s_shape():
    # the measured shape: 125,120 tokens, 40 heads, blocks of 128 (978 blocks)
    rows, heads, block = 31 * 48 * 84 + 128, 40, 128
    q, k, qw, kw = inputs(rows, heads, False)
    rope = h3.make_rope(GRID["T"], GRID["H"], GRID["W"], GRID["A"], GRID["split"])
    qo, ko, ws, nb = run_pool(q, k, qw, kw, rope, block)
    qp, kp = torch.empty_like(qo), torch.empty_like(ko)
    h3.h3f_qk_rmsnorm_rope3d(qp, kp, q, k, qw, kw, rope)
    assert torch.equal(qo, qp) and torch.equal(ko, kp)
    del qp, kp, q, k
    _, keep, _ = h3.h3f_subblock_plan(rows, heads, 128, block, 0.8, 10)
    kv = torch.empty(heads, nb, keep, dtype=torch.int32, device=DEV)
    sc = h3.scores_view(heads, nb, DEV)  # 128-byte rows, as the benchmark launches it
    h3.h3f_subblock_route_pooled(kv, sc, rows, heads, block, 0.8, 10, ws)
    kv, sc = to_np(kv), to_np(sc.contiguous())
    check_selection_on_own_scores(kv[::9], sc[::9])
    qblocks = np.array([0, 500, 977])
    for h in (0, 27):
        qh, kh = host_bits(qo[:, h:h + 1]), host_bits(ko[:, h:h + 1])
        pq = oracle.subblock_pool(qh, block)[:, qblocks]
        pk = oracle.subblock_pool(kh, block)
        ref = oracle.subblock_scores(pq, pk)[0]
        tol = score_tol(ref[None], block_abs_means(qh, block)[:, qblocks],
                        block_abs_means(kh, block), block)[0]
        assert_scores(sc[h, qblocks], ref, tol, f"scores head {h}", plain_fp32=True)
        check_selection_valid(kv[h, qblocks], ref, tol)
