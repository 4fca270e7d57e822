"""GPU parity of the block-sparse attention router (h3f_subblock_route) against
the CPU oracle.

Block scores are fp32 outputs of a two-level reduction -- an fp32 mean of n
tokens per block, then a 128-term fp32 dot product -- so near-zero scores can
come from heavy cancellation.  Their tolerance is the fp32 output tolerance
plus the standard forward-error bound of that arithmetic (Higham, "Accuracy
and Stability of Numerical Algorithms", sec. 3.1, gamma_m = m u / (1 - m u),
u = 2^-24): with a_q, a_k the block means of |q|, |k|,
  |err| <= 1e-6 + 1e-5 |ref| + (2 gamma_n + gamma_130) sum_d a_q[d] a_k[d],
covering the rounding of each mean (gamma_n of the mean of |x|) and of the
dot product of the rounded means.  Calls with blocks of 64 tokens or more (the
5 s and 10 s shapes among them) are also held to the plain fp32 tolerance.
The kept key blocks are an integer decision taken from floating point, where
several answers can be right when two scores are within rounding of each
other, so they are checked as follows:
  - exact on their own input: each row keeps blocks whose GPU scores are all
    >= every skipped block's GPU score, equal scores going to the lower index,
    listed strictly ascending (this pins the selection kernel bit for bit);
  - valid against the oracle: no skipped block's oracle score exceeds a kept
    block's oracle score by more than the two scores' tolerances (the bound
    above);
  - where scores are exact by construction (planted inputs), identical to the
    oracle's selection.
"""
import numpy as np
import pytest
import torch

import h3gen
import oracle
from gpu_util import DEV, dev_tensor, to_np
from tolerance import FP32_ATOL, FP32_RTOL, as_f64

pytestmark = pytest.mark.gpu

h3 = pytest.importorskip("video_diffusion_transformer_h3f_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    h3.lib()
    h3gen.dev_lib()
    yield
    torch.cuda.synchronize()


def qk_tensors(rows, heads, packed=False, seed=0):
    """bf16 q, k [rows, heads, 128] on the GPU (views of one packed qkv buffer
    when packed) and the matching host arrays."""
    cols = heads * 128
    if packed:
        buf = torch.full((rows, 3, heads, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
        q, k = buf[:, 0], buf[:, 1]
        flat = buf.view(rows, 3 * cols)
        h3gen.fill_device(flat[:, :cols], "q", seed=seed)
        h3gen.fill_device(flat[:, cols:2 * cols], "k", seed=seed)
    else:
        q = dev_tensor("q", rows, cols, "bf16", seed=seed).view(rows, heads, 128)
        k = dev_tensor("k", rows, cols, "bf16", seed=seed).view(rows, heads, 128)
    qh = h3gen.host_rows("q", rows, cols, "bf16", seed=seed).reshape(rows, heads, 128)
    kh = h3gen.host_rows("k", rows, cols, "bf16", seed=seed).reshape(rows, heads, 128)
    return q, k, qh, kh


def padded_stride(nb):
    """Score row stride of 128-byte rows, as the benchmark allocates them."""
    return -(-nb // 32) * 32


def run_route(q, k, block, sparsity, step, sentinel=None, stride=None, pad_out=None):
    """kv, scores of one route call; scores rows `stride` floats apart (dense when
    None).  pad_out (a list) receives the pad columns of padded rows."""
    rows, heads, _ = q.shape
    nb, keep, _ = h3.h3f_subblock_plan(rows, heads, 128, block, sparsity, step)
    kv = torch.full((heads, nb, keep), -7, dtype=torch.int32, device=DEV)
    buf = torch.full((heads, nb, stride or nb), float("nan") if sentinel is None else sentinel,
                     dtype=torch.float32, device=DEV)
    sc = buf[:, :, :nb]
    h3.h3f_subblock_route(kv, sc, q, k, block, sparsity, step)
    torch.cuda.synchronize()
    if pad_out is not None:
        pad_out.append(to_np(buf[:, :, nb:].contiguous()))
    return to_np(kv), to_np(sc.contiguous())


def check_selection_on_own_scores(kv, sc):
    """Every row of kv is the top-keep of its own row of sc (ties: lower index)."""
    heads, nbq, keep = kv.shape
    nbk = sc.shape[2]
    assert kv.min() >= 0 and kv.max() < nbk
    assert (np.diff(kv, axis=2) > 0).all(), "kept blocks must be strictly ascending"
    kept = np.zeros(sc.shape, dtype=bool)
    np.put_along_axis(kept, kv.astype(np.int64), True, axis=2)
    if keep == nbk:
        return
    s = sc.astype(np.float64)
    lo = np.where(kept, s, np.inf).min(axis=2)          # smallest kept score
    hi = np.where(kept, -np.inf, s).max(axis=2)         # largest skipped score
    assert (lo >= hi).all(), "a skipped block outscores a kept block"
    # equal to the threshold and skipped: must come after every kept block of that score
    thr = lo[..., None]
    idx = np.arange(nbk)
    last_kept_at_thr = np.where(kept & (s == thr), idx, -1).max(axis=2)
    first_skipped_at_thr = np.where(~kept & (s == thr), idx, nbk).min(axis=2)
    assert (first_skipped_at_thr > last_kept_at_thr).all(), "ties must go to the lower index"


U = 2.0 ** -24


def gamma(m):
    return m * U / (1.0 - m * U)


def block_abs_means(x, block):
    """[heads, n_blocks, 128] means of |x| over each block's tokens (x: host bf16 bits)."""
    a = np.abs(as_f64(x))                       # [rows, heads, 128]
    starts = np.arange(0, a.shape[0], block)
    sums = np.add.reduceat(a, starts, axis=0)   # [n_blocks, heads, 128]
    counts = np.minimum(block, a.shape[0] - starts).astype(np.float64)
    return np.ascontiguousarray((sums / counts[:, None, None]).transpose(1, 0, 2))


def score_tol(ref, aq, ak, block):
    """Tolerance of each block score: fp32 output tolerance + rounding bound."""
    return FP32_ATOL + FP32_RTOL * np.abs(ref) + (2 * gamma(block) + gamma(130)) * (aq @ ak.transpose(0, 2, 1))


# Blocks of at least this many tokens have block means well below 1 and scores
# that also meet the plain fp32 output tolerance, which is then asserted too;
# blocks of 1 - 3 tokens give O(10) scores formed with cancellation, held to
# the derived bound alone.
PLAIN_FP32_MIN_BLOCK = 64


def assert_scores(sc, ref, tol, what, plain_fp32=False):
    """Scores within tol; with plain_fp32 also within the plain fp32 output tolerance."""
    err = np.abs(sc.astype(np.float64) - ref)
    worst = float((err / tol).max())
    plain = float((err / (FP32_ATOL + FP32_RTOL * np.abs(ref))).max())
    print(f"  {what}: max err/tol {worst:.3g}; against the plain fp32 tolerance {plain:.3g}")
    assert worst <= 1.0, f"{what}: max err/tol {worst:.3f}"
    if plain_fp32:
        assert plain <= 1.0, f"{what}: max err / plain fp32 tolerance {plain:.3f}"


def check_selection_valid(kv, ref_scores, tol):
    """No skipped block's oracle score beats a kept block's by more than the tolerances."""
    s = ref_scores
    kept = np.zeros(s.shape, dtype=bool)
    np.put_along_axis(kept, kv.astype(np.int64), True, axis=-1)
    if kept.all():
        return
    lo = np.where(kept, s + tol, np.inf).min(axis=-1)
    hi = np.where(kept, -np.inf, s - tol).max(axis=-1)
    assert (lo >= hi).all(), "selection inconsistent with the oracle's scores"


@pytest.mark.parametrize("rows,heads,block,packed", [
    (4096 + 77, 3, 128, False),   # ragged last block, a partial group of heads
    (4096, 8, 64, True),          # strided q / k inside a packed qkv buffer
    (5000, 2, 1000, False),       # long blocks, ragged
    (4096 + 77, 1, 4096 + 77, False),  # a single block
    (4096, 2, 3, False),          # 1366 blocks (the select kernel's 32-key-per-lane form)
    (4096 + 3, 1, 2, False),      # 2050 blocks (its 128-key-per-lane form)
    (4096 + 50, 9, 128, False),   # 9 dense heads: the strided pool form, not the flat one
    (4470, 2, 128, False),        # 35 blocks: 3 columns past the last 4-column group
], ids=["ragged", "packed", "long-blocks", "one-block", "nb1366", "nb2050", "heads9", "nb35"])
@pytest.mark.parametrize("sparsity", [0.8, 0.75])
def test_router_matches_oracle(rows, heads, block, packed, sparsity):
    print(f"router rows={rows} heads={heads} block={block} packed={packed} s={sparsity}", flush=True)
    q, k, qh, kh = qk_tensors(rows, heads, packed=packed, seed=3)
    kv, sc = run_route(q, k, block, sparsity, step=10)
    kv_ref, sc_ref = oracle.subblock_route(qh, kh, block, sparsity, 10)
    assert kv.shape == kv_ref.shape and sc.shape == sc_ref.shape
    tol = score_tol(sc_ref, block_abs_means(qh, block), block_abs_means(kh, block), block)
    assert_scores(sc, sc_ref, tol, "block scores", plain_fp32=block >= PLAIN_FP32_MIN_BLOCK)
    check_selection_on_own_scores(kv, sc)
    check_selection_valid(kv, sc_ref, tol)
    agree = np.mean([len(np.intersect1d(a, b)) / kv.shape[2]
                     for a, b in zip(kv.reshape(-1, kv.shape[2]), kv_ref.reshape(-1, kv.shape[2]))])
    print(f"  kept sets agree with the oracle's on {agree:.4%} of entries")


@pytest.mark.parametrize("block", [128, 32])  # 33 blocks (sorted directly), 130 (probed first)
def test_router_planted_scores_exact(block):
    # Every query token is e0; every token of key block j is alpha_j * e0 (head h
    # uses (-1)^h alpha).  Block means and scores are exact in fp32, so the kept
    # blocks must equal the oracle's exactly, ties included (alpha repeats).
    rows, heads = 4096 + 40, 5
    nb = (rows + block - 1) // block
    rng = np.random.default_rng(11)
    alpha = rng.integers(-16, 17, size=nb).astype(np.float32) / 8.0   # many ties
    q = np.zeros((rows, heads, 128), np.float32)
    k = np.zeros((rows, heads, 128), np.float32)
    q[:, :, 0] = 1.0
    sign = np.array([(-1.0) ** h for h in range(heads)], np.float32)
    k[:, :, 0] = alpha[np.arange(rows) // block][:, None] * sign[None, :]
    qb = torch.from_numpy(q).to(torch.bfloat16).to(DEV)
    kb = torch.from_numpy(k).to(torch.bfloat16).to(DEV)
    qh = qb.cpu().view(torch.int16).numpy().view(np.uint16)
    kh = kb.cpu().view(torch.int16).numpy().view(np.uint16)
    for sparsity in (0.8, 0.5, 0.0):
        kv, sc = run_route(qb, kb, block, sparsity, step=12)
        kv_ref, sc_ref = oracle.subblock_route(qh, kh, block, sparsity, 12)
        assert np.array_equal(sc.astype(np.float64), sc_ref)
        assert np.array_equal(kv, kv_ref), f"sparsity {sparsity}"


def test_router_planted_outliers_exact():
    # As above, with a few key blocks of +-4096 among values in [-2, 2]: the
    # select kernel's first probe (the row's mean + z * std, which assumes a
    # roughly normal row) lands far from the threshold, and the search must still
    # end on the oracle's kept blocks.  1023 blocks of 8 tokens (16 keys per lane).
    block, heads = 8, 2
    rows = 1023 * block
    nb = 1023
    rng = np.random.default_rng(23)
    alpha = rng.integers(-16, 17, size=nb).astype(np.float32) / 8.0
    alpha[rng.choice(nb, 5, replace=False)] = 4096.0
    alpha[rng.choice(nb, 3, replace=False)] = -4096.0
    q = np.zeros((rows, heads, 128), np.float32)
    k = np.zeros((rows, heads, 128), np.float32)
    q[:, :, 0] = 1.0
    sign = np.array([(-1.0) ** h for h in range(heads)], np.float32)
    k[:, :, 0] = alpha[np.arange(rows) // block][:, None] * sign[None, :]
    qb = torch.from_numpy(q).to(torch.bfloat16).to(DEV)
    kb = torch.from_numpy(k).to(torch.bfloat16).to(DEV)
    qh = qb.cpu().view(torch.int16).numpy().view(np.uint16)
    kh = kb.cpu().view(torch.int16).numpy().view(np.uint16)
    for sparsity in (0.8, 0.995, 0.3):
        kv, sc = run_route(qb, kb, block, sparsity, step=12)
        kv_ref, sc_ref = oracle.subblock_route(qh, kh, block, sparsity, 12)
        assert np.array_equal(sc.astype(np.float64), sc_ref)
        assert np.array_equal(kv, kv_ref), f"sparsity {sparsity}"


def test_router_all_scores_equal_keeps_lowest_blocks():
    # zero queries: every score is +0 or -0 (0 times a negative mean), which rank
    # equal, so each query block keeps the lowest-numbered key blocks
    rows, heads, block = 8192 + 5, 3, 64
    q = torch.zeros(rows, heads, 128, dtype=torch.bfloat16, device=DEV)
    k = dev_tensor("k", rows, heads * 128, "bf16", seed=6).view(rows, heads, 128)
    kv, sc = run_route(q, k, block, 0.8, step=10)
    nb, keep = 129, 129 - int(0.8 * 129)
    assert kv.shape == (heads, nb, keep) and (sc == 0).all()
    assert (kv == np.arange(keep, dtype=np.int32)).all()


def test_router_dense_steps_keep_everything():
    q, k, _, _ = qk_tensors(4096 + 5, 2, seed=1)
    kv, sc = run_route(q, k, 128, 0.8, step=9, sentinel=123.0)
    nb = 33
    assert kv.shape == (2, nb, nb)
    assert (kv == np.arange(nb, dtype=np.int32)).all()
    assert (sc == 123.0).all(), "a dense step must not write scores"


def test_router_sparsity_zero_keeps_all_in_order():
    q, k, _, _ = qk_tensors(4096, 2, seed=2)
    kv, sc = run_route(q, k, 256, 0.0, step=10)
    assert (kv == np.arange(16, dtype=np.int32)).all()
    assert np.isfinite(sc).all()


def test_router_deterministic():
    q, k, _, _ = qk_tensors(8192 + 100, 4, seed=4)
    a = run_route(q, k, 128, 0.8, step=20)
    b = run_route(q, k, 128, 0.8, step=20)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


def test_router_full_10s_sampled():
    # the 10 s sequence (246,208 tokens -> 1924 blocks, 385 kept at 0.8), as the
    # benchmark's 10 s workload runs it; sampled heads and query blocks
    rows, heads, block = 61 * 48 * 84 + 256, 40, 128
    q = dev_tensor("q", rows, heads * 128, "bf16").view(rows, heads, 128)
    k = dev_tensor("k", rows, heads * 128, "bf16").view(rows, heads, 128)
    kv, sc = run_route(q, k, block, 0.8, step=10, stride=padded_stride(1924))
    del q, k
    assert kv.shape == (40, 1924, 385)
    check_selection_on_own_scores(kv[::7], sc[::7])
    qblocks = np.array([0, 961, 1923])
    for h in (5, 33):
        qh = h3gen.host_cols("q", rows, heads * 128, h * 128, 128).reshape(rows, 1, 128)
        kh = h3gen.host_cols("k", rows, heads * 128, h * 128, 128).reshape(rows, 1, 128)
        pq = oracle.subblock_pool(qh, block)[:, qblocks]
        pk = oracle.subblock_pool(kh, block)
        ref = oracle.subblock_scores(pq, pk)[0]
        tol = score_tol(ref[None], block_abs_means(qh, block)[:, qblocks],
                        block_abs_means(kh, block), block)[0]
        assert_scores(sc[h, qblocks], ref, tol, f"scores head {h}", plain_fp32=True)
        check_selection_valid(kv[h, qblocks], ref, tol)


def test_router_full_5s_sampled():
    # The 5 s sequence (125,120 tokens, 40 heads of 128, blocks of 128 -> 978
    # blocks, sparsity 0.8 -> 196 kept), launched as the benchmark launches it.
    # The oracle recomputes every block mean of sampled heads and the score rows
    # of sampled query blocks (the first, a middle and the short last one); the
    # selection property is checked on every row.
    rows, heads, block = 31 * 48 * 84 + 128, 40, 128
    q, k, _, _ = (dev_tensor("q", rows, heads * 128, "bf16").view(rows, heads, 128),
                  dev_tensor("k", rows, heads * 128, "bf16").view(rows, heads, 128), None, None)
    kv, sc = run_route(q, k, block, 0.8, step=10, stride=padded_stride(978))
    assert kv.shape == (40, 978, 196)
    check_selection_on_own_scores(kv, sc)
    qblocks = np.array([0, 1, 500, 977])
    for h in (0, 17, 39):
        qh = h3gen.host_cols("q", rows, heads * 128, h * 128, 128).reshape(rows, 1, 128)
        kh = h3gen.host_cols("k", rows, heads * 128, h * 128, 128).reshape(rows, 1, 128)
        pq = oracle.subblock_pool(qh, block)[:, qblocks]
        pk = oracle.subblock_pool(kh, block)
        ref = oracle.subblock_scores(pq, pk)[0]
        tol = score_tol(ref[None], block_abs_means(qh, block)[:, qblocks],
                        block_abs_means(kh, block), block)[0]
        # blocks of 128 tokens: the means are small, and the scores also meet the
        # plain fp32 output tolerance
        assert_scores(sc[h, qblocks], ref, tol, f"scores head {h}", plain_fp32=True)
        check_selection_valid(kv[h, qblocks], ref, tol)


@pytest.mark.parametrize("rows,heads,block", [
    (4096 + 77, 3, 128),   # 33 blocks (odd: 4- and 8-byte stores at the row end)
    (4096, 2, 3),          # 1366 blocks (2 mod 4)
    (4096, 8, 64),         # 64 blocks (whole 16-byte groups)
], ids=["nb33", "nb1366", "nb64"])
@pytest.mark.parametrize("extra", [0, 5], ids=["rows128B", "rows-odd"])
def test_router_padded_score_rows(rows, heads, block, extra):
    # scores rows further apart than n_blocks: the same scores (bit for bit) and
    # kept lists as dense rows, and the pad columns are never written; extra = 5
    # makes a stride that is not a multiple of 4 (rows only 4-byte aligned)
    q, k, _, _ = qk_tensors(rows, heads, seed=4)
    nb, _, _ = h3.h3f_subblock_plan(rows, heads, 128, block, 0.8, 10)
    kv_d, sc_d = run_route(q, k, block, 0.8, 10)
    pads = []
    kv_p, sc_p = run_route(q, k, block, 0.8, 10, sentinel=-7.0, stride=padded_stride(nb) + extra,
                           pad_out=pads)
    assert np.array_equal(sc_p.view(np.uint32), sc_d.view(np.uint32))
    assert np.array_equal(kv_p, kv_d)
    assert pads[0].size == heads * nb * (padded_stride(nb) + extra - nb)
    assert (pads[0] == -7.0).all(), "a pad column of the scores was written"


def test_router_maximum_blocks():
    # 8192 blocks, the largest call the select kernel takes (128 keys per lane, every
    # slot filled); one-token blocks, one head
    rows, heads, block = 8192, 1, 1
    q, k, qh, kh = qk_tensors(rows, heads, seed=5)
    kv, sc = run_route(q, k, block, 0.75, step=30)
    assert kv.shape == (1, 8192, 8192 - 6144)
    check_selection_on_own_scores(kv, sc)
    kv_ref, sc_ref = oracle.subblock_route(qh, kh, block, 0.75, 30)
    tol = score_tol(sc_ref, block_abs_means(qh, block), block_abs_means(kh, block), block)
    assert_scores(sc, sc_ref, tol, "block scores at 8192 blocks")
    check_selection_valid(kv, sc_ref, tol)
    # one block more is refused before any launch
    with pytest.raises(h3.H3FError):
        h3.h3f_subblock_plan(8193, 1, 128, 1, 0.75, 30)
