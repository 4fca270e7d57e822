"""The fused calls captured in a HIP graph and replayed.

One DiT block's calls (AdaLN, QK RMSNorm + 3D RoPE, gated residual, AdaLN,
SwiGLU, gated residual), the residual-difference reduction and the block-sparse
router (separate, and with its pooling fused into QK) are captured once with
torch.cuda.graph (the binding launches on the current stream, which is the
capture stream inside the context) and replayed several times, with eager work
and synchronisations between the replays.  Every
replay must reproduce the eager calls bit for bit, and a replay after the
inputs change must follow the new contents (the graph holds pointers, not
data).  The library issues kernel launches only (no memset, copy or allocation
nodes), so nothing in the graph depends on replay order."""
import pytest
import torch

import h3gen
from gpu_util import DEV, dev_tensor

pytestmark = pytest.mark.gpu

h3 = pytest.importorskip("video_diffusion_transformer_h3f_amd")

S5 = dict(T=31, H=48, W=84, A=128, D=5120, heads=40, Dh=128, split=(32, 48, 48))
ROWS, F = 4096 + 37, 2048


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    h3.lib()
    h3gen.dev_lib()
    yield
    torch.cuda.synchronize()


def _buffers():
    D, H, Dh = S5["D"], S5["heads"], S5["Dh"]
    t = {n: dev_tensor(n, ROWS, D, "bf16") for n in ("x", "h", "h2", "x_prev")}
    t["x0"] = t["x"].clone()
    for n in ("shift", "scale", "gate", "shift2", "scale2", "gate2"):
        t[n] = dev_tensor(n, 1, D, "bf16")
    t["q"] = dev_tensor("q", ROWS, H * Dh, "bf16").view(ROWS, H, Dh)
    t["k"] = dev_tensor("k", ROWS, H * Dh, "bf16").view(ROWS, H, Dh)
    t["q_weight"] = dev_tensor("q_weight", 1, Dh, "bf16").view(Dh)
    t["k_weight"] = dev_tensor("k_weight", 1, Dh, "bf16").view(Dh)
    t["gate_up"] = dev_tensor("gate_up", ROWS, 2 * F, "bf16")
    nb, keep, ws = h3.h3f_subblock_plan(ROWS, H, Dh, 128, 0.8, 12)
    outs = {
        "y1": torch.empty(ROWS, D, dtype=torch.bfloat16, device=DEV),
        "y2": torch.empty(ROWS, D, dtype=torch.bfloat16, device=DEV),
        "q_out": torch.empty(ROWS, H, Dh, dtype=torch.bfloat16, device=DEV),
        "k_out": torch.empty(ROWS, H, Dh, dtype=torch.bfloat16, device=DEV),
        "act": torch.empty(ROWS, F, dtype=torch.bfloat16, device=DEV),
        "l1": torch.empty(3, dtype=torch.float64, device=DEV),
        "kv": torch.empty(H, nb, keep, dtype=torch.int32, device=DEV),
        "scores": torch.empty(H, nb, nb, dtype=torch.float32, device=DEV),
        "q_out2": torch.empty(ROWS, H, Dh, dtype=torch.bfloat16, device=DEV),
        "k_out2": torch.empty(ROWS, H, Dh, dtype=torch.bfloat16, device=DEV),
        "kv2": torch.empty(H, nb, keep, dtype=torch.int32, device=DEV),
        "scores2": h3.scores_view(H, nb, DEV),  # rows padded to 128 bytes
        "x": t["x"],
    }
    t["l1_ws"] = torch.empty(max(h3.h3f_residual_l1_workspace_bytes(ROWS, D, torch.bfloat16), 16),
                             dtype=torch.uint8, device=DEV)
    t["route_ws"] = torch.empty(max(ws, 16), dtype=torch.uint8, device=DEV)
    t["pool_ws"] = torch.empty(max(ws, 16), dtype=torch.uint8, device=DEV)
    return t, outs


def _block(t, o, rope):
    h3.h3f_stream_copy(t["x"], t["x0"])  # every replay starts from the same residual stream
    h3.h3f_adaln_modulate(o["y1"], t["x"], t["shift"], t["scale"])
    h3.h3f_qk_rmsnorm_rope3d(o["q_out"], o["k_out"], t["q"], t["k"], t["q_weight"],
                             t["k_weight"], rope)
    h3.h3f_gated_residual(t["x"], t["h"], t["gate"])
    h3.h3f_adaln_modulate(o["y2"], t["x"], t["shift2"], t["scale2"])
    h3.h3f_swiglu(o["act"], t["gate_up"])
    h3.h3f_gated_residual(t["x"], t["h2"], t["gate2"])
    h3.h3f_residual_l1(o["l1"], t["x"], t["x_prev"], workspace=t["l1_ws"])
    h3.h3f_subblock_route(o["kv"], o["scores"], o["q_out"], o["k_out"], 128, 0.8, 12,
                          workspace=t["route_ws"])
    # the same route with the pooling fused into the QK operator
    h3.h3f_qk_rmsnorm_rope3d_pool(o["q_out2"], o["k_out2"], t["q"], t["k"], t["q_weight"],
                                  t["k_weight"], rope, 128, t["pool_ws"])
    h3.h3f_subblock_route_pooled(o["kv2"], o["scores2"], ROWS, S5["heads"], 128, 0.8, 12,
                                 t["pool_ws"])


def _snapshot(o):
    torch.cuda.synchronize()
    return {n: v.clone() for n, v in o.items()}


def _clear(o):
    for n, v in o.items():
        if n != "x":
            v.zero_()


def _assert_equal(got, want, what):
    for n in want:
        assert torch.equal(got[n], want[n]), f"{what}: {n} differs from the eager calls"


def test_block_graph_replays_match_eager():
    t, o = _buffers()
    rope = h3.make_rope(S5["T"], S5["H"], S5["W"], S5["A"], S5["split"], token_offset=124000)
    _block(t, o, rope)
    want = _snapshot(o)

    g = torch.cuda.CUDAGraph()
    _clear(o)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        _block(t, o, rope)
    torch.cuda.synchronize()

    scratch = torch.empty(1 << 22, dtype=torch.float32, device=DEV)
    for rep in range(4):
        _clear(o)
        scratch.normal_()  # unrelated eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        _assert_equal(_snapshot(o), want, f"replay {rep}")

    # new input contents, same buffers: the replay follows them
    t["x0"].mul_(0.5)
    t["gate_up"].neg_()
    t["q"].mul_(-2.0)
    _block(t, o, rope)
    want2 = _snapshot(o)
    assert not torch.equal(want2["y1"], want["y1"])
    assert not torch.equal(want2["act"], want["act"])
    for rep in range(2):
        _clear(o)
        g.replay()
        _assert_equal(_snapshot(o), want2, f"replay {rep} after new inputs")


def test_two_graphs_interleaved_with_eager_calls():
    # two captures over separate buffers, replayed alternately with eager calls on a
    # third set; each stays equal to its own eager result
    rope = h3.make_rope(S5["T"], S5["H"], S5["W"], S5["A"], S5["split"])
    sets = [_buffers() for _ in range(3)]
    sets[1][0]["x0"].mul_(3.0)
    wants = []
    for t, o in sets[:2]:
        _block(t, o, rope)
        wants.append(_snapshot(o))
    graphs = []
    for t, o in sets[:2]:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            _block(t, o, rope)
        graphs.append(g)
    torch.cuda.synchronize()
    te, oe = sets[2]
    for rep in range(3):
        for i, g in enumerate(graphs):
            _clear(sets[i][1])
            g.replay()
            _block(te, oe, rope)
            _assert_equal(_snapshot(sets[i][1]), wants[i], f"graph {i} replay {rep}")
