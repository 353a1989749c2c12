"""Parallel decoding as one HIP graph (ParallelVLM notes, "parallel
decoding": the draft produces the next window while the target verifies the
last): the dense-verify launches on one stream and the draft launches on a
second stream, captured as two branches of one graph, give bit for bit the
outputs of the same calls made one after the other without a graph.

Each branch has its own workspace (calls that overlap in time must not share
one).  The graph is replayed several times with eager work and
synchronisations between the replays, and every replay is checked, so a
node that only works on the first replay would fail here."""
import pytest

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

from tests._util import log  # noqa: E402


def _layers(L, Hq, Hkv, D, n_verify, n_draft, gamma, seed):
    g = torch.Generator(device="cuda:0").manual_seed(seed)
    dev = "cuda:0"
    kv = torch.randn(2, L, Hkv, n_verify, D, generator=g, device=dev).to(torch.bfloat16)
    kd = torch.randn(2, L, Hkv, n_draft, D, generator=g, device=dev).to(torch.bfloat16)
    qv = torch.randn(L, 1, gamma + 1, Hq, D, generator=g, device=dev).to(torch.bfloat16)
    qd = torch.randn(L, 1, 1, Hq, D, generator=g, device=dev).to(torch.bfloat16)
    return kv, kd, qv, qd


@pytest.mark.parametrize("L,n_verify,n_draft", [(4, 25222, 2638), (6, 3000, 700)])
def test_two_branch_graph_equals_serial_calls(L, n_verify, n_draft):
    from visual_kv_pruning_amd import ops
    Hq, Hkv, D, gamma = 64, 8, 128, 5
    log(f"parallel graph case L={L} verify keys={n_verify} draft keys={n_draft}")
    kv, kd, qv, qd = _layers(L, Hq, Hkv, D, n_verify, n_draft, gamma, seed=11)
    dev = "cuda:0"
    lv = torch.full((1,), n_verify, dtype=torch.int32, device=dev)
    ld = torch.full((1,), n_draft, dtype=torch.int32, device=dev)
    ws_v = torch.empty(max(256, ops.decode_attn_workspace_bytes(1, gamma + 1, Hq, Hkv, D, n_verify)),
                       dtype=torch.uint8, device=dev)
    ws_d = torch.empty(max(256, ops.decode_attn_workspace_bytes(1, 1, Hq, Hkv, D, n_draft)),
                       dtype=torch.uint8, device=dev)
    ov = torch.empty(L, 1, gamma + 1, Hq, D, device=dev)
    sv = torch.empty(L, 1, gamma + 1, Hq, device=dev)
    od = torch.empty(L, 1, 1, Hq, D, device=dev)
    sd = torch.empty(L, 1, 1, Hq, device=dev)

    def verify(l):
        ops.decode_attn(qv[l], kv[0, l], kv[1, l], lv, True, out=ov[l], lse=sv[l], ws=ws_v)

    def draft(l):
        ops.decode_attn(qd[l], kd[0, l], kd[1, l], ld, False, out=od[l], lse=sd[l], ws=ws_d)

    # eager, one after the other
    for l in range(L):
        verify(l)
    for l in range(L):
        draft(l)
    torch.cuda.synchronize()
    want = [t.clone() for t in (ov, sv, od, sd)]

    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        main = torch.cuda.current_stream()
        side.wait_stream(main)
        with torch.cuda.stream(side):
            for l in range(L):
                draft(l)
        for l in range(L):
            verify(l)
        main.wait_stream(side)
    for rep in range(4):
        for t in (ov, sv, od, sd):
            t.fill_(float("nan"))        # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(("verify out", "verify lse", "draft out", "draft lse"), (ov, sv, od, sd), want):
            assert torch.equal(got, ref), f"replay {rep}: {name} differs from the serial calls"
        # an eager call between replays, on the same buffers the graph uses
        verify(0)
        torch.cuda.synchronize()
        assert torch.equal(ov[0], want[0][0])
