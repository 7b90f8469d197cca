"""The library inside a captured HIP graph: one gemm_bf16 call (split K with
its reduction kernel, an unsplit call, and a hybrid plan) captured once on a
stream whose workspace was reserved beforehand, then replayed several times
with new integer inputs copied into the captured buffers between replays,
eager work and synchronisations in between; every replay must equal the
oracle bit for bit.  Nothing in the path allocates, synchronises or records a
memset, so the captured launches are the whole call."""
import numpy as np
import pytest

from synthetic_inputs import int_bf16

pytestmark = pytest.mark.gpu


# a split-K plan (GEMM + reduction), an unsplit one, and a hybrid plan (a
# split launch for the last tile columns, its reduction, then the unsplit
# launch for the rest)
@pytest.mark.parametrize("shape", [(256, 8192, 2048), (512, 512, 512), (300, 11008, 2048)])
def test_graph_replays_match_oracle(shape):
    import torch

    import dense_gemm_bf16_amd as g
    import oracle

    M, N, K = shape
    plan = g.config_name(M, N, K)
    print(shape, plan, flush=True)
    if M == 300:
        assert "_h" in plan, plan
    s = torch.cuda.Stream()
    g.reserve_workspace(max(g.workspace_size(M, N, K), 256), s)
    dA = torch.zeros((M, K), dtype=torch.int16, device="cuda")
    dB = torch.zeros((N, K), dtype=torch.int16, device="cuda")
    dC = torch.zeros((M, N), dtype=torch.int16, device="cuda")
    with torch.cuda.stream(s):
        g.gemm_bf16(M, N, K, dA, K, dB, K, dC, N)  # eager call on the capture stream
    s.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        g.gemm_bf16(M, N, K, dA, K, dB, K, dC, N)
    torch.cuda.synchronize()
    for rep in range(3):
        A = int_bf16(M, K, seed=800 + 2 * rep)
        B = int_bf16(N, K, seed=801 + 2 * rep)
        dA.copy_(torch.from_numpy(A.view(np.int16)))
        dB.copy_(torch.from_numpy(B.view(np.int16)))
        dC.fill_(0x7FC0)  # NaN everywhere, so a missed store shows
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref16, _ = oracle.gemm(A, B)
        got = dC.cpu().numpy().view(np.uint16)
        bad = int(np.count_nonzero(got != ref16))
        print(shape, "replay", rep, "mismatches", bad, flush=True)
        assert bad == 0, (shape, rep, bad)


# The refused call enqueues nothing, so torch warns that the graph it captured is empty.
@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")
def test_capture_that_needs_a_larger_workspace_is_refused():
    """A call captured on a stream whose workspace is too small returns
    GEMM_ERR_CAPTURE without allocating, synchronising or enqueueing, so the
    capture itself stays valid; the same call made eagerly afterwards
    allocates and is exact."""
    import torch

    import dense_gemm_bf16_amd as g
    import oracle

    # larger partials than the other tests reserve on any stream (torch hands
    # out its streams from a pool, so this stream may have been used before)
    M, N, K = 256, 12800, 4608
    assert g.workspace_size(M, N, K) > 32 << 20
    A = int_bf16(M, K, seed=850)
    B = int_bf16(N, K, seed=851)
    dA = torch.from_numpy(A.view(np.int16)).cuda()
    dB = torch.from_numpy(B.view(np.int16)).cuda()
    dC = torch.zeros((M, N), dtype=torch.int16, device="cuda")
    s = torch.cuda.Stream()  # a new stream: no workspace reserved for it
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        rc = g.gemm_bf16_status(M, N, K, dA, K, dB, K, dC, N, stream=s.cuda_stream)
    print("status under capture", rc, g.status_string(rc), flush=True)
    assert rc == g.GEMM_ERR_CAPTURE
    with torch.cuda.stream(s):
        g.gemm_bf16(M, N, K, dA, K, dB, K, dC, N, stream=s)
    torch.cuda.synchronize()
    ref16, _ = oracle.gemm(A, B)
    assert np.array_equal(dC.cpu().numpy().view(np.uint16), ref16)
