"""Split-K calls on several streams at once, workspace growth while work is
still queued, and release followed by reuse.

The C interface keeps one split-K workspace per (device, stream), so calls
on different streams may overlap on the GPU, and a buffer they shared would
mix their partial sums.  Growth retires the old buffer without freeing it,
so a call already queued on the stream still writes valid memory.  Integer
inputs make every result exact (fp32 sums of products of small integers), so
each output is compared with the oracle bit for bit."""
import numpy as np
import pytest

from synthetic_inputs import int_bf16

pytestmark = pytest.mark.gpu

# The 256 x 128 direct-to-LDS tile with K split k ways (fixed-order reduction).
SPLIT = "t256x128x64_w2x2_s3_x3_p10_k{}_g4"


def _case(M, N, K, seed):
    import torch

    import oracle

    A = int_bf16(M, K, seed=seed)
    B = int_bf16(N, K, seed=seed + 1)
    ref16, _ = oracle.gemm(A, B, want_f64=False)
    dA = torch.from_numpy(A.view(np.int16)).cuda()
    dB = torch.from_numpy(B.view(np.int16)).cuda()
    return dA, dB, ref16


def _mismatches(dC, ref16):
    return int(np.count_nonzero(dC.cpu().numpy().view(np.uint16) != ref16))


def test_split_k_on_two_streams_at_once():
    """Two streams, each with its own split-K shape and inputs, enqueued
    alternately with no synchronisation between the calls; every call writes
    its own output buffer, and all of them must be exact."""
    import torch

    import dense_gemm_bf16_amd as g

    shapes = [(256, 1024, 2048, 4, 900), (200, 1000, 1536, 3, 910)]
    cases = [_case(M, N, K, seed) for M, N, K, _, seed in shapes]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    reps = 12
    outs = [[torch.empty((M, N), dtype=torch.int16, device="cuda") for _ in range(reps)]
            for M, N, _, _, _ in shapes]
    torch.cuda.synchronize()
    for r in range(reps):
        for (M, N, K, splits, _), (dA, dB, _), s, out in zip(shapes, cases, streams, outs):
            g.gemm_bf16_ex(SPLIT.format(splits), M, N, K, dA, K, dB, K, out[r], N, stream=s)
    torch.cuda.synchronize()
    for (M, N, K, splits, _), (_, _, ref16), out in zip(shapes, cases, outs):
        bad = [_mismatches(c, ref16) for c in out]
        print((M, N, K), "split", splits, "mismatches per call", bad, flush=True)
        assert not any(bad), ((M, N, K), bad)


def test_workspace_growth_with_work_queued_then_release_and_reuse():
    """On one stream with no workspace: a small split call, then, before it
    can have finished, one that needs a larger workspace (the library
    allocates a new buffer and keeps the old one for the queued call), then
    the small call again.  Then every workspace is released and the large
    call runs once more on the same stream."""
    import torch

    import dense_gemm_bf16_amd as g

    g.release_workspace()  # no stream starts with a workspace
    small = (256, 512, 2048, 4)
    large = (256, 2048, 2048, 4)
    assert g.workspace_size(*large[:3]) > g.workspace_size(*small[:3]) > 0
    ds = _case(*small[:3], seed=920)
    dl = _case(*large[:3], seed=930)
    s = torch.cuda.Stream()
    outs = [torch.empty((M, N), dtype=torch.int16, device="cuda")
            for M, N, _, _ in (small, large, small, large)]
    torch.cuda.synchronize()

    def call(shape, case, out):
        M, N, K, splits = shape
        dA, dB, _ = case
        g.gemm_bf16_ex(SPLIT.format(splits), M, N, K, dA, K, dB, K, out, N, stream=s)

    call(small, ds, outs[0])
    call(large, dl, outs[1])  # grows the workspace while the first call is queued
    call(small, ds, outs[2])
    torch.cuda.synchronize()
    g.release_workspace()
    call(large, dl, outs[3])  # allocates again
    torch.cuda.synchronize()
    bad = [_mismatches(o, c[2]) for o, c in zip(outs, (ds, dl, ds, dl))]
    print("mismatches small, large, small, large after release:", bad, flush=True)
    assert not any(bad), bad
