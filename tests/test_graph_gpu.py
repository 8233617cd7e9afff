"""HIP graph capture: the forward, the split-key path and the backward captured
in one graph (torch.cuda.CUDAGraph on ROCm records HIP graphs) and replayed
several times, with new inputs copied in and eager work between the replays;
every replay must give the eager results bit for bit (the kernels use no
atomics and no memsets, and take caller-owned workspaces)."""
import pytest

pytestmark = pytest.mark.gpu


def test_capture_and_replay_matches_eager():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import flashattention_forward_fa2_amd as fa
    dev = torch.device("cuda:0")
    B, H, N, d = 2, 4, 700, 128
    gen = torch.Generator(device=dev).manual_seed(3)
    mk = lambda *s: torch.randn(*s, device=dev, generator=gen).to(torch.bfloat16)
    q, k, v, dout = (mk(B, H, N, d) for _ in range(4))
    qd = mk(B, H, 8, d)                                            # a short query block for the split path
    out, lse = torch.empty_like(q), torch.empty(B, H, N, device=dev)
    outd, lsed = torch.empty_like(qd), torch.empty(B, H, 8, device=dev)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws_split = torch.empty(fa.splitkv_workspace_bytes(B, H, 8, N, d, 4), dtype=torch.uint8, device=dev)
    ws_bwd = torch.empty(fa.bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)

    def work():
        fa.fa_fwd(q, k, v, causal=True, out=out, lse=lse)
        fa.fa_fwd_splitkv(qd, k, v, causal=False, out=outd, lse=lsed, num_splits=4, workspace=ws_split)
        fa.fa_bwd(q, k, v, out, lse, dout, causal=True, dq=dq, dk=dk, dv=dv, workspace=ws_bwd)

    def snapshot():
        return [t.clone() for t in (out, lse, outd, lsed, dq, dk, dv)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()                                                     # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work()
    torch.cuda.synchronize()

    for rep in range(3):
        for t in (q, k, v, dout, qd):                              # new inputs in the captured buffers
            t.copy_(mk(*t.shape))
        _ = (q.float() @ k.float().transpose(-1, -2)).sum()        # unrelated eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        got = snapshot()
        work()                                                     # eager on the same inputs
        torch.cuda.synchronize()
        want = snapshot()
        for a, b in zip(got, want):
            assert torch.equal(a, b), "replay %d differs from eager" % rep
