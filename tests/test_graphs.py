"""The library enqueues kernels only (no allocation, memset or synchronisation
inside a call), so a caller can capture its calls into a HIP graph.  These
GPU tests capture the forward + backward (on a shared workspace) and the
Gram selection + cascade through torch's graph API, replay each graph
several times with eager work and synchronisation in between (outputs
refilled with NaN), and check every replay bit for bit against an eager run
of the same calls (the kernels are deterministic).
"""
import numpy as np
import pytest

from bwd_rope_apply_amd import workloads as W
import harness as Hn

pytestmark = pytest.mark.gpu


def _capture_and_replay(run, outs, replays=3):
    import torch
    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on a side stream, as torch recommends before capture
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for i in range(replays):
        for t in outs:
            if t.is_floating_point():
                t.fill_(float("nan"))
            else:
                t.fill_(7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, (x, y) in enumerate(zip(outs, ref)):
            assert torch.equal(x, y), (i, k)
    return ref


def test_attention_graph_replays():
    import torch
    from bwd_rope_apply_amd import _lib
    wl = W.get("long_8k", B=1, H=2, N=700)
    inp = W.make_inputs(wl)
    q, k, v, do = (Hn.to_device(getattr(inp, n)) for n in ("q", "k", "v", "do"))
    a = Hn.to_device(inp.alpha)
    B, H, N, D = 1, 2, 700, 128
    f32 = dict(dtype=torch.float32, device="cuda")
    o, lse = torch.empty((B, H, N, D), **f32), torch.empty((B, H, N), **f32)
    dq, dk, dv = (torch.empty((B, H, N, D), **f32) for _ in range(3))
    da = torch.empty((D // 2,), **f32)
    ws = torch.empty(_lib.workspace_bytes("bwd", B, H, N, D, _lib.BF16, True), dtype=torch.uint8,
                     device="cuda")
    bwd_stages = _lib.STAGE_ALL & ~_lib.STAGE_PREP | _lib.STAGE_PREP_GRAD

    def run():
        _lib.fwd(q, k, v, wl.base, a, True, workspace=ws, out=(o, lse))
        _lib.bwd(q, k, v, o, do, lse, wl.base, a, True, workspace=ws, out=(dq, dk, dv, da),
                 stages=bwd_stages)

    ref = _capture_and_replay(run, [o, lse, dq, dk, dv, da])
    for t in ref:
        assert torch.isfinite(t).all()


def test_gram_graph_replays():
    import torch
    from bwd_rope_apply_amd import _lib
    wl = W.get_tokens("gram_gptj_512")
    x0s, x1s = (a[0] for a in W.make_tokens(wl, layers=2))
    x0, x1 = Hn.to_device(x0s), Hn.to_device(x1s)
    T, d = wl.T, wl.d
    lib = _lib.load()
    ws = torch.empty(int(lib.gram_select_workspace_bytes(1, T, d)), dtype=torch.uint8, device="cuda")
    wsc = torch.empty(int(lib.gram_cascade_workspace_bytes(T, d)), dtype=torch.uint8, device="cuda")
    m = torch.empty((1, T), dtype=torch.float32, device="cuda")
    rep = torch.empty((1, T), dtype=torch.uint8, device="cuda")
    cnt = torch.empty((1,), dtype=torch.int32, device="cuda")
    mc = torch.empty((T,), dtype=torch.float32, device="cuda")
    repc = torch.empty((T,), dtype=torch.uint8, device="cuda")
    cntc = torch.empty((1,), dtype=torch.int32, device="cuda")

    def run():
        _lib.gram_select(x0, wl.tau, workspace=ws, out=(m, rep, cnt))
        _lib.gram_cascade(x1, wl.tau, rep[0], workspace=wsc, out=(mc, repc, cntc))

    ref = _capture_and_replay(run, [m, rep, cnt, mc, repc, cntc])
    assert int(ref[2][0]) == int(ref[1].sum()) and int(ref[5][0]) == int(ref[4].sum())
    assert np.isfinite(ref[0].cpu().numpy()[0, 1:]).all()
