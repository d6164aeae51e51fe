"""A kda_fwd call captured in a HIP graph and replayed.

The call allocates nothing, never synchronises and records no memset (the
index kernel clears the counters itself), so it can be captured.  Every
replay is checked against an eager call on the same inputs, with the
program's own eager work and synchronisations between the replays.  The eager
reference calls run on the graph's own workspace, or on a workspace of their
own, so that the graph's workspace sees only replays back to back: a replay
keeps the captured call's epoch, and the flags each replay leaves behind must
not pass for the next one's (the second pass clears them).  At lower bound
-0.1 no segment's transition vanishes, and every replay merges and reruns."""
import pytest

import kda_inputs
import kimi_delta_attention_02_amd as kda

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cp,ref_ws,lb", [("off", "same", -5.0), ("force", "same", -5.0),
                                          ("force", "separate", -5.0), ("force", "separate", -0.1)])
def test_graph_replays_equal_eager_calls(cp, ref_ws, lb):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests.gpu_util import dev_inputs

    w = kda_inputs.custom(seqlens=[300, 90, 257], H=2, lower_bound=lb, seed=51, name=f"graph {cp}")
    d = dev_inputs(kda_inputs.make_inputs(w))
    x = kda_inputs.make_inputs(w)
    N, H = w.N, w.H
    ws = torch.empty(kda.get_workspace_size(w.B * w.T, H, N, cp, 5), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(d["q"])
    fin = torch.empty((N, H, 128, 128), dtype=torch.float32, device="cuda")
    init = d["initial_state"].clone()

    ws_ref = ws if ref_ws == "same" else torch.empty_like(ws)

    def call(o, f, wsp=ws):
        kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], x["scale"], o, A_log=d["A_log"], dt_bias=d["dt_bias"],
                lower_bound=x["lower_bound"], workspace=wsp, initial_state=init, final_state=f,
                cu_seqlens=d["cu_seqlens"], cp_mode=cp, seg_chunks=5)

    call(out, fin)  # warm up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(out, fin)
    gen = torch.Generator(device="cuda").manual_seed(7)
    for rep in range(3):
        # new inputs in the captured buffers, eager work, then the replay
        for name in ("q", "k", "v"):
            d[name].copy_(torch.randn(d[name].shape, generator=gen, device="cuda").to(torch.bfloat16))
        init.copy_(0.05 * torch.randn(init.shape, generator=gen, device="cuda"))
        _ = (d["q"].float() * 2).sum()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        o_ref = torch.empty_like(out)
        f_ref = torch.empty_like(fin)
        call(o_ref, f_ref, ws_ref)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), o_ref.view(torch.int16)), f"replay {rep}: output differs"
        assert torch.equal(fin, f_ref), f"replay {rep}: final state differs"
