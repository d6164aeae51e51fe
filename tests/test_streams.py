"""Calls on two streams at once, each with its own workspace.

A call keeps all of its state in its own workspace and outputs (the epoch
that tags its hand-off words comes from an atomic counter), and no block of
one launch waits for another block, so calls on different streams may run
side by side on the device.  Two different calls, segmented and serial, and
two calls of the same segmented shape, are launched on two streams without
a wait in between, three times, and must give the bits each gives alone."""
import pytest

import kda_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _setup(w, cp, seg):
    import kimi_delta_attention_02_amd as kda
    from tests.gpu_util import dev_inputs

    x = kda_inputs.make_inputs(w)
    d = dev_inputs(x)
    ws = torch.empty(kda.get_workspace_size(w.B * w.T, w.H, w.N, cp, seg), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(d["q"])
    fin = torch.empty((w.N, w.H, 128, 128), dtype=torch.float32, device="cuda")

    def call(o, f):
        kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], x["scale"], o, A_log=d["A_log"], dt_bias=d["dt_bias"],
                lower_bound=x["lower_bound"], workspace=ws, initial_state=d["initial_state"], final_state=f,
                cu_seqlens=d["cu_seqlens"], cp_mode=cp, seg_chunks=seg)

    return call, out, fin


@pytest.mark.parametrize("pair", ["different", "same_shape"])
def test_two_streams_give_the_bits_of_separate_calls(pair):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wa = kda_inputs.custom(seqlens=[3000, 90, 2570], H=8, lower_bound=-1.0, seed=61, name="stream a")
    if pair == "different":
        wb = kda_inputs.custom(B=2, T=2900, H=8, lower_bound=-3.0, seed=62, name="stream b")
        cb = _setup(wb, "auto", 0)
    else:
        wb = kda_inputs.custom(seqlens=[3000, 90, 2570], H=8, lower_bound=-0.1, seed=63, name="stream b")
        cb = _setup(wb, "force", 16)
    ca = _setup(wa, "force", 16)
    refs = []
    for call, out, fin in (ca, cb):  # alone, one after the other
        call(out, fin)
        torch.cuda.synchronize()
        refs.append((out.clone(), fin.clone()))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        for _, out, fin in (ca, cb):
            out.fill_(float("nan"))
            fin.fill_(float("nan"))
        torch.cuda.synchronize()
        for (call, out, fin), s in ((ca, s1), (cb, s2)):
            with torch.cuda.stream(s):
                call(out, fin)
        torch.cuda.synchronize()
        for (_, out, fin), (o_ref, f_ref) in zip((ca, cb), refs):
            assert torch.equal(out.view(torch.int16), o_ref.view(torch.int16)), f"rep {rep}: output differs"
            assert torch.equal(fin, f_ref), f"rep {rep}: final state differs"
