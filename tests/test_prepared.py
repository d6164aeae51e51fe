"""The prepared call (kda.prepare): checked and marshalled once, then launched
on each call.  It must give the bits of an fwd call on the same tensors, also
after rebind() to other tensors; and fwd(check=True) must surface what the
kernels record in the workspace counters."""
import numpy as np
import pytest

import kda_inputs
from tests.gpu_util import dev_inputs, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kimi_delta_attention_02_amd as kda

    kda.load_library()


def _same(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16)) if a.dtype == torch.bfloat16 else torch.equal(a, b)


@pytest.mark.parametrize("cp,seg", [("off", 0), ("force", 4)])
def test_prepared_call_equals_fwd_and_rebinds(cp, seg):
    import kimi_delta_attention_02_amd as kda

    w = kda_inputs.custom(B=2, T=300, H=4, lower_bound=-2.0, seed=61, name="prepared")
    say(f"case prepared {w.name} cp={cp} seg={seg}")
    x = kda_inputs.make_inputs(w)
    d = dev_inputs(x)
    final_p = torch.empty(w.N, w.H, 128, 128, dtype=torch.float32, device="cuda")
    kw = dict(A_log=d["A_log"], dt_bias=d["dt_bias"], lower_bound=x["lower_bound"], cp_mode=cp, seg_chunks=seg)
    call = kda.prepare(d["q"], d["k"], d["v"], d["g"], d["beta"], x["scale"], initial_state=d["initial_state"],
                       final_state=final_p, **kw)
    for rep in range(2):
        call()
        torch.cuda.synchronize()
        final_f = torch.empty_like(final_p)
        out_f = kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], x["scale"], initial_state=d["initial_state"],
                        final_state=final_f, check=True, **kw)
        torch.cuda.synchronize()
        assert _same(call.out, out_f) and _same(final_p, final_f), f"call {rep}"
    # other inputs of the same shapes: the prepared call follows the new tensors
    q2 = torch.flip(d["q"], dims=[1]).contiguous()
    call.rebind(q=q2)
    call()
    out_f = kda.fwd(q2, d["k"], d["v"], d["g"], d["beta"], x["scale"], initial_state=d["initial_state"],
                    final_state=torch.empty_like(final_p), **kw)
    torch.cuda.synchronize()
    assert _same(call.out, out_f)
    with pytest.raises(ValueError, match="has shape"):
        call.rebind(q=d["q"][:, :10].contiguous())
    with pytest.raises(TypeError, match="bfloat16"):
        call.rebind(k=d["k"].float())
    with pytest.raises(ValueError, match="presence"):
        call.rebind(initial_state=None)


def test_check_flag_raises_on_clamped_offsets():
    import kimi_delta_attention_02_amd as kda

    w = kda_inputs.custom(seqlens=[10, 30, 20], H=1, seed=29, name="badcu-check")
    x = kda_inputs.make_inputs(w)
    x["cu_seqlens"] = np.array([0, 40, 25, 90], dtype=np.int32)  # decreasing, and past the end
    d = dev_inputs(x)
    with pytest.raises(kda.KdaError, match="cu_seqlens was malformed"):
        kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], x["scale"], A_log=d["A_log"], dt_bias=d["dt_bias"],
                lower_bound=x["lower_bound"], cu_seqlens=d["cu_seqlens"], cp_mode="off", check=True)
    # a well-formed call passes the same check, and its counters are readable
    ws = torch.empty(kda.get_workspace_size(60, 1, 3, "off"), dtype=torch.uint8, device="cuda")
    good = torch.tensor([0, 10, 40, 60], dtype=torch.int32, device="cuda")
    kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], x["scale"], A_log=d["A_log"], dt_bias=d["dt_bias"],
            lower_bound=x["lower_bound"], cu_seqlens=good, cp_mode="off", workspace=ws, check=True)
    cnt = kda.read_counters(ws, 60, 1, 3, "off")
    assert cnt == {"chunks": 1 + 2 + 2, "segments": 3, "flags": 0, "early_stops": 0, "seg_chunks": 0,
                   "longest_first": True}  # a serial varlen plan: sequences longest first
