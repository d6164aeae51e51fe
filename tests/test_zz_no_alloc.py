"""The no-allocation entry point (kda_fwd_noalloc) against kda_fwd.

Both run the same kernels on the same plan, so their results must agree bit
for bit.  Two calls in a row, the second smaller, so that the second one runs
over the scratch array the first left behind (nothing in it may be assumed to
start at zero).  Both also stay within the oracle's tolerance."""
import pytest

import kda_inputs
from tests.gpu_util import check_against_oracle, dev_inputs, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kimi_delta_attention_02_amd as kda

    kda.load_library()


def _both(w, cp_mode, seg_chunks, heads):
    import kimi_delta_attention_02_amd as kda

    say(f"case noalloc {w.name} cp={cp_mode} seg={seg_chunks}")
    x = kda_inputs.make_inputs(w)
    d = dev_inputs(x)
    sdt = torch.float32 if w.state_dtype == "fp32" else torch.bfloat16
    need = kda.get_workspace_size(w.B * w.T, w.H, w.N, cp_mode, seg_chunks)
    assert need <= kda.NOALLOC_SCRATCH_BYTES
    res = {}
    for name in ("fwd", "noalloc"):
        out = torch.full_like(d["q"], float("nan"))
        final = torch.full((w.N, w.H, 128, 128), float("nan"), dtype=sdt, device=d["q"].device)
        kw = dict(A_log=d["A_log"], dt_bias=d["dt_bias"], lower_bound=x["lower_bound"],
                  initial_state=d["initial_state"], final_state=final, cu_seqlens=d["cu_seqlens"], cp_mode=cp_mode,
                  seg_chunks=seg_chunks)
        if name == "fwd":
            kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], x["scale"], out, check=True, **kw)
        else:
            kda.fwd_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], x["scale"], out, **kw)
        torch.cuda.synchronize()
        res[name] = (out, final)
    (o1, f1), (o2, f2) = res["fwd"], res["noalloc"]
    same_o = torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    same_f = torch.equal(f1.view(torch.int16) if sdt == torch.bfloat16 else f1.view(torch.int32),
                         f2.view(torch.int16) if sdt == torch.bfloat16 else f2.view(torch.int32))
    say(f"noalloc {w.name}: out identical={same_o} final identical={same_f}")
    assert same_o and same_f
    check_against_oracle(w, x, o2, f2, heads=heads, final_dtype=w.state_dtype)


def test_noalloc_equals_fwd_two_calls_second_smaller():
    # 1: B=2 T=4096 H=16, fp32 states, the automatic segment plan (about 90 MiB of scratch)
    _both(kda_inputs.WORKLOADS["cfg2"], "auto", 0, heads=[0, 15])
    # 2: a smaller varlen call over the same scratch, bf16 states, forced short segments
    w = kda_inputs.custom(seqlens=[300, 17, 0, 520], H=4, lower_bound=-1.0, state_dtype="bf16", seed=41,
                          name="noalloc_varlen4_H4")
    _both(w, "force", 3, heads=None)
