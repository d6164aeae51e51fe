"""The no-allocation entry point (kda_fwd_noalloc) against kda_fwd.

Both run the same kernels on the same plan, so their results must agree bit
for bit.  Two calls in a row, the second smaller, so that the second one runs
over the scratch array the first left behind (nothing in it may be assumed to
start at zero).  Both also stay within the oracle's tolerance.  A skewed
varlen batch of 256 chains shows that the array counts as room for the
automatic plan's split, as a kda_fwd workspace of the segmented size does."""
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


def _both(w, cp_mode, seg_chunks, heads, groups=None):
    """groups: lists of sequences compared with the oracle separately (each
    against its own RMS); by default all at once."""
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
    for seqs in groups or [None]:
        check_against_oracle(w, x, o2, f2, seqs=seqs, heads=heads, final_dtype=w.state_dtype)
    return x, d, o2


def test_noalloc_equals_fwd_two_calls_second_smaller():
    # 1: B=2 T=4096 H=16, fp32 states, the automatic segment plan (about 90 MiB of scratch)
    _both(kda_inputs.WORKLOADS["cfg2"], "auto", 0, heads=[0, 15])
    # 2: a smaller varlen call over the same scratch, bf16 states, forced short segments
    w = kda_inputs.custom(seqlens=[300, 17, 0, 520], H=4, lower_bound=-1.0, state_dtype="bf16", seed=41,
                          name="noalloc_varlen4_H4")
    _both(w, "force", 3, heads=None)


def test_noalloc_splits_a_skewed_batch_like_fwd():
    import kimi_delta_attention_02_amd as kda

    # one 3000-token sequence among 255 of 4 tokens, H = 1: 256 chains, which the
    # automatic plan keeps serial unless the workspace holds the segmented layout
    # (89 MiB here, within the array; fwd allocates it for such calls).  At lower
    # bound 0 the segmented result differs from the serial one in its low bits,
    # so equal bits mean that both calls took the split.  Without decay the long
    # sequence's state grows to ~6 times the short ones' RMS, so the two kinds are
    # held to the oracle's tolerance each against their own RMS.
    lens = [3000] + [4] * 255
    assert kda.varlen_seg_choice(lens, 1) == (16, True)
    assert kda.get_workspace_size(sum(lens), 1, len(lens), "force", 0) <= kda.NOALLOC_SCRATCH_BYTES
    w = kda_inputs.custom(seqlens=lens, H=1, lower_bound=0.0, state_dtype="fp32", seed=47,
                          name="noalloc_skewed_256x1")
    x, d, o2 = _both(w, "auto", 0, heads=None, groups=[[0], list(range(1, len(lens)))])
    serial = torch.full_like(o2, float("nan"))
    kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], x["scale"], serial, A_log=d["A_log"], dt_bias=d["dt_bias"],
            lower_bound=x["lower_bound"], initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"], cp_mode="off",
            check=True)
    torch.cuda.synchronize()
    assert not torch.equal(serial.view(torch.int16), o2.view(torch.int16))
