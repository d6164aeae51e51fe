"""The chunk_kda call (flash-linear-attention's name and flags) on top of fwd,
and the caller's state in either layout ([v][k] or [k][v] per head)."""
import numpy as np
import pytest

import kda_inputs
import kimi_delta_attention_02_amd as kda

torch = pytest.importorskip("torch")


def test_unsupported_flags_are_rejected_before_any_device_work():
    x = torch.zeros(1, 16, 1, 128, dtype=torch.bfloat16)  # CPU: never reached
    for flag in ("use_gate_in_kernel", "use_qk_l2norm_in_kernel", "use_beta_sigmoid_in_kernel", "safe_gate"):
        with pytest.raises(ValueError, match=flag):
            kda.chunk_kda(x, x, x, x, x[..., 0], A_log=None, dt_bias=None, lower_bound=-1.0, **{flag: False})


@pytest.mark.gpu
@pytest.mark.parametrize("sdt", ["fp32", "bf16"])
@pytest.mark.parametrize("cp", ["off", "force"])
def test_state_layouts_agree_bit_for_bit(sdt, cp):
    """transpose_state_layout=False takes and returns the transposed states;
    the output and the (transposed) final state equal the [v][k] call's bits,
    on the serial path and on the segmented one (whose final state can come
    from the first pass's R: lb = -5 decays fast)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests.gpu_util import check_against_oracle, dev_inputs

    w = kda_inputs.custom(seqlens=[400, 37, 260], H=2, lower_bound=-5.0, state_dtype=sdt, seed=41,
                          name=f"layouts {sdt} {cp}")
    x = kda_inputs.make_inputs(w)
    d = dev_inputs(x)
    common = dict(A_log=d["A_log"], dt_bias=d["dt_bias"], lower_bound=x["lower_bound"], cu_seqlens=d["cu_seqlens"],
                  cp_mode=cp)
    o1, f1 = kda.chunk_kda(d["q"], d["k"], d["v"], d["g"], d["beta"], x["scale"], d["initial_state"], True,
                           **common)
    init_kv = d["initial_state"].transpose(-1, -2).contiguous()
    o2, f2 = kda.chunk_kda(d["q"], d["k"], d["v"], d["g"], d["beta"], x["scale"], init_kv, True,
                           transpose_state_layout=False, **common)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(f1, f2.transpose(-1, -2))
    check_against_oracle(w, x, o1, f1, final_dtype=sdt)


@pytest.mark.gpu
def test_chunk_kda_matches_fwd_and_final_only():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests.gpu_util import dev_inputs

    w = kda_inputs.custom(B=2, T=100, H=2, lower_bound=-1.0, seed=42, name="chunk_kda")
    x = kda_inputs.make_inputs(w)
    d = dev_inputs(x)
    o, f = kda.chunk_kda(d["q"], d["k"], d["v"], d["g"], d["beta"], x["scale"], None, True, A_log=d["A_log"],
                         dt_bias=d["dt_bias"], lower_bound=x["lower_bound"])
    assert f.dtype == torch.float32 and f.shape == (2, 2, 128, 128)
    fin = torch.empty_like(f)
    o_ref = kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], x["scale"], A_log=d["A_log"], dt_bias=d["dt_bias"],
                    lower_bound=x["lower_bound"], final_state=fin)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)) and torch.equal(f, fin)
    o2, f2 = kda.chunk_kda(d["q"], d["k"], d["v"], d["g"], d["beta"], A_log=d["A_log"], dt_bias=d["dt_bias"],
                           lower_bound=x["lower_bound"])
    assert f2 is None and o2.shape == o.shape


@pytest.mark.gpu
@pytest.mark.parametrize("sdt", ["fp32", "bf16"])
@pytest.mark.parametrize("layout", ["vk", "kv"])
def test_final_state_decided_at_checkpoint(sdt, layout):
    """Segments of 6 chunks, past the 4-chunk checkpoint, with fast decay
    (lb = -5): the second pass decides every such segment at its checkpoint, and
    for the last segment of a sequence (the 480-token one) the final state is
    then the first pass's zero-start state R, written straight into the caller's
    dtype and layout.  The 200-token sequence ends in a 1-chunk segment with no
    checkpoint, which the second pass runs whole.  Output and final state equal
    the serial call's bits and the oracle."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests.gpu_util import check_against_oracle, dev_inputs, read_ws

    w = kda_inputs.custom(seqlens=[480, 96, 200], H=2, lower_bound=-5.0, state_dtype=sdt, seed=43,
                          name=f"checkpoint final {sdt} {layout}")
    x = kda_inputs.make_inputs(w)
    d = dev_inputs(x)
    init = d["initial_state"] if layout == "vk" else d["initial_state"].transpose(-1, -2).contiguous()
    st = torch.float32 if sdt == "fp32" else torch.bfloat16

    def call(cp, seg):
        final = torch.full((w.N, w.H, 128, 128), float("nan"), dtype=st, device="cuda")
        ws = torch.empty(kda.get_workspace_size(w.B * w.T, w.H, w.N, cp, seg), dtype=torch.uint8, device="cuda")
        out = kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], x["scale"], A_log=d["A_log"], dt_bias=d["dt_bias"],
                      lower_bound=x["lower_bound"], workspace=ws, initial_state=init, final_state=final,
                      cu_seqlens=d["cu_seqlens"], cp_mode=cp, seg_chunks=seg, state_layout=layout)
        torch.cuda.synchronize()
        return out, final, ws

    o_ser, f_ser, _ = call("off", 0)
    o_seg, f_seg, ws = call("force", 6)
    offs = kda.workspace_offsets(w.B * w.T, w.H, w.N, "force", 6)
    stops = int(read_ws(ws, offs, "counters", 4, np.int32)[3])
    # checkpointed segments: 4 of the 480-token sequence, 1 of the 200-token one; per head
    assert stops == 5 * w.H, stops
    assert torch.equal(o_seg.view(torch.int16), o_ser.view(torch.int16))
    assert torch.equal(f_seg.view(torch.int16) if sdt == "bf16" else f_seg,
                       f_ser.view(torch.int16) if sdt == "bf16" else f_ser)
    f_vk = f_seg if layout == "vk" else f_seg.transpose(-1, -2).contiguous()
    check_against_oracle(w, x, o_seg, f_vk, final_dtype=sdt)
