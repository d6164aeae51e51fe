"""Grouped value heads: H heads for v, g, beta, out and the states, and
H_qk < H heads for q and k, head h reading q/k head h // (H // H_qk).  The
reading taken of "HV > H" on the cuLA PR #106 page: a grouped call is the
same computation as a plain call whose q and k repeat each q/k head over its
group, so it must give the same bits, and both match the oracle on the
expanded inputs."""
import numpy as np
import pytest

import kda_inputs
import kimi_delta_attention_02_amd as kda

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("H,Hqk,cp", [(4, 2, "off"), (4, 1, "force"), (6, 3, "force")])
def test_grouped_heads_equal_repeated_qk(H, Hqk, cp):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests.gpu_util import check_against_oracle, dev_inputs

    w = kda_inputs.custom(seqlens=[300, 45, 200], H=H, lower_bound=-2.0, seed=61, name=f"gva {H}/{Hqk} {cp}")
    x = kda_inputs.make_inputs(w)
    grp = H // Hqk
    lead = list(range(0, H, grp))  # one q/k head per group
    rep = [h // grp * grp for h in range(H)]  # the group leader of each head
    xg = dict(x)
    for n in ("q", "k"):
        xg[n] = np.ascontiguousarray(x[n][:, :, rep])  # plain call: q/k repeated over each group
    d = dev_inputs(xg)
    common = dict(A_log=d["A_log"], dt_bias=d["dt_bias"], lower_bound=x["lower_bound"], cu_seqlens=d["cu_seqlens"],
                  cp_mode=cp)
    f1 = torch.empty((w.N, H, 128, 128), dtype=torch.float32, device="cuda")
    o1 = kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], x["scale"], initial_state=d["initial_state"],
                 final_state=f1, **common)
    qg = d["q"][:, :, lead].contiguous()
    kg = d["k"][:, :, lead].contiguous()
    f2 = torch.empty_like(f1)
    o2 = kda.fwd(qg, kg, d["v"], d["g"], d["beta"], x["scale"], initial_state=d["initial_state"], final_state=f2,
                 **common)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(f1, f2)
    check_against_oracle(w, xg, o2, f2, final_dtype="fp32")
