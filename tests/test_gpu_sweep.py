"""Seeded random sweep of the forward call against the fp64 oracle.

Each case draws its shape and options from one counter-based seed: fixed
length or varlen (lengths 0, 1-16, whole chunks, or ragged up to 2048), H and a grouped
q/k head count, the lower bound, scale, state dtype, layout, presence and
aliasing, and the plan (serial, forced segments of 1-12 chunks, or the
library's own).  Every chain of every case is compared with the oracle (the
token recurrence), with the tolerance of the other parity tests, and the
prepared call and the no-allocation entry point must give the same bits as
fwd.  The sizes keep the oracle to about a second per case."""
import math

import numpy as np
import pytest

import kda_inputs
from tests.gpu_util import check_against_oracle, dev_inputs, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SWEEP_SEED = 20261203
N_CASES = 96


def _draw_case(i):
    rng = np.random.Generator(np.random.PCG64([SWEEP_SEED, i]))

    def length():
        r = rng.random()
        if r < 0.1:
            return 0
        if r < 0.3:
            return int(rng.integers(1, 17))
        if r < 0.5:
            return 16 * int(rng.integers(1, 24))
        if r < 0.6:
            return int(rng.integers(640, 2049))
        return int(rng.integers(17, 640))

    varlen = bool(rng.random() < 0.6)
    H = int(rng.choice([1, 2, 3, 4, 6, 8]))
    Hqk = H if rng.random() < 0.6 else int(rng.choice([d for d in range(1, H + 1) if H % d == 0]))
    if varlen:
        lens = [length() for _ in range(int(rng.integers(1, 6)))]
        if sum(lens) == 0:
            lens[0] = int(rng.integers(1, 40))
        B, T = 1, sum(lens)
    else:
        B, T = int(rng.integers(1, 4)), max(1, length())
        lens = None
    lb = float(rng.choice([-5.0, -3.0, -1.0, -0.3, 0.0, float(np.float32(rng.uniform(-5.0, 0.0)))]))
    init = bool(rng.random() < 0.7)
    final = bool(rng.random() < 0.8)
    cp = str(rng.choice(["off", "force", "auto"]))
    return dict(
        varlen=varlen, lens=lens, B=B, T=T, H=H, Hqk=Hqk, lb=lb,
        scale=float(rng.choice([0.125, 1.0 / math.sqrt(128.0), 0.3])),
        sdt=str(rng.choice(["fp32", "bf16"])), layout=str(rng.choice(["vk", "kv"])),
        init=init, final=final, alias=bool(init and final and rng.random() < 0.3),
        cp=cp, seg=int(rng.integers(1, 13)) if cp == "force" and rng.random() < 0.8 else 0,
    )


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case_matches_oracle(i):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kimi_delta_attention_02_amd as kda

    c = _draw_case(i)
    say(f"sweep case {i}: {c}")
    w = kda_inputs.custom(B=c["B"], T=c["T"], H=c["H"], seqlens=c["lens"], lower_bound=c["lb"], scale=c["scale"],
                          init_std=0.05 if c["init"] else None, state_dtype=c["sdt"], want_final=c["final"],
                          seed=1000 + i, name=f"sweep{i}")
    x = kda_inputs.make_inputs(w)
    H, Hqk = c["H"], c["Hqk"]
    grp = H // Hqk
    lead = list(range(0, H, grp))  # the q/k head each group reads
    rep = [h // grp * grp for h in range(H)]
    xg = dict(x)
    for n in ("q", "k"):  # what the oracle sees: each group's q/k head repeated over the group
        xg[n] = np.ascontiguousarray(x[n][:, :, rep])
    d = dev_inputs(xg)
    q = d["q"][:, :, lead].contiguous()
    k = d["k"][:, :, lead].contiguous()
    kv = c["layout"] == "kv"
    sdt = torch.float32 if c["sdt"] == "fp32" else torch.bfloat16
    init = d["initial_state"]
    if init is not None and kv:
        init = init.transpose(-1, -2).contiguous()
    final = None
    if c["final"]:
        if c["alias"]:
            init = init.clone()
            final = init
        else:
            final = torch.full((w.N, H, 128, 128), float("nan"), dtype=sdt, device="cuda")
    out = kda.fwd(q, k, d["v"], d["g"], d["beta"], x["scale"], A_log=d["A_log"], dt_bias=d["dt_bias"],
                  lower_bound=x["lower_bound"], initial_state=init, final_state=final, cu_seqlens=d["cu_seqlens"],
                  cp_mode=c["cp"], seg_chunks=c["seg"], state_layout=c["layout"], check=True)
    torch.cuda.synchronize()
    fin_vk = None
    if final is not None:
        fin_vk = final.transpose(-1, -2).contiguous() if kv else final
    check_against_oracle(w, xg, out, fin_vk, init=c["init"], final_dtype=c["sdt"])
    if c["alias"]:
        return  # a repeated call would start from the state the first one wrote
    # the prepared call and the no-allocation entry point give the same bits
    args = dict(A_log=d["A_log"], dt_bias=d["dt_bias"], lower_bound=x["lower_bound"], initial_state=init,
                cu_seqlens=d["cu_seqlens"], cp_mode=c["cp"], seg_chunks=c["seg"], state_layout=c["layout"])
    f2 = torch.full_like(final, float("nan")) if final is not None else None
    prep = kda.prepare(q, k, d["v"], d["g"], d["beta"], x["scale"], final_state=f2, **args)
    out2 = prep()
    f3 = torch.full_like(final, float("nan")) if final is not None else None
    out3 = torch.full_like(out, float("nan"))
    if kda.get_workspace_size(w.B * w.T, H, w.N, c["cp"], c["seg"]) <= kda.NOALLOC_SCRATCH_BYTES:
        kda.fwd_noalloc(q, k, d["v"], d["g"], d["beta"], x["scale"], out3, final_state=f3, **args)
    else:
        out3, f3 = out2, f2
    torch.cuda.synchronize()
    for o, f in ((out2, f2), (out3, f3)):
        assert torch.equal(o.view(torch.int16), out.view(torch.int16))
        if final is not None:
            assert torch.equal(f.view(torch.int16) if f.dtype == torch.bfloat16 else f,
                               final.view(torch.int16) if final.dtype == torch.bfloat16 else final)
