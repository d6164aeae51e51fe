"""Calls whose tensors pass 2^31 and 2^32 elements.

Element (t, h, c) of a [tokens, H, 128] tensor lies at (H t + h) 128 + c, so
at H = 16 token 1,048,576 starts the 2^31st element of q, k, v, g and out, and
token 2,097,152 the 2^32nd: every address past them needs 64-bit arithmetic
(the beta, state and table offsets stay far below).  One fixed-length batch
of 528 rows of 4,000 tokens (2,112,000 tokens; 8.65 GB per bf16 tensor,
about 60 GB of device memory in all) is drawn on the device from a seeded
generator, and run
  - on the library's own plan (8,448 chains: serial) and on 128-chunk
    segments, which must give the same bits over the whole output and final
    state (the gate's lower bound is -5, as for the 64K workload);
  - as one varlen call over the same memory, with ragged sequence lengths
    (the index tables then take the two-launch form: 132,000 chunk rows).
In each call the chains that cross those two boundaries, and the last one,
are compared with the fp64 oracle (the token recurrence) on three heads, from
host copies of just their inputs.

Two more limits: the largest head count the interface accepts (65535, so that
a token's row of H x 128 elements stays under the 2^24 of the kernels' 24-bit
row multiplies), fixed length and varlen; and 300,000 ragged sequences at one
head (a grid of as many chains, and the two-launch index tables)."""
import numpy as np
import pytest

import kda_inputs
from tests.gpu_util import check_against_oracle, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

B, T, H, D = 528, 4000, 16, 128
EDGE_TOKENS = ((1 << 31) // (H * D), (1 << 32) // (H * D))
HEADS = [0, 9, 15]
NEED_BYTES = 70 << 30


@pytest.fixture(scope="module")
def big():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    free, _ = torch.cuda.mem_get_info()
    if free < NEED_BYTES:
        pytest.skip(f"needs {NEED_BYTES >> 30} GiB of free device memory, {free >> 30} GiB free")
    w = kda_inputs.custom(B=B, T=T, H=H, lower_bound=-5.0, init_std=0.05, state_dtype="fp32", seed=41,
                          name="kda_fwd_B528_T4000_H16")
    say(f"drawing {w.name} on the device ({B * T} tokens, {B * T * H * D} elements per tensor)")
    d = kda_inputs.make_device_inputs(w, "cuda")
    d["A_log_dev"] = torch.from_numpy(d["A_log"]).cuda()
    d["dt_bias_dev"] = torch.from_numpy(d["dt_bias"]).cuda()
    torch.cuda.synchronize()
    yield w, d
    d.clear()
    torch.cuda.empty_cache()


def _flat(t):
    return t.view((1, -1) + tuple(t.shape[2:]))


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _call(d, q, k, v, g, beta, init, final, cu=None, cp_mode="auto", seg_chunks=0):
    import kimi_delta_attention_02_amd as kda

    out = torch.full_like(q, float("nan"))
    kda.fwd(q, k, v, g, beta, d["scale"], out, A_log=d["A_log_dev"], dt_bias=d["dt_bias_dev"],
            lower_bound=d["lower_bound"], initial_state=init, final_state=final, cu_seqlens=cu, cp_mode=cp_mode,
            seg_chunks=seg_chunks, check=True)
    torch.cuda.synchronize()
    return out


def _check_spans(name, d, out, final, spans, heads=HEADS, n_heads=H, init=None):
    """spans: (state index, first token in the flattened token order, length)
    of the chains to compare; their inputs are copied to the host and run
    through the oracle as one varlen problem (init: the initial states, by
    default the inputs' own)."""
    lens = [L for _, _, L in spans]
    x = {}
    for n in ("q", "k", "v", "g", "beta"):
        f = _flat(d[n])
        x[n] = np.concatenate([_bits(f[:, t0:t0 + L]) for _, t0, L in spans], axis=1)
    idx = torch.tensor([i for i, _, _ in spans], device="cuda")
    s0 = d["initial_state"] if init is None else init
    x["initial_state"] = None if s0 is False else s0[idx].cpu().numpy()
    for n in ("A_log", "dt_bias", "scale", "lower_bound"):
        x[n] = d[n]
    cu = np.zeros(len(spans) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    x["cu_seqlens"] = cu
    w = kda_inputs.custom(seqlens=lens, H=n_heads, lower_bound=d["lower_bound"], name=name)
    out_sub = torch.cat([_flat(out)[:, t0:t0 + L] for _, t0, L in spans], dim=1)
    check_against_oracle(w, x, out_sub, None if final is None else final[idx], heads=heads,
                         init=s0 is not False, final_dtype="fp32")


def _covering(starts, lens, tokens):
    """Indices of the chains that contain the given tokens, and the last chain."""
    ends = np.asarray(starts) + np.asarray(lens)
    pick = [int(np.searchsorted(ends, t, side="right")) for t in tokens] + [len(lens) - 1]
    return sorted(set(pick))


def _device_inputs(w, need):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    free, _ = torch.cuda.mem_get_info()
    if free < need:
        pytest.skip(f"needs {need >> 30} GiB of free device memory, {free >> 30} GiB free")
    say(f"drawing {w.name} on the device")
    d = kda_inputs.make_device_inputs(w, "cuda")
    d["A_log_dev"] = torch.from_numpy(d["A_log"]).cuda()
    d["dt_bias_dev"] = torch.from_numpy(d["dt_bias"]).cuda()
    return d


def test_maximum_head_count():
    Hm = 65535
    w = kda_inputs.custom(B=1, T=21, H=Hm, lower_bound=-1.0, init_std=0.05, state_dtype="fp32", seed=43,
                          name="kda_fwd_B1_T21_H65535")
    d = _device_inputs(w, 30 << 30)
    heads = [0, 1, 40000, Hm - 1]
    fin = torch.full((1, Hm, D, D), float("nan"), dtype=torch.float32, device="cuda")
    say(f"{w.name}: fixed length, {Hm} chains of one chunk and a 5-token tail")
    out = _call(d, d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"], fin)
    _check_spans(w.name, d, out, fin, [(0, 0, 21)], heads=heads, n_heads=Hm)
    del fin
    # the same tokens as two sequences (5 and 16 tokens), no initial state
    fin2 = torch.full((2, Hm, D, D), float("nan"), dtype=torch.float32, device="cuda")
    cu = torch.tensor([0, 5, 21], dtype=torch.int32, device="cuda")
    say(f"{w.name}: varlen 5 + 16 tokens, {2 * Hm} chains")
    out2 = _call(d, d["q"], d["k"], d["v"], d["g"], d["beta"], None, fin2, cu=cu)
    _check_spans(f"{w.name} varlen", d, out2, fin2, [(0, 0, 5), (1, 5, 16)], heads=heads, n_heads=Hm, init=False)
    del d, out, out2, fin2
    torch.cuda.empty_cache()


def test_many_sequences():
    rng = np.random.Generator(np.random.PCG64(44))
    lens = rng.integers(0, 41, size=300000)
    lens[:5] = [0, 1, 16, 17, 0]
    total = int(lens.sum())
    w = kda_inputs.custom(B=1, T=total, H=1, lower_bound=-3.0, init_std=None, seed=45, name="varlen300000_H1")
    d = _device_inputs(w, 40 << 30)
    N = len(lens)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), device="cuda")
    fin = torch.full((N, 1, D, D), float("nan"), dtype=torch.float32, device="cuda")
    say(f"{w.name}: {N} sequences, {total} tokens")
    out = _call(d, d["q"], d["k"], d["v"], d["g"], d["beta"], None, fin, cu=cu)
    pick = sorted(set(list(range(6)) + rng.choice(N, size=40, replace=False).tolist() + [N - 1]))
    # every chain has an end state (zero for an empty sequence), every token an output
    assert not torch.isnan(fin).any().item()
    assert not torch.isnan(out).any().item()
    empty = torch.from_numpy(np.flatnonzero(lens == 0)).cuda()
    assert not fin[empty].any().item()
    _check_spans(w.name, d, out, fin, [(i, int(starts[i]), int(lens[i])) for i in pick], heads=[0], n_heads=1,
                 init=False)
    del d, out, fin
    torch.cuda.empty_cache()


def test_fixed_length_past_2_32_elements(big):
    w, d = big
    assert B * T * H * D > 1 << 32
    rows = _covering([b * T for b in range(B)], [T] * B, EDGE_TOKENS)
    say(f"{w.name}: rows {rows} cover tokens {EDGE_TOKENS} and the end")
    fin_a = torch.full((B, H, D, D), float("nan"), dtype=torch.float32, device="cuda")
    out_a = _call(d, d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"], fin_a)
    _check_spans(f"{w.name} (library's plan)", d, out_a, fin_a, [(b, b * T, T) for b in rows])
    fin_b = torch.full_like(fin_a, float("nan"))
    out_b = _call(d, d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"], fin_b, cp_mode="force",
                  seg_chunks=128)
    say(f"{w.name}: 128-chunk segments against the library's plan, whole output and final state")
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
    assert torch.equal(fin_a, fin_b)
    _check_spans(f"{w.name} (128-chunk segments)", d, out_b, fin_b, [(b, b * T, T) for b in rows])


def test_varlen_past_2_32_elements(big):
    w, d = big
    rng = np.random.Generator(np.random.PCG64(42))
    lens = []
    while sum(lens) < B * T:
        lens.append(int(min(rng.integers(1, 12001), B * T - sum(lens))))
    assert len(lens) <= B  # the fixed batch's initial states cover them
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), device="cuda")
    N = len(lens)
    pick = _covering(starts, lens, EDGE_TOKENS)
    say(f"varlen over {w.name}'s memory: {N} sequences, checking {[(i, int(starts[i]), lens[i]) for i in pick]}")
    init = d["initial_state"][:N]
    fin = torch.full((N, H, D, D), float("nan"), dtype=torch.float32, device="cuda")
    out = _call(d, _flat(d["q"]), _flat(d["k"]), _flat(d["v"]), _flat(d["g"]), _flat(d["beta"]), init, fin, cu=cu)
    assert not torch.isnan(out).any().item()
    assert not torch.isnan(fin).any().item()
    _check_spans("varlen past 2^32 elements", d, out, fin, [(i, int(starts[i]), lens[i]) for i in pick])
