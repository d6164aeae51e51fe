"""GPU parity: the HIP path against the fp64 oracle on the same seeded inputs,
plus the bitwise invariants of the GPU path itself.  All calls go through the
C ABI (via the ctypes binding)."""
import numpy as np
import pytest

import kda_inputs
from oracle import kda_oracle as O
from tests.gpu_util import (assert_close, check_against_oracle, dev_inputs, read_ws, run_gpu, say,
                            to_f64)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kimi_delta_attention_02_amd as kda

    kda.load_library()


def _case(w, cp_mode="auto", seg_chunks=0, seqs=None, heads=None, init=True, want_final=True, alias=False):
    say(f"case {w.name} seed={w.seed} cp={cp_mode} seg={seg_chunks} init={init} final={want_final} alias={alias}")
    x = kda_inputs.make_inputs(w)
    d = dev_inputs(x)
    out, final, ws = run_gpu(w, x, d, cp_mode, seg_chunks, want_final=want_final, init=init, alias=alias)
    check_against_oracle(w, x, out, final, seqs=seqs, heads=heads, init=init and x["initial_state"] is not None,
                         final_dtype=w.state_dtype)
    return x, d, out, final, ws


# ------------------------------------------------------------------- small shapes, every chain checked
def test_config1_full():
    _case(kda_inputs.WORKLOADS["cfg1"])


@pytest.mark.parametrize("lens", [[1], [15], [16], [17], [33, 1, 16, 70], [0, 5, 0, 40]])
def test_ragged_varlen(lens):
    _case(kda_inputs.custom(seqlens=lens, H=3, lower_bound=-5.0, seed=sum(lens) + len(lens), name=f"varlen{lens}"))


@pytest.mark.parametrize("lb", [0.0, -1.0, -5.0])
def test_lower_bound_range(lb):
    _case(kda_inputs.custom(B=2, T=100, H=2, lower_bound=lb, seed=21, name=f"lb{lb}"))


@pytest.mark.parametrize("init,final", [(False, False), (False, True), (True, False), (True, True)])
@pytest.mark.parametrize("sdt", ["fp32", "bf16"])
def test_state_presence_combinations(init, final, sdt):
    w = kda_inputs.custom(B=2, T=50, H=2, state_dtype=sdt, seed=22, name=f"state_{sdt}_{init}_{final}")
    _case(w, init=init, want_final=final)


@pytest.mark.parametrize("sdt", ["fp32", "bf16"])
def test_final_state_may_alias_initial(sdt):
    _case(kda_inputs.custom(B=1, T=90, H=2, state_dtype=sdt, seed=23, name=f"alias_{sdt}"), alias=True)


@pytest.mark.parametrize("alias", [False, True])
@pytest.mark.parametrize("layout_sdt", ["fp32", "bf16"])
def test_segmented_final_state_with_and_without_alias(alias, layout_sdt):
    # Segmented: without aliasing the first pass writes the final state of a
    # sequence's last segment itself; with aliasing the second pass does.
    w = kda_inputs.custom(B=2, T=700, H=2, lower_bound=-3.0, state_dtype=layout_sdt, seed=25,
                          name=f"segfinal_{layout_sdt}_{alias}")
    _case(w, cp_mode="force", seg_chunks=8, alias=alias)


@pytest.mark.parametrize("seg", [1, 2, 3])
def test_segment_path_small(seg):
    w = kda_inputs.custom(seqlens=[200, 16, 48, 1, 130], H=2, lower_bound=-1.0, seed=24, name=f"segsmall{seg}")
    _case(w, cp_mode="force", seg_chunks=seg)


def test_segment_path_slow_decay():
    # lb = 0: no decay at all, the merge must carry the full transition M
    w = kda_inputs.custom(B=1, T=400, H=2, lower_bound=0.0, seed=25, name="segnodecay")
    _case(w, cp_mode="force", seg_chunks=4)


def _early_stops(w, ws, cp_mode, seg_chunks):
    """(segment, head) pairs whose second pass stopped at the checkpoint."""
    import kimi_delta_attention_02_amd as kda

    offs = kda.workspace_offsets(w.B * w.T, w.H, w.N, cp_mode, seg_chunks)
    return int(read_ws(ws, offs, "counters", 4, np.int32)[3])


@pytest.mark.parametrize("seg,lb", [(5, -5.0), (9, -1.0), (12, 0.0)])
def test_segment_checkpoint(seg, lb):
    """Segments longer than the 4-chunk checkpoint.  The first pass writes their
    output from the zero-start state; the second pass redoes the first 4 chunks
    from the true start state and stops there only if its state equals the
    zero-start one bit for bit, else it runs to the segment's end.  Strong decay
    (lb = -5) reaches that equality; no decay (lb = 0) never does.  Both are
    checked against the oracle."""
    w = kda_inputs.custom(seqlens=[300, 16, 90, 1, 257], H=2, lower_bound=lb, seed=28, name=f"segchk{seg}/{lb}")
    x, d, out, final, ws = _case(w, cp_mode="force", seg_chunks=seg)
    stops = _early_stops(w, ws, "force", seg)
    say(f"{w.name}: early stops {stops}")
    if lb == 0.0:
        assert stops == 0
    if lb == -5.0:
        assert stops > 0


def test_zero_tokens_with_final_state():
    w = kda_inputs.custom(seqlens=[0, 0], H=2, seed=26, name="empty")
    x = kda_inputs.make_inputs(w)
    d = dev_inputs(x)
    out, final, _ = run_gpu(w, x, d)
    np.testing.assert_array_equal(to_f64(final), O.widen(x["initial_state"]))


# ------------------------------------------------------------------- chunk prep at every chunk size
@pytest.mark.parametrize("lb,init_std", [(-5.0, 0.05), (-0.5, 0.5)])
def test_every_chunk_tail(lb, init_std):
    """Sequences of 1..16 tokens are one chunk of each possible size, 17..32 a
    full chunk then a ragged one.  A one-chunk output is the chunk prep (norms,
    decays, beta, the WY inverse, Aqk) applied to the initial state and V, so
    each tail size of the prep is checked on its own sequence."""
    w = kda_inputs.custom(seqlens=list(range(1, 33)), H=2, lower_bound=lb, init_std=init_std, seed=27,
                          name=f"tails lb={lb}")
    x = kda_inputs.make_inputs(w)
    d = dev_inputs(x)
    out, final, _ = run_gpu(w, x, d, cp_mode="off")
    check_against_oracle(w, x, out, final)


# The shape of the pages' own benchmark (64 heads, no initial state) on a varlen
# mix of irregular lengths, serial (64 heads x 4 sequences already fill the
# chip) and split into 16-chunk segments.
@pytest.mark.parametrize("cp,seg", [("auto", 0), ("force", 16)])
def test_sixty_four_heads_no_initial_state(cp, seg):
    w = kda_inputs.custom(seqlens=[1000, 3000, 37, 2048], H=64, lower_bound=-5.0, init_std=None, seed=71,
                          name=f"H64 no-init {cp}")
    _case(w, cp_mode=cp, seg_chunks=seg, heads=[0, 31, 63])


# Degenerate inputs: all-zero query or key rows (the norm gives a zero vector, no
# NaN), beta logits of +-30 (sigmoid 1 and ~1e-13) and gate inputs of +-30 (the
# log decay saturates at lower_bound or at 0).
@pytest.mark.parametrize("cp,seg", [("off", 0), ("force", 5)])
def test_degenerate_rows_and_saturated_gates(cp, seg):
    w = kda_inputs.custom(seqlens=[300, 77], H=4, lower_bound=-5.0, seed=73, name=f"degenerate {cp}")
    say(f"case {w.name} seed={w.seed} cp={cp} seg={seg}")
    x = kda_inputs.make_inputs(w)
    x = dict(x)
    for n in ("q", "k", "beta", "g"):
        x[n] = x[n].copy()
    pos, neg = np.uint16(0x41F0), np.uint16(0xC1F0)  # bf16 30.0 and -30.0
    x["q"][0, 5::23] = 0
    x["k"][0, 11::29] = 0
    x["q"][0, 150:160, 1] = 0
    x["k"][0, 150:160, 1] = 0
    x["beta"][0, 3::17] = pos
    x["beta"][0, 7::19] = neg
    x["g"][0, 2::13, :, :40] = pos
    x["g"][0, 9::31, :, 60:] = neg
    d = dev_inputs(x)
    out, final, _ = run_gpu(w, x, d, cp, seg)
    check_against_oracle(w, x, out, final, final_dtype=w.state_dtype)


def _scale_bf16(a: np.ndarray, p2) -> np.ndarray:
    """bf16 bit patterns times 2**p2 (exact while the values stay normal)."""
    f = (a.astype(np.uint32) << 16).view(np.float32) * np.float32(2.0 ** p2)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


# Values far from 1: V and the start state times 2^20 or 2^-20.  The update's
# fp16 operand U then leaves the range it is used in unscaled, and every tile
# takes the power-of-two scaled form; the result must not depend on the scale.
@pytest.mark.parametrize("p2", [20, -20])
@pytest.mark.parametrize("cp,seg", [("off", 0), ("force", 5)])
def test_value_scale_extremes(p2, cp, seg):
    w = kda_inputs.custom(seqlens=[300, 77], H=4, lower_bound=-5.0, seed=91, name=f"v x 2^{p2} {cp}")
    say(f"case {w.name} seed={w.seed} cp={cp} seg={seg}")
    x = dict(kda_inputs.make_inputs(w))
    x["v"] = _scale_bf16(x["v"], p2)
    x["initial_state"] = (x["initial_state"] * np.float32(2.0 ** p2)).astype(np.float32)
    d = dev_inputs(x)
    out, final, _ = run_gpu(w, x, d, cp, seg)
    check_against_oracle(w, x, out, final, final_dtype=w.state_dtype)


# Column blocks of V at different scales (2^20, 2^-20, 1): the scaled and
# unscaled forms run side by side in one call, each tile deciding on its own
# values, so the 4-consumer first pass (two tiles per wavefront) and the
# 8-consumer second pass give the serial call's bits; each block is checked
# against the oracle at its own scale.
def test_mixed_value_scales_segmented_bit_identical():
    w = kda_inputs.custom(seqlens=[4096], H=2, lower_bound=-5.0, seed=92, name="mixed V scales")
    say(f"case {w.name} seed={w.seed}")
    x = dict(kda_inputs.make_inputs(w))
    v = x["v"].copy()
    s0 = x["initial_state"].copy()
    blocks = {(0, 16): 20, (16, 32): -20, (48, 64): 20, (96, 112): -20}
    for (a, b), p2 in blocks.items():
        v[..., a:b] = _scale_bf16(v[..., a:b], p2)
        s0[:, :, a:b, :] *= np.float32(2.0 ** p2)  # state layout [N, H, V, K]
    x["v"] = v
    x["initial_state"] = s0
    d = dev_inputs(x)
    out_s, fin_s, _ = run_gpu(w, x, d, cp_mode="off")
    out_c, fin_c, _ = run_gpu(w, x, d, cp_mode="force", seg_chunks=128)
    same_o = torch.equal(out_c.view(torch.int16), out_s.view(torch.int16))
    same_f = torch.equal(fin_c, fin_s)
    say(f"mixed scales: out identical={same_o} final identical={same_f}")
    assert same_o and same_f
    outs, finals = O.kda_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["A_log"], x["dt_bias"], x["scale"],
                                 x["lower_bound"], x["initial_state"], x["cu_seqlens"], seqs=[0], heads=[0])
    got = to_f64(out_s[0, :, [0]]).reshape(4096, 1, -1)
    ref = outs[0].reshape(4096, 1, -1)
    for (a, b) in list(blocks) + [(32, 48), (112, 128)]:
        assert_close(got[..., a:b].reshape(-1), ref[..., a:b].reshape(-1), f"out columns {a}:{b}")


# ------------------------------------------------------------------- index tables, bit-exact
def _zero_inputs(w):
    """Inputs of the workload's shapes, all zero, made on the device (the index
    tables depend on the sequence lengths only)."""
    z = {n: torch.zeros((w.B, w.T, w.H, 128), dtype=torch.bfloat16, device="cuda") for n in ("q", "k", "v", "g")}
    z["beta"] = torch.zeros((w.B, w.T, w.H), dtype=torch.bfloat16, device="cuda")
    z["A_log"] = torch.zeros(w.H, dtype=torch.float32, device="cuda")
    z["dt_bias"] = torch.zeros((w.H, 128), dtype=torch.float32, device="cuda")
    z["initial_state"] = None
    cu = None
    if w.seqlens is not None:
        cu = np.concatenate([[0], np.cumsum(np.asarray(w.seqlens, dtype=np.int64))]).astype(np.int32)
        z["cu_seqlens"] = torch.from_numpy(cu).to("cuda")
    else:
        z["cu_seqlens"] = None
    x = {"scale": float(np.float32(w.scale)), "lower_bound": float(np.float32(w.lower_bound)), "cu_seqlens": cu}
    return x, z


@pytest.mark.parametrize("lens,seg,fixed,H,mode", [
    ([1023, 1025, 1, 16, 4097, 8191, 65537], 64, False, 1, None), ([0, 1, 15, 16, 17, 0], 1, False, 1, None),
    ([65536] + [1024] * 5, 0, False, 1, None), ([65537], 37, False, 1, None),
    # past the one-workgroup form's limits (4095 sequences, 16384 rows): the two-launch form
    ([3] * 5000, 0, False, 1, None), ([300000], 64, False, 1, None),
    # fixed length (no cu_seqlens): the closed-form tables
    ([100] * 3, 2, True, 1, None), ([4096] * 2, 32, True, 1, None), ([33] * 7, 0, True, 1, None),
    ([512], 16, True, 1, None),
    # the library's own plan at H = 16: the segment length follows the placement model
    # (varlen: chosen on the device, one and two-launch forms; fixed length: on the host)
    ([65536] + [1024] * 5, 0, False, 16, "auto"), ([1023, 1025, 1, 16, 4097, 8191, 65537], 0, False, 16, "auto"),
    ([300000, 5000, 70], 0, False, 16, "auto"), ([8192] * 3, 0, True, 16, "auto"), ([65536], 0, False, 16, "auto"),
    ([24000, 3000, 1000], 0, False, 16, "auto"),
    # the two-launch form with the shorter segments longest first
    ([41621, 4127, 111604, 20239, 3299, 75763, 1774, 16070], 0, False, 16, "auto"),
    # the two-launch form, serial, sequences longest first
    ([70000] * 4 + [1000] * 20, 0, False, 1, "off"),
    # the two-launch form, a skewed batch of N*H >= 256 chains split on the
    # automatic plan (a workspace of the segmented size)
    ([200000] + [2000] * 40, 0, False, 8, "auto-split")])
def test_index_tables_bit_exact(lens, seg, fixed, H, mode):
    from tests.span_model import chosen_plan, rest_cost

    if fixed:
        w = kda_inputs.custom(B=len(lens), T=lens[0], H=H, seed=28, name="tables fixed", init_std=None)
    else:
        w = kda_inputs.custom(seqlens=lens, H=H, seed=28, name="tables", init_std=None)
    x, d = _zero_inputs(w)
    mode = mode or ("force" if seg else "off")
    import kimi_delta_attention_02_amd as kda

    split = mode == "auto-split"
    mode = "auto" if split else mode
    big = kda.get_workspace_size(w.B * w.T, w.H, w.N, "force", 0) if split else None
    _, _, ws = run_gpu(w, x, d, cp_mode=mode, seg_chunks=seg, want_final=False,
                       workspace=None if big is None else torch.empty(big, dtype=torch.uint8, device="cuda"))

    if fixed:  # kda_fwd computes these rows in closed form without storing them
        kda.write_fixed_tables(w.B, w.T, w.H, mode, seg, ws)
        torch.cuda.synchronize()

    offs = kda.workspace_offsets(w.B * w.T, w.H, w.N, "force" if split else mode, seg)
    planned = kda.plan_seg_chunks(w.B * w.T, w.H, w.N, mode, seg)
    used, desc = chosen_plan(planned, lens, H, varlen=not fixed) if seg == 0 else (planned, False)
    if used == 0 and not fixed and len(lens) <= 256:
        desc = True  # a serial varlen plan goes longest first
    if split:  # the host replay of the device's split decision
        used, desc = kda.varlen_seg_choice(lens, H)
        assert used > 0 and desc
    if mode == "auto":
        assert used > 0
        if fixed:
            assert kda.fixed_seg_chunks(w.B, w.T, w.H, mode, seg) == used
    say(f"tables {len(lens)} sequences H={H} {mode}: planned {planned}, used {used}, longest first {desc}")
    ref = O.index_tables(lens, 16, used if used else None)
    N = len(lens)
    cnt = read_ws(ws, offs, "counters", 6, np.int32)
    assert cnt[0] == ref["seq_chunk_off"][-1] and cnt[1] == ref["seq_seg_off"][-1] and cnt[2] == 0
    assert cnt[4] == used and cnt[5] == int(desc)
    np.testing.assert_array_equal(read_ws(ws, offs, "seq_chunk_off", N + 1, np.int32), ref["seq_chunk_off"])
    np.testing.assert_array_equal(read_ws(ws, offs, "seq_seg_off", N + 1, np.int32), ref["seq_seg_off"])
    nch, nsg = int(cnt[0]), int(cnt[1])
    np.testing.assert_array_equal(read_ws(ws, offs, "chunk_tab", 2 * nch, np.int32).reshape(-1, 2), ref["chunk_tab"])
    np.testing.assert_array_equal(read_ws(ws, offs, "seg_tab", 4 * nsg, np.int32).reshape(-1, 4), ref["seg_tab"])
    np.testing.assert_array_equal(read_ws(ws, offs, "seq_len", N, np.int32), lens)
    # rows past the live counts are -1
    mc, ms = offs["max_chunks"], offs["max_segs"]
    assert (read_ws(ws, offs, "chunk_tab", 2 * mc, np.int32)[2 * nch:] == -1).all()
    assert (read_ws(ws, offs, "seg_tab", 4 * ms, np.int32)[4 * nsg:] == -1).all()
    # dispatch order: every full-length segment (seg chunks) in segment order,
    # then the others in segment order or, where the call chose it, longest
    # first by first-pass cost (serial: every sequence counts as full); a row
    # also carries its sequence's first token and length and the segment length
    # in use
    st = ref["seg_tab"]
    starts = np.concatenate([[0], np.cumsum(lens)])
    full = [i for i in range(nsg) if not used or st[i][2] - st[i][1] == used]
    rest = [i for i in range(nsg) if used and st[i][2] - st[i][1] != used]
    nch_of = [(L + 15) // 16 for L in lens]
    if desc and used:
        rest = sorted(rest, key=lambda i: (-rest_cost(nch_of[st[i][0]], used), i))
    elif desc:  # serial: every sequence, longest first
        full = sorted(full, key=lambda i: (-nch_of[st[i][0]], i))
    want = np.array([[i, *st[i], starts[st[i][0]], lens[st[i][0]], used] for i in full + rest],
                    dtype=np.int32).reshape(-1, 8)
    unit = read_ws(ws, offs, "unit_tab", 8 * ms, np.int32).reshape(-1, 8)
    np.testing.assert_array_equal(unit[:nsg], want)
    assert (unit[nsg:] == -1).all()


def test_malformed_offsets_are_clamped():
    """Decreasing or out-of-range offsets are clamped into a non-decreasing
    sequence inside [0, total] (memory-safe), and flagged in the counters."""
    w = kda_inputs.custom(seqlens=[10, 30, 20], H=1, seed=29, name="badcu")
    x = kda_inputs.make_inputs(w)
    x["cu_seqlens"] = np.array([0, 40, 25, 90], dtype=np.int32)  # 25 < 40; 90 > total 60
    d = dev_inputs(x)
    _, _, ws = run_gpu(w, x, d, cp_mode="off", want_final=False)
    import kimi_delta_attention_02_amd as kda

    offs = kda.workspace_offsets(60, 1, 3, "off", 0)
    np.testing.assert_array_equal(read_ws(ws, offs, "seq_start", 4, np.int32), [0, 40, 40, 60])
    np.testing.assert_array_equal(read_ws(ws, offs, "seq_len", 3, np.int32), [40, 0, 20])
    assert read_ws(ws, offs, "counters", 4, np.int32)[2] != 0


# ------------------------------------------------------------------- bitwise invariants of the GPU path
def test_deterministic_and_varlen_equals_separate_calls():
    lens = [37, 16, 80, 5]
    w = kda_inputs.custom(seqlens=lens, H=2, seed=30, name="bitwise")
    x = kda_inputs.make_inputs(w)
    d = dev_inputs(x)
    out1, fin1, _ = run_gpu(w, x, d, cp_mode="off")
    out2, fin2, _ = run_gpu(w, x, d, cp_mode="off")
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16)) and torch.equal(fin1, fin2)
    cu = x["cu_seqlens"]
    for i, L in enumerate(lens):
        wi = kda_inputs.custom(B=1, T=L, H=2, seed=30, name="part")
        xi = dict(x)
        for n in ("q", "k", "v", "g", "beta"):
            xi[n] = np.ascontiguousarray(x[n][:, cu[i]:cu[i + 1]])
        xi["initial_state"] = x["initial_state"][i:i + 1]
        xi["cu_seqlens"] = None
        di = dev_inputs(xi)
        oi, fi, _ = run_gpu(wi, xi, di, cp_mode="off")
        assert torch.equal(oi.view(torch.int16), out1[:, cu[i]:cu[i + 1]].view(torch.int16))
        assert torch.equal(fi, fin1[i:i + 1])


def test_state_chaining_bitwise():
    """fwd(x1 || x2) == fwd(x2; S0 = final(x1)) bit for bit when len(x1) % 16 == 0 (fp32 state)."""
    w = kda_inputs.custom(B=1, T=160, H=2, seed=31, name="chain")
    x = kda_inputs.make_inputs(w)
    d = dev_inputs(x)
    out, fin, _ = run_gpu(w, x, d, cp_mode="off")
    parts = []
    state = d["initial_state"]
    for a, b in ((0, 64), (64, 160)):
        wi = kda_inputs.custom(B=1, T=b - a, H=2, seed=31, name="chainpart")
        xi = dict(x)
        for n in ("q", "k", "v", "g", "beta"):
            xi[n] = np.ascontiguousarray(x[n][:, a:b])
        di = dev_inputs(xi)
        di["initial_state"] = state
        oi, fi, _ = run_gpu(wi, xi, di, cp_mode="off")
        parts.append(oi)
        state = fi
    assert torch.equal(torch.cat(parts, 1).view(torch.int16), out.view(torch.int16))
    assert torch.equal(state, fin)


# ------------------------------------------------------------------- the five workloads at full size
def _full(name, seqs, heads, cp_mode="auto"):
    w = kda_inputs.WORKLOADS[name]
    return _case(w, cp_mode=cp_mode, seqs=seqs, heads=heads)


def test_config2_full_size():
    _full("cfg2", seqs=[0, 1], heads=[0, 7, 15])


def test_config3_full_size():
    _full("cfg3", seqs=[0, 1, 2, 3, 4, 5, 6], heads=[0, 3, 15])


def test_config5_full_size():
    _full("cfg5", seqs=[0, 7], heads=[0, 31])


@pytest.mark.parametrize("name", ["cfg4a", "cfg4b"])
def test_config4_segmented_bit_identical_to_serial(name):
    w = kda_inputs.WORKLOADS[name]
    say(f"case {name} serial vs segmented")
    x = kda_inputs.make_inputs(w)
    d = dev_inputs(x)
    out_s, fin_s, _ = run_gpu(w, x, d, cp_mode="off")
    check_against_oracle(w, x, out_s, fin_s, seqs=[0] if name == "cfg4a" else [0, 5], heads=[0, 5, 15],
                         final_dtype=w.state_dtype)
    for seg in (0, 64):
        out_c, fin_c, ws = run_gpu(w, x, d, cp_mode="force", seg_chunks=seg)
        same_o = torch.equal(out_c.view(torch.int16), out_s.view(torch.int16))
        same_f = torch.equal(fin_c, fin_s)
        stops = _early_stops(w, ws, "force", seg)
        say(f"{name} seg={seg}: out identical={same_o} final identical={same_f} early stops={stops}")
        assert same_o and same_f
        assert stops > 0  # the checkpoint path is the one measured at this size


@pytest.mark.parametrize("kind", ["fixed", "varlen"])
def test_lengthened_segments_bit_identical_to_serial(kind):
    """Calls whose segment length the library lengthens past the planned one:
    B=3 T=8192 H=16 (planned 96, chosen on the host: 102, so each sequence ends
    in a 2-chunk segment that the first pass skips) and the varlen
    40000+20000+9000 H=16 (planned 270, chosen in the index kernel).  Against
    the serial call bit for bit, and against the oracle on sampled chains."""
    from tests.span_model import chosen_seg
    import kimi_delta_attention_02_amd as kda

    if kind == "fixed":
        w = kda_inputs.custom(B=3, T=8192, H=16, lower_bound=-5.0, seed=44, name="B3_T8192_H16")
        lens = [8192] * 3
    else:
        lens = [40000, 20000, 9000]
        w = kda_inputs.custom(seqlens=lens, H=16, lower_bound=-5.0, seed=45, name="varlen_40000+20000+9000_H16")
    say(f"case {w.name} lengthened segments")
    x = kda_inputs.make_inputs(w)
    d = dev_inputs(x)
    planned = kda.plan_seg_chunks(w.B * w.T, w.H, w.N, "auto")
    used = chosen_seg(planned, lens, w.H, varlen=kind == "varlen")
    assert used > planned
    if kind == "fixed":
        assert kda.fixed_seg_chunks(w.B, w.T, w.H) == used
    out_s, fin_s, _ = run_gpu(w, x, d, cp_mode="off")
    out_c, fin_c, ws = run_gpu(w, x, d, cp_mode="auto")
    offs = kda.workspace_offsets(w.B * w.T, w.H, w.N, "auto", 0)
    cnt = read_ws(ws, offs, "counters", 6, np.int32)
    stops = int(cnt[3])
    say(f"{w.name}: planned {planned}, used {int(cnt[4])}, early stops {stops}")
    assert cnt[4] == used
    assert torch.equal(out_c.view(torch.int16), out_s.view(torch.int16)) and torch.equal(fin_c, fin_s)
    assert stops > 0
    check_against_oracle(w, x, out_c, fin_c, seqs=[2], heads=[1, 14], final_dtype=w.state_dtype)


@pytest.mark.parametrize("i", range(6))
def test_random_varlen_mix_segment_choice(i):
    """Seeded random varlen mixes at H=16 (2-15 sequences, 33-60K tokens) on
    the library's own plan, where the index kernel chooses the segment length
    and the order of the shorter segments: both equal the placement model's
    choice, the result equals
    the serial call bit for bit (lower bound -5), and sampled chains match the
    oracle."""
    from tests.span_model import chosen_plan
    import kimi_delta_attention_02_amd as kda

    rng = np.random.Generator(np.random.PCG64([7001, i]))
    N = int(rng.integers(2, 16))  # N * H < 256: the automatic plan splits
    total = int(rng.integers(33000, 60001))
    lens = np.floor(rng.dirichlet(np.full(N, 0.6)) * total).astype(int).tolist()
    w = kda_inputs.custom(seqlens=lens, H=16, lower_bound=-5.0, seed=7100 + i, name=f"mix{i}")
    say(f"case {w.name}: lengths {lens}")
    x = kda_inputs.make_inputs(w)
    d = dev_inputs(x)
    planned = kda.plan_seg_chunks(w.T, w.H, w.N, "auto")
    want, desc = chosen_plan(planned, lens, w.H, varlen=True)
    out_s, fin_s, _ = run_gpu(w, x, d, cp_mode="off")
    out_c, fin_c, ws = run_gpu(w, x, d, cp_mode="auto")
    offs = kda.workspace_offsets(w.T, w.H, w.N, "auto", 0)
    cnt = read_ws(ws, offs, "counters", 6, np.int32)
    say(f"{w.name}: planned {planned}, model {want} (longest first {desc}), used {int(cnt[4])} "
        f"(longest first {bool(cnt[5])}), early stops {int(cnt[3])}")
    assert cnt[4] == want and cnt[5] == int(desc) and cnt[2] == 0
    assert torch.equal(out_c.view(torch.int16), out_s.view(torch.int16)) and torch.equal(fin_c, fin_s)
    short = min((j for j in range(N) if lens[j] > 0), key=lambda j: lens[j])
    check_against_oracle(w, x, out_c, fin_c, seqs=[short], heads=[3, 12], final_dtype=w.state_dtype)


@pytest.mark.parametrize("kind", ["skewed", "balanced"])
def test_skewed_varlen_batch_splits_on_the_automatic_plan(kind):
    """32 sequences at H=16 (512 chains, which the automatic plan keeps
    serial): with a workspace that also holds the segmented layout, a skewed
    batch (32768 + 31 x 1024 tokens) splits on the device, a balanced one
    (32 x 1536) stays serial, as kda_varlen_seg_choice says; the tables follow
    the segmented layout's offsets; the result equals the serial call bit for
    bit and matches the oracle on sampled chains.  With a workspace of the
    automatic size only, the call stays serial."""
    import kimi_delta_attention_02_amd as kda

    lens = [32768] + [1024] * 31 if kind == "skewed" else [1536] * 32
    w = kda_inputs.custom(seqlens=lens, H=16, lower_bound=-5.0, seed=53, name=f"{kind} 32 sequences")
    say(f"case {w.name}")
    x = kda_inputs.make_inputs(w)
    d = dev_inputs(x)
    out_s, fin_s, _ = run_gpu(w, x, d, cp_mode="off")
    want, _ = kda.varlen_seg_choice(lens, w.H)
    assert (want > 0) == (kind == "skewed")
    ws = torch.empty(kda.get_workspace_size(w.T, w.H, w.N, "force", 0), dtype=torch.uint8, device="cuda")
    fin = torch.empty_like(fin_s)
    out = kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], x["scale"], A_log=d["A_log"], dt_bias=d["dt_bias"],
                  lower_bound=x["lower_bound"], workspace=ws, initial_state=d["initial_state"], final_state=fin,
                  cu_seqlens=d["cu_seqlens"], cp_mode="auto", check=True)
    cnt = kda.read_counters(ws, w.T, w.H, w.N, "auto")
    say(f"{w.name}: segment length in use {cnt['seg_chunks']} (host replay {want}), early stops {cnt['early_stops']}")
    assert cnt["seg_chunks"] == want and cnt["flags"] == 0
    if want:
        offs = kda.workspace_offsets(w.T, w.H, w.N, "force", 0)
        ref = O.index_tables(lens, 16, want)
        assert cnt["segments"] == ref["seq_seg_off"][-1] and cnt["early_stops"] > 0
        np.testing.assert_array_equal(read_ws(ws, offs, "seq_seg_off", w.N + 1, np.int32), ref["seq_seg_off"])
        np.testing.assert_array_equal(read_ws(ws, offs, "seg_tab", 4 * cnt["segments"], np.int32).reshape(-1, 4),
                                      ref["seg_tab"])
        # the full segments in segment order, then the shorter units longest first
        from tests.span_model import rest_cost

        st = ref["seg_tab"]
        nch_of = [(L + 15) // 16 for L in lens]
        full = [i for i in range(len(st)) if st[i][2] - st[i][1] == want]
        rest = sorted((i for i in range(len(st)) if st[i][2] - st[i][1] != want),
                      key=lambda i: (-rest_cost(nch_of[st[i][0]], want), i))
        assert cnt["longest_first"]
        unit = read_ws(ws, offs, "unit_tab", 8 * cnt["segments"], np.int32).reshape(-1, 8)
        np.testing.assert_array_equal(unit[:, 0], full + rest)
        assert (unit[:, 7] == want).all()
    assert torch.equal(out.view(torch.int16), out_s.view(torch.int16)) and torch.equal(fin, fin_s)
    check_against_oracle(w, x, out, fin, seqs=[0, 5], heads=[0, 9], final_dtype=w.state_dtype)
    # a workspace of the automatic plan's size: serial, as before
    ws2 = torch.empty(kda.get_workspace_size(w.T, w.H, w.N, "auto", 0), dtype=torch.uint8, device="cuda")
    kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], x["scale"], A_log=d["A_log"], dt_bias=d["dt_bias"],
            lower_bound=x["lower_bound"], workspace=ws2, initial_state=d["initial_state"], final_state=fin,
            cu_seqlens=d["cu_seqlens"], cp_mode="auto", check=True)
    assert kda.read_counters(ws2, w.T, w.H, w.N, "auto")["seg_chunks"] == 0


def test_config4_slow_decay_segmented():
    """T=65536 H=16 at lower_bound -0.1: the start state's influence has not
    decayed after a segment's first 4 chunks, so the second pass runs every
    segment >= 1 again from its merged start state.  Segmented against serial
    and both against the oracle; whether the bits agree is reported."""
    w = kda_inputs.WORKLOADS["cfg4a_slow"]
    say(f"case {w.name} serial vs segmented (slow decay)")
    x = kda_inputs.make_inputs(w)
    d = dev_inputs(x)
    out_s, fin_s, _ = run_gpu(w, x, d, cp_mode="off")
    out_c, fin_c, ws = run_gpu(w, x, d, cp_mode="auto")
    import kimi_delta_attention_02_amd as kda

    seg = kda.plan_seg_chunks(w.B * w.T, w.H, w.N, "auto")
    assert seg > 0
    stops = _early_stops(w, ws, "auto", 0)
    same_o = torch.equal(out_c.view(torch.int16), out_s.view(torch.int16))
    same_f = torch.equal(fin_c, fin_s)
    say(f"{w.name} seg={seg}: out identical={same_o} final identical={same_f} early stops={stops}")
    for got_o, got_f in ((out_s, fin_s), (out_c, fin_c)):
        check_against_oracle(w, x, got_o, got_f, heads=[0, 11], final_dtype=w.state_dtype)
    # segmented against serial, every chain: the oracle's tolerance with serial as the reference
    assert_close(to_f64(out_c).reshape(-1), to_f64(out_s).reshape(-1), "segmented vs serial out", stored="bf16")
    assert_close(to_f64(fin_c).reshape(-1), to_f64(fin_s).reshape(-1), "segmented vs serial final", stored="fp32")


def test_config4_no_decay_segmented():
    """T=65536 H=16 at lower_bound 0: no decay, so every segment's M stays
    nonzero and the second pass merges each start state through all the
    earlier segments' maps (fp32 products) before running the segment again.
    Segmented against serial within the tolerance, both against the oracle."""
    w = kda_inputs.WORKLOADS["cfg4a_nodecay"]
    say(f"case {w.name} serial vs segmented (no decay)")
    x = kda_inputs.make_inputs(w)
    d = dev_inputs(x)
    out_s, fin_s, _ = run_gpu(w, x, d, cp_mode="off")
    out_c, fin_c, ws = run_gpu(w, x, d, cp_mode="auto")
    import kimi_delta_attention_02_amd as kda

    seg = kda.plan_seg_chunks(w.B * w.T, w.H, w.N, "auto")
    assert seg > 0
    stops = _early_stops(w, ws, "auto", 0)
    say(f"{w.name} seg={seg}: out identical={torch.equal(out_c.view(torch.int16), out_s.view(torch.int16))} "
        f"early stops={stops}")
    for got_o, got_f in ((out_s, fin_s), (out_c, fin_c)):
        check_against_oracle(w, x, got_o, got_f, heads=[0, 11], final_dtype=w.state_dtype)
    assert_close(to_f64(out_c).reshape(-1), to_f64(out_s).reshape(-1), "segmented vs serial out", stored="bf16")
    assert_close(to_f64(fin_c).reshape(-1), to_f64(fin_s).reshape(-1), "segmented vs serial final", stored="fp32")


def test_two_launch_index_path_end_to_end():
    """5000 sequences of 3..40 tokens (past the one-workgroup index form's
    4095): the index scan + fill launches, then the chunk kernel, every chain
    against the oracle, serial and in 2-chunk segments."""
    rng = np.random.Generator(np.random.PCG64(77))
    lens = rng.integers(3, 41, size=5000).tolist()
    w = kda_inputs.custom(seqlens=lens, H=2, lower_bound=-2.0, seed=77, state_dtype="bf16", name="varlen5000_H2")
    say(f"case {w.name} tokens={w.T}")
    x = kda_inputs.make_inputs(w)
    d = dev_inputs(x)
    outs, finals = O.kda_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["A_log"], x["dt_bias"], x["scale"],
                                 x["lower_bound"], x["initial_state"], x["cu_seqlens"])
    ref_o = np.concatenate([o.reshape(-1) for o in outs])
    for cp, seg in (("off", 0), ("force", 2)):
        out, final, ws = run_gpu(w, x, d, cp_mode=cp, seg_chunks=seg)
        import kimi_delta_attention_02_amd as kda

        offs = kda.workspace_offsets(w.T, w.H, w.N, cp, seg)
        cnt = read_ws(ws, offs, "counters", 4, np.int32)
        assert cnt[0] == sum((L + 15) // 16 for L in lens) and cnt[2] == 0
        got_o = to_f64(out[0]).reshape(-1)
        assert_close(got_o, ref_o, f"{w.name} {cp} out", stored="bf16")
        assert_close(to_f64(final).reshape(-1), finals.reshape(-1), f"{w.name} {cp} final", stored="bf16")
