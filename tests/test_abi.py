"""C ABI checks that need no GPU: the library loads, exports every function
include/kda.h declares, plans and sizes workspaces consistently, and rejects
invalid calls before any HIP call is made (so these run on a CPU host)."""
import ctypes
import os
import re
import subprocess

import pytest

import kimi_delta_attention_02_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.library_path()):
        pytest.fail("libkda.so is not built (python -m kimi_delta_attention_02_amd.build)")
    return kda.load_library()


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert "kda_fwd" in names and "kda_get_workspace_size" in names
    out = subprocess.run(["nm", "-D", "--defined-only", kda.library_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (kda_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, f"declared but not exported: {missing}"
    for n in names:
        getattr(lib, n)  # resolvable through ctypes


def test_version_and_strerror(lib):
    assert b"gfx950" in lib.kda_version()
    assert lib.kda_strerror(0) == b"ok"
    assert lib.kda_strerror(-3) == b"workspace too small"


def test_plan_modes():
    # OFF is always serial; FORCE always splits; AUTO splits only few, long chains
    assert kda.plan_seg_chunks(65536, 16, 1, "off") == 0
    assert kda.plan_seg_chunks(1024, 16, 1, "force") > 0
    assert kda.plan_seg_chunks(65536, 16, 1, "auto") > 0
    assert kda.plan_seg_chunks(8 * 8192, 32, 8, "auto") == 0  # 256 chains fill the chip
    assert kda.plan_seg_chunks(1023, 16, 1, "auto") == 0  # too short to split
    assert kda.plan_seg_chunks(65536, 16, 1, "auto", 64) == 64
    # about one (segment, head) unit per CU: ceil(chunks * heads / 256) chunks per segment
    assert kda.plan_seg_chunks(65536, 16, 1, "auto") == 256
    assert kda.plan_seg_chunks(2 * 4096, 16, 2, "auto") == 32
    assert kda.plan_seg_chunks(65536, 16, 1, "off", 64) == 0
    with pytest.raises(kda.KdaError):
        kda.plan_seg_chunks(100, 0, 1)


def test_placement_model_worked_example():
    """Three sequences of 8192 tokens (512 chunks) at H = 16, planned length 96,
    by hand: 15 full segments of 96 + 4 run-on chunks (finish at 104 with the
    start cost), then three last segments of 32.  Per XCD a segment is two
    workgroups, local indices 2r and 2r + 1, so even rows take engines 0 and 1
    and odd rows engines 2 and 3; the 8 even full rows fill engines 0 and 1.
    The odd last segment starts at once, but the even one after it waits for
    engine 0/1 until 104 and ends at 104 + 32 + 4 = 140, the next in order with
    it.  At 102, 512 = 5 * 102 + 2: the last segments (2 <= K chunks) end at once
    and the fifth full segment runs on no further, so the span is 102 + 4 + 4."""
    from tests.span_model import chosen_seg, first_pass_span, unit_costs

    assert unit_costs(96, [512] * 3) == [100] * 15 + [32] * 3
    assert first_pass_span(96, [512] * 3, 16) == 140
    assert first_pass_span(102, [512] * 3, 16) == 110
    assert chosen_seg(96, [8192] * 3, 16) == 102
    # a single sequence that splits evenly is kept: 16 units of 256 (+4) fill the chip once
    assert chosen_seg(256, [65536], 16) == 256


def test_fixed_seg_chunks_follows_placement_model():
    """Where the library chooses the plan, a fixed-length call may lengthen
    the planned segment length, by at most a quarter and 63 chunks, to the one
    the placement model predicts fastest; explicit lengths, serial plans and
    shapes outside the model (more than 16 sequences, H not a multiple of 8)
    keep the planned one."""
    from tests.span_model import chosen_seg

    for B, T, H in [(1, 65536, 16), (2, 4096, 16), (3, 8192, 16), (1, 70656, 16), (3, 20000, 16), (5, 7777, 16),
                    (2, 100000, 8), (7, 5000, 8), (16, 2000, 8), (1, 65536, 32), (4, 10000, 8), (2, 30000, 24),
                    (2, 30000, 12), (17, 9000, 8)]:
        p = kda.plan_seg_chunks(B * T, H, B, "auto")
        got = kda.fixed_seg_chunks(B, T, H)
        assert got == chosen_seg(p, [T] * B, H), (B, T, H)
        assert p <= got <= p + min(p // 4, 63)
        assert kda.fixed_seg_chunks(B, T, H, "force") == chosen_seg(kda.plan_seg_chunks(B * T, H, B, "force"),
                                                                    [T] * B, H)
    assert kda.fixed_seg_chunks(3, 8192, 16) == 102
    assert kda.fixed_seg_chunks(3, 8192, 16, "auto", 96) == 96
    assert kda.fixed_seg_chunks(3, 8192, 16, "off") == 0
    assert kda.fixed_seg_chunks(2, 30000, 12) == kda.plan_seg_chunks(60000, 12, 2, "auto")
    with pytest.raises(kda.KdaError):
        kda.fixed_seg_chunks(0, 100, 16)
    with pytest.raises(kda.KdaError):
        kda.fixed_seg_chunks(1, 100, 0)


def test_varlen_seg_choice_follows_placement_model():
    """The library's varlen choice (replayed on the host by
    kda_varlen_seg_choice, the index kernel's arithmetic) against the literal
    placement model of tests/span_model.py, which places every workgroup on
    every XCD: seeded random mixes at H = 8, 16, 24, 32, 64 (each with its own
    form of the replay), both orders of the shorter segments, empty and tiny
    sequences included."""
    import numpy as np

    from tests.span_model import chosen_plan

    rng = np.random.Generator(np.random.PCG64(4242))
    n_long = 0
    for t in range(160):
        H = int(rng.choice([8, 16, 24, 32, 64]))
        N = int(rng.integers(1, min(16, 255 // H) + 1))
        total = int(rng.integers(10000, 400000))
        lens = np.floor(rng.dirichlet(np.full(N, float(rng.choice([0.3, 1.0, 3.0])))) * total).astype(int).tolist()
        if rng.random() < 0.2:
            lens[int(rng.integers(0, N))] = int(rng.choice([0, 1, 15, 16, 17]))
        planned = kda.plan_seg_chunks(sum(lens), H, N, "auto")
        got = kda.varlen_seg_choice(lens, H)
        want = chosen_plan(planned, lens, H, varlen=True) if planned else (0, True)  # serial: longest first
        assert got == want, (H, lens, planned, got, want)
        n_long += got[1]
    assert n_long > 10  # both orders were chosen
    # N*H >= 256 chains: serial on the automatic plan unless the longest
    # sequence has more than 5/4 of the segmented plan's length
    skew = [32768] + [1024] * 31
    f = kda.plan_seg_chunks(sum(skew), 16, 32, "force")
    assert kda.plan_seg_chunks(sum(skew), 16, 32, "auto") == 0
    assert kda.varlen_seg_choice(skew, 16) == (f, True) and f > 0  # shorter units longest first
    assert kda.varlen_seg_choice([1536] * 32, 16) == (0, True)  # serial, longest first
    # the boundary: 39 x 1536 tokens and one of 5072 (317 chunks) plan 254-chunk
    # segments; 317 <= 5/4 x 254 = 317.5 stays serial, 318 chunks split
    assert kda.plan_seg_chunks(39 * 1536 + 5072, 16, 40, "force") == 254
    assert kda.varlen_seg_choice([1536] * 39 + [5072], 16) == (0, True)
    assert kda.varlen_seg_choice([1536] * 39 + [5088], 16) == (254, True)
    assert kda.varlen_seg_choice(skew, 16, "off") == (0, True)
    assert kda.varlen_seg_choice([100] * 300, 16, "off") == (0, False)  # over 256 sequences: sequence order
    # explicit lengths and serial plans are kept; bad arguments raise
    assert kda.varlen_seg_choice([65536, 1024], 16, "auto", 300) == (300, False)
    assert kda.varlen_seg_choice([65536, 1024], 16, "off") == (0, True)
    with pytest.raises(kda.KdaError):
        kda.varlen_seg_choice([100, -1], 16)


def test_automatic_workspace_makes_room_for_a_split_up_to_the_cap():
    """fwd and prepare allocate the segmented layout's workspace for a varlen
    call on the automatic plan with N*H >= 256 chains (so that a skewed batch
    can split), but only up to SPLIT_WORKSPACE_CAP; otherwise the plan's own."""
    from types import SimpleNamespace as C

    def alloc(N, H, T, cp="auto", seg=0, varlen=True):
        return kda._alloc_bytes(C(B=1, T=T, H=H, N=N), kda._CP[cp], seg, varlen)

    def size(N, H, T, cp, seg=0):
        return kda.get_workspace_size(T, H, N, cp, seg)

    for N, H, T in [(32, 8, 64512), (41, 8, 280000), (32, 16, 65536)]:  # N*H >= 256, split size under the cap
        assert size(N, H, T, "force") <= kda.SPLIT_WORKSPACE_CAP
        assert alloc(N, H, T) == max(size(N, H, T, "auto"), size(N, H, T, "force"))
        assert alloc(N, H, T, varlen=False) == size(N, H, T, "auto")
        assert alloc(N, H, T, cp="off") == size(N, H, T, "off")
        assert alloc(N, H, T, seg=4) == size(N, H, T, "auto", 4)
    assert alloc(15, 16, 65536) == size(15, 16, 65536, "auto")  # N*H = 240 < 256
    for N, H, T in [(64, 32, 131072), (256, 16, 262144)]:  # split size over the cap
        assert size(N, H, T, "force") > kda.SPLIT_WORKSPACE_CAP
        assert alloc(N, H, T) == size(N, H, T, "auto")


def test_workspace_layout_consistent():
    for args in [(256, 2, 1, "off", 0), (8192, 16, 2, "auto", 0), (79890, 16, 7, "force", 64), (0, 4, 3, "auto", 0)]:
        size = kda.get_workspace_size(*args)
        off = kda.workspace_offsets(*args)
        assert off["total"] == size
        prev = -1
        for name in kda.WS_FIELDS[:16]:
            assert off[name] % kda.WS_ALIGN == 0
            assert off[name] >= prev
            prev = off[name]
        total, H, N = args[0], args[1], args[2]
        assert off["max_chunks"] == (total + 15 * N) // 16
        seg = kda.plan_seg_chunks(*args)
        assert off["max_segs"] == (off["max_chunks"] // seg + N if seg else N)
        assert off["seg_m"] - off["seg_tab"] >= 16 * off["max_segs"]
        mat = off["max_segs"] * H * 128 * 128 * 4
        if seg == 0:
            assert off["seg_s"] == off["seg_r"] == off["seg_m"] == off["seg_mnz"] == off["seg_chk"] == off["seq_full_off"]
        else:
            assert off["seg_r"] - off["seg_m"] >= mat and off["seg_s"] - off["seg_r"] >= mat
            assert off["seg_mnz"] - off["seg_s"] >= mat
            assert off["seg_chk"] - off["seg_mnz"] >= off["max_segs"] * H * 8 * 4
            assert off["seq_full_off"] - off["seg_chk"] >= mat
        assert off["unit_tab"] - off["seq_full_off"] >= 4 * (N + 1)
        assert off["seg_fix"] - off["unit_tab"] >= 32 * off["max_segs"]
        assert off["seg_sync"] - off["seg_fix"] >= (mat if seg else 0)
        assert off["total"] - off["seg_sync"] >= (off["max_segs"] * H * 16 * 4 if seg else 0)


def _call(lib, **kw):
    """kda_fwd with fake, never-dereferenced pointers (every case here fails
    validation before any device access or HIP call)."""
    P = ctypes.c_void_p(0x10000)
    a = dict(q=P, k=P, v=P, g=P, beta=P, scale=0.1, out=P, A_log=P, dt_bias=P, lower_bound=-1.0,
             initial_state=None, final_state=None, state_dtype=1, state_layout=0, cu_seqlens=None, num_seqs=0, B=1, T=64, H=2,
             H_qk=0, D=128, workspace=ctypes.c_void_p(0x100000), workspace_bytes=1 << 40, cp_mode=0, seg_chunks=0,
             stream=None)
    a.update(kw)
    return lib.kda_fwd(*a.values())


@pytest.mark.parametrize("kw,status,msg", [
    (dict(D=64), -2, "head dimension"),
    (dict(lower_bound=0.5), -1, "lower_bound"),
    (dict(lower_bound=-5.5), -1, "lower_bound"),
    (dict(lower_bound=float("nan")), -1, "lower_bound"),
    (dict(scale=float("inf")), -1, "scale"),
    (dict(state_dtype=7), -1, "state_dtype"),
    (dict(state_layout=2), -1, "state_layout"),
    (dict(H=4, H_qk=3), -1, "H_qk"),
    (dict(H=2, H_qk=4), -1, "H_qk"),
    (dict(B=2, cu_seqlens=ctypes.c_void_p(0x2000), num_seqs=2), -1, "B == 1"),
    (dict(cu_seqlens=ctypes.c_void_p(0x2000), num_seqs=0), -1, "num_seqs"),
    (dict(B=2, num_seqs=3), -1, "num_seqs"),
    (dict(q=None), -1, "non-NULL"),
    (dict(out=None), -1, "non-NULL"),
    (dict(A_log=None), -1, "A_log"),
    (dict(H=0), -1, "H="),
    (dict(T=-1), -1, ">= 0"),
    (dict(workspace=None), -1, "workspace"),
    (dict(workspace=ctypes.c_void_p(0x100010)), -1, "aligned"),
    (dict(workspace_bytes=1024), -3, "need"),
    (dict(cp_mode=5), -1, "cp_mode"),
    (dict(seg_chunks=-2), -1, "seg_chunks"),
    # token offsets and table rows are int32
    (dict(B=2, T=2 ** 30), -1, "B*T too large"),
    (dict(T=2 ** 30, H=64, cp_mode=2, seg_chunks=1), -1, "too large for the index tables"),
])
def test_fwd_rejects_before_launch(lib, kw, status, msg):
    st = _call(lib, **kw)
    assert st == status
    assert msg in lib.kda_last_error().decode()


def test_empty_call_is_a_no_op(lib):
    # B*T == 0 without a final state returns OK with no launch (and no HIP call)
    assert _call(lib, T=0) == 0
    assert _call(lib, B=0, T=10) == 0


def _call_noalloc(lib, **kw):
    """kda_fwd_noalloc with fake, never-dereferenced pointers (every case here
    fails validation before any device access or HIP call)."""
    P = ctypes.c_void_p(0x10000)
    a = dict(q=P, k=P, v=P, g=P, beta=P, scale=0.1, out=P, A_log=P, dt_bias=P, lower_bound=-1.0,
             initial_state=None, final_state=None, state_dtype=1, state_layout=0, cu_seqlens=None, num_seqs=0, B=1,
             T=64, H=2, H_qk=0, D=128, cp_mode=0, seg_chunks=0, stream=None)
    a.update(kw)
    return lib.kda_fwd_noalloc(*a.values())


def test_noalloc_scratch_size_matches_header():
    src = open(HEADER).read()
    m = re.search(r"#define KDA_NOALLOC_SCRATCH_BYTES \((\d+)ll << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == kda.NOALLOC_SCRATCH_BYTES


@pytest.mark.parametrize("kw,status,msg", [
    # one-chunk segments over 64K tokens at H = 16: 4097 x 16 units of 320 KiB
    (dict(T=65536, H=16, cp_mode=2, seg_chunks=1), -3, "scratch"),
    (dict(D=64), -2, "head dimension"),
    (dict(lower_bound=0.5), -1, "lower_bound"),
    (dict(q=None), -1, "non-NULL"),
    (dict(B=2, cu_seqlens=ctypes.c_void_p(0x2000), num_seqs=2), -1, "B == 1"),
])
def test_noalloc_rejects_before_launch(lib, kw, status, msg):
    st = _call_noalloc(lib, **kw)
    assert st == status
    assert msg in lib.kda_last_error().decode()


def test_noalloc_limit_covers_every_workload_plan():
    import kda_inputs

    for w in kda_inputs.WORKLOADS.values():
        for cp in ("auto", "off"):
            assert kda.get_workspace_size(w.B * w.T, w.H, w.N, cp) <= kda.NOALLOC_SCRATCH_BYTES, (w.name, cp)
