"""MI355X (gfx950) Kimi Delta Attention forward prefill.

Thin ctypes binding over libkda.so (include/kda.h).  It only checks and
marshals arguments: every step of the forward runs in the library's HIP
kernels, on the tensors' device and the current HIP stream.  PyTorch provides
device memory and streams.  There is no CPU path: if the library is missing,
importing the binding's entry points raises.

Interface (pages: "How to Use FlashKDA as a Backend for flash-linear-attention",
"Kernel API and Tensor Requirements"; "How FlashKDA Integrates with CUTLASS",
"Practical Implementation Example"):

    fwd(q, k, v, g, beta, scale=..., out=..., A_log=..., dt_bias=...,
        lower_bound=..., workspace=None, initial_state=None, final_state=None,
        cu_seqlens=None, cp_mode="auto", seg_chunks=0)

No implicit conversions are made: a tensor of the wrong dtype, device, shape
or layout is an error (the cuLA PR #106 review asks for errors over hidden
conversions).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "fwd",
    "fwd_noalloc",
    "prepare",
    "PreparedFwd",
    "read_counters",
    "chunk_kda",
    "get_workspace_size",
    "plan_seg_chunks",
    "fixed_seg_chunks",
    "varlen_seg_choice",
    "workspace_offsets",
    "library_path",
    "load_library",
    "KdaError",
    "WS_FIELDS",
    "STAGES",
    "profile_enable",
    "profile_collect",
    "profile_host",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libkda.so")
_lib = None

HEAD_DIM = 128
CHUNK = 16
WS_ALIGN = 256
WS_FIELDS = [
    "counters", "seq_start", "seq_len", "seq_chunk_off", "seq_seg_off", "chunk_tab", "seg_tab",
    "seg_m", "seg_r", "seg_s", "seg_mnz", "seg_chk", "seq_full_off", "unit_tab", "seg_fix", "seg_sync", "max_chunks",
    "max_segs", "total",
]
_CP = {"auto": 0, "off": 1, "force": 2, None: 0, False: 1, True: 2}
_STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported", -3: "workspace too small", -4: "HIP error"}


class KdaError(RuntimeError):
    """A library call returned a negative status."""

    def __init__(self, status: int, message: str):
        super().__init__(f"kda: {_STATUS.get(status, status)}: {message}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libkda.so (built in-tree); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it with `python -m kimi_delta_attention_02_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(_LIB_PATH)
    i32, i64, sz, vp, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
    lib.kda_plan_seg_chunks.argtypes = [i64, i32, i32, i32, i32]
    lib.kda_plan_seg_chunks.restype = i32
    lib.kda_fixed_seg_chunks.argtypes = [i32, i64, i32, i32, i32]
    lib.kda_fixed_seg_chunks.restype = i32
    lib.kda_varlen_seg_choice.argtypes = [ctypes.POINTER(i32), i32, i32, i32, i32, ctypes.POINTER(i32),
                                          ctypes.POINTER(i32)]
    lib.kda_varlen_seg_choice.restype = i32
    lib.kda_get_workspace_size.argtypes = [i64, i32, i32, i32, i32]
    lib.kda_get_workspace_size.restype = sz
    lib.kda_workspace_offsets.argtypes = [i64, i32, i32, i32, i32, ctypes.POINTER(i64)]
    lib.kda_workspace_offsets.restype = i32
    lib.kda_write_fixed_tables.argtypes = [i32, i64, i32, i32, i32, vp, sz, vp]
    lib.kda_write_fixed_tables.restype = i32
    lib.kda_fwd.argtypes = [vp, vp, vp, vp, vp, f32, vp, vp, vp, f32, vp, vp, i32, i32, vp, i32, i32, i64, i32, i32,
                            i32, vp, sz, i32, i32, vp]
    lib.kda_fwd.restype = i32
    lib.kda_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, f32, vp, vp, vp, f32, vp, vp, i32, i32, vp, i32, i32, i64, i32,
                                    i32, i32, i32, i32, vp]
    lib.kda_fwd_noalloc.restype = i32
    lib.kda_profile_enable.argtypes = [i32]
    lib.kda_profile_enable.restype = i32
    lib.kda_profile_collect.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64), i32]
    lib.kda_profile_collect.restype = i32
    lib.kda_profile_host.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]
    lib.kda_profile_host.restype = i32
    lib.kda_strerror.argtypes = [i32]
    lib.kda_strerror.restype = ctypes.c_char_p
    lib.kda_last_error.argtypes = []
    lib.kda_last_error.restype = ctypes.c_char_p
    lib.kda_version.argtypes = []
    lib.kda_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _cp(cp_mode) -> int:
    if isinstance(cp_mode, int) and not isinstance(cp_mode, bool):
        if cp_mode not in (0, 1, 2):
            raise ValueError(f"cp_mode must be 0 (auto), 1 (off) or 2 (force), got {cp_mode}")
        return cp_mode
    if isinstance(cp_mode, str):
        cp_mode = cp_mode.lower()
    if cp_mode not in _CP:
        raise ValueError(f"cp_mode must be 'auto', 'off' or 'force' (or None/False/True), got {cp_mode!r}")
    return _CP[cp_mode]


def _raise(status: int):
    lib = load_library()
    raise KdaError(status, lib.kda_last_error().decode())


def plan_seg_chunks(total_tokens: int, num_heads: int, num_seqs: int = 1, cp_mode="auto", seg_chunks: int = 0) -> int:
    """Planned segment length (chunks of 16 tokens); 0 = serial.  It sizes the
    workspace; with seg_chunks 0 a call may use a longer one (fixed_seg_chunks
    for a fixed-length call; a varlen call's is in its workspace counters)."""
    r = load_library().kda_plan_seg_chunks(int(total_tokens), int(num_heads), int(num_seqs), _cp(cp_mode),
                                           int(seg_chunks))
    if r < 0:
        _raise(r)
    return r


def fixed_seg_chunks(B: int, T: int, num_heads: int, cp_mode="auto", seg_chunks: int = 0) -> int:
    """Segment length a fixed-length call (B sequences of T tokens) uses; 0 = serial."""
    r = load_library().kda_fixed_seg_chunks(int(B), int(T), int(num_heads), _cp(cp_mode), int(seg_chunks))
    if r < 0:
        _raise(r)
    return r


def varlen_seg_choice(seq_lens, num_heads: int, cp_mode="auto", seg_chunks: int = 0):
    """(segment length, longest first) a varlen call with these sequence
    lengths takes; (0, False) = serial."""
    lens = [int(x) for x in seq_lens]
    arr = (ctypes.c_int32 * max(1, len(lens)))(*lens)
    seg, order = ctypes.c_int32(), ctypes.c_int32()
    r = load_library().kda_varlen_seg_choice(arr, len(lens), int(num_heads), _cp(cp_mode), int(seg_chunks),
                                             ctypes.byref(seg), ctypes.byref(order))
    if r < 0:
        _raise(r)
    return seg.value, bool(order.value)


def get_workspace_size(total_tokens: int, num_heads: int, num_seqs: int = 1, cp_mode="auto",
                       seg_chunks: int = 0) -> int:
    """Workspace bytes for a call over total_tokens = B*T tokens (the pages'
    get_workspace_size(B*T, H), plus the sequence count and segment plan)."""
    lib = load_library()
    n = lib.kda_get_workspace_size(int(total_tokens), int(num_heads), int(num_seqs), _cp(cp_mode), int(seg_chunks))
    if n == 0:
        raise KdaError(-1, lib.kda_last_error().decode())
    return int(n)


def workspace_offsets(total_tokens: int, num_heads: int, num_seqs: int = 1, cp_mode="auto",
                      seg_chunks: int = 0) -> dict:
    """Byte offsets of the workspace regions (names in WS_FIELDS)."""
    arr = (ctypes.c_int64 * len(WS_FIELDS))()
    st = load_library().kda_workspace_offsets(int(total_tokens), int(num_heads), int(num_seqs), _cp(cp_mode),
                                              int(seg_chunks), arr)
    if st != 0:
        _raise(st)
    return dict(zip(WS_FIELDS, [int(x) for x in arr]))


def write_fixed_tables(B: int, T: int, H: int, cp_mode, seg_chunks: int, workspace) -> None:
    """Write the index tables of a fixed-length call (B sequences of T tokens)
    into workspace, on the current stream; kda_fwd computes them in closed
    form without storing them (for inspection and tests)."""
    import torch

    _check(workspace, "workspace", torch.uint8)
    _check_devices((("workspace", workspace),))
    with torch.cuda.device_of(workspace):
        stream = torch.cuda.current_stream(workspace.device).cuda_stream
        st = load_library().kda_write_fixed_tables(int(B), int(T), int(H), _cp(cp_mode), int(seg_chunks),
                                                   workspace.data_ptr(), workspace.numel(), stream)
    if st != 0:
        _raise(st)


STAGES = ["index", "recur0", "merge", "recur1"]


PROFILE_KERNELS = 1
PROFILE_HOST = 2


def profile_enable(on: bool = True, host: bool = False) -> None:
    """Record HIP events around each kernel stage of every fwd on this thread
    (on), and the host time each forward call spends inside the library (host)."""
    load_library().kda_profile_enable((PROFILE_KERNELS if on else 0) | (PROFILE_HOST if host else 0))


def profile_host() -> tuple:
    """(host microseconds, calls) of the forward calls timed since the last
    call, inside the C ABI; then resets."""
    us = ctypes.c_double()
    n = ctypes.c_int64()
    load_library().kda_profile_host(ctypes.byref(us), ctypes.byref(n))
    return float(us.value), int(n.value)


def profile_collect() -> dict:
    """Wait for the recorded events; return {stage: (total_ms, launches)} and reset."""
    n = len(STAGES)
    ms = (ctypes.c_double * n)()
    calls = (ctypes.c_int64 * n)()
    st = load_library().kda_profile_collect(ms, calls, n)
    if st != 0:
        _raise(st)
    return {STAGES[i]: (float(ms[i]), int(calls[i])) for i in range(n)}


def _check(t, name, dtype, shape=None):
    """Type, dtype, layout and shape of one tensor (the device is checked once
    for all tensors of a call, last: _check_devices)."""
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype}); no implicit conversion is made")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _check_devices(named):
    """Every given tensor is a GPU tensor, all on the first one's device."""
    dev = None
    for name, t in named:
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a GPU tensor (got device {t.device})")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"all tensors must be on the same device ({name} is on {t.device}, not {dev})")


class _Checked:
    """The checked shapes and dtypes of one forward call."""

    __slots__ = ("B", "T", "H", "Hqk", "D", "N", "sdt", "out", "device")


SPLIT_WORKSPACE_CAP = 512 << 20


def _alloc_bytes(c, cpm, seg_chunks, varlen) -> int:
    """Workspace bytes fwd and prepare allocate: the plan's, or for a varlen
    call on the automatic plan with N*H >= 256 chains the segmented layout's
    when larger, so that a skewed batch can split (kda_fwd, cp_mode).  The
    segmented layout takes about (256 + N*H) x 320 KiB; beyond
    SPLIT_WORKSPACE_CAP bytes the plan's is allocated (the call then stays
    serial; pass a larger workspace to let it split)."""
    need = get_workspace_size(c.B * c.T, c.H, c.N, cpm, seg_chunks)
    if varlen and cpm == _CP["auto"] and int(seg_chunks) == 0 and c.N * c.H >= 256:
        split = get_workspace_size(c.B * c.T, c.H, c.N, _CP["force"], 0)
        if split <= SPLIT_WORKSPACE_CAP:
            need = max(need, split)
    return need


def _check_fwd(q, k, v, g, beta, out, A_log, dt_bias, initial_state, final_state, cu_seqlens, state_layout,
               workspace=None) -> _Checked:
    """Every check of a forward call's tensors, before any device work
    (allocates out when it is None)."""
    import torch

    _check(q, "q", torch.bfloat16)
    _check(v, "v", torch.bfloat16)
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q and v must be [B, T, heads, D]")
    B, T, Hqk, D = q.shape
    H = v.shape[2]
    if D != HEAD_DIM:
        raise ValueError(f"head dimension must be {HEAD_DIM} (got {D})")
    if tuple(v.shape) != (B, T, H, D) or H % Hqk != 0:
        raise ValueError(f"v has shape {tuple(v.shape)}: expected [B, T, H, D] with H a multiple of q's {Hqk} heads")
    dev = q.device
    _check(k, "k", torch.bfloat16, q.shape)
    _check(g, "g", torch.bfloat16, v.shape)
    _check(beta, "beta", torch.bfloat16, (B, T, H))
    _check(A_log, "A_log", torch.float32, (H,))
    _check(dt_bias, "dt_bias", torch.float32, (H, D))
    if cu_seqlens is not None:
        _check(cu_seqlens, "cu_seqlens", torch.int32)
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
            raise ValueError("cu_seqlens must be 1-D with N + 1 >= 2 entries")
        if B != 1:
            raise ValueError("cu_seqlens requires B == 1")
        N = cu_seqlens.numel() - 1
    else:
        N = B
    sdt = None
    for name, st in (("initial_state", initial_state), ("final_state", final_state)):
        if st is None:
            continue
        if not isinstance(st, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if st.dtype not in (torch.float32, torch.bfloat16):
            raise TypeError(f"{name} must be float32 or bfloat16 (got {st.dtype})")
        _check(st, name, st.dtype, (N, H, D, D))
        if sdt is not None and st.dtype != sdt:
            raise TypeError("initial_state and final_state must have the same dtype")
        sdt = st.dtype
    if out is not None:
        _check(out, "out", torch.bfloat16, v.shape)
    if workspace is not None:
        _check(workspace, "workspace", torch.uint8)
    if state_layout not in ("vk", "kv"):
        raise ValueError(f"state_layout must be 'vk' or 'kv' (got {state_layout!r})")
    _check_devices((("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("out", out), ("A_log", A_log),
                    ("dt_bias", dt_bias), ("initial_state", initial_state), ("final_state", final_state),
                    ("cu_seqlens", cu_seqlens), ("workspace", workspace)))
    if out is None:
        out = torch.empty_like(v)
    c = _Checked()
    c.B, c.T, c.H, c.Hqk, c.D, c.N, c.sdt, c.out, c.device = B, T, H, Hqk, D, N, sdt, out, dev
    return c


def _ptr(t):
    return t.data_ptr() if t is not None else None


def _fwd_args(c: _Checked, q, k, v, g, beta, scale, A_log, dt_bias, lower_bound, initial_state, final_state,
              cu_seqlens, state_layout):
    """kda_fwd's arguments before the workspace (shared with kda_fwd_noalloc)."""
    import torch

    return (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(c.out), _ptr(A_log), _ptr(dt_bias),
            float(lower_bound), _ptr(initial_state), _ptr(final_state),
            1 if c.sdt in (None, torch.float32) else 0, 1 if state_layout == "kv" else 0,
            _ptr(cu_seqlens), c.N if cu_seqlens is not None else 0, c.B, c.T, c.H, c.Hqk, c.D)


def _log_call(c: _Checked, cpm: int, seg_chunks: int):
    if os.environ.get("KDA_LOG") == "1":
        import sys

        seg = plan_seg_chunks(c.B * c.T, c.H, c.N, cpm, seg_chunks)
        print(f"[kda] fwd B={c.B} T={c.T} H={c.H} N={c.N} plan={'serial' if seg == 0 else f'segments of {seg} chunks'}",
              file=sys.stderr)


# counters[2] bits: repaired cu_seqlens faults (0x1-0x8), a chunk-kernel wait that gave up (0x100, 0x200)
FLAG_OFFSETS_REPAIRED = 0x00F
FLAG_WAIT_GAVE_UP = 0x300


def read_counters(workspace, total_tokens: int, num_heads: int, num_seqs: int = 1, cp_mode="auto",
                  seg_chunks: int = 0) -> dict:
    """The counters a call left in its workspace (copies 24 bytes to the host,
    which waits for the call): chunks, segments, flags (FLAG_* bits),
    early_stops, the segment length in use (0: serial) and whether the shorter
    segments were dispatched longest first.  The sizes and plan must be the
    call's."""
    import numpy as np

    offs = workspace_offsets(total_tokens, num_heads, num_seqs, cp_mode, seg_chunks)
    o = offs["counters"]
    c = workspace[o:o + 24].cpu().numpy().view(np.int32)
    return {"chunks": int(c[0]), "segments": int(c[1]), "flags": int(c[2]), "early_stops": int(c[3]),
            "seg_chunks": int(c[4]), "longest_first": bool(c[5])}


def _raise_on_flags(workspace, c: _Checked, cpm: int, seg_chunks: int):
    cnt = read_counters(workspace, c.B * c.T, c.H, c.N, cpm, seg_chunks)
    f = cnt["flags"]
    if f & FLAG_WAIT_GAVE_UP:
        raise KdaError(-4, f"a chunk-kernel wait gave up (counters flags {f:#x}): the results are not valid")
    if f & FLAG_OFFSETS_REPAIRED:
        raise KdaError(-1, f"cu_seqlens was malformed and clamped on the device (counters flags {f:#x})")


def fwd(q, k, v, g, beta, scale: float, out=None, *, A_log, dt_bias, lower_bound: float, workspace=None,
        initial_state=None, final_state=None, cu_seqlens=None, cp_mode="auto", seg_chunks: int = 0,
        state_layout: str = "vk", check: bool = False):
    """KDA forward.  Returns out (allocated if None).

    q, k, v, g: bf16 [B, T, H, 128]; beta: bf16 [B, T, H]; A_log: fp32 [H];
    q and k may have fewer heads H_qk (dividing H): head h then uses q/k head
    h // (H // H_qk) (grouped value heads);
    dt_bias: fp32 [H, 128]; lower_bound in [-5, 0];
    initial_state / final_state: None or [N, H, 128, 128] in bf16 or fp32
    (both the same dtype when both are given), [v][k] per head when
    state_layout is "vk", [k][v] when it is "kv"; cu_seqlens: None or int32
    [N + 1] (then B == 1); workspace: uint8 device buffer of at least
    get_workspace_size(B*T, H, N, cp_mode, seg_chunks) bytes, 256-byte
    aligned (allocated here when None); cp_mode: "auto" | "off" | "force".

    The call is asynchronous.  A wait inside the kernels that gives up, or a
    malformed cu_seqlens that the kernels clamped, is recorded only in the
    workspace's counters; check=True waits for the call, reads them and raises
    KdaError when either is set (read_counters does the same for a caller's
    workspace).
    """
    import torch

    lib = load_library()
    cpm = _cp(cp_mode)
    c = _check_fwd(q, k, v, g, beta, out, A_log, dt_bias, initial_state, final_state, cu_seqlens, state_layout,
                   workspace)
    need = get_workspace_size(c.B * c.T, c.H, c.N, cpm, seg_chunks)
    with torch.cuda.device_of(q):
        if workspace is None:
            workspace = torch.empty(_alloc_bytes(c, cpm, seg_chunks, cu_seqlens is not None), dtype=torch.uint8,
                                    device=c.device)
        stream = torch.cuda.current_stream(c.device).cuda_stream
        st = lib.kda_fwd(*_fwd_args(c, q, k, v, g, beta, scale, A_log, dt_bias, lower_bound, initial_state,
                                    final_state, cu_seqlens, state_layout),
                         workspace.data_ptr(), workspace.numel(), cpm, int(seg_chunks), stream)
    if st != 0:
        _raise(st)
    _log_call(c, cpm, seg_chunks)
    if check:
        _raise_on_flags(workspace, c, cpm, seg_chunks)
    return c.out


NOALLOC_SCRATCH_BYTES = 128 << 20  # KDA_NOALLOC_SCRATCH_BYTES of include/kda.h


def fwd_noalloc(q, k, v, g, beta, scale: float, out, *, A_log, dt_bias, lower_bound: float, initial_state=None,
                final_state=None, cu_seqlens=None, cp_mode="auto", seg_chunks: int = 0, state_layout: str = "vk"):
    """fwd for callers that cannot allocate: the library's per-GPU scratch
    array (NOALLOC_SCRATCH_BYTES) replaces the workspace, and out must be
    given.  Calls that may overlap on one GPU race on that array.  A call that
    needs more scratch raises KdaError (status -3) before any launch."""
    import torch

    if out is None:
        raise ValueError("fwd_noalloc needs out: it allocates nothing")
    lib = load_library()
    cpm = _cp(cp_mode)
    c = _check_fwd(q, k, v, g, beta, out, A_log, dt_bias, initial_state, final_state, cu_seqlens, state_layout)
    with torch.cuda.device_of(q):
        stream = torch.cuda.current_stream(c.device).cuda_stream
        st = lib.kda_fwd_noalloc(*_fwd_args(c, q, k, v, g, beta, scale, A_log, dt_bias, lower_bound, initial_state,
                                            final_state, cu_seqlens, state_layout),
                                 cpm, int(seg_chunks), stream)
    if st != 0:
        _raise(st)
    _log_call(c, cpm, seg_chunks)
    return c.out


class PreparedFwd:
    """A forward call checked and marshalled once (prepare()), for callers that
    repeat the same call on the same buffers: __call__ only launches it, on the
    stream chosen at preparation, with the ctypes arguments already built.
    Refill the input tensors in place between calls; rebind() swaps tensors of
    the same shape, dtype and device."""

    _NAMES = ("q", "k", "v", "g", "beta", "out", "A_log", "dt_bias", "initial_state", "final_state", "cu_seqlens",
              "workspace")

    def __init__(self, tensors: dict, scale, lower_bound, cp_mode, seg_chunks, state_layout, stream):
        import torch

        lib = load_library()
        t = dict(tensors)
        cpm = _cp(cp_mode)
        c = _check_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["out"], t["A_log"], t["dt_bias"],
                       t["initial_state"], t["final_state"], t["cu_seqlens"], state_layout, t["workspace"])
        t["out"] = c.out
        need = get_workspace_size(c.B * c.T, c.H, c.N, cpm, seg_chunks)
        if t["workspace"] is None:
            t["workspace"] = torch.empty(_alloc_bytes(c, cpm, seg_chunks, t["cu_seqlens"] is not None),
                                         dtype=torch.uint8, device=c.device)
        elif t["workspace"].numel() < need:
            raise ValueError(f"workspace of {t['workspace'].numel()} bytes, need {need}")
        if stream is None:
            stream = torch.cuda.current_stream(c.device)
        self._c, self._cpm, self._seg = c, cpm, int(seg_chunks)
        self._scale, self._lb, self._layout = float(scale), float(lower_bound), state_layout
        self._t = t
        self._stream = stream
        # the function without argtypes, called with ready ctypes values
        fn = ctypes.CDLL(_LIB_PATH).kda_fwd
        fn.restype = ctypes.c_int32
        self._fn = fn
        self._types = lib.kda_fwd.argtypes
        self._build()

    def _build(self):
        t, c = self._t, self._c
        raw = _fwd_args(c, t["q"], t["k"], t["v"], t["g"], t["beta"], self._scale, t["A_log"], t["dt_bias"], self._lb,
                        t["initial_state"], t["final_state"], t["cu_seqlens"], self._layout) + (
            t["workspace"].data_ptr(), t["workspace"].numel(), self._cpm, self._seg, self._stream.cuda_stream)
        self._args = tuple(ty(x) if x is not None else ty() for ty, x in zip(self._types, raw))

    @property
    def out(self):
        return self._t["out"]

    @property
    def workspace(self):
        return self._t["workspace"]

    def rebind(self, **tensors):
        """Use other tensors of the same shapes, dtypes and device (names as in fwd)."""
        for name, new in tensors.items():
            if name not in self._NAMES:
                raise ValueError(f"unknown tensor {name!r}")
            old = self._t[name]
            if (old is None) != (new is None):
                raise ValueError(f"{name}: presence cannot change after prepare()")
            if old is not None:
                _check(new, name, old.dtype, old.shape)
                if new.device != old.device:
                    raise ValueError(f"{name} must stay on {old.device}")
        self._t.update(tensors)
        self._build()

    def __call__(self):
        st = self._fn(*self._args)
        if st != 0:
            _raise(st)
        return self._t["out"]


def prepare(q, k, v, g, beta, scale: float, out=None, *, A_log, dt_bias, lower_bound: float, workspace=None,
            initial_state=None, final_state=None, cu_seqlens=None, cp_mode="auto", seg_chunks: int = 0,
            state_layout: str = "vk", stream=None) -> PreparedFwd:
    """Check and marshal a fwd call once; the returned object launches it
    (on `stream`, default: the current stream now) each time it is called.
    out and the workspace are allocated here when None."""
    tensors = dict(q=q, k=k, v=v, g=g, beta=beta, out=out, A_log=A_log, dt_bias=dt_bias, initial_state=initial_state,
                   final_state=final_state, cu_seqlens=cu_seqlens, workspace=workspace)
    return PreparedFwd(tensors, scale, lower_bound, cp_mode, seg_chunks, state_layout, stream)


def chunk_kda(q, k, v, g, beta, scale=None, initial_state=None, output_final_state: bool = False, *, A_log,
              dt_bias, lower_bound: float, use_gate_in_kernel: bool = True, use_qk_l2norm_in_kernel: bool = True,
              use_beta_sigmoid_in_kernel: bool = True, safe_gate: bool = True, transpose_state_layout: bool = True,
              cu_seqlens=None, cp_mode="auto"):
    """The chunk_kda call of the flash-linear-attention integration ("How to Use
    FlashKDA as a Backend for flash-linear-attention", "Running Inference with
    chunk_kda"), served by this library.  Returns (out, final_state), with
    final_state None unless output_final_state.

    Same tensors as fwd.  scale None means 1/sqrt(128).  With
    transpose_state_layout the states are [N, H, V, K] per head, otherwise
    [N, H, K, V]; the kernels read and write either layout directly.  The final
    state is allocated in the initial state's dtype (float32 without one);
    out and the workspace are allocated here too.

    The kernels always apply the L2 norm of q and k, the beta sigmoid and the
    lower-bounded gate; the integration page routes other settings of those
    flags to a different implementation, which this library does not have, so
    they raise ValueError.
    """
    import torch

    for name, val in (("use_gate_in_kernel", use_gate_in_kernel),
                      ("use_qk_l2norm_in_kernel", use_qk_l2norm_in_kernel),
                      ("use_beta_sigmoid_in_kernel", use_beta_sigmoid_in_kernel), ("safe_gate", safe_gate)):
        if val is not True:
            raise ValueError(f"{name}={val!r} is not supported: the kernels compute only the {name}=True form")
    if scale is None:
        scale = HEAD_DIM ** -0.5
    if not isinstance(v, torch.Tensor) or v.dim() != 4:
        raise ValueError("v must be a [B, T, H, D] tensor")
    B, T, H, D = v.shape
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    final = None
    if output_final_state:
        sdt = initial_state.dtype if initial_state is not None else torch.float32
        final = torch.empty((N, H, D, D), dtype=sdt, device=q.device)
    out = fwd(q, k, v, g, beta, scale, None, A_log=A_log, dt_bias=dt_bias, lower_bound=lower_bound,
              initial_state=initial_state, final_state=final, cu_seqlens=cu_seqlens, cp_mode=cp_mode,
              state_layout="vk" if transpose_state_layout else "kv")
    return out, final
