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
    "chunk_kda",
    "get_workspace_size",
    "plan_seg_chunks",
    "workspace_offsets",
    "library_path",
    "load_library",
    "KdaError",
    "WS_FIELDS",
    "STAGES",
    "profile_enable",
    "profile_collect",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libkda.so")
_lib = None

HEAD_DIM = 128
CHUNK = 16
WS_ALIGN = 256
WS_FIELDS = [
    "counters", "seq_start", "seq_len", "seq_chunk_off", "seq_seg_off", "chunk_tab", "seg_tab",
    "seg_m", "seg_r", "seg_s", "seg_mnz", "seg_chk", "seq_full_off", "unit_tab", "seg_fix", "max_chunks", "max_segs", "total",
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
    lib.kda_get_workspace_size.argtypes = [i64, i32, i32, i32, i32]
    lib.kda_get_workspace_size.restype = sz
    lib.kda_workspace_offsets.argtypes = [i64, i32, i32, i32, i32, ctypes.POINTER(i64)]
    lib.kda_workspace_offsets.restype = i32
    lib.kda_write_fixed_tables.argtypes = [i32, i64, i32, i32, i32, vp, sz, vp]
    lib.kda_write_fixed_tables.restype = i32
    lib.kda_fwd.argtypes = [vp, vp, vp, vp, vp, f32, vp, vp, vp, f32, vp, vp, i32, i32, vp, i32, i32, i64, i32, i32,
                            i32, vp, sz, i32, i32, vp]
    lib.kda_fwd.restype = i32
    lib.kda_profile_enable.argtypes = [i32]
    lib.kda_profile_enable.restype = i32
    lib.kda_profile_collect.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64), i32]
    lib.kda_profile_collect.restype = i32
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
    """Segment length (chunks of 16 tokens) the library will use; 0 = serial."""
    r = load_library().kda_plan_seg_chunks(int(total_tokens), int(num_heads), int(num_seqs), _cp(cp_mode),
                                           int(seg_chunks))
    if r < 0:
        _raise(r)
    return r


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
    with torch.cuda.device_of(workspace):
        stream = torch.cuda.current_stream(workspace.device).cuda_stream
        st = load_library().kda_write_fixed_tables(int(B), int(T), int(H), _cp(cp_mode), int(seg_chunks),
                                                   workspace.data_ptr(), workspace.numel(), stream)
    if st != 0:
        _raise(st)


STAGES = ["index", "recur0", "merge", "recur1"]


def profile_enable(on: bool = True) -> None:
    """Record HIP events around each kernel stage of every fwd on this thread."""
    load_library().kda_profile_enable(1 if on else 0)


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
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got device {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype}); no implicit conversion is made")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def fwd(q, k, v, g, beta, scale: float, out=None, *, A_log, dt_bias, lower_bound: float, workspace=None,
        initial_state=None, final_state=None, cu_seqlens=None, cp_mode="auto", seg_chunks: int = 0,
        state_layout: str = "vk"):
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
    """
    import torch

    lib = load_library()
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
        if st.dtype not in (torch.float32, torch.bfloat16):
            raise TypeError(f"{name} must be float32 or bfloat16 (got {st.dtype})")
        _check(st, name, st.dtype, (N, H, D, D))
        if sdt is not None and st.dtype != sdt:
            raise TypeError("initial_state and final_state must have the same dtype")
        sdt = st.dtype
    if out is None:
        out = torch.empty_like(v)
    else:
        _check(out, "out", torch.bfloat16, v.shape)
    tensors = [q, k, v, g, beta, out, A_log, dt_bias, initial_state, final_state, cu_seqlens, workspace]
    for t in tensors:
        if t is not None and t.device != dev:
            raise ValueError("all tensors must be on the same device")
    if state_layout not in ("vk", "kv"):
        raise ValueError(f"state_layout must be 'vk' or 'kv' (got {state_layout!r})")
    cpm = _cp(cp_mode)
    need = get_workspace_size(B * T, H, N, cpm, seg_chunks)
    with torch.cuda.device_of(q):
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        _check(workspace, "workspace", torch.uint8)
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = lib.kda_fwd(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), beta.data_ptr(), float(scale), out.data_ptr(),
            A_log.data_ptr(), dt_bias.data_ptr(), float(lower_bound),
            initial_state.data_ptr() if initial_state is not None else None,
            final_state.data_ptr() if final_state is not None else None,
            1 if sdt in (None, torch.float32) else 0, 1 if state_layout == "kv" else 0,
            cu_seqlens.data_ptr() if cu_seqlens is not None else None, N if cu_seqlens is not None else 0,
            B, T, H, Hqk, D, workspace.data_ptr(), workspace.numel(), cpm, int(seg_chunks), stream)
    if st != 0:
        _raise(st)
    if os.environ.get("KDA_LOG") == "1":
        import sys

        seg = plan_seg_chunks(B * T, H, N, cpm, seg_chunks)
        print(f"[kda] fwd B={B} T={T} H={H} N={N} plan={'serial' if seg == 0 else f'segments of {seg} chunks'}",
              file=sys.stderr)
    return out


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
