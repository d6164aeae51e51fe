"""KDA forward prefill benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config cfg4a] [--cp auto]

One step = one kda_fwd call (index tables: a launch for varlen calls, closed form
inside the chunk kernel for fixed-length ones; chunk prep fused with the
recurrence and, when the plan splits sequences, a second pass that merges each
segment's start state and redoes its first chunks where needed) over one batch
of seeded synthetic inputs already resident in HBM.  The default workload is
the long single sequence, B=1 T=65536 H=16 (the 64K end of the metric's range).
Untimed calls first run for --preheat-ms of wall time (default 300 ms): the
GPU's clock rises over the first tens of milliseconds of sustained load (the
per-step time falls by 13-17 % over them), and the steps are meant to be
timed at the clock the chip holds under load.  Then W untimed steps, then
exactly K steps timed with HIP events on the stream the library launches on
(events made for timing only, without the system-scope fence that would flush
the L2 after every step), bracketed by device synchronisation.  Prints ONE
JSON line.

Per-kernel time comes from the library's own timing hook
(kda_profile_enable / kda_profile_collect: every kernel launched with a pair
of HIP events that take its own start and end, on the library's stream) over
a second run of K steps; the step time comes from the first, uninstrumented
run.  The roofline object is computed for the chunk kernel (chunk prep +
recurrence), summed over its launches in a step, against the vendor HBM peak
and, beside it, the bandwidth of a plain device copy measured in the same run.
Host time per call is reported under "path" three ways: fwd() from Python,
the prepared call (kda.prepare: checked and marshalled once), and the C ABI's
own share (the library's host timer).  The same call is also captured once in
a HIP graph and replayed K times, last, after the same preheat and warmup
as the plain calls (the capture leaves the device idle and the clock falls).

The CPU baseline times the fp64 oracle (unchanged) on a bounded sample of the
same workload, before any GPU work starts: its first tokens (whole sequences
in order, the last cut to a prefix), all heads, one head per worker process,
sized to about --cpu-seconds; and one head on one core, scaled to all heads.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s at H=16,D=128, T=4K–64K; % of MFMA/HBM roofline"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, vendor figure
PEAK_BF16_TFLOPS = 2500.0  # dense bf16 MFMA, vendor figure
D = 128
C = 16
# algorithmic work per token-head (one token of one head)
BYTES_IN = 4 * 2 * D + 2  # q, k, v, g bf16 + beta bf16
BYTES_OUT = 2 * D  # out bf16
FLOPS_PATH = 6 * D * D + 10 * C * D  # 3 chunk GEMMs of 2*16*128*128 per 16 tokens + five 16x16x128 products


def _code_only(text: str) -> str:
    """C/C++/HIP source without its comments and blank space, so that editing
    a comment does not change what counts as the kernel's source.  String and
    character literals are kept as they are."""
    import re

    tok = re.compile(r'"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'|//[^\n]*|/\*.*?\*/|\s+', re.S)

    def keep(m):
        t = m.group(0)
        if t.startswith("//") or t.startswith("/*") or t.isspace():
            return " "
        return t

    return " ".join(tok.sub(keep, text).split())


def kernel_source_sha() -> str:
    """Short hash of the HIP sources' code (comments and blank space
    removed), to tell whether committed counter data still describes the
    kernels being run."""
    import glob
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "kimi_delta_attention_02_amd", "csrc")
    for f in sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.h"))):
        h.update(os.path.basename(f).encode())
        h.update(_code_only(open(f, encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, modes):
    """HBM bytes (read + write) of one call's chunk-kernel launches, one per
    mode in `modes` (0 serial; 1 and 2 the two passes of a segmented plan),
    whichever consumer variant ran, from the committed rocprofv3 counter runs
    (profiles/pmc_traffic.txt, one row per kernel and dispatch), or None when
    they were taken on other kernel sources, another workload or another plan."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.txt")
    if not os.path.exists(path):
        return None
    sha = kernel_source_sha()
    rows = {}
    for line in open(path):
        f = line.split()
        if len(f) == 5 and not line.startswith("#") and f[0] == workload and f[2] == sha \
                and f[1].startswith("kda_chunk_kernel") and f[1].endswith(">"):
            rows[f[1][f[1].index("<") + 1:-1]] = int(f[3]) + int(f[4])
    if any(str(m) not in rows for m in modes):
        return None
    return sum(rows[str(m)] for m in modes)


class HipTimingEvents:
    """HIP events for timing only (hipEventDisableSystemFence), on a given
    stream.  Reaching one of torch's events runs a system-scope fence, which
    writes back and invalidates the L2; recorded after every step, that adds a
    cache flush the calls do not otherwise have.  These come from the HIP
    runtime already loaded in the process (torch's, found by soname)."""

    FLAGS = 0x20000000  # hipEventDisableSystemFence

    def __init__(self):
        import ctypes

        self.c = ctypes
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.events = []

    def _ok(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed: hipError {rc}")

    def create(self):
        e = self.c.c_void_p()
        self._ok(self.lib.hipEventCreateWithFlags(self.c.byref(e), self.FLAGS), "hipEventCreateWithFlags")
        self.events.append(e)
        return e

    def record(self, e, stream):
        self._ok(self.lib.hipEventRecord(e, self.c.c_void_p(stream.cuda_stream)), "hipEventRecord")

    def elapsed_ms(self, a, b):
        self._ok(self.lib.hipEventSynchronize(b), "hipEventSynchronize")
        ms = self.c.c_float()
        self._ok(self.lib.hipEventElapsedTime(self.c.byref(ms), a, b), "hipEventElapsedTime")
        return ms.value

    def close(self):
        for e in self.events:
            self.lib.hipEventDestroy(e)
        self.events = []


_CPU_X = None  # inputs shared with the forked baseline workers
CPU_SHARE = 16  # host cores a one-GPU machine grants a job (worker pools are sized to it)


def _sample_spans(w, x, tokens: int):
    """The first `tokens` tokens of the workload, sequence by sequence in
    order (the last one cut to a prefix): [(row, first token, length, seq)]."""
    from oracle import kda_oracle as O

    out, left = [], tokens
    for i, (b, t0, L) in enumerate(O.sequence_spans(w.B, w.T, x["cu_seqlens"])):
        if left <= 0:
            break
        n = min(L, left)
        if n > 0:
            out.append((b, t0, n, i))
            left -= n
    return out


def _oracle_on(x, spans, head):
    """The oracle, unchanged, over the given sequence prefixes of one head."""
    from oracle import kda_oracle as O

    for b, t0, n, i in spans:
        sl = (slice(b, b + 1), slice(t0, t0 + n))
        init = None if x["initial_state"] is None else x["initial_state"][i:i + 1]
        O.kda_forward(x["q"][sl], x["k"][sl], x["v"][sl], x["g"][sl], x["beta"][sl], x["A_log"], x["dt_bias"],
                      x["scale"], x["lower_bound"], init, None, heads=[head])


def _cpu_worker(args):
    head, spans, reps = args
    from threadpoolctl import threadpool_limits

    with threadpool_limits(1):
        t = time.perf_counter()
        for _ in range(reps):
            _oracle_on(_CPU_X, spans, head)
        return time.perf_counter() - t


def cpu_baseline(name: str, target_s: float) -> dict:
    """The oracle, unchanged, over a bounded sample of the workload: its first
    tokens (whole sequences in order, the last one cut to a prefix), all
    heads, one head per worker process, sized so that the timed work lasts
    about target_s seconds; plus the same oracle on one core."""
    import multiprocessing as mp

    from threadpoolctl import threadpool_limits

    import kda_inputs

    global _CPU_X
    w = kda_inputs.WORKLOADS[name]
    _CPU_X = kda_inputs.make_inputs(w)
    host_cores = os.cpu_count() or 1
    workers = max(1, min(CPU_SHARE, host_cores, w.H))
    rounds = math.ceil(w.H / workers)
    # one core: one head over a growing prefix until about 2 s of work
    n, t1 = 256, 0.0
    with threadpool_limits(1):
        while True:
            sp = _sample_spans(w, _CPU_X, n)
            t = time.perf_counter()
            _oracle_on(_CPU_X, sp, 0)
            t1 = time.perf_counter() - t
            done = sum(s[2] for s in sp)
            if t1 >= 2.0 or done < n:
                break
            n = int(n * min(8.0, max(2.0, 2.0 / max(t1, 1e-3))))
    per_head_tok_s = done / t1
    # all cores: a prefix sized for target_s
    tokens = max(16, int(target_s * per_head_tok_s / rounds))
    spans = _sample_spans(w, _CPU_X, tokens)
    tokens = sum(s[2] for s in spans)
    reps = 1
    ctx = mp.get_context("fork")
    t = time.perf_counter()
    with ctx.Pool(workers) as pool:
        pool.map(_cpu_worker, [(h, spans, reps) for h in range(w.H)])
    wall = time.perf_counter() - t
    desc = ", ".join(f"seq {i}: {n} of its tokens" for _, _, n, i in spans)
    return {
        "value": tokens * reps / wall,
        "unit": "tokens/s",
        "cores": workers,
        "kind": "oracle",
        "host_cores": host_cores,
        "one_core": {"value": per_head_tok_s / w.H, "unit": "tokens/s",
                     "sample": f"head 0 over the first {done} tokens, {t1:.1f} s, scaled to all {w.H} heads"},
        "sample": f"{w.name}: the first {tokens} tokens ({desc}), all {w.H} heads, fp64 token recurrence, one "
                  f"head per process ({workers} processes of the {host_cores} host cores), {wall:.1f} s wall",
    }


def copy_bandwidth(dev, mib: int = 1024, reps: int = 20) -> dict:
    """Device-to-device copy bandwidth (read + write bytes per second) of a
    plain torch copy of `mib` MiB, timed with fence-free HIP events: the box's
    measured HBM figure, reported beside the vendor peak."""
    import torch

    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream(dev)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    tev = HipTimingEvents()
    a, b = tev.create(), tev.create()
    tev.record(a, stream)
    for _ in range(reps):
        dst.copy_(src)
    tev.record(b, stream)
    ms = tev.elapsed_ms(a, b) / reps
    tev.close()
    del src, dst
    return {"GBs": round(2 * n / (ms / 1e3) / 1e9, 1), "bytes": n, "ms": round(ms, 4)}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--preheat-ms", type=float, default=300.0,
                    help="untimed calls for this much wall time before the warmup steps (0 = none)")
    ap.add_argument("--config", default="cfg4a",
                    help="workload: cfg1..cfg5 (cfg4a/cfg4b), cfg4a_slow (T=65536 H=16 at lower_bound -0.1) or "
                         "cfg4a_nodecay (the same at lower_bound 0)")
    ap.add_argument("--cp", default="auto", help="auto | off | force")
    ap.add_argument("--seg", type=int, default=0, help="segment length in chunks (0 = library choice)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target wall time of the CPU baseline's all-core sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-copy-bw", action="store_true", help="skip the device copy bandwidth measurement")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (scale reference for HBM counters)")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {a.gpus}): the library has no multi-GPU path",
              file=sys.stderr)
        return 2

    import kda_inputs

    w = kda_inputs.WORKLOADS[a.config]
    cpu = None if a.no_cpu_baseline else cpu_baseline(a.config, a.cpu_seconds)

    import numpy as np
    import torch

    import kimi_delta_attention_02_amd as kda

    if not torch.cuda.is_available():
        print("no GPU available", file=sys.stderr)
        return 1
    kda.load_library()
    dev = torch.device("cuda:0")
    x = kda_inputs.make_inputs(w)

    def bf(arr):
        return torch.from_numpy(np.ascontiguousarray(arr)).view(torch.bfloat16).to(dev)

    q, k, v, g, beta = (bf(x[n]) for n in ("q", "k", "v", "g", "beta"))
    A_log = torch.from_numpy(x["A_log"]).to(dev)
    dt_bias = torch.from_numpy(x["dt_bias"]).to(dev)
    sdt = torch.float32 if w.state_dtype == "fp32" else torch.bfloat16
    init = None
    if x["initial_state"] is not None:
        init = bf(x["initial_state"]) if w.state_dtype == "bf16" else torch.from_numpy(x["initial_state"]).to(dev)
    final = torch.empty(w.N, w.H, D, D, dtype=sdt, device=dev) if w.want_final else None
    cu = None if x["cu_seqlens"] is None else torch.from_numpy(x["cu_seqlens"]).to(dev)
    out = torch.empty_like(q)
    total = w.B * w.T
    seg = kda.plan_seg_chunks(total, w.H, w.N, a.cp, a.seg)
    need = kda.get_workspace_size(total, w.H, w.N, a.cp, a.seg)
    if cu is not None and a.cp == "auto" and a.seg == 0:
        # as the binding allocates: room for the segmented layout lets a skewed
        # varlen batch split where the automatic plan would stay serial
        split = kda.get_workspace_size(total, w.H, w.N, "force", 0)
        need = max(need, split) if split <= kda.SPLIT_WORKSPACE_CAP else need
    ws = torch.empty(need, dtype=torch.uint8, device=dev)

    def step():
        kda.fwd(q, k, v, g, beta, x["scale"], out, A_log=A_log, dt_bias=dt_bias, lower_bound=x["lower_bound"],
                workspace=ws, initial_state=init, final_state=final, cu_seqlens=cu, cp_mode=a.cp, seg_chunks=a.seg)

    def preheat(fn):
        """Batches of calls, each waited for, until --preheat-ms of wall time
        has passed (the device is busy for nearly all of it); returns the
        calls made and the time taken."""
        calls = 0
        h0 = time.perf_counter()
        batch = 1
        while (time.perf_counter() - h0) * 1e3 < a.preheat_ms:
            for _ in range(batch):
                fn()
            torch.cuda.synchronize()
            calls += batch
            batch = min(2 * batch, 64)
        return calls, (time.perf_counter() - h0) * 1e3

    preheat_calls, preheat_ms = preheat(step)
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    # the segment length the calls used (with the library's own plan it may be
    # longer than the planned one once the sequence lengths are known)
    c0 = kda.workspace_offsets(total, w.H, w.N, a.cp, a.seg)["counters"]
    seg = int(ws[c0:c0 + 20].cpu().numpy().view(np.int32)[4])
    stream = torch.cuda.current_stream(dev)
    # Timed region 1: the K steps as a caller runs them (events only around
    # whole steps).  Timed region 2, right after it: the same K steps again
    # with the library's per-kernel events on, for the stage split and the
    # chunk kernel's own duration (the roofline); region 2 does not feed
    # ms_per_step.  The graph replays come last, after W untimed replays of
    # their own, so that nothing timed for the line follows them.
    tev = HipTimingEvents()
    evs = [tev.create() for _ in range(a.steps + 1)]
    tev.record(evs[0], stream)
    h0 = time.perf_counter()
    for i in range(a.steps):
        step()
        tev.record(evs[i + 1], stream)
    host_us = (time.perf_counter() - h0) / a.steps * 1e6  # submission only: the loop never waits
    torch.cuda.synchronize()
    total_ms = tev.elapsed_ms(evs[0], evs[-1])
    per = sorted(tev.elapsed_ms(evs[i], evs[i + 1]) for i in range(a.steps))
    kda.profile_enable(True)
    for i in range(a.steps):
        step()
    torch.cuda.synchronize()
    kda.profile_enable(False)
    stages = kda.profile_collect()
    # Host time per call on the fast path: the call checked and marshalled once
    # (kda.prepare), then only launched; inside it, the C ABI's own share
    # (validation, planning and the launches), from the library's host timer.
    prep = kda.prepare(q, k, v, g, beta, x["scale"], out, A_log=A_log, dt_bias=dt_bias, lower_bound=x["lower_bound"],
                       workspace=ws, initial_state=init, final_state=final, cu_seqlens=cu, cp_mode=a.cp,
                       seg_chunks=a.seg)
    for _ in range(a.warmup):
        prep()
    torch.cuda.synchronize()
    kda.profile_enable(False, host=True)
    h0 = time.perf_counter()
    for i in range(a.steps):
        prep()
    prep_host_us = (time.perf_counter() - h0) / a.steps * 1e6
    kda.profile_enable(False, host=False)
    cabi_us, cabi_calls = kda.profile_host()
    torch.cuda.synchronize()
    # Timed region 3: the same call captured once in a HIP graph and replayed K
    # times (the call allocates nothing and never synchronises, so it can be
    # captured); reported beside the plain calls, not as the value.
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    # the capture and instantiation leave the device idle, and the clock
    # falls; the replays get the plain calls' preheat and warmup
    graph_preheat_calls, _ = preheat(graph.replay)
    for _ in range(a.warmup):
        graph.replay()
    torch.cuda.synchronize()
    gev = [tev.create() for _ in range(2)]
    tev.record(gev[0], stream)
    h0 = time.perf_counter()
    for i in range(a.steps):
        graph.replay()
    graph_host_us = (time.perf_counter() - h0) / a.steps * 1e6
    tev.record(gev[1], stream)
    torch.cuda.synchronize()
    graph_ms = tev.elapsed_ms(gev[0], gev[1]) / a.steps
    tev.close()
    del graph
    copy = None if a.no_copy_bw else copy_bandwidth(dev)
    q1, q3 = len(per) // 4, len(per) - len(per) // 4
    iqr_mean = float(np.mean(per[q1:q3])) if q3 > q1 else float(np.mean(per))
    ms = total_ms / a.steps
    th = total * w.H  # token-heads per step
    state_bytes = 0
    if init is not None:
        state_bytes += init.numel() * init.element_size()
    if final is not None:
        state_bytes += final.numel() * final.element_size()

    # Roofline of the chunk kernel, the kernel that does the path's work (chunk
    # prep fused with the recurrence).  It runs once per step on a serial plan
    # and twice on a segmented one (first pass + segment pass); every
    # token-head's output is written by exactly one of those launches, so the
    # algorithmic work of a step (1282 B and 6 D^2 + 10 C D flops per
    # token-head, plus the state read and write) is set against the summed
    # duration of the chunk-kernel launches of a step.  The index tables and
    # the segment hand-off traffic are overhead and earn nothing.
    chunk_stages = [n for n in ("recur0", "recur1") if stages.get(n, (0.0, 0))[1]]
    chunk_ms = sum(stages[n][0] for n in chunk_stages) / a.steps
    launches = sum(stages[n][1] for n in chunk_stages) / a.steps
    bytes_d = th * (BYTES_IN + BYTES_OUT) + state_bytes
    flops_d = th * FLOPS_PATH
    t_s = chunk_ms / 1e3
    gbs = bytes_d / t_s / 1e9 if t_s > 0 else 0.0
    tfl = flops_d / t_s / 1e12 if t_s > 0 else 0.0
    if bytes_d / (PEAK_HBM_GBS * 1e9) >= flops_d / (PEAK_BF16_TFLOPS * 1e12):
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None}
    else:
        roof = {"bound": "mfma", "achieved": round(tfl, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tfl / PEAK_BF16_TFLOPS, 4), "traffic": None}
    roof["traffic"] = measured_traffic(w.name, (1, 2) if seg > 0 else (0,))
    if roof["bound"] == "hbm" and copy is not None:
        roof["measured_copy_GBs"] = copy["GBs"]
        roof["frac_of_measured_copy"] = round(gbs / copy["GBs"], 4)
    roof["kernel"] = "kda_chunk_kernel"
    roof["launches_per_step"] = launches
    roof["kernel_ms_per_step"] = round(chunk_ms, 4)
    roof["flops_frac"] = round(tfl / PEAK_BF16_TFLOPS, 4)

    path_bytes = th * (BYTES_IN + BYTES_OUT) + state_bytes
    path_flops = th * FLOPS_PATH
    res = {
        "metric": METRIC,
        "value": round(total / (ms / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "preheat": {"calls": preheat_calls, "ms": round(preheat_ms, 1)},
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 inputs, see kda_inputs)",
        "config": {
            "workload": w.name, "B": w.B, "T": w.T, "H": w.H, "D": D, "num_seqs": w.N,
            "global_batch": w.B, "seq_len": w.T, "lower_bound": w.lower_bound,
            "state": w.state_dtype, "plan": "serial" if seg == 0 else f"segments of {seg} chunks",
            "parallelism": "single GPU",
        },
        "roofline": roof,
        "cpu_baseline": cpu,
        "path": {
            "token_heads_per_s": round(th / (ms / 1e3), 1),
            "achieved_GBs": round(path_bytes / (ms / 1e3) / 1e9, 1),
            "achieved_TFLOPs": round(path_flops / (ms / 1e3) / 1e12, 2),
            "hbm_frac": round(path_bytes / (ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
            "mfma_frac": round(path_flops / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "iqr_mean_ms": round(iqr_mean, 4),
            # host time to submit one call: fwd() from Python (argument checks, ctypes,
            # C ABI validation, launches); the prepared call (kda.prepare) on the
            # same buffers; and the C ABI's own share of the prepared call
            "host_us_per_call": round(host_us, 1),
            "prepared_host_us_per_call": round(prep_host_us, 2),
            "c_abi_host_us_per_call": round(cabi_us / max(cabi_calls, 1), 2),
            # the call captured in a HIP graph, replayed K times (after
            # graph_preheat_calls untimed replays and W more)
            "graph_ms_per_step": round(graph_ms, 4),
            "graph_preheat_calls": graph_preheat_calls,
            "graph_host_us_per_call": round(graph_host_us, 1),
        },
        "stages_ms_per_step": {n: round(t / a.steps, 4) for n, (t, c) in stages.items() if c},
    }
    res["copy_bandwidth"] = copy
    if a.copy_probe_mib > 0:
        n = a.copy_probe_mib * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_probe_bytes"] = n
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
