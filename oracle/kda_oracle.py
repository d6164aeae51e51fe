"""fp64 CPU oracle for the Kimi Delta Attention (KDA) forward prefill.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports, links or runs this
file; only the tests, the package's smoke check and the benchmark's CPU-baseline
leg call it.  It shares no code with the HIP path: the only common module is the
seeded input generator, which holds none of the method's arithmetic.

What it computes (one chain = one sequence x one head, K = V = 128):

  q^_t = q_t / sqrt(|q_t|^2 + eps)          k^_t likewise           (q/k L2 norm in kernel)
  b_t  = sigmoid(beta_t)                                             (beta sigmoid in kernel)
  l_t  = lower_bound * sigmoid(exp(A_log[h]) * (g_t + dt_bias[h]))   (gate in kernel, safe gate)
  a_t  = exp(l_t)                                                    per key channel
  S_t  = (I - b_t k^_t k^_t^T) Diag(a_t) S_{t-1} + b_t k^_t v_t^T       (S is K x V)
  o_t  = scale * S_t^T q^_t
  state tensors hold S^T, i.e. element [v][k] = S[k][v]              (transposed state layout)

Sources, all from the pages' text:
  * "How to Use FlashKDA as a Backend for flash-linear-attention", section
    "Running Inference with chunk_kda": the flags use_gate_in_kernel,
    use_qk_l2norm_in_kernel, use_beta_sigmoid_in_kernel, safe_gate, A_log,
    dt_bias, lower_bound, transpose_state_layout; section "Kernel API and Tensor
    Requirements": shapes, dtypes and lower_bound in [-5, 0]; section "State
    Handling and Variable-Length Batches": state [B,H,V,K] or [N,H,V,K] with
    cu_seqlens and B = 1.
  * cuLA PR #106 ("feat(kda): SM90 FlashKDA prefill, intracard CP, and backend
    dispatch"), commit list: K1 prepares decayed q/k, beta and the WY inverse,
    K2 runs the inter-chunk recurrence, CHUNK = 16, forward only; long
    sequences split into segments (K1 once -> pre_scan -> merge -> segment K2);
    description: an exact segment transition M is kept.
The pages print no equations; the update above is the plain reading of a
gated delta rule whose decay is per key channel and applied before the delta
correction, with the output read after the update.  Every such reading is
listed with the tests that pin it.

Pins (tests/test_oracle_pins.py): hand-derived fixtures under tests/golden/,
closed forms (beta = 0, one token, gate at g + dt_bias = 0), the textbook delta
rule at lower_bound = 0, the unit-key write invariant, linearity, chunked vs
token form, forward substitution vs numpy.linalg.solve, varlen vs per-sequence
calls, state chaining, exact segment merge, and hand-checked index tables.
"""
from __future__ import annotations

from typing import Iterable, Optional, Sequence

import numpy as np

EPS_L2 = 1e-6  # reading: q/k norm is x / sqrt(sum(x^2) + 1e-6); the pages give no epsilon
CHUNK = 16  # cuLA PR #106 commit list: CHUNK = 16


# ----------------------------------------------------------------------------
# input widening (exact)
# ----------------------------------------------------------------------------
def widen(x) -> np.ndarray:
    """bf16 bit patterns (uint16) or fp32/fp64 arrays -> fp64, exactly."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp64 -> nearest bf16 value (ties to even), returned as fp64.  Used to
    express a result in the storage type it is written in."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# token activations
# ----------------------------------------------------------------------------
def sigmoid(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    e = np.exp(x[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def l2_normalize(x: np.ndarray) -> np.ndarray:
    """Row-wise L2 normalisation over the last axis (use_qk_l2norm_in_kernel)."""
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + EPS_L2)


def log_decay(g: np.ndarray, a_log: np.ndarray, dt_bias: np.ndarray, lower_bound: float) -> np.ndarray:
    """Per-channel log decay l = lower_bound * sigmoid(exp(A_log) * (g + dt_bias)).

    g: [..., H, K]; a_log: [H]; dt_bias: [H, K].  With lower_bound in [-5, 0]
    the result lies in [lower_bound, 0] (safe_gate, lower_bound range from the
    "Kernel API and Tensor Requirements" section).
    """
    a = np.exp(np.asarray(a_log, dtype=np.float64))[:, None]
    return float(lower_bound) * sigmoid(a * (g + np.asarray(dt_bias, dtype=np.float64)))


# ----------------------------------------------------------------------------
# token recurrence (the definition)
# ----------------------------------------------------------------------------
def delta_rule_recurrence(qh, kh, v, lam, beta, scale, S0):
    """Token-by-token gated delta rule for H independent chains.

    qh, kh: [L, H, K] (already normalised); v: [L, H, V]; lam: [L, H, K] log
    decays; beta: [L, H] (already through the sigmoid); S0: [H, K, V].
    Returns o [L, H, V] and the state after the last token [H, K, V].
    """
    S = np.array(S0, dtype=np.float64, copy=True)
    L = qh.shape[0]
    o = np.empty((L, S.shape[0], S.shape[2]), dtype=np.float64)
    for t in range(L):
        S = np.exp(lam[t])[:, :, None] * S  # Diag(a_t) S_{t-1}
        pred = np.einsum("hk,hkv->hv", kh[t], S)  # (Diag(a_t) S_{t-1})^T k^_t
        S = S + beta[t][:, None, None] * kh[t][:, :, None] * (v[t] - pred)[:, None, :]
        o[t] = scale * np.einsum("hk,hkv->hv", qh[t], S)
    return o, S


# ----------------------------------------------------------------------------
# chunked (WY) form, written from the K1/K2 description
# ----------------------------------------------------------------------------
def forward_substitution_inverse(A: np.ndarray) -> np.ndarray:
    """(I + A)^{-1} for strictly lower-triangular A, row by row:
    T_ii = 1, T_ij = -sum_{p=j}^{i-1} A_ip T_pj for j < i."""
    m = A.shape[0]
    T = np.zeros_like(A)
    for i in range(m):
        T[i, i] = 1.0
        for j in range(i):
            T[i, j] = -np.dot(A[i, j:i], T[j:i, j])
    return T


def chunk_quantities(qh, kh, v, lam, beta, scale):
    """Per-chunk quantities for one chain and one chunk of m <= CHUNK tokens.

    qh, kh: [m, K]; v: [m, V]; lam: [m, K]; beta: [m].  Returns a dict with the
    cumulative log decay G, gamma_C = exp(G_last), the decayed operands
    Qbar = scale q^ exp(G), Kbar = k^ exp(G), Ktil = k^ exp(-G),
    Khat = k^ exp(G_last - G), A = StrictLower(Diag(b) Kbar Ktil^T), its WY
    inverse T = (I + A)^{-1}, W = T Diag(b) Kbar, Ut = T Diag(b) V and
    Aqk = LowerInclusive(Qbar Ktil^T).
    """
    G = np.cumsum(lam, axis=0)
    gam = np.exp(G)
    igam = np.exp(-G)
    gam_C = gam[-1]
    Qbar = scale * qh * gam
    Kbar = kh * gam
    Ktil = kh * igam
    Khat = kh * np.exp(G[-1][None, :] - G)
    A = np.tril(beta[:, None] * (Kbar @ Ktil.T), k=-1)
    T = forward_substitution_inverse(A)
    W = T @ (beta[:, None] * Kbar)
    Ut = T @ (beta[:, None] * v)
    Aqk = np.tril(Qbar @ Ktil.T)
    return dict(G=G, gamma_C=gam_C, Qbar=Qbar, Kbar=Kbar, Ktil=Ktil, Khat=Khat, A=A, T=T, W=W, Ut=Ut, Aqk=Aqk)


def chunk_step(c: dict, S: np.ndarray):
    """K2 step for one chunk: U = Ut - W S; O = Qbar S + Aqk U;
    S_next = Diag(gamma_C) S + Khat^T U."""
    U = c["Ut"] - c["W"] @ S
    O = c["Qbar"] @ S + c["Aqk"] @ U
    S_next = c["gamma_C"][:, None] * S + c["Khat"].T @ U
    return O, S_next


def chunked_recurrence(qh, kh, v, lam, beta, scale, S0, C: int = CHUNK, keep: bool = False):
    """Chunked form for one chain: qh, kh, lam [L, K]; v [L, V]; beta [L]; S0 [K, V].

    Chunks of C tokens from the sequence start; the last one may be shorter.
    Returns (o [L, V], S_L [K, V], list of per-chunk dicts if keep else None).
    """
    L = qh.shape[0]
    S = np.array(S0, dtype=np.float64, copy=True)
    o = np.empty((L, S.shape[1]), dtype=np.float64)
    kept = [] if keep else None
    for c0 in range(0, L, C):
        sl = slice(c0, min(c0 + C, L))
        c = chunk_quantities(qh[sl], kh[sl], v[sl], lam[sl], beta[sl], scale)
        o[sl], S = chunk_step(c, S)
        if keep:
            kept.append(c)
    return o, S, kept


def chunk_affine_map(c: dict):
    """A chunk maps the entering state affinely: S -> Mc S + Rc with
    Mc = Diag(gamma_C) - Khat^T W and Rc = Khat^T Ut."""
    Mc = np.diag(c["gamma_C"]) - c["Khat"].T @ c["W"]
    Rc = c["Khat"].T @ c["Ut"]
    return Mc, Rc


def segment_transition(chunks: Sequence[dict]):
    """Exact transition of a run of chunks (pre-scan): M = product of Mc
    (later chunks on the left, starting from I) and R, the state the run
    produces from a zero start."""
    K = chunks[0]["Khat"].shape[1]
    V = chunks[0]["Ut"].shape[1]
    M = np.eye(K)
    R = np.zeros((K, V))
    for c in chunks:
        Mc, Rc = chunk_affine_map(c)
        M = Mc @ M
        R = Mc @ R + Rc
    return M, R


def merge(M: np.ndarray, R: np.ndarray, S: np.ndarray) -> np.ndarray:
    """State after a segment from the state before it."""
    return M @ S + R


# ----------------------------------------------------------------------------
# index tables for fixed-length and varlen batches
# ----------------------------------------------------------------------------
def index_tables(seqlens: Sequence[int], C: int = CHUNK, seg_chunks: Optional[int] = None) -> dict:
    """Brute-force chunk and segment tables.

    Sequence i has ceil(len_i / C) chunks; chunks never cross a sequence start.
      seq_chunk_off [N+1]  : prefix sums of the chunk counts
      chunk_tab [n_chunks, 2] : (sequence, chunk index inside the sequence)
      seq_seg_off [N+1]    : prefix sums of the segment counts; every sequence
                             has max(1, ceil(chunks / seg_chunks)) segments
                             (one segment when seg_chunks is None)
      seg_tab [n_segs, 4]  : (sequence, first global chunk, end global chunk,
                             segment index inside the sequence)
    """
    N = len(seqlens)
    seq_chunk_off = [0]
    chunk_tab = []
    for i in range(N):
        n = 0
        t = 0
        while t < seqlens[i]:
            chunk_tab.append((i, n))
            n += 1
            t += C
        seq_chunk_off.append(seq_chunk_off[-1] + n)
    seq_seg_off = [0]
    seg_tab = []
    for i in range(N):
        first, end = seq_chunk_off[i], seq_chunk_off[i + 1]
        nch = end - first
        if seg_chunks is None or nch == 0:
            nseg = 1
        else:
            nseg = 0
            while nseg * seg_chunks < nch:
                nseg += 1
        for j in range(nseg):
            if seg_chunks is None:
                b, e = first, end
            else:
                b = min(first + j * seg_chunks, end)
                e = min(first + (j + 1) * seg_chunks, end)
            seg_tab.append((i, b, e, j))
        seq_seg_off.append(seq_seg_off[-1] + nseg)
    return dict(
        seq_chunk_off=np.asarray(seq_chunk_off, dtype=np.int32),
        chunk_tab=np.asarray(chunk_tab, dtype=np.int32).reshape(-1, 2),
        seq_seg_off=np.asarray(seq_seg_off, dtype=np.int32),
        seg_tab=np.asarray(seg_tab, dtype=np.int32).reshape(-1, 4),
    )


# ----------------------------------------------------------------------------
# the forward call, as the library's interface defines it
# ----------------------------------------------------------------------------
def sequence_spans(B: int, T: int, cu_seqlens=None):
    """(batch row, first token, length) for every sequence."""
    if cu_seqlens is None:
        return [(b, 0, T) for b in range(B)]
    cu = [int(x) for x in np.asarray(cu_seqlens)]
    return [(0, cu[i], cu[i + 1] - cu[i]) for i in range(len(cu) - 1)]


def kda_forward(q, k, v, g, beta, A_log, dt_bias, scale, lower_bound, initial_state=None,
                cu_seqlens=None, seqs: Optional[Iterable[int]] = None, heads: Optional[Iterable[int]] = None,
                chunked: Optional[int] = None):
    """KDA forward over a batch, in fp64.

    q, k, v, g: [B, T, H, 128] (bf16 bits or floats); beta: [B, T, H] logits;
    A_log: [H]; dt_bias: [H, 128]; initial_state: [N, H, V, K] or None;
    cu_seqlens: [N + 1] offsets (then B == 1) or None.
    seqs / heads select a subset of chains (default: all).
    chunked: None for the token recurrence, or a chunk size for the chunked form.

    Returns (outs, finals): outs[i] is [len_i, len(heads), V] for each selected
    sequence i (in the order given), finals is [len(seqs), len(heads), V, K]
    (the transposed state layout).
    """
    B, T, H, D = np.shape(q)
    spans = sequence_spans(B, T, cu_seqlens)
    seqs = list(range(len(spans))) if seqs is None else list(seqs)
    heads = list(range(H)) if heads is None else list(heads)
    hs = np.asarray(heads)
    a_log = np.asarray(A_log, dtype=np.float64)[hs]
    dtb = np.asarray(dt_bias, dtype=np.float64)[hs]
    scale = float(np.float32(scale))
    lower_bound = float(np.float32(lower_bound))
    outs = []
    finals = np.zeros((len(seqs), len(heads), D, D), dtype=np.float64)
    for si, i in enumerate(seqs):
        b, t0, L = spans[i]
        sl = (b, slice(t0, t0 + L))
        qi = l2_normalize(widen(np.asarray(q)[sl][:, hs]))
        ki = l2_normalize(widen(np.asarray(k)[sl][:, hs]))
        vi = widen(np.asarray(v)[sl][:, hs])
        lam = log_decay(widen(np.asarray(g)[sl][:, hs]), a_log, dtb, lower_bound)
        bi = sigmoid(widen(np.asarray(beta)[sl][:, hs]))
        if initial_state is None:
            S0 = np.zeros((len(heads), D, D))
        else:
            S0 = np.swapaxes(widen(np.asarray(initial_state)[i][hs]), -1, -2)  # [V][K] -> S [K][V]
        if chunked is None:
            o, S = delta_rule_recurrence(qi, ki, vi, lam, bi, scale, S0)
        else:
            o = np.empty((L, len(heads), D))
            S = np.empty_like(S0)
            for hj in range(len(heads)):
                o[:, hj], S[hj], _ = chunked_recurrence(qi[:, hj], ki[:, hj], vi[:, hj], lam[:, hj],
                                                        bi[:, hj], scale, S0[hj], C=chunked)
        outs.append(o)
        finals[si] = np.swapaxes(S, -1, -2)
    return outs, finals
