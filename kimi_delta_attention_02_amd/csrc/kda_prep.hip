// Chunk preparation ("K1" on the cuLA PR #106 page: K1 prepares decayed q/k,
// beta and the WY inverse; CHUNK = 16, D = 128, forward only).
//
// One wavefront per (chunk, head).  For the chunk's m <= 16 tokens (rows past
// m are zero keys/values with zero log decay and zero beta, so they change
// nothing) it computes, in fp32:
//   q^ = q / sqrt(|q|^2 + 1e-6), k^ likewise           (use_qk_l2norm_in_kernel)
//   b  = sigmoid(beta)                                   (use_beta_sigmoid_in_kernel)
//   l  = lower_bound * sigmoid(exp(A_log) (g + dt_bias)) (gate in kernel, safe gate;
//        lower_bound in [-5, 0] keeps |cumulative l| <= 80 over 16 tokens, so
//        exp(+-G) below stays finite in fp32 and bf16)
//   G  = cumulative sum of l over the chunk, gamma = exp(G), gamma_C = gamma_last
//   Qbar = scale q^ gamma, Kbar = k^ gamma, Ktil = k^ / gamma, Khat = Ktil gamma_C
//   A  = StrictLower(Diag(b) Kbar Ktil^T), T = (I + A)^{-1} by forward substitution
//   W  = T Diag(b) Kbar,  Ut = T Diag(b) V,  Aqk = LowerInclusive(Qbar Ktil^T)
// and writes W, Qbar (bf16), Khat and Aqk (bf16 high/low pairs), Ut and
// gamma_C (fp32) into the chunk record in the recurrence kernel's operand order.
//
// Precision: the small products A, Aqk, W and Ut take their operands as bf16
// high/low pairs, each packed into one 16x16x32 MFMA (the K dimension carries
// both halves), so they are accurate to ~2^-16 instead of bf16's 2^-8; the
// largest outputs are ~10x the output RMS, where plain bf16 operands alone
// would exceed a 3% of RMS error.
//
// Lane L owns key channels 2L and 2L+1 for all 16 tokens while loading (each
// load instruction reads one 256-byte token row) and while forming the decays
// (the cumulative sum runs in registers).  The bf16 tiles go through LDS:
// token-major rows for the products over channels, then (same storage)
// channel-major rows for the products over tokens.
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int ROWP = 136;  // token-major bf16 row pitch (272 B: 16-B aligned, conflict-free b128 reads)
constexpr int COLP = 20;   // channel-major bf16 row pitch (40 B: conflict-free b64 reads)
constexpr int MP = 20;     // fp32 16x16 matrix pitch (80 B: 16-B aligned rows)
constexpr int ROWT = C * ROWP;  // one token-major tile
constexpr int COLT = D * COLP;  // one channel-major tile

struct PrepSmem {
  // phase 1: Kbar hi/lo, Ktil hi/lo, Qbar hi/lo as token-major rows (6 tiles);
  // phase 2: Kbar hi/lo, Khat hi/lo, V as channel-major rows (5 tiles)
  uint16_t buf[6 * ROWT > 5 * COLT ? 6 * ROWT : 5 * COLT];
  float A[C * MP];
  float Tp[C * MP];
  float beta[C];
};

__device__ __forceinline__ float lane_read(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

__device__ __forceinline__ void store_col16(uint16_t* row, const float* x) {
  // 16 consecutive tokens of one channel -> 4 x 8-byte LDS writes
  u32x2* p = reinterpret_cast<u32x2*>(row);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    u32x2 w;
    w.x = pack2(x[4 * i + 0], x[4 * i + 1]);
    w.y = pack2(x[4 * i + 2], x[4 * i + 3]);
    p[i] = w;
  }
}

// writes hi = bf16(x) and lo = bf16(x - hi) for 16 tokens of one channel
__device__ __forceinline__ void store_col16_split(uint16_t* row_hi, uint16_t* row_lo, const float* x) {
  float h[C], l[C];
#pragma unroll
  for (int i = 0; i < C; ++i) {
    h[i] = hi_part(x[i]);
    l[i] = x[i] - h[i];
  }
  store_col16(row_hi, h);
  store_col16(row_lo, l);
}

__device__ __forceinline__ void store_row2_split(uint16_t* hi, uint16_t* lo, int off, float a, float b) {
  const float ha = hi_part(a), hb = hi_part(b);
  *reinterpret_cast<uint32_t*>(hi + off) = pack2(ha, hb);
  *reinterpret_cast<uint32_t*>(lo + off) = pack2(a - ha, b - hb);
}

// sum_k X[m][k] Y[n][k] over the 128 channels of two token-major tiles given as
// high/low pairs: X_hi Y_hi + X_hi Y_lo + X_lo Y_hi (4 k-steps of 32 channels)
__device__ __forceinline__ f32x4 rows_dot_split(const uint16_t* xh, const uint16_t* xl, const uint16_t* yh,
                                                const uint16_t* yl, int c, int g) {
  f32x4 acc = zero4();
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int o = c * ROWP + 32 * s + 8 * g;
    const u32x4 a_h = *reinterpret_cast<const u32x4*>(xh + o);
    const u32x4 a_l = *reinterpret_cast<const u32x4*>(xl + o);
    const u32x4 b_h = *reinterpret_cast<const u32x4*>(yh + o);
    const u32x4 b_l = *reinterpret_cast<const u32x4*>(yl + o);
    acc = mfma_k32(a_h, b_h, acc);
    acc = mfma_k32(a_h, b_l, acc);
    acc = mfma_k32(a_l, b_h, acc);
  }
  return acc;
}

}  // namespace

__global__ __launch_bounds__(64) void kda_prep_kernel(Problem p, Tables t, uint8_t* __restrict__ rec) {
  __shared__ PrepSmem sm;
  const int chunk = blockIdx.x;
  const int h = blockIdx.y;
  if (chunk >= t.counters[CNT_N_CHUNKS]) return;
  const int L = threadIdx.x;
  const int g = L >> 4;
  const int c = L & 15;
  const int H = p.H;

  const int seq = t.chunk_tab[2 * chunk];
  const int cis = t.chunk_tab[2 * chunk + 1];
  const long long tok0 = (long long)t.seq_start[seq] + (long long)C * cis;
  const int m = min(C, t.seq_len[seq] - C * cis);
  uint8_t* r = rec + ((long long)chunk * H + h) * REC_BYTES;

  const int c0 = 2 * L;
  const float a = expf(p.A_log[h]);
  const float adt0 = a * p.dt_bias[h * D + c0];
  const float adt1 = a * p.dt_bias[h * D + c0 + 1];

  // ---- load the chunk (lane owns channels c0, c0+1; rows past m are zero).
  // Every load is issued unconditionally (rows past m re-read row m-1, which
  // exists since m >= 1) so all 64 are in flight together; padding is zeroed
  // afterwards with selects.
  uint32_t qq[C], kk[C], vv[C], gg[C];
#pragma unroll
  for (int i = 0; i < C; ++i) {
    const long long off = ((tok0 + min(i, m - 1)) * H + h) * D + c0;
    qq[i] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p.q + off));
    kk[i] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p.k + off));
    vv[i] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p.v + off));
    gg[i] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p.g + off));
  }
  float q0[C], q1[C], k0[C], k1[C], v0[C], v1[C], l0[C], l1[C];
#pragma unroll
  for (int i = 0; i < C; ++i) {
    const bool ok = i < m;
    const uint32_t qi = ok ? qq[i] : 0u, ki = ok ? kk[i] : 0u, vi = ok ? vv[i] : 0u;
    q0[i] = __uint_as_float(qi << 16);
    q1[i] = __uint_as_float(qi & 0xFFFF0000u);
    k0[i] = __uint_as_float(ki << 16);
    k1[i] = __uint_as_float(ki & 0xFFFF0000u);
    v0[i] = __uint_as_float(vi << 16);
    v1[i] = __uint_as_float(vi & 0xFFFF0000u);
    const float x0 = fmaf(a, __uint_as_float(gg[i] << 16), adt0);
    const float x1 = fmaf(a, __uint_as_float(gg[i] & 0xFFFF0000u), adt1);
    l0[i] = ok ? p.lower_bound * __builtin_amdgcn_rcpf(1.0f + __expf(-x0)) : 0.f;
    l1[i] = ok ? p.lower_bound * __builtin_amdgcn_rcpf(1.0f + __expf(-x1)) : 0.f;
  }
  if (L < C) {
    const float bl = bf16_to_f32(p.beta[(tok0 + min(L, m - 1)) * H + h]);
    sm.beta[L] = (L < m) ? __builtin_amdgcn_rcpf(1.0f + __expf(-bl)) : 0.f;
  }

  // ---- squared norms of the 16 q rows and 16 k rows: butterfly reduction of
  // 32 values over 64 lanes; afterwards lane L holds value index L >> 1 ----
  float red[2 * C];
#pragma unroll
  for (int i = 0; i < C; ++i) {
    red[i] = fmaf(q0[i], q0[i], q1[i] * q1[i]);
    red[C + i] = fmaf(k0[i], k0[i], k1[i] * k1[i]);
  }
#pragma unroll
  for (int lvl = 0; lvl < 5; ++lvl) {
    const int off = 32 >> lvl;
    const int half = 16 >> lvl;
    const bool up = (L & off) != 0;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const float send = up ? red[i] : red[i + half];
      const float keep = up ? red[i + half] : red[i];
      red[i] = keep + __shfl_xor(send, off, 64);
    }
  }
  const float ssq = red[0] + __shfl_xor(red[0], 1, 64);
  const float rn = rsqrtf(ssq + 1e-6f);

  // ---- decays: cumulative log decay per channel over the 16 rows ----
  float G0 = 0.f, G1 = 0.f;
#pragma unroll
  for (int i = 0; i < C; ++i) {
    G0 += l0[i];
    G1 += l1[i];
    l0[i] = G0;  // l now holds G
    l1[i] = G1;
  }
  const float gC0 = __expf(G0);
  const float gC1 = __expf(G1);
  reinterpret_cast<f32x2*>(r + REC_GC)[L] = f32x2{gC0, gC1};

  uint16_t* const kbh = sm.buf;
  uint16_t* const kbl = sm.buf + ROWT;
  uint16_t* const kth = sm.buf + 2 * ROWT;
  uint16_t* const ktl = sm.buf + 3 * ROWT;
  uint16_t* const qbh = sm.buf + 4 * ROWT;
  uint16_t* const qbl = sm.buf + 5 * ROWT;
  float kb0[C], kb1[C], kt0[C], kt1[C];
#pragma unroll
  for (int i = 0; i < C; ++i) {
    const float sq = p.scale * lane_read(rn, 2 * i);       // scale / |q_i|
    const float rk = lane_read(rn, 2 * (C + i));           // 1 / |k_i|
    const float e0 = __expf(l0[i]), e1 = __expf(l1[i]);    // gamma
    const float i0 = __expf(-l0[i]), i1 = __expf(-l1[i]);  // 1 / gamma
    const float kh0 = k0[i] * rk, kh1 = k1[i] * rk;
    kb0[i] = kh0 * e0;
    kb1[i] = kh1 * e1;
    kt0[i] = kh0 * i0;
    kt1[i] = kh1 * i1;
    const int o = i * ROWP + c0;
    store_row2_split(kbh, kbl, o, kb0[i], kb1[i]);
    store_row2_split(kth, ktl, o, kt0[i], kt1[i]);
    store_row2_split(qbh, qbl, o, q0[i] * sq * e0, q1[i] * sq * e1);
  }
  __syncthreads();

  // ---- A_raw = Kbar Ktil^T and Aqk^T = Ktil Qbar^T over the 128 channels ----
  const f32x4 Araw = rows_dot_split(kbh, kbl, kth, ktl, c, g);  // D[4g+i][c] = Kbar_{4g+i} . Ktil_c
  const f32x4 AqkT = rows_dot_split(kth, ktl, qbh, qbl, c, g);  // D[4g+i][c] = Aqk[c][4g+i]
  {
    f32x4 aq;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * g + i;
      sm.A[row * MP + c] = (c < row) ? sm.beta[row] * Araw[i] : 0.f;
      aq[i] = (row <= c) ? AqkT[i] : 0.f;
    }
    u32x2 ah, al;
    split4(aq, ah, al);
    reinterpret_cast<u32x2*>(r + REC_AQK_HI)[L] = ah;
    reinterpret_cast<u32x2*>(r + REC_AQK_LO)[L] = al;
  }
  // Qbar (high part) in the recurrence's operand order, before the rows are reused
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const u32x2 lo = *reinterpret_cast<const u32x2*>(&qbh[c * ROWP + 32 * s + 4 * g]);
    const u32x2 hi = *reinterpret_cast<const u32x2*>(&qbh[c * ROWP + 32 * s + 16 + 4 * g]);
    reinterpret_cast<u32x4*>(r + REC_Q)[s * 64 + L] = cat(lo, hi);
  }
  __syncthreads();

  // ---- phase 2: channel-major tiles (same storage) ----
  uint16_t* const kbch = sm.buf;
  uint16_t* const kbcl = sm.buf + COLT;
  uint16_t* const khch = sm.buf + 2 * COLT;
  uint16_t* const khcl = sm.buf + 3 * COLT;
  uint16_t* const vc = sm.buf + 4 * COLT;
  {
    store_col16_split(&kbch[c0 * COLP], &kbcl[c0 * COLP], kb0);
    store_col16_split(&kbch[(c0 + 1) * COLP], &kbcl[(c0 + 1) * COLP], kb1);
#pragma unroll
    for (int i = 0; i < C; ++i) {
      kt0[i] *= gC0;  // Khat = Ktil gamma_C
      kt1[i] *= gC1;
    }
    store_col16_split(&khch[c0 * COLP], &khcl[c0 * COLP], kt0);
    store_col16_split(&khch[(c0 + 1) * COLP], &khcl[(c0 + 1) * COLP], kt1);
    store_col16(&vc[c0 * COLP], v0);
    store_col16(&vc[(c0 + 1) * COLP], v1);
  }

  // ---- T = (I + A)^{-1} by forward substitution; lane c owns column c ----
  {
    float tc[C];
#pragma unroll
    for (int i = 0; i < C; ++i) {
      float acc = 0.f;
#pragma unroll
      for (int pp = 0; pp < i; ++pp) acc = fmaf(sm.A[i * MP + pp], tc[pp], acc);
      tc[i] = (i == c) ? 1.f : ((i < c) ? 0.f : -acc);
    }
    if (L < C) {
      const float bc = sm.beta[c];
#pragma unroll
      for (int i = 0; i < C; ++i) sm.Tp[i * MP + c] = tc[i] * bc;  // T' = T Diag(b)
    }
  }
  __syncthreads();

  u32x2 tf_h, tf_l;  // T'[c][4g..4g+3] as a high/low pair
  split4(*reinterpret_cast<const f32x4*>(&sm.Tp[c * MP + 4 * g]), tf_h, tf_l);
  const u32x4 tf_hl = cat(tf_h, tf_l);

  // ---- W^T = Kbar^T T'^T, one channel tile per MFMA pair:
  // [Kbar^T_hi | Kbar^T_hi] [T'^T_hi ; T'^T_lo] + [Kbar^T_lo | Kbar^T_lo] [T'^T_hi ; T'^T_lo]
  f32x4 WT[8];
#pragma unroll
  for (int tt = 0; tt < 8; ++tt) {
    const int o = (16 * tt + c) * COLP + 4 * g;
    const u32x2 kh = *reinterpret_cast<const u32x2*>(&kbch[o]);
    const u32x2 kl = *reinterpret_cast<const u32x2*>(&kbcl[o]);
    f32x4 acc = mfma_k32(cat(kh, kh), tf_hl, zero4());
    WT[tt] = mfma_k32(cat(kl, kl), tf_hl, acc);  // D[4g+i][c] = W[token c][16tt+4g+i]
  }
#pragma unroll
  for (int s = 0; s < 4; ++s)
    reinterpret_cast<u32x4*>(r + REC_W)[s * 64 + L] = cat(pack4(WT[2 * s]), pack4(WT[2 * s + 1]));

  // ---- Ut = T' V = [T'_hi | T'_lo] [V ; V] (column tiles over value columns) ----
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const u32x2 vT = *reinterpret_cast<const u32x2*>(&vc[(16 * jj + c) * COLP + 4 * g]);
    reinterpret_cast<f32x4*>(r + REC_UT)[jj * 64 + L] = mfma_k32(tf_hl, cat(vT, vT), zero4());
  }

  // ---- Khat high/low in the recurrence's operand order ----
#pragma unroll
  for (int tt = 0; tt < 8; ++tt) {
    const int o = (16 * tt + c) * COLP + 4 * g;
    reinterpret_cast<u32x2*>(r + REC_KH_HI)[tt * 64 + L] = *reinterpret_cast<const u32x2*>(&khch[o]);
    reinterpret_cast<u32x2*>(r + REC_KH_LO)[tt * 64 + L] = *reinterpret_cast<const u32x2*>(&khcl[o]);
  }
}

hipError_t launch_prep(const Problem& p, Tables t, uint8_t* rec, int64_t max_chunks, hipStream_t st) {
  if (max_chunks <= 0) return hipSuccess;
  hipLaunchKernelGGL(kda_prep_kernel, dim3((unsigned)max_chunks, (unsigned)p.H), dim3(64), 0, st, p, t, rec);
  return hipGetLastError();
}

}  // namespace kda
