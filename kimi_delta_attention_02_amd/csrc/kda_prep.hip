// Chunk preparation ("K1" on the cuLA PR #106 page: K1 prepares decayed q/k,
// beta and the WY inverse; CHUNK = 16, D = 128, forward only).
//
// One wavefront per (chunk, head).  For the chunk's m <= 16 tokens (rows past
// m are zero keys/values with zero log decay and zero beta, so they change
// nothing) it computes, in fp32:
//   q^ = q / sqrt(|q|^2 + 1e-6), k^ likewise         (use_qk_l2norm_in_kernel)
//   b  = sigmoid(beta)                                 (use_beta_sigmoid_in_kernel)
//   l  = lower_bound * sigmoid(exp(A_log) (g + dt_bias)) (gate in kernel, safe gate;
//        lower_bound in [-5, 0] keeps |cumulative l| <= 80 over 16 tokens, so
//        exp(+-G) below stays finite in fp32 and bf16)
//   G  = cumulative sum of l over the chunk, gamma = exp(G), gamma_C = gamma_last
//   Qbar = scale q^ gamma, Kbar = k^ gamma, Ktil = k^ / gamma, Khat = Ktil gamma_C
//   A  = StrictLower(Diag(b) Kbar Ktil^T), T = (I + A)^{-1} by forward substitution
//   W  = T Diag(b) Kbar,  Ut = T Diag(b) V,  Aqk = LowerInclusive(Qbar Ktil^T)
// and writes W, Qbar, Khat (bf16), Ut (fp32), Aqk (bf16) and gamma_C (fp32)
// into the chunk record in the recurrence kernel's operand order.
//
// Lane L owns key channels 2L and 2L+1 for all 16 tokens while loading (each
// load instruction reads one 256-byte token row) and while forming the decays
// (the cumulative sum runs in registers).  The bf16 tiles go to LDS twice:
// token-major rows for the 16x16x32 products over channels, channel-major rows
// for the 16x16x16 products over tokens.
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int ROWP = 136;  // token-major bf16 row pitch (272 B: 16-B aligned, conflict-free b128 reads)
constexpr int COLP = 20;   // channel-major bf16 row pitch (40 B: conflict-free b64 reads)
constexpr int MP = 20;     // fp32 16x16 matrix pitch (80 B: 16-B aligned rows)

struct PrepSmem {
  uint16_t qrow[C * ROWP];
  uint16_t kbrow[C * ROWP];
  uint16_t ktrow[C * ROWP];
  uint16_t kbcol[D * COLP];
  uint16_t khcol[D * COLP];
  uint16_t vcol[D * COLP];
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

  // ---- load the chunk (lane owns channels c0, c0+1; rows past m are zero) ----
  float q0[C], q1[C], k0[C], k1[C], v0[C], v1[C], l0[C], l1[C];
#pragma unroll
  for (int i = 0; i < C; ++i) {
    uint32_t qq = 0, kk = 0, vv = 0, gg = 0;
    if (i < m) {
      const long long off = ((tok0 + i) * H + h) * D + c0;
      qq = *reinterpret_cast<const uint32_t*>(p.q + off);
      kk = *reinterpret_cast<const uint32_t*>(p.k + off);
      vv = *reinterpret_cast<const uint32_t*>(p.v + off);
      gg = *reinterpret_cast<const uint32_t*>(p.g + off);
    }
    q0[i] = __uint_as_float(qq << 16);
    q1[i] = __uint_as_float(qq & 0xFFFF0000u);
    k0[i] = __uint_as_float(kk << 16);
    k1[i] = __uint_as_float(kk & 0xFFFF0000u);
    v0[i] = __uint_as_float(vv << 16);
    v1[i] = __uint_as_float(vv & 0xFFFF0000u);
    if (i < m) {
      const float x0 = fmaf(a, __uint_as_float(gg << 16), adt0);
      const float x1 = fmaf(a, __uint_as_float(gg & 0xFFFF0000u), adt1);
      l0[i] = p.lower_bound * __builtin_amdgcn_rcpf(1.0f + __expf(-x0));
      l1[i] = p.lower_bound * __builtin_amdgcn_rcpf(1.0f + __expf(-x1));
    } else {
      l0[i] = 0.f;
      l1[i] = 0.f;
    }
  }
  if (L < C) {
    float b = 0.f;
    if (L < m) b = __builtin_amdgcn_rcpf(1.0f + __expf(-bf16_to_f32(p.beta[(tok0 + L) * H + h])));
    sm.beta[L] = b;
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

  float qb0[C], qb1[C], kb0[C], kb1[C], kt0[C], kt1[C];
#pragma unroll
  for (int i = 0; i < C; ++i) {
    const float sq = p.scale * lane_read(rn, 2 * i);     // scale / |q_i|
    const float rk = lane_read(rn, 2 * (C + i));         // 1 / |k_i|
    const float e0 = __expf(l0[i]), e1 = __expf(l1[i]);  // gamma
    const float i0 = __expf(-l0[i]), i1 = __expf(-l1[i]);  // 1 / gamma
    const float kh0 = k0[i] * rk, kh1 = k1[i] * rk;
    qb0[i] = q0[i] * sq * e0;
    qb1[i] = q1[i] * sq * e1;
    kb0[i] = kh0 * e0;
    kb1[i] = kh1 * e1;
    kt0[i] = kh0 * i0;
    kt1[i] = kh1 * i1;
    *reinterpret_cast<uint32_t*>(&sm.qrow[i * ROWP + c0]) = pack2(qb0[i], qb1[i]);
    *reinterpret_cast<uint32_t*>(&sm.kbrow[i * ROWP + c0]) = pack2(kb0[i], kb1[i]);
    *reinterpret_cast<uint32_t*>(&sm.ktrow[i * ROWP + c0]) = pack2(kt0[i], kt1[i]);
  }
  {
    float kh0c[C], kh1c[C];
#pragma unroll
    for (int i = 0; i < C; ++i) {
      kh0c[i] = kt0[i] * gC0;
      kh1c[i] = kt1[i] * gC1;
    }
    store_col16(&sm.kbcol[c0 * COLP], kb0);
    store_col16(&sm.kbcol[(c0 + 1) * COLP], kb1);
    store_col16(&sm.khcol[c0 * COLP], kh0c);
    store_col16(&sm.khcol[(c0 + 1) * COLP], kh1c);
    store_col16(&sm.vcol[c0 * COLP], v0);
    store_col16(&sm.vcol[(c0 + 1) * COLP], v1);
  }
  __syncthreads();

  // ---- A_raw = Kbar Ktil^T and Aqk^T = Ktil Qbar^T over the 128 channels ----
  f32x4 Araw = zero4(), AqkT = zero4();
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int o = c * ROWP + 32 * s + 8 * g;
    const u32x4 kb = *reinterpret_cast<const u32x4*>(&sm.kbrow[o]);
    const u32x4 kt = *reinterpret_cast<const u32x4*>(&sm.ktrow[o]);
    const u32x4 qb = *reinterpret_cast<const u32x4*>(&sm.qrow[o]);
    Araw = mfma_k32(kb, kt, Araw);  // D[4g+i][c] = Kbar_{4g+i} . Ktil_c
    AqkT = mfma_k32(kt, qb, AqkT);  // D[4g+i][c] = Ktil_{4g+i} . Qbar_c = Aqk[c][4g+i]
  }
  {
    f32x4 aq;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * g + i;
      sm.A[row * MP + c] = (c < row) ? sm.beta[row] * Araw[i] : 0.f;
      aq[i] = (row <= c) ? AqkT[i] : 0.f;
    }
    reinterpret_cast<u32x2*>(r + REC_AQK)[L] = pack4(aq);
  }
  __syncthreads();

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

  const u32x2 tf = pack4(*reinterpret_cast<const f32x4*>(&sm.Tp[c * MP + 4 * g]));  // T'[c][4g..4g+3]

  // ---- W^T = Kbar^T T'^T (row tiles over channels); stored as W rows ----
  f32x4 WT[8];
#pragma unroll
  for (int tt = 0; tt < 8; ++tt) {
    const u32x2 kbT = *reinterpret_cast<const u32x2*>(&sm.kbcol[(16 * tt + c) * COLP + 4 * g]);
    WT[tt] = mfma_k16(kbT, tf, zero4());  // D[4g+i][c] = W[token c][16tt+4g+i]
  }
#pragma unroll
  for (int s = 0; s < 4; ++s)
    reinterpret_cast<u32x4*>(r + REC_W)[s * 64 + L] = cat(pack4(WT[2 * s]), pack4(WT[2 * s + 1]));

  // ---- Ut = T' V (column tiles over value columns) ----
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const u32x2 vT = *reinterpret_cast<const u32x2*>(&sm.vcol[(16 * jj + c) * COLP + 4 * g]);
    reinterpret_cast<f32x4*>(r + REC_UT)[jj * 64 + L] = mfma_k16(tf, vT, zero4());
  }

  // ---- Qbar and Khat in the recurrence's operand order ----
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const u32x2 lo = *reinterpret_cast<const u32x2*>(&sm.qrow[c * ROWP + 32 * s + 4 * g]);
    const u32x2 hi = *reinterpret_cast<const u32x2*>(&sm.qrow[c * ROWP + 32 * s + 16 + 4 * g]);
    reinterpret_cast<u32x4*>(r + REC_Q)[s * 64 + L] = cat(lo, hi);
  }
#pragma unroll
  for (int tt = 0; tt < 8; ++tt)
    reinterpret_cast<u32x2*>(r + REC_KH)[tt * 64 + L] =
        *reinterpret_cast<const u32x2*>(&sm.khcol[(16 * tt + c) * COLP + 4 * g]);
}

hipError_t launch_prep(const Problem& p, Tables t, uint8_t* rec, int64_t max_chunks, hipStream_t st) {
  if (max_chunks <= 0) return hipSuccess;
  hipLaunchKernelGGL(kda_prep_kernel, dim3((unsigned)max_chunks, (unsigned)p.H), dim3(64), 0, st, p, t, rec);
  return hipGetLastError();
}

}  // namespace kda
