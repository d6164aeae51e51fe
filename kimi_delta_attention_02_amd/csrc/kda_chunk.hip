// Chunk kernel: chunk preparation ("K1" on the cuLA PR #106 page: decayed q/k,
// beta and the WY inverse) and the inter-chunk recurrence ("K2") or the segment
// pre-scan ("pre_scan"), in one workgroup, with the prepared operands handed
// from producer to consumer wavefronts through an LDS ring (no HBM hand-off).
//
// Workgroup = 8 wavefronts for one (segment, head):
//   producers 0..3 : wavefront p prepares chunks p, p+4, p+8, ... of the
//                    segment, each one alone (lane (g, c) = token c with key
//                    channels {32s+4g+0..3, 32s+16+4g+0..3}, s = 0..3, the
//                    consumers' own operand order), into ring slot (chunk % 6)
//   consumers 4..7 : wavefront 4+w walks the chunks in order and applies them
//                    to value columns 32w..32w+31 of the state (RECUR), or of
//                    both R and M (pre-scan), held in MFMA accumulators.
// Producers and consumers meet at per-slot flags in LDS (ready: the chunk a
// slot holds; done: the last chunk each consumer finished with it).  Every
// wait is bounded, so a wavefront always exits; a wait that gives up sets an
// error flag in the workspace counters.
//
// Per chunk of m <= 16 tokens (rows past m: zero keys/values/queries, zero
// log decay, zero beta):
//   q^ = q / sqrt(|q|^2 + 1e-6), k^ likewise; b = sigmoid(beta);
//   l = lower_bound * sigmoid(exp(A_log) (g + dt_bias)); G = cumulative sum of
//   l over the chunk (DPP scan along the 16 lanes of a row), gamma_C = e^{G_last};
//   Qbar = scale q^ e^G, Kbar = k^ e^G, Ktil = k^ e^-G, Khat = Ktil gamma_C;
//   A = StrictLower(Diag(b) Kbar Ktil^T), T = (I + A)^{-1} by forward
//   substitution (4 lanes per column, DPP quad sums), T' = T Diag(b);
//   Aqk = LowerInclusive(Qbar Ktil^T)
// and the consumers, with S the K x V state entering the chunk:
//   Y = Kbar S;  X = T' Y (= W S, W = T' Kbar);  Ut = T' V;  U = Ut - X
//   O = Qbar S + Aqk U;  S <- Diag(gamma_C) S + Khat^T U
// (pre-scan: M starts at I with Ut = 0, R starts at 0; neither writes O).
//
// Every product is a 16x16x32 bf16 MFMA with fp32 accumulation; A, Aqk, T', U
// and Khat enter as bf16 high/low pairs (x = x_hi + x_lo, ~16 significant
// bits) packed into the 32-long K dimension: the largest outputs and state
// entries are ~10x their RMS, where plain bf16 operands cost more than 3% of
// the RMS.  A 16x16 accumulator tile holds rows 4g..4g+3 of column c in lane
// 16g+c, which is also the bf16 operand layout of the next chunk's products,
// so the state never leaves registers within a segment.
#include "kda_internal.h"

namespace kda {

namespace {

enum Role { RECUR = 0, PRE = 1 };

constexpr int NSLOT = 6;
constexpr int MP = 20;                 // fp32 16x16 matrix pitch
constexpr int SPIN_LIMIT = 1 << 24;    // polls (each with s_sleep) before a wait gives up

struct Slot {
  u32x4 kbf[4][64];       // Kbar (bf16) operand fragment per k-step s
  u32x4 qbf[4][64];       // Qbar (bf16) operand fragment per k-step s
  uint16_t khT[2][D][C];  // Khat^T high / low part, [channel][token]
  float gC[D];            // gamma_C per key channel
  u32x4 tf[64];           // [T'_hi | T'_lo] fragment: T'[c][4g..4g+3]
  u32x4 aq[64];           // (Aqk_hi, Aqk_lo) fragment: Aqk[c][4g..4g+3]
};

struct Smem {
  Slot slot[NSLOT];
  float Aq[4][C][16];     // per producer: A rows arranged for the quad-parallel solve
  float Tp[4][C * MP];    // per producer: T'
  float bt[4][C];         // per producer: beta of the chunk's tokens
  float adt[D];           // exp(A_log) * dt_bias of the head
  int ready[NSLOT];
  int done[NSLOT][4];
};

// raw inputs of one chunk for one producer lane
struct ProdIn {
  u32x2 q[8], k[8], g[8];  // index 2s+h: channels 32s+16h+4g+0..3 of token c
  uint32_t b;
};

// Orders this wavefront's LDS writes before its later LDS reads by other lanes
// (LDS executes one wavefront's operations in order; this only stops the
// compiler from moving accesses across the point).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// flag reads are made wavefront-uniform so that every wait loop is a scalar loop
__device__ __forceinline__ int wg_load(int* p) {
  return __builtin_amdgcn_readfirstlane(__hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP));
}
__device__ __forceinline__ void wg_store(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

template <int CTRL>
__device__ __forceinline__ float dppz(float x) {  // lanes with no source read 0
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// inclusive prefix sum over the 16 lanes of each row
__device__ __forceinline__ float row_scan(float x) {
  x += dppz<0x111>(x);  // row_shr:1
  x += dppz<0x112>(x);  // row_shr:2
  x += dppz<0x114>(x);  // row_shr:4
  x += dppz<0x118>(x);  // row_shr:8
  return x;
}

// value of lane 15 of each row, broadcast to the row (row_newbcast:15)
__device__ __forceinline__ float row_last(float x) { return dppz<0x15F>(x); }

__device__ __forceinline__ void unpack4(u32x2 v, float* f) {
  f[0] = __uint_as_float(v.x << 16);
  f[1] = __uint_as_float(v.x & 0xFFFF0000u);
  f[2] = __uint_as_float(v.y << 16);
  f[3] = __uint_as_float(v.y & 0xFFFF0000u);
}

__device__ __forceinline__ void split8(const float* x, u32x4& hi, u32x4& lo) {
  float h[8], l[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h[e] = hi_part(x[e]);
    l[e] = x[e] - h[e];
  }
  hi = u32x4{pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7])};
  lo = u32x4{pack2(l[0], l[1]), pack2(l[2], l[3]), pack2(l[4], l[5]), pack2(l[6], l[7])};
}

__device__ __forceinline__ void load_prod(ProdIn& in, const Problem& p, long long tok0, int m, int h, int g, int c) {
  const long long row = ((tok0 + min(c, m - 1)) * p.H + h) * D + 4 * g;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int off = 32 * (i >> 1) + 16 * (i & 1);
    in.q[i] = *reinterpret_cast<const u32x2*>(p.q + row + off);
    in.k[i] = *reinterpret_cast<const u32x2*>(p.k + row + off);
    in.g[i] = *reinterpret_cast<const u32x2*>(p.g + row + off);
  }
  in.b = p.beta[(tok0 + min(c, m - 1)) * p.H + h];
}

// V[4g+0..3][col] of one 16-column tile as raw bf16 values; masked and packed
// only where they are used, so a prefetch is not waited for where it is issued
struct VRaw {
  uint32_t r[4];
};

__device__ __forceinline__ void load_v(VRaw& x, const Problem& p, long long tok0, int m, int h, int g, int col) {
#pragma unroll
  for (int i = 0; i < 4; ++i) x.r[i] = p.v[((tok0 + min(4 * g + i, m - 1)) * p.H + h) * D + col];
}

__device__ __forceinline__ u32x2 pack_v(const VRaw& x, int m, int g) {
  uint32_t t[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) t[i] = (4 * g + i < m) ? x.r[i] : 0u;  // rows past the chunk end are zero
  return u32x2{t[0] | (t[1] << 16), t[2] | (t[3] << 16)};
}

// ---------------------------------------------------------------- producer
// Prepares one chunk into a ring slot.  want_q: also Qbar and Aqk (RECUR).
__device__ __forceinline__ void produce(Smem& sm, Slot& sl, int pw, const ProdIn& in, const Problem& p, int m,
                                        float a, bool want_q, int L, int g, int c) {
  const bool ok = c < m;
  // squared norms of q_c, k_c over the 128 channels
  float sq = 0.f, sk = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float qf[4], kf[4];
    unpack4(in.q[i], qf);
    unpack4(in.k[i], kf);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sq = fmaf(qf[e], qf[e], sq);
      sk = fmaf(kf[e], kf[e], sk);
    }
  }
  sq += __shfl_xor(sq, 16, 64);
  sq += __shfl_xor(sq, 32, 64);
  sk += __shfl_xor(sk, 16, 64);
  sk += __shfl_xor(sk, 32, 64);
  const float rq = ok ? p.scale * __builtin_amdgcn_rsqf(sq + 1e-6f) : 0.f;  // zero rows past m
  const float rk = ok ? __builtin_amdgcn_rsqf(sk + 1e-6f) : 0.f;
  const float bt = ok ? __builtin_amdgcn_rcpf(1.0f + __expf(-__uint_as_float(in.b << 16))) : 0.f;
  sm.bt[pw][c] = bt;  // the four lanes of a token store the same value
  wave_lds_sync();

  f32x4 Araw = zero4(), AqkT = zero4();
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    float qf[8], kf[8], gf[8];
    unpack4(in.q[2 * s], qf);
    unpack4(in.q[2 * s + 1], qf + 4);
    unpack4(in.k[2 * s], kf);
    unpack4(in.k[2 * s + 1], kf + 4);
    unpack4(in.g[2 * s], gf);
    unpack4(in.g[2 * s + 1], gf + 4);
    float Kb[8], Kt[8], Qb[8], Kh[8], gce[8], adt[8];
    *reinterpret_cast<f32x4*>(&adt[0]) = *reinterpret_cast<const f32x4*>(&sm.adt[32 * s + 4 * g]);
    *reinterpret_cast<f32x4*>(&adt[4]) = *reinterpret_cast<const f32x4*>(&sm.adt[32 * s + 16 + 4 * g]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = fmaf(a, gf[e], adt[e]);
      const float l = ok ? p.lower_bound * __builtin_amdgcn_rcpf(1.0f + __expf(-x)) : 0.f;
      const float G = row_scan(l);
      const float ep = __expf(G), em = __expf(-G);
      gce[e] = row_last(ep);
      const float kh = kf[e] * rk;
      Kb[e] = kh * ep;
      Kt[e] = kh * em;
      Qb[e] = qf[e] * rq * ep;
      Kh[e] = Kt[e] * gce[e];
    }
    u32x4 kbh, kbl, kth, ktl;
    split8(Kb, kbh, kbl);
    split8(Kt, kth, ktl);
    Araw = mfma_k32(kbh, kth, Araw);  // D[4g+i][c] += Kbar_{4g+i} . Ktil_c over this k-step
    Araw = mfma_k32(kbh, ktl, Araw);
    Araw = mfma_k32(kbl, kth, Araw);
    sl.kbf[s][L] = kbh;
    if (want_q) {
      u32x4 qbh, qbl;
      split8(Qb, qbh, qbl);
      AqkT = mfma_k32(kth, qbh, AqkT);  // D[4g+i][c] += Ktil_{4g+i} . Qbar_c = Aqk[c][4g+i]
      AqkT = mfma_k32(kth, qbl, AqkT);
      AqkT = mfma_k32(ktl, qbh, AqkT);
      sl.qbf[s][L] = qbh;
    }
    // Khat^T (channel-major) high / low, and gamma_C
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int ch = 32 * s + 16 * (e >> 2) + 4 * g + (e & 3);
      const float hh = hi_part(Kh[e]);
      const uint32_t pk = pack2(hh, Kh[e] - hh);
      sl.khT[0][ch][c] = (uint16_t)(pk & 0xFFFFu);
      sl.khT[1][ch][c] = (uint16_t)(pk >> 16);
    }
    if (c == 0) {
      *reinterpret_cast<f32x4*>(&sl.gC[32 * s + 4 * g]) = f32x4{gce[0], gce[1], gce[2], gce[3]};
      *reinterpret_cast<f32x4*>(&sl.gC[32 * s + 16 + 4 * g]) = f32x4{gce[4], gce[5], gce[6], gce[7]};
    }
  }

  // A = StrictLower(Diag(b) A_raw) into the solve layout Aq[i][4(p%4) + p/4] = A[i][p]
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * g + i;
    sm.Aq[pw][row][4 * (c & 3) + (c >> 2)] = (c < row) ? sm.bt[pw][row] * Araw[i] : 0.f;
  }
  if (want_q) {
    f32x4 aq;
#pragma unroll
    for (int i = 0; i < 4; ++i) aq[i] = (4 * g + i <= c) ? AqkT[i] : 0.f;
    u32x2 ah, al;
    split4(aq, ah, al);
    sl.aq[L] = cat(ah, al);
  }

  wave_lds_sync();
  // T = (I + A)^{-1} by forward substitution: lane 4j+q owns column j and the
  // rows p = q, q+4, q+8, q+12; row i's dot product is split over the quad
  {
    const int j = L >> 2, q = L & 3;
    float t0 = 0.f, t1 = 0.f, t2 = 0.f, t3 = 0.f;  // T[q+4k][j]
#pragma unroll
    for (int i = 0; i < C; ++i) {
      const f32x4 ar = *reinterpret_cast<const f32x4*>(&sm.Aq[pw][i][4 * q]);  // A[i][q+4k], k = 0..3
      float part = ar[0] * t0;
      part = fmaf(ar[1], t1, part);
      part = fmaf(ar[2], t2, part);
      part = fmaf(ar[3], t3, part);
      part += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(part), 0xB1, 0xF, 0xF, false));  // quad xor 1
      part += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(part), 0x4E, 0xF, 0xF, false));  // quad xor 2
      const float tij = (i == j) ? 1.f : ((i < j) ? 0.f : -part);
      if ((i & 3) == q) {
        if ((i >> 2) == 0) t0 = tij;
        else if ((i >> 2) == 1) t1 = tij;
        else if ((i >> 2) == 2) t2 = tij;
        else t3 = tij;
      }
    }
    const float bj = sm.bt[pw][j];
    sm.Tp[pw][(q + 0) * MP + j] = t0 * bj;  // T' = T Diag(b)
    sm.Tp[pw][(q + 4) * MP + j] = t1 * bj;
    sm.Tp[pw][(q + 8) * MP + j] = t2 * bj;
    sm.Tp[pw][(q + 12) * MP + j] = t3 * bj;
  }
  wave_lds_sync();
  u32x2 th, tl;
  split4(*reinterpret_cast<const f32x4*>(&sm.Tp[pw][c * MP + 4 * g]), th, tl);
  sl.tf[L] = cat(th, tl);
}

// ---------------------------------------------------------------- consumer
// A state column tile is f32x4 S[8]: S[t] holds rows 16t+4g+0..3 of column c.

// U = Ut - T'(Kbar S) of one column tile as a high/low pair (Ut = T'V, or 0 when v is null)
__device__ __forceinline__ u32x4 tile_u(const u32x2 (&Sb)[8], const u32x4 (&kb)[4], u32x4 tf, const u32x2* v) {
  f32x4 Y = zero4();
#pragma unroll
  for (int s = 0; s < 4; ++s) Y = mfma_k32(kb[s], cat(Sb[2 * s], Sb[2 * s + 1]), Y);
  const u32x2 Yb = pack4(Y);
  const f32x4 X = mfma_k32(tf, cat(Yb, Yb), zero4());
  const f32x4 U = v ? mfma_k32(tf, cat(*v, *v), zero4()) - X : -X;
  u32x2 uh, ul;
  split4(U, uh, ul);
  return cat(uh, ul);
}

// S <- Diag(gamma_C) S + Khat^T U for NT column tiles; the Khat / gamma_C
// fragments of a row tile are read once and used by every column tile
template <int NT>
__device__ __forceinline__ void tiles_update(f32x4 (&S)[NT][8], const u32x4 (&Uhl)[NT], const Slot& sl, int g, int c) {
#pragma unroll
  for (int tt = 0; tt < 8; ++tt) {
    const int ch = 16 * tt + c;
    const u32x2 kh = *reinterpret_cast<const u32x2*>(&sl.khT[0][ch][4 * g]);
    const u32x2 kl = *reinterpret_cast<const u32x2*>(&sl.khT[1][ch][4 * g]);
    const f32x4 gc = *reinterpret_cast<const f32x4*>(&sl.gC[16 * tt + 4 * g]);
#pragma unroll
    for (int jj = 0; jj < NT; ++jj) {
      const f32x4 acc = mfma_k32(cat(kh, kh), Uhl[jj], S[jj][tt] * gc);
      S[jj][tt] = mfma_k32(cat(kl, kl), Uhl[jj], acc);
    }
  }
}

__device__ __forceinline__ void pack_tile(const f32x4 (&S)[8], u32x2 (&Sb)[8]) {
#pragma unroll
  for (int tt = 0; tt < 8; ++tt) Sb[tt] = pack4(S[tt]);
}

// All loads are issued before any value is converted, so they overlap.
template <int NT>
__device__ __forceinline__ void load_state(f32x4 (&S)[NT][8], const void* src, bool f32, long long base, int col0,
                                           int g, int c) {
  if (!src) {
#pragma unroll
    for (int jj = 0; jj < NT; ++jj)
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) S[jj][tt] = zero4();
  } else if (f32) {
    const float* s = static_cast<const float*>(src) + base;
#pragma unroll
    for (int jj = 0; jj < NT; ++jj)
#pragma unroll
      for (int tt = 0; tt < 8; ++tt)
        S[jj][tt] = *reinterpret_cast<const f32x4*>(s + (long long)(col0 + 16 * jj + c) * D + 16 * tt + 4 * g);
  } else {
    const uint16_t* s = static_cast<const uint16_t*>(src) + base;
    u32x2 raw[NT][8];
#pragma unroll
    for (int jj = 0; jj < NT; ++jj)
#pragma unroll
      for (int tt = 0; tt < 8; ++tt)
        raw[jj][tt] = *reinterpret_cast<const u32x2*>(s + (long long)(col0 + 16 * jj + c) * D + 16 * tt + 4 * g);
#pragma unroll
    for (int jj = 0; jj < NT; ++jj)
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        float f[4];
        unpack4(raw[jj][tt], f);
        S[jj][tt] = f32x4{f[0], f[1], f[2], f[3]};
      }
  }
}

template <int NT>
__device__ __forceinline__ void store_state(const f32x4 (&S)[NT][8], float* dst32, uint16_t* dst16, long long base,
                                            int col0, int g, int c) {
#pragma unroll
  for (int jj = 0; jj < NT; ++jj) {
    const int col = col0 + 16 * jj + c;
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      const long long off = base + (long long)col * D + 16 * tt + 4 * g;
      if (dst32) *reinterpret_cast<f32x4*>(dst32 + off) = S[jj][tt];
      if (dst16) *reinterpret_cast<u32x2*>(dst16 + off) = pack4(S[jj][tt]);
    }
  }
}

}  // namespace

template <int ROLE>
__device__ __forceinline__ void chunk_body(Smem& sm, const Problem& p, const Tables& t, float* __restrict__ segM,
                                           float* __restrict__ segR, float* __restrict__ segS, int phase,
                                           int sidx, int h) {
  if (sidx >= t.counters[CNT_N_SEGS]) return;
  const int seq = t.seg_tab[4 * sidx + 0];
  const int cb = t.seg_tab[4 * sidx + 1];
  const int ce = t.seg_tab[4 * sidx + 2];
  const int j = t.seg_tab[4 * sidx + 3];
  const int ns = t.seq_seg_off[seq + 1] - t.seq_seg_off[seq];
  if (ROLE == RECUR) {
    if (phase == 0 ? (j != 0) : (j == 0)) return;
  } else {
    if (!(j > 0 && j < ns - 1)) return;
  }

  const int H = p.H;
  const int wave = threadIdx.x >> 6;
  const int L = threadIdx.x & 63;
  const int g = L >> 4;
  const int c = L & 15;
  const int nch = ce - cb;
  const int first_chunk = t.seq_chunk_off[seq];
  const long long seq_tok0 = t.seq_start[seq];
  const int seq_len = t.seq_len[seq];
  auto chunk_m = [&](int lc) { return min(C, seq_len - C * (cb + lc - first_chunk)); };
  auto chunk_tok0 = [&](int lc) { return seq_tok0 + (long long)C * (cb + lc - first_chunk); };

  if (threadIdx.x < D) sm.adt[threadIdx.x] = expf(p.A_log[h]) * p.dt_bias[h * D + threadIdx.x];
  if (threadIdx.x < NSLOT) sm.ready[threadIdx.x] = -1;
  if (threadIdx.x < NSLOT * 4) sm.done[threadIdx.x >> 2][threadIdx.x & 3] = -1;
  __syncthreads();

  if (wave < 4) {
    // ======================= producer =======================
    const int pw = wave;
    const float a = expf(p.A_log[h]);
    ProdIn inA, inB;
    auto run = [&](const ProdIn& in, int lc) -> bool {
      const int slot = lc % NSLOT;
      if (lc >= NSLOT) {  // wait until every consumer is done with chunk lc - NSLOT
        int it = 0;
        while (true) {
          const int d = min(min(wg_load(&sm.done[slot][0]), wg_load(&sm.done[slot][1])),
                            min(wg_load(&sm.done[slot][2]), wg_load(&sm.done[slot][3])));
          if (d >= lc - NSLOT) break;
          if (++it > SPIN_LIMIT) {
            if (L == 0) atomicOr(&t.counters[CNT_FLAGS], 0x100);
            return false;
          }
          __builtin_amdgcn_s_sleep(1);
        }
      }
      produce(sm, sm.slot[slot], pw, in, p, chunk_m(lc), a, ROLE == RECUR, L, g, c);
      wg_store(&sm.ready[slot], lc);
      return true;
    };
    // the next chunk's inputs are loaded before this one is prepared; past the
    // last chunk the load repeats the current one (always in bounds, unused)
    auto load = [&](ProdIn& in, int lc) {
      const int lcc = lc < nch ? lc : lc - 4;
      load_prod(in, p, chunk_tok0(lcc), chunk_m(lcc), h, g, c);
    };
    int lc = pw;
    if (lc < nch) load(inA, lc);
    while (lc < nch) {
      load(inB, lc + 4);
      if (!run(inA, lc)) break;
      lc += 4;
      if (lc >= nch) break;
      load(inA, lc + 4);
      if (!run(inB, lc)) break;
      lc += 4;
    }
    return;
  }

  // ======================= consumer =======================
  const int cw = wave - 4;
  const int col0 = 32 * cw;
  const long long state_base = ((long long)seq * H + h) * D * D;
  const long long seg_base = ((long long)sidx * H + h) * D * D;

  auto wait_ready = [&](int slot, int lc) -> bool {
    int it = 0;
    while (wg_load(&sm.ready[slot]) != lc) {
      if (++it > SPIN_LIMIT) {
        if (L == 0) atomicOr(&t.counters[CNT_FLAGS], 0x200);
        return false;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    return true;
  };

  // V of the next chunk is loaded before this one is applied; past the last
  // chunk the load repeats the last one (always in bounds, unused)
  VRaw vA[2], vB[2];
  auto loadv = [&](VRaw (&v)[2], int lc) {
    const int lcc = min(lc, nch - 1);
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) load_v(v[jj], p, chunk_tok0(lcc), chunk_m(lcc), h, g, col0 + 16 * jj + c);
  };

  if (ROLE == RECUR) {
    f32x4 S[2][8];
    {
      const bool from_seg = (phase == 1);
      load_state<2>(S, from_seg ? (const void*)(segS + seg_base) : p.init_state, from_seg || p.state_fp32,
                    from_seg ? 0 : state_base, col0, g, c);
    }
    auto step = [&](const VRaw (&vr)[2], int lc) -> bool {
      const int slot = lc % NSLOT;
      if (!wait_ready(slot, lc)) return false;
      const Slot& sl = sm.slot[slot];
      u32x4 kb[4], qb[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        kb[s] = sl.kbf[s][L];
        qb[s] = sl.qbf[s][L];
      }
      const u32x4 tf = sl.tf[L];
      const u32x4 aqf = sl.aq[L];
      const u32x4 aqh = u32x4{aqf.x, aqf.y, aqf.x, aqf.y};
      const u32x4 aql = u32x4{aqf.z, aqf.w, aqf.z, aqf.w};
      const int m = chunk_m(lc);
      const long long tok = chunk_tok0(lc) + c;
      const u32x2 v[2] = {pack_v(vr[0], m, g), pack_v(vr[1], m, g)};
      u32x4 Uhl[2];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        u32x2 Sb[8];
        pack_tile(S[jj], Sb);
        Uhl[jj] = tile_u(Sb, kb, tf, &v[jj]);
        // O^T = S^T Qbar^T + U^T Aqk^T
        f32x4 Ot = zero4();
#pragma unroll
        for (int s = 0; s < 4; ++s) Ot = mfma_k32(cat(Sb[2 * s], Sb[2 * s + 1]), qb[s], Ot);
        Ot = mfma_k32(Uhl[jj], aqh, Ot);
        Ot = mfma_k32(Uhl[jj], aql, Ot);
        if (c < m) *reinterpret_cast<u32x2*>(p.out + (tok * H + h) * D + col0 + 16 * jj + 4 * g) = pack4(Ot);
      }
      tiles_update<2>(S, Uhl, sl, g, c);
      wg_store(&sm.done[slot][cw], lc);
      return true;
    };
    if (nch > 0) loadv(vA, 0);
    for (int lc = 0; lc < nch; lc += 2) {
      loadv(vB, lc + 1);
      if (!step(vA, lc)) break;
      if (lc + 1 >= nch) break;
      loadv(vA, lc + 2);
      if (!step(vB, lc + 1)) break;
    }
    float* dst32 = nullptr;
    uint16_t* dst16 = nullptr;
    long long base = 0;
    if (j == ns - 1) {
      if (p.final_state) {
        base = state_base;
        if (p.state_fp32)
          dst32 = static_cast<float*>(p.final_state);
        else
          dst16 = static_cast<uint16_t*>(p.final_state);
      }
    } else {
      dst32 = segS;  // start state of the next segment of this sequence (slot sidx + 1)
      base = seg_base + (long long)H * D * D;
    }
    store_state<2>(S, dst32, dst16, base, col0, g, c);
  } else {
    // pre-scan on the same columns: X[0..1] = R (start 0, with Ut), X[2..3] = M (start I, Ut = 0)
    f32x4 X[4][8];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        X[jj][tt] = zero4();
        f32x4 x;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = (16 * tt + 4 * g + i == col0 + 16 * jj + c) ? 1.f : 0.f;
        X[2 + jj][tt] = x;
      }
    auto step = [&](const VRaw (&vr)[2], int lc) -> bool {
      const int slot = lc % NSLOT;
      if (!wait_ready(slot, lc)) return false;
      const Slot& sl = sm.slot[slot];
      u32x4 kb[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) kb[s] = sl.kbf[s][L];
      const u32x4 tf = sl.tf[L];
      const int m = chunk_m(lc);
      const u32x2 v[2] = {pack_v(vr[0], m, g), pack_v(vr[1], m, g)};
      u32x4 Uhl[4];
#pragma unroll
      for (int x = 0; x < 4; x += 2) {  // two tiles at a time: enough independent MFMAs, bounded live range
        u32x2 Sb0[8], Sb1[8];
        pack_tile(X[x], Sb0);
        pack_tile(X[x + 1], Sb1);
        Uhl[x] = tile_u(Sb0, kb, tf, x < 2 ? &v[0] : nullptr);
        Uhl[x + 1] = tile_u(Sb1, kb, tf, x < 2 ? &v[1] : nullptr);
        __builtin_amdgcn_sched_barrier(0);
      }
      tiles_update<4>(X, Uhl, sl, g, c);
      wg_store(&sm.done[slot][cw], lc);
      return true;
    };
    if (nch > 0) loadv(vA, 0);
    for (int lc = 0; lc < nch; lc += 2) {
      loadv(vB, lc + 1);
      if (!step(vA, lc)) break;
      if (lc + 1 >= nch) break;
      loadv(vA, lc + 2);
      if (!step(vB, lc + 1)) break;
    }
    store_state<2>(*reinterpret_cast<f32x4(*)[2][8]>(&X[0]), segR, nullptr, seg_base, col0, g, c);
    store_state<2>(*reinterpret_cast<f32x4(*)[2][8]>(&X[2]), segM, nullptr, seg_base, col0, g, c);
  }
}

// MODE 0: recurrence of the segments the phase selects (one block per segment).
// MODE 1: first pass of a segmented call, blocks [0, n) pre-scan the middle
// segments and blocks [n, 2n) run the recurrence over the first segments.
template <int MODE>
__global__ __launch_bounds__(512) void kda_chunk_kernel(Problem p, Tables t, float* __restrict__ segM,
                                                        float* __restrict__ segR, float* __restrict__ segS,
                                                        int phase) {
  __shared__ Smem sm;
  if (MODE == 0) {
    chunk_body<RECUR>(sm, p, t, segM, segR, segS, phase, blockIdx.x, blockIdx.y);
  } else {
    const int half = gridDim.x / 2;
    if ((int)blockIdx.x < half)
      chunk_body<PRE>(sm, p, t, segM, segR, segS, 0, blockIdx.x, blockIdx.y);
    else
      chunk_body<RECUR>(sm, p, t, segM, segR, segS, 0, blockIdx.x - half, blockIdx.y);
  }
}

hipError_t launch_chunks(const Problem& p, Tables t, float* segM, float* segR, float* segS, int64_t max_segs,
                         int phase, bool segmented, hipStream_t st) {
  if (max_segs <= 0) return hipSuccess;
  if (phase == 0 && segmented) {
    hipLaunchKernelGGL(kda_chunk_kernel<1>, dim3((unsigned)(2 * max_segs), (unsigned)p.H), dim3(512), 0, st, p, t,
                       segM, segR, segS, 0);
  } else {
    hipLaunchKernelGGL(kda_chunk_kernel<0>, dim3((unsigned)max_segs, (unsigned)p.H), dim3(512), 0, st, p, t, segM,
                       segR, segS, phase);
  }
  return hipGetLastError();
}

}  // namespace kda
