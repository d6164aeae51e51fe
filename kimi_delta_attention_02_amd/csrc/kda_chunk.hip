// Chunk kernel: chunk preparation ("K1" on the cuLA PR #106 page: decayed q/k,
// beta and the WY inverse) and the inter-chunk recurrence ("K2") in one
// workgroup, with the prepared operands handed from producer to consumer
// wavefronts through an LDS ring (no HBM hand-off).
//
// Workgroup = 12 wavefronts (3 per SIMD) for one (segment, head), or 8 in the
// build with 4 consumers:
//   producers 0..3  : wavefront p prepares chunks p, p+4, p+8, ... of the
//                     segment, each one alone (lane (g, c) = token c with key
//                     channels {32s+4g+0..3, 32s+16+4g+0..3}, s = 0..3, the
//                     consumers' own operand order), into ring slot chunk % 6
//   consumers       : wavefront 4+w walks the chunks in order and applies them
//                     to value columns 16w..16w+15 (two such tiles with 4
//                     consumers) of the state, held in MFMA accumulators
//                     (first pass of a segment >= 1: the zero-start state R,
//                     plus the transition M while it is nonzero).
// V goes through the slot as whole rows (the producer loads 256-byte token rows
// with the chunk's other inputs); each consumer reads its column slice and
// overwrites it with its slice of the output, and the producer that next reuses
// the slot writes the output rows out whole, so HBM sees full rows both ways.
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
//   Y = Kbar S;  U = T' V - T' Y (one accumulation: the consumers hold -Kbar)
//   O = Qbar S + Aqk U;  S <- Diag(gamma_C) (S + Ktil^T U)  (Khat = Ktil gamma_C)
// (M starts at I with Ut = 0 and writes no output).
//
// Every product is a 16x16x32 bf16 MFMA with fp32 accumulation; Aqk (and its
// factors Qbar, Ktil), T', U and Ktil in the update enter as bf16 high/low pairs (x = x_hi + x_lo, ~16 significant
// bits) packed into the 32-long K dimension: the largest outputs and state
// entries are ~10x their RMS, where plain bf16 operands cost more than 3% of
// the RMS.  A 16x16 accumulator tile holds rows 4g..4g+3 of column c in lane
// 16g+c, which is also the bf16 operand layout of the next chunk's products,
// so the state never leaves registers within a segment.
#include <cfloat>
#include <type_traits>

#include "kda_internal.h"

namespace kda {

namespace {

// Consumer wavefronts: 8, one 16-column state tile each (kda_chunk_kernel).
// The file is also built with KDA_CONSUMERS=4, two tiles each, into
// kda_chunk_kernel_c4: a consumer then shares its per-chunk operand loads,
// waits and loop overhead between two tiles, which is faster on long units
// and slower on short ones.  Each state column goes through the same
// instructions in both, so they give the same bits.
#ifndef KDA_CONSUMERS
#define KDA_CONSUMERS 8
#endif
// Row tiles of the state update whose LDS operands a consumer step reads
// together with the chunk's other operands, before its first product (the
// rest are read during the update).  Four measured best in both builds
// (1.5-2.8 % faster than none; eight spills in the first-pass kernels).
#ifndef KDA_HOIST
#define KDA_HOIST 4
#endif
constexpr int NPW = 4;                  // producer wavefronts
constexpr int NCW = KDA_CONSUMERS;      // consumer wavefronts
constexpr int TPW = (D / 16) / NCW;     // 16-column state tiles per consumer wavefront
constexpr int NTHREADS = 64 * (NPW + NCW);
#ifndef KDA_NSLOT
#define KDA_NSLOT 8
#endif
constexpr int NSLOT = KDA_NSLOT;  // ring slots
constexpr int MP = 20;               // fp32 16x16 matrix pitch
constexpr int SPIN_LIMIT = 1 << 24;  // polls (each with s_sleep) before a wait gives up
constexpr float LOG2E = 1.4426950408889634f;

// One prepared chunk.  Every fragment is stored in the register order of the
// MFMA operand that reads it, so the consumers read 16 bytes per lane and use
// them as they are.
struct Slot {
  u32x4 kbf[4][64];   // -Kbar bf16, A operand of -Kbar S: k-step s, lane (g, c) = token c (negated:
                      // its product is -Y, whose bf16 is the operand U = T' V + T' (-Yb) needs)
  u32x4 qbf[4][64];   // Qbar bf16, B operand of S^T Qbar^T, same arrangement
  u32x2 ktp[D][4];    // [channel][(g + (channel % 16) / 4) % 4]: Khat = Ktil gamma_C (at most 1 in
                      // magnitude) as fp16, tokens 4g..4g+3 (the rotation spreads a column read
                      // over the LDS banks)
  float gC[D];        // gamma_C per key channel
  u32x4 tf[64];       // [T'_hi | T'_lo] of row c, columns 4g..4g+3
  u32x2 aq[64];       // Aqk as fp16, row c, columns 4g..4g+3
  uint16_t vo[C][D + 8];  // V rows of the chunk (producer), overwritten column slice by column slice
                          // with O by the consumer owning those columns; written out whole rows
                          // (16 bytes of padding per row move consecutive rows to other banks)
};

struct Smem {
  Slot slot[NSLOT];
  float Aq[4][C][20];   // per producer: A rows arranged for the quad-parallel solve (pitch 20:
                        // the two halves of a wavefront write to different banks)
  float Tp[4][C * MP];  // per producer: T'
  float bt[4][C];       // per producer: beta of the chunk's tokens
  float adt[D];         // log2(e) exp(A_log) dt_bias of the head
  int ready[NSLOT];
  int done[NSLOT][NCW];
  int go;    // producers allowed to issue their first loads (staggered start)
  int vote;  // second pass at the checkpoint: +1 per consumer whose columns match, +0x100 per mismatch
};

// raw inputs of one chunk for one producer lane: q[s], k[s], g[s] hold token c,
// channels 32s+4g+0..3 then 32s+16+4g+0..3 (the k-step-s MFMA operand order)
struct ProdIn {
  u32x4 q[4], k[4], g[4];
  uint32_t b;
  u32x4 v[4];  // V of token L/4, columns 32(L%4) .. 32(L%4)+31
};

// Orders this wavefront's LDS writes before its later LDS reads by other lanes
// (LDS executes one wavefront's operations in order; this only stops the
// compiler from moving accesses across the point).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The chunks a second-pass block runs, from the checkpoint vote word v (+1 per
// consumer whose state matched, +0x100 per one that did not): k once all
// consumers matched, nch once any did not, -1 while votes are missing.
// (A function of values: a lambda selecting between captured variables makes
// the compiler keep its closure in scratch memory.)
__device__ __forceinline__ int vote_chunks(int v, int k, int nch) {
  if ((v & 0xFF) + (v >> 8) < NCW) return -1;
  return v == NCW ? k : nch;
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

__device__ __forceinline__ void unpack4(u32x2 v, float* f) {
  f[0] = __uint_as_float(v.x << 16);
  f[1] = __uint_as_float(v.x & 0xFFFF0000u);
  f[2] = __uint_as_float(v.y << 16);
  f[3] = __uint_as_float(v.y & 0xFFFF0000u);
}

// Where one chunk's producer inputs are: wavefront-uniform bases (chunk start,
// head) plus 32-bit lane offsets; rows past the chunk end repeat its last row.
// q and k are read at head hq of their Hqk heads (hq = h with one q/k head
// per head), g, v and beta at head h.
struct InAddr {
  const uint16_t *q, *k, *g, *b, *v;
  uint32_t row, qrow, brow, vrow;
};

__device__ __forceinline__ InAddr in_addr(const Problem& p, long long tok0, int m, int h, int hq, int g, int c) {
  const long long base = (tok0 * p.H + h) * D;
  const long long qbase = (tok0 * p.Hqk + hq) * D;
  InAddr a;
  a.q = p.q + qbase;
  a.k = p.k + qbase;
  a.g = p.g + base;
  a.b = p.beta + tok0 * p.H + h;
  a.row = __umul24((uint32_t)min(c, m - 1), (uint32_t)(p.H * D)) + 4 * g;
  a.qrow = __umul24((uint32_t)min(c, m - 1), (uint32_t)(p.Hqk * D)) + 4 * g;
  a.brow = __umul24((uint32_t)min(c, m - 1), (uint32_t)p.H);
  const int L = threadIdx.x & 63;
  a.v = p.v + base;
  a.vrow = __umul24((uint32_t)min(L >> 2, m - 1), (uint32_t)(p.H * D)) + 32 * (L & 3);
  return a;
}

// V rows of a chunk, 64 bytes per lane (coalesced 256-byte rows)
__device__ __forceinline__ void load_vrows(ProdIn& in, const InAddr& a) {
#pragma unroll
  for (int i = 0; i < 4; ++i) in.v[i] = *reinterpret_cast<const u32x4*>(a.v + a.vrow + 8 * i);
}

// k-step s of q, k and g: channels 32s+4g+0..3, then 32s+16+4g+0..3
__device__ __forceinline__ void load_part(ProdIn& in, const InAddr& a, int s) {
  const uint32_t o = a.row + 32 * s, oq = a.qrow + 32 * s;
  in.q[s] = cat(*reinterpret_cast<const u32x2*>(a.q + oq), *reinterpret_cast<const u32x2*>(a.q + oq + 16));
  in.k[s] = cat(*reinterpret_cast<const u32x2*>(a.k + oq), *reinterpret_cast<const u32x2*>(a.k + oq + 16));
  in.g[s] = cat(*reinterpret_cast<const u32x2*>(a.g + o), *reinterpret_cast<const u32x2*>(a.g + o + 16));
}

__device__ __forceinline__ void load_prod(ProdIn& in, const InAddr& a) {
#pragma unroll
  for (int s = 0; s < 4; ++s) load_part(in, a, s);
  in.b = a.b[a.brow];
  load_vrows(in, a);
}

// V[4g+0..3][col] of a chunk from its slot (the producer stored rows past the
// chunk end as zeros)
__device__ __forceinline__ u32x2 slot_v(const Slot& sl, int g, int col) {
  uint32_t t[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) t[i] = sl.vo[4 * g + i][col];
  return u32x2{t[0] | (t[1] << 16), t[2] | (t[3] << 16)};
}

// ---------------------------------------------------------------- producer
// a.lo b.lo + a.hi b.hi + acc for two packed bf16 pairs
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), acc,
                                         false);
}

// x summed over the lanes L, L^16, L^32, L^48 (the four lane groups g of one
// c); every lane of the four gets the same bits (each step adds two values in
// either order)
__device__ __forceinline__ float sum_lane_groups(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Prepares one chunk into a ring slot: V rows, Kbar, Ktil, Qbar, gamma_C, beta,
// Aqk and T' (the first pass of a segmented call needs Qbar and Aqk too, since
// it writes the outputs of every chunk after the checkpoint).
// a2 = log2(e) exp(A_log); the log decays are kept in base 2 (G2 = G log2 e),
// so every exponential is one v_exp_f32.
// Each part of `in` is reloaded from `next` (the producer's next chunk) as soon
// as it has been used, so the inputs of one chunk are in flight while the
// previous one is prepared, in the same registers.
__device__ __forceinline__ void produce(Smem& sm, Slot& sl, int pw, ProdIn& in, const InAddr& next,
                                        const Problem& p, int m, float a2, int L, int g, int c) {
  const bool ok = c < m;
  {  // V rows into the slot (rows past the chunk end as zeros), then the next
     // chunk's V into the same registers
    const int L = threadIdx.x & 63;
    if (m == C) {
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(&sl.vo[L >> 2][32 * (L & 3) + 8 * i]) = in.v[i];
    } else {
      const uint32_t keep = (L >> 2) < m ? 0xFFFFFFFFu : 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(&sl.vo[L >> 2][32 * (L & 3) + 8 * i]) = in.v[i] & keep;
    }
    load_vrows(in, next);
  }
  // |q_c|^2, |k_c|^2: this lane's 32 channels by bf16 pair dot products (the
  // products are exact in fp32), then the sum over the four lanes of token c
  float sq0 = 0.f, sq1 = 0.f, sk0 = 0.f, sk1 = 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int i = 0; i < 4; i += 2) {
      sq0 = dot2_bf16(in.q[s][i], in.q[s][i], sq0);
      sq1 = dot2_bf16(in.q[s][i + 1], in.q[s][i + 1], sq1);
      sk0 = dot2_bf16(in.k[s][i], in.k[s][i], sk0);
      sk1 = dot2_bf16(in.k[s][i + 1], in.k[s][i + 1], sk1);
    }
  const float sq = sum_lane_groups(sq0 + sq1);
  const float sk = sum_lane_groups(sk0 + sk1);
  // rows past the chunk end: zero key, query, beta and log decay
  const float rq = ok ? p.scale * __builtin_amdgcn_rsqf(sq + 1e-6f) : 0.f;
  const float rk = ok ? __builtin_amdgcn_rsqf(sk + 1e-6f) : 0.f;
  // 1 / (log2(e) lower_bound); rows past the chunk end, and a bound of 0, take
  // -FLT_MAX, whose reciprocal below is 0 or a denormal that adds nothing to a
  // log decay (exp2 of it is 1)
  const float lb2 = p.lower_bound * LOG2E;
  const float ilb = (ok && lb2 < -1e-30f) ? 1.0f / lb2 : -FLT_MAX;
  const float bt =
      ok ? __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-LOG2E * __uint_as_float(in.b << 16))) : 0.f;
  sm.bt[pw][c] = bt;  // the four lanes of a token store the same value
  in.b = next.b[next.brow];

  // A_raw = Kbar Ktil^T from bf16 operands (one MFMA per k-step), Aqk^T =
  // Ktil Qbar^T from bf16 high/low operands (hi.hi + hi.lo + lo.hi).
  // Khat = Ktil gamma_C of token c, channel ch goes to ktp[ch][(c/4 + (ch % 16)/4) % 4],
  // element c % 4, as fp16; (ch % 16) / 4 = g for every channel this lane holds
  uint16_t* khp16 = reinterpret_cast<uint16_t*>(&sl.ktp[0][0]) + 4 * (((c >> 2) + g) & 3) + (c & 3);
  f32x4 Araw = zero4(), AqkT = zero4();
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const f32x4 adt0 = *reinterpret_cast<const f32x4*>(&sm.adt[32 * s + 4 * g]);
    const f32x4 adt1 = *reinterpret_cast<const f32x4*>(&sm.adt[32 * s + 16 + 4 * g]);
    uint32_t kbh[4], kth[4], ktl[4], qbh[4], qbl[4];
    float ep_last[8];  // e^G of token 15 = gamma_C (rows past the chunk end add no decay)
    // element pairs (2i, 2i+1): channels 32s + 16(i/2) + 4g + 2(i%2) + 0, 1,
    // split into bf16 high/low pairs as soon as both are formed
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t qw = in.q[s][i], kw = in.k[s][i], gw = in.g[s][i];
      float Kb[2], Kt[2], Qb[2], Kh[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float qv = __uint_as_float(h ? (qw & 0xFFFF0000u) : (qw << 16));
        const float kv = __uint_as_float(h ? (kw & 0xFFFF0000u) : (kw << 16));
        const float gv = __uint_as_float(h ? (gw & 0xFFFF0000u) : (gw << 16));
        const int e = 2 * i + h;
        const float ad = (e < 4) ? adt0[e] : adt1[e - 4];
        // l2 = log2(e) lower_bound sigmoid(exp(A_log) (g + dt_bias)), formed as
        // 1 / ((1 + e^-x) / (log2(e) lower_bound))
        const float x2 = fmaf(a2, gv, ad);
        const float ex = __builtin_amdgcn_exp2f(-x2);
        const float l2 = __builtin_amdgcn_rcpf(fmaf(ex, ilb, ilb));
        const float G2 = row_scan(l2);
        const float ep = __builtin_amdgcn_exp2f(G2), em = __builtin_amdgcn_exp2f(-G2);
        ep_last[e] = ep;
        const float kr = kv * rk;
        Kb[h] = -(kr * ep);  // -Kbar (see Slot::kbf)
        Kt[h] = kr * em;
        Qb[h] = (qv * rq) * ep;
        // gamma_C of this channel is e^G of token 15, held by lane 15 of the row
        Kh[h] = Kt[h] * __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(ep), 0x15F, 0xF, 0xF, false));
      }
      kbh[i] = pack2(Kb[0], Kb[1]);
      split_pair(Kt[0], Kt[1], kth[i], ktl[i]);
      split_pair(Qb[0], Qb[1], qbh[i], qbl[i]);
      // Khat, channel-major (16 fp16 per channel row)
      const int ch = 32 * s + 16 * (i >> 1) + 4 * g + 2 * (i & 1);
      const uint32_t kh = pack2_f16(Kh[0], Kh[1]);
      khp16[16 * ch] = (uint16_t)(kh & 0xFFFFu);
      khp16[16 * (ch + 1)] = (uint16_t)(kh >> 16);
    }
    const u32x4 kbh4 = {kbh[0], kbh[1], kbh[2], kbh[3]};
    const u32x4 kth4 = {kth[0], kth[1], kth[2], kth[3]}, ktl4 = {ktl[0], ktl[1], ktl[2], ktl[3]};
    Araw = mfma_k32(kbh4, kth4, Araw);  // D[4g+i][c] -= Kbar_{4g+i} . Ktil_c over this k-step
    sl.kbf[s][L] = kbh4;
    {
      const u32x4 qbh4 = {qbh[0], qbh[1], qbh[2], qbh[3]}, qbl4 = {qbl[0], qbl[1], qbl[2], qbl[3]};
      AqkT = mfma_k32(kth4, qbh4, AqkT);  // D[4g+i][c] += Ktil_{4g+i} . Qbar_c = Aqk[c][4g+i]
      AqkT = mfma_k32(kth4, qbl4, AqkT);
      AqkT = mfma_k32(ktl4, qbh4, AqkT);
      sl.qbf[s][L] = qbh4;
    }
    if (c == C - 1) {
      *reinterpret_cast<f32x4*>(&sl.gC[32 * s + 4 * g]) = f32x4{ep_last[0], ep_last[1], ep_last[2], ep_last[3]};
      *reinterpret_cast<f32x4*>(&sl.gC[32 * s + 16 + 4 * g]) = f32x4{ep_last[4], ep_last[5], ep_last[6], ep_last[7]};
    }
    load_part(in, next, s);
  }
  wave_lds_sync();

  // A = StrictLower(Diag(b) A_raw) into the solve layout Aq[i][4(p%4) + p/4] = A[i][p]
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * g + i;
    sm.Aq[pw][row][4 * (c & 3) + (c >> 2)] = (c < row) ? -(sm.bt[pw][row] * Araw[i]) : 0.f;  // Araw = -A_raw
  }
  {
    f32x4 aq;
#pragma unroll
    for (int i = 0; i < 4; ++i) aq[i] = (4 * g + i <= c) ? AqkT[i] : 0.f;
    sl.aq[L] = pack4_f16(aq);
  }

  wave_lds_sync();
  // T = (I + A)^{-1} by forward substitution: lane 4j+q owns column j and the
  // rows p = q, q+4, q+8, q+12; row i's dot product is split over the quad
  {
    const int j = L >> 2, q = L & 3;
    // T[p][j] = 0 for p < j, so a row above the diagonal sums to zero and the
    // diagonal entry (which also sums to zero) is set to 1 beforehand and kept
    const bool d0 = (j == q), d1 = (j == q + 4), d2 = (j == q + 8), d3 = (j == q + 12);
    float t0 = d0 ? 1.f : 0.f, t1 = d1 ? 1.f : 0.f, t2 = d2 ? 1.f : 0.f, t3 = d3 ? 1.f : 0.f;  // T[q+4k][j]
#pragma unroll
    for (int i = 1; i < C; ++i) {
      const f32x4 ar = *reinterpret_cast<const f32x4*>(&sm.Aq[pw][i][4 * q]);  // A[i][q+4k], k = 0..3
      // A[i][p] = 0 for p >= i, so only the terms k <= (i - 1) / 4 can be nonzero
      const int kmax = (i - 1) >> 2;
      float part;
      if (kmax == 0) part = ar[0] * t0;
      else if (kmax == 1) part = fmaf(ar[1], t1, ar[0] * t0);
      else if (kmax == 2) part = fmaf(ar[2], t2, fmaf(ar[1], t1, ar[0] * t0));
      else part = fmaf(ar[1], t1, ar[0] * t0) + fmaf(ar[3], t3, ar[2] * t2);
      part += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(part), 0xB1, 0xF, 0xF, false));  // quad xor 1
      part += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(part), 0x4E, 0xF, 0xF, false));  // quad xor 2
      // row i is held by the lanes with q = i % 4, as t_{i/4}
      const bool own = ((i & 3) == q) && (i != j);
      if ((i >> 2) == 0) t0 = own ? -part : t0;
      else if ((i >> 2) == 1) t1 = own ? -part : t1;
      else if ((i >> 2) == 2) t2 = own ? -part : t2;
      else t3 = own ? -part : t3;
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
// U of a column tile is the fp16 B operand of the state update Khat^T U and
// the A operand of Aqk U (U^T is the A operand of O^T += U^T Aqk^T): lane
// (g, c) holds U[4g+i][c], i = 0..3, times sc = 2^k.  k = 0 while the tile's
// largest |U| lies in [2^-12, 2^15) (or the tile is zero): fp16 then keeps 11
// bits of every value down to 2^-14 and an absolute error of at most 2^-25
// below, small against that largest value.  Outside that range (or for
// non-finite values) 2^k brings the largest |U| to [2^13, 2^14); the state
// tile is scaled by 2^k around the update and by isc = 2^-k after it, exactly.
// The pre-scan's M (up = false) is only scaled down: its values shrink to
// exact zero as the start state's influence dies out, and small ones weigh
// nothing against R, so they are left to fp16's range.
struct U16 {
  u32x2 u;
  float sc, isc;
  uint32_t scaled;  // wavefront-uniform (a word, not a bool: keeps the struct in whole registers)
};

__device__ __forceinline__ U16 to_u16(f32x4 U, bool up = true) {
  const float m = fmaxf(fmaxf(fabsf(U[0]), fabsf(U[1])), fmaxf(fabsf(U[2]), fabsf(U[3])));
  const uint64_t big = __builtin_amdgcn_ballot_w64(!(m < 32768.f));
  const uint64_t fit = __builtin_amdgcn_ballot_w64(m >= 0x1p-12f);
  const uint64_t nz = __builtin_amdgcn_ballot_w64(m != 0.f);
  U16 r;
  r.scaled = (big != 0 || (up && fit == 0 && nz != 0)) ? 1u : 0u;
  r.sc = 1.f;
  r.isc = 1.f;
  if (r.scaled) {
    float w = m;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) w = fmaxf(w, __shfl_xor(w, o, 64));
    w = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(w)));  // every lane holds the maximum
    const int e = __builtin_isfinite(w) ? __builtin_amdgcn_frexp_expf(w) : 0;  // w in [2^(e-1), 2^e)
    r.sc = __builtin_ldexpf(1.f, 14 - e);
    r.isc = __builtin_ldexpf(1.f, e - 14);
    U = U * r.sc;
  }
  r.u = pack4_f16(U);
  return r;
}

__device__ __forceinline__ void pack_tile(const f32x4 (&S)[8], u32x2 (&Sb)[8]) {
#pragma unroll
  for (int tt = 0; tt < 8; ++tt) Sb[tt] = pack4(S[tt]);
}

// -Y = -Kbar S for NT column tiles (kb holds -Kbar), interleaved so
// consecutive MFMAs are independent
template <int NT>
__device__ __forceinline__ void tiles_y(const u32x2 (&Sb)[NT][8], const u32x4 (&kb)[4], f32x4 (&Y)[NT]) {
#pragma unroll
  for (int jj = 0; jj < NT; ++jj) Y[jj] = zero4();
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int jj = 0; jj < NT; ++jj) Y[jj] = mfma_k32(kb[s], cat(Sb[jj][2 * s], Sb[jj][2 * s + 1]), Y[jj]);
}

// U = T' V + T' (-Yb) (no V term when v is null) in fp32, from nY = -Y =
// -Kbar S; the second product accumulates onto the first
__device__ __forceinline__ f32x4 tile_u(f32x4 nY, u32x4 tf, const u32x2* v) {
  const u32x2 nYb = pack4(nY);
  const f32x4 Ut = v ? mfma_k32(tf, cat(*v, *v), zero4()) : zero4();
  return mfma_k32(tf, cat(nYb, nYb), Ut);
}

template <int NT>
__device__ __forceinline__ void scale_tiles(f32x4 (&S)[NT][8], const U16 (&u)[NT], bool before) {
#pragma unroll
  for (int jj = 0; jj < NT; ++jj)
    if (u[jj].scaled) {
      const float f = before ? u[jj].sc : u[jj].isc;
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) S[jj][tt] = S[jj][tt] * f;
    }
}

// S <- Diag(gamma_C) S + Khat^T U for NT column tiles, one fp16 product per
// row tile (Khat = Ktil gamma_C = k^ e^(G_C - G)); the Khat / gamma_C
// fragments of a row tile are read once and used by every column tile.
template <int NT>
__device__ __forceinline__ void tiles_update(f32x4 (&S)[NT][8], const U16 (&u)[NT], u32x2 (&kp)[8],
                                             f32x4 (&gc)[8], const Slot& sl, int g, int c) {
#pragma unroll
  for (int tt = KDA_HOIST; tt < 8; ++tt) {
    kp[tt] = sl.ktp[16 * tt + c][(g + (c >> 2)) & 3];
    gc[tt] = *reinterpret_cast<const f32x4*>(&sl.gC[16 * tt + 4 * g]);
  }
  scale_tiles<NT>(S, u, true);
#pragma unroll
  for (int tt = 0; tt < 8; ++tt) {
#pragma unroll
    for (int jj = 0; jj < NT; ++jj) S[jj][tt] = mfma_f16_k16(kp[tt], u[jj].u, S[jj][tt] * gc[tt]);
  }
  scale_tiles<NT>(S, u, false);
}

// The Khat and gamma_C fragments of the update, for the first row tiles
__device__ __forceinline__ void update_operands(const Slot& sl, int g, int c, u32x2 (&kp)[8], f32x4 (&gc)[8]) {
#pragma unroll
  for (int tt = 0; tt < KDA_HOIST; ++tt) {
    kp[tt] = sl.ktp[16 * tt + c][(g + (c >> 2)) & 3];
    gc[tt] = *reinterpret_cast<const f32x4*>(&sl.gC[16 * tt + 4 * g]);
  }
}

// The same update for two sets of column tiles (R and M of the pre-scan);
// returns the OR of the bit patterns of the new S2 entries
template <int NT>
__device__ __forceinline__ uint32_t tiles_update2(f32x4 (&S1)[NT][8], const U16 (&u1)[NT], f32x4 (&S2)[NT][8],
                                                  const U16 (&u2)[NT], const Slot& sl, int g, int c) {
  scale_tiles<NT>(S1, u1, true);
  scale_tiles<NT>(S2, u2, true);
#pragma unroll
  for (int tt = 0; tt < 8; ++tt) {
    const u32x2 kp = sl.ktp[16 * tt + c][(g + (c >> 2)) & 3];
    const f32x4 gc = *reinterpret_cast<const f32x4*>(&sl.gC[16 * tt + 4 * g]);
#pragma unroll
    for (int jj = 0; jj < NT; ++jj) {
      S1[jj][tt] = mfma_f16_k16(kp, u1[jj].u, S1[jj][tt] * gc);
      S2[jj][tt] = mfma_f16_k16(kp, u2[jj].u, S2[jj][tt] * gc);
    }
  }
  scale_tiles<NT>(S1, u1, false);
  scale_tiles<NT>(S2, u2, false);
  uint32_t bits = 0;
#pragma unroll
  for (int jj = 0; jj < NT; ++jj)
#pragma unroll
    for (int tt = 0; tt < 8; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) bits |= __float_as_uint(S2[jj][tt][i]);
  return bits;
}

// O^T += U^T Aqk^T for one column tile (fp16 product, scaled back by isc)
__device__ __forceinline__ f32x4 add_aqk_u(f32x4 Ot, const U16& u, u32x2 aq) {
  const f32x4 P = mfma_f16_k16(u.u, aq, zero4());
  f32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = fmaf(P[i], u.isc, Ot[i]);
  return r;
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

// The caller's state in the [K][V] layout: element (k, v) at k D + v.  Lane
// (g, c) holds rows k = 16tt + 4g + i of column v = col0 + 16jj + c, so each
// scalar access is coalesced over the 16 lanes of a row group.
template <int NT>
__device__ __forceinline__ void load_state_kv(f32x4 (&S)[NT][8], const void* src, bool f32, long long base,
                                              int col0, int g, int c) {
#pragma unroll
  for (int jj = 0; jj < NT; ++jj)
#pragma unroll
    for (int tt = 0; tt < 8; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const long long off = base + (long long)(16 * tt + 4 * g + i) * D + col0 + 16 * jj + c;
        S[jj][tt][i] = f32 ? static_cast<const float*>(src)[off] : bf16_to_f32(static_cast<const uint16_t*>(src)[off]);
      }
}

template <int NT>
__device__ __forceinline__ void store_state_kv(const f32x4 (&S)[NT][8], float* dst32, uint16_t* dst16,
                                               long long base, int col0, int g, int c) {
#pragma unroll
  for (int jj = 0; jj < NT; ++jj)
#pragma unroll
    for (int tt = 0; tt < 8; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const long long off = base + (long long)(16 * tt + 4 * g + i) * D + col0 + 16 * jj + c;
        if (dst32) dst32[off] = S[jj][tt][i];
        if (dst16) dst16[off] = (uint16_t)(pack2(S[jj][tt][i], 0.f) & 0xFFFFu);
      }
}

// A state handed between blocks of one launch, which may run on different
// XCDs, each with its own L2: it is written and read with device-coherent
// accesses (the sc1 cache policy, which agent-scope atomics also use), 16 bytes
// per lane, so no cache needs to be written back or invalidated around it and
// every store fills whole 64-byte pieces of a column.  [V][K] fp32 layout as
// store_state; the buffer resource spans the one 128x128 state at dst + base.
constexpr int CPOL_SC1 = 16;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t state_rsrc(const float* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p), 0, D * D * 4, 0x00020000);
}

__device__ __forceinline__ int state_off(int col0, int jj, int tt, int g, int c) {
  return 4 * ((col0 + 16 * jj + c) * D + 16 * tt + 4 * g);
}

template <int NT>
__device__ __forceinline__ void store_state_coherent(const f32x4 (&S)[NT][8], float* dst, long long base, int col0,
                                                     int g, int c) {
  const __amdgpu_buffer_rsrc_t r = state_rsrc(dst + base);
#pragma unroll
  for (int jj = 0; jj < NT; ++jj)
#pragma unroll
    for (int tt = 0; tt < 8; ++tt)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, S[jj][tt]), r, state_off(col0, jj, tt, g, c),
                                             0, CPOL_SC1);
}

// True if every state entry of this lane equals the state at src bit for bit
// (device-coherent loads, all issued before any compare).
template <int NT>
__device__ __forceinline__ bool same_bits_coherent(const f32x4 (&S)[NT][8], float* src, long long base, int col0,
                                                   int g, int c) {
  const __amdgpu_buffer_rsrc_t r = state_rsrc(src + base);
  u32x4 x[NT][8];
#pragma unroll
  for (int jj = 0; jj < NT; ++jj)
#pragma unroll
    for (int tt = 0; tt < 8; ++tt)
      x[jj][tt] = __builtin_amdgcn_raw_buffer_load_b128(r, state_off(col0, jj, tt, g, c), 0, CPOL_SC1);
  uint32_t diff = 0;
#pragma unroll
  for (int jj = 0; jj < NT; ++jj)
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      const u32x4 d = __builtin_bit_cast(u32x4, S[jj][tt]) ^ x[jj][tt];
      diff |= d.x | d.y | d.z | d.w;
    }
  return diff == 0u;
}

// Segment merge for this wavefront's column tiles: S <- M S + R, the affine map
// of one segment (M from a start state, R from zero).  M and R are stored
// [v][k] like the states (Mt[p][k] = M[k][p]); bit b of nz is set when columns
// 16b..16b+15 of M (the reduction index) are nonzero, and zero blocks, which
// the first pass leaves unstored, are skipped.  fp32 products on
// v_mfma_f32_16x16x4_f32: for output row tile `to`, K slot g of the MFMA for
// (tt, i) is reduction index p = 16tt + 4g + i, whose S value this lane holds.
template <int NT>
__device__ __forceinline__ void apply_map(f32x4 (&S)[NT][8], const float* Mt, const float* Rt, uint32_t nz, int col0,
                                          int g, int c) {
  f32x4 acc[NT][8];
  load_state<NT>(acc, Rt, true, 0, col0, g, c);
  for (int tt = 0; tt < 8; ++tt) {
    if (!((nz >> tt) & 1u)) continue;
#pragma unroll
    for (int to = 0; to < 8; ++to)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = Mt[(long long)(16 * tt + 4 * g + i) * D + 16 * to + c];
#pragma unroll
        for (int jj = 0; jj < NT; ++jj) acc[jj][to] = mfma_f32_k4(a, S[jj][tt][i], acc[jj][to]);
      }
  }
#pragma unroll
  for (int jj = 0; jj < NT; ++jj)
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) S[jj][tt] = acc[jj][tt];
}

// Whole-block work on one 128x128 fp32 state: thread x takes 16-byte pieces
// x + NTHREADS r, r < PIECES, and issues all its loads before using any, so
// the block waits for one memory round trip rather than one per piece.
constexpr int PIECES = (D * D / 4 + NTHREADS - 1) / NTHREADS;

// A segment's R as the caller's final state (its dtype and layout): piece i
// of the state, (v, k) = (4i / D, 4i % D + 0..3).
__device__ __forceinline__ void store_final_piece(const Problem& p, long long state_base, int i, f32x4 v) {
  if (p.state_kv) {
    const long long o = state_base + (long long)(4 * i % D) * D + 4 * i / D;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (p.state_fp32)
        static_cast<float*>(p.final_state)[o + e * D] = v[e];
      else
        static_cast<uint16_t*>(p.final_state)[o + e * D] = (uint16_t)(pack2(v[e], 0.f) & 0xFFFFu);
    }
  } else if (p.state_fp32) {
    reinterpret_cast<f32x4*>(static_cast<float*>(p.final_state) + state_base)[i] = v;
  } else {
    reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.final_state) + state_base)[i] = pack4(v);
  }
}

// A segment's R written to the caller's final state by the whole block (all
// loads issued before any store).
__device__ __forceinline__ void final_from_R(const Problem& p, const Seg& sg, long long seg_base, long long state_base) {
  const f32x4* r = reinterpret_cast<const f32x4*>(sg.R + seg_base);
  f32x4 vr[PIECES];
#pragma unroll
  for (int q = 0; q < PIECES; ++q) vr[q] = r[min((int)threadIdx.x + NTHREADS * q, D * D / 4 - 1)];
#pragma unroll
  for (int q = 0; q < PIECES; ++q) {
    const int i = threadIdx.x + NTHREADS * q;
    if (i < D * D / 4) store_final_piece(p, state_base, i, vr[q]);
  }
}

// Second pass, before any chunk (every thread of the block calls it): true if
// the state the first pass reached after this segment's first K chunks (fix,
// run from the previous segment's R) equals the segment's checkpoint bit for
// bit, and that R was the segment's start state: the previous segment is
// segment 0 (nzf null) or its M is exactly zero (the flags nzf[0..D/16) all
// zero).  The segment's outputs are then all final; for the sequence's last
// segment (LAST) the end state is R, written to the caller's final state here.
// Every load (flags, fix, checkpoint, and R for LAST) is issued before any is
// used, so the block waits for one memory round trip.
template <bool LAST>
__device__ __forceinline__ bool decided_at_checkpoint(const Problem& p, const Seg& sg, const int32_t* nzf,
                                                      long long seg_base, long long state_base) {
  const u32x4* x = reinterpret_cast<const u32x4*>(sg.fix + seg_base);
  const u32x4* y = reinterpret_cast<const u32x4*>(sg.chk + seg_base);
  const f32x4* r = reinterpret_cast<const f32x4*>(sg.R + seg_base);
  // Threads past the last piece load (and compare) the last piece again: no
  // load sits in a branch, whose end would wait for all loads issued before it.
  u32x4 va[PIECES], vb[PIECES];
  f32x4 vr[PIECES];
#pragma unroll
  for (int q = 0; q < PIECES; ++q) {
    const int i = min((int)threadIdx.x + NTHREADS * q, D * D / 4 - 1);
    va[q] = x[i];
    vb[q] = y[i];
    if (LAST) vr[q] = r[i];
  }
  uint32_t diff = 0;
  if (nzf) {
#pragma unroll
    for (int b = 0; b < D / 16; ++b) diff |= (uint32_t)nzf[b];
  }
#pragma unroll
  for (int q = 0; q < PIECES; ++q) {
    const u32x4 d = va[q] ^ vb[q];
    diff |= d.x | d.y | d.z | d.w;
  }
  if (__syncthreads_or(diff != 0u)) return false;
  if (LAST) {
#pragma unroll
    for (int q = 0; q < PIECES; ++q) {
      const int i = threadIdx.x + NTHREADS * q;
      if (i < D * D / 4) store_final_piece(p, state_base, i, vr[q]);
    }
  }
  return true;
}

}  // namespace

// One row of the dispatch table: segment (row of the segment tables), its
// sequence, its chunk range [cb, ce) in global chunk numbers, its index in the
// sequence, the sequence's first token and length, and the segment length of
// the call (0: serial).
struct Unit {
  int sidx, seq, cb, ce, j, start, len, seg;
};

// MODE 0: a sequence of a serial call from its initial state.
// MODE 1: first pass of a segmented call: segment 0 of each sequence from the
//         initial state, every later segment (pre) from a zero state, with its
//         transition M while that is nonzero.
// MODE 2: second pass of a segmented call: segments >= 1 from their start states.
template <int MODE>
__device__ __forceinline__ void chunk_body(Smem& sm, const Problem& p, const Tables& t, const Seg& sg,
                                           const Unit& u, int h) {
  constexpr int phase = MODE == 2 ? 1 : 0;
  const int sidx = u.sidx;
  const int seq = u.seq;
  const int cb = u.cb;
  const int ce = u.ce;
  const int j = u.j;
  // the sequence's chunk and segment counts, its first chunk and the next
  // segment's length follow from its length and the segment length (serial:
  // one segment per sequence)
  const int seq_len = u.len;
  const int seq_nc = (seq_len + C - 1) / C;
  const int seg_c = u.seg;
  const int ns = seg_c > 0 ? (seq_nc > 0 ? (seq_nc + seg_c - 1) / seg_c : 1) : 1;
  const int first_chunk = cb - j * seg_c;
  if (MODE == 2 && j == 0) return;  // segment 0 has its true start state in the first pass
  const bool pre = MODE == 1 && j > 0;

  const int H = p.H;
  const int hq = h / (H / p.Hqk);  // q/k head of this head
  const int wave = threadIdx.x >> 6;
  const int L = threadIdx.x & 63;
  const int g = L >> 4;
  const int c = L & 15;
  const int nch = ce - cb;
  const long long seq_tok0 = u.start;
  auto chunk_m = [&](int lc) { return min(C, seq_len - C * (cb + lc - first_chunk)); };
  auto chunk_tok0 = [&](int lc) { return seq_tok0 + (long long)C * (cb + lc - first_chunk); };

  // Segments >= 1 longer than K = chk_chunks chunks: the first pass (PRE)
  // writes the output of chunks >= K from its zero-start state R and keeps R
  // after K chunks; the second pass redoes chunks < K from the true start
  // state and stops there if its state equals that checkpoint bit for bit
  // (the rest is then the same computation on the same bits, already done),
  // else it runs to the end.  The state's value columns evolve independently,
  // so each consumer compares its own columns; the block stops when all agree.
  const int K = sg.chk_chunks;
  const bool has_chk = j > 0 && K > 0 && nch > K;
  const int o_from = pre ? (has_chk ? K : nch) : 0;  // first chunk whose output this pass writes
  const bool may_stop = MODE == 2 && has_chk;
  // a last segment without a checkpoint: the first pass has nothing to hand on
  // (no segment after it needs its map, and the second pass runs it whole)
  if (pre && j == ns - 1 && !has_chk) return;
  // The first pass goes on for K chunks into the next segment of the sequence
  // (when that one has a checkpoint) from its own end state, which is the next
  // segment's start state when this is segment 0 or its M is exactly zero.
  // It writes those chunks' output and stores its state after them (fix): the
  // second pass keeps them if that state equals the next segment's checkpoint
  // bit for bit, and then has nothing left to compute.
  int ext = 0;
  if (phase == 0 && K > 0 && j < ns - 1) {
    const int nn = min(seg_c, seq_nc - (j + 1) * seg_c);  // the next segment's chunks
    if (nn > K) ext = K;
  }
  const int ntot = nch + ext;  // chunks this block runs
  const long long seg_base = ((long long)sidx * H + h) * D * D;
  const long long state_base = ((long long)seq * H + h) * D * D;

  // Second pass: the first pass already ran this segment's first K chunks from
  // its start state (the previous segment's R, kept when that segment's M is
  // zero; or S_1).  If the state it reached equals the checkpoint bit for bit,
  // every output of the segment is final and the block has nothing to do.
  // The previous segment's block compared the two at its end, per 16-column
  // block, and left the results in this segment's sync words (1: equal, 2:
  // not, 3: not compared, that block's fix columns stored for the comparison
  // here).  The sync words have served the first pass once read; they are
  // cleared for the next call, so that a later call (a replayed graph, whose
  // epoch does not change, too) never reads this call's words.
  if (MODE == 2) {
    uint32_t* sy = sg.sync + ((long long)sidx * H + h) * 16;
    uint32_t w[D / 16];
#pragma unroll
    for (int b = 0; b < D / 16; ++b) w[b] = sy[8 + b];
    __syncthreads();  // every thread has read them before they are cleared
    if (threadIdx.x < 16) sy[threadIdx.x] = 0u;
    if (has_chk) {
      const int32_t* nzf = j >= 2 ? sg.mnz + ((long long)(sidx - 1) * H + h) * (D / 16) : nullptr;
      bool nz = false;  // the previous segment's M is not exactly zero: its R is not this start state
      int n_equal = 0, n_differ = 0;
#pragma unroll
      for (int b = 0; b < D / 16; ++b) {
        if (nzf) nz = nz || nzf[b] != 0;
        const uint32_t code = (w[b] >> 2) == (sg.epoch & 0x3FFFFFFFu) ? (w[b] & 3u) : 3u;
        n_equal += code == 1u;
        n_differ += code == 2u;
      }
      // the final state is this segment's R; the first pass wrote it already
      // unless it may alias the initial state
      const bool last_final = j == ns - 1 && p.final_state && !p.final_early;
      bool decided = false;
      if (!nz && n_differ == 0) {
        if (n_equal == D / 16) {
          decided = true;
          if (last_final) final_from_R(p, sg, seg_base, state_base);
        } else {
          decided = last_final ? decided_at_checkpoint<true>(p, sg, nzf, seg_base, state_base)
                               : decided_at_checkpoint<false>(p, sg, nzf, seg_base, state_base);
        }
      }
      if (decided) {
        if (threadIdx.x == 0) atomicAdd(&t.counters[CNT_EARLY_STOPS], 1);
        return;
      }
    }
  }

  // Producer p prepares chunks p, p + NPW, ...; its inputs are loaded a chunk
  // ahead into `in`.  Past the last chunk the next-chunk address repeats the
  // current one (always in bounds, loaded and unused).
  ProdIn in;
  auto addr = [&](int lc) {
    const int lcc = lc < ntot ? lc : lc - NPW;
    return in_addr(p, chunk_tok0(lcc), chunk_m(lcc), h, hq, g, c);
  };
  // The inputs of chunk 0, which every consumer waits for, are requested
  // first, so that their latency overlaps that of the gate constants below
  // and of the workgroup barrier.
  if (wave == 0 && ntot > 0) load_prod(in, addr(0));

  const float a2 = LOG2E * expf(p.A_log[h]);
  if (threadIdx.x < D) sm.adt[threadIdx.x] = a2 * p.dt_bias[h * D + threadIdx.x];
  if (threadIdx.x < NSLOT) sm.ready[threadIdx.x] = -1;
  if (threadIdx.x < NSLOT * NCW) sm.done[threadIdx.x / NCW][threadIdx.x % NCW] = -1;
  if (threadIdx.x == 0) sm.vote = 0;
  if (threadIdx.x == 0) sm.go = 0;
  __syncthreads();

  if (wave < NPW) {
    // ======================= producer =======================
    const int pw = wave;
    // chunks the block runs: nch, or K once the consumers agreed to stop
    // there; -1 while their vote is incomplete
    auto n_run = [&]() -> int { return may_stop ? vote_chunks(wg_load(&sm.vote), K, nch) : ntot; };
    // 1 once every consumer is done with chunk y, 0 if the block stopped
    // before y, -1 when the (bounded) wait gives up
    auto wait_done = [&](int y) -> int {
      const int slot = y % NSLOT;
      int it = 0;
      while (true) {
        int d = wg_load(&sm.done[slot][0]);
#pragma unroll
        for (int w = 1; w < NCW; ++w) d = min(d, wg_load(&sm.done[slot][w]));
        if (d >= y) return 1;
        if (may_stop) {
          const int n = n_run();
          if (n >= 0 && y >= n) return 0;
        }
        if (++it > SPIN_LIMIT) {
          if (L == 0) atomicOr(&t.counters[CNT_FLAGS], 0x100);
          return -1;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    };
    // the output rows of chunk lc, left in its slot by the consumers: whole
    // 256-byte rows, 64 bytes per lane
    auto flush = [&](int lc) {
      const Slot& sl = sm.slot[lc % NSLOT];
      const int tok = L >> 2;
      if (tok < chunk_m(lc)) {
        // a wavefront-uniform chunk base and a 32-bit lane offset
        uint16_t* ob = p.out + (chunk_tok0(lc) * H + h) * D;
        const uint32_t o = __umul24((uint32_t)tok, (uint32_t)(H * D)) + 32 * (L & 3);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<u32x4*>(ob + o + 8 * i) =
              *reinterpret_cast<const u32x4*>(&sl.vo[tok][32 * (L & 3) + 8 * i]);
      }
    };
    // Producer pw takes chunks lc = pw, pw + NPW, ...: before preparing chunk
    // lc it waits until the slot's previous chunk lc - NSLOT is consumed and
    // writes that chunk's output rows; past the last chunk it goes on only to
    // write out the outputs of the last NSLOT chunks.
    // Staggered start: producer pw issues its first chunk's loads once those of
    // producer pw - 1 have returned.  Every block starts at once, and this keeps
    // the inputs of chunk 0, which the consumers wait for, from queueing behind
    // those of chunks 1..3.  The wait only orders loads: it is bounded, and
    // going on after it gives up changes no result.
    if (pw > 0) {
      int it = 0;
      while (wg_load(&sm.go) < pw && ++it < 4096) __builtin_amdgcn_s_sleep(1);
    }
    if (pw < ntot) {
      if (pw > 0) load_prod(in, addr(pw));  // producer 0's are in flight since the start
      asm volatile("" ::"v"(in.v[3]));  // a use of the last load issued: waits for all of them
    }
    if (pw + 1 < NPW) wg_store(&sm.go, pw + 1);
    for (int lc = pw; lc < ntot + NSLOT; lc += NPW) {
      const int y = lc - NSLOT;
      if (y >= 0) {
        if (wait_done(y) <= 0) break;
        if (y >= o_from) flush(y);
      }
      if (lc < ntot) {
        // chunks past the checkpoint wait for the vote (the block usually stops
        // there, and a chunk prepared meanwhile would slow the consumers)
        int n = n_run();
        if (may_stop && lc >= K) {
          int it = 0;
          while (n < 0) {
            if (++it > SPIN_LIMIT) {
              if (L == 0) atomicOr(&t.counters[CNT_FLAGS], 0x100);
              break;
            }
            __builtin_amdgcn_s_sleep(1);
            n = n_run();
          }
          if (n < 0) break;
        }
        if (n >= 0 && lc >= n) continue;  // stopped before this chunk
        // Qbar and Aqk are prepared for every chunk, also the first pass's
        // first chunks, whose output it does not write: one inlined copy of the
        // preparation keeps the loop's scalar registers from spilling.
        produce(sm, sm.slot[lc % NSLOT], pw, in, addr(lc + NPW), p, chunk_m(lc), a2, L, g, c);
        wg_store(&sm.ready[lc % NSLOT], lc);
      }
    }
    return;
  }

  // ======================= consumer =======================
  const int cw = wave - NPW;
  const int col0 = 16 * TPW * cw;
  const long long fix_base = seg_base + (long long)H * D * D;  // the next segment's slot

  // The next chunk's ready flag is read early (relaxed) and looked at only
  // after this chunk is done; a chunk seen ready there needs no wait.  The
  // slot reads stay behind that load: a signal fence keeps the compiler from
  // moving them, and LDS performs one wavefront's accesses in order.
  int seen = -1;
  auto peek_ready = [&](int lc) {
    return __hip_atomic_load(&sm.ready[lc % NSLOT], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  };
  auto wait_ready = [&](int slot, int lc) -> bool {
    if (seen == lc) return true;  // seen by the early read
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
  using NoOut = std::integral_constant<bool, false>;
  using WithOut = std::integral_constant<bool, true>;

  // One chunk applied to the state columns S; with the output (WithOut):
  //   O^T = S^T Qbar^T + U^T Aqk^T into the slot's V rows (this wavefront has
  //   read its V columns), written out by a producer.
  // The state update is the same instruction sequence with or without it.
  auto step_s = [&](int lc, f32x4 (&S)[TPW][8], auto wo) -> bool {
    constexpr bool WO = decltype(wo)::value;
    const int slot = lc % NSLOT;
    if (!wait_ready(slot, lc)) return false;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const Slot& sl = sm.slot[slot];
    const int peek = peek_ready(lc + 1);
    u32x4 kb[4], qb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      kb[s] = sl.kbf[s][L];
      if (WO) qb[s] = sl.qbf[s][L];
    }
    const u32x4 tf = sl.tf[L];
    u32x2 kp[8];
    f32x4 gc[8];
    update_operands(sl, g, c, kp, gc);
    u32x2 v[TPW];
#pragma unroll
    for (int jj = 0; jj < TPW; ++jj) v[jj] = slot_v(sl, g, col0 + 16 * jj + c);
    // every read of the slot is issued here, before any of it is used
    __builtin_amdgcn_sched_barrier(0);
    u32x2 Sb[TPW][8];
#pragma unroll
    for (int jj = 0; jj < TPW; ++jj) pack_tile(S[jj], Sb[jj]);
    // -Y = -Kbar S and O^T: independent MFMA chains
    f32x4 Y[TPW], Ot[TPW];
    tiles_y<TPW>(Sb, kb, Y);
    if constexpr (WO) {
#pragma unroll
      for (int jj = 0; jj < TPW; ++jj) Ot[jj] = zero4();
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int jj = 0; jj < TPW; ++jj) Ot[jj] = mfma_k32(cat(Sb[jj][2 * s], Sb[jj][2 * s + 1]), qb[s], Ot[jj]);
    }
    U16 u[TPW];
#pragma unroll
    for (int jj = 0; jj < TPW; ++jj) u[jj] = to_u16(tile_u(Y[jj], tf, &v[jj]));
    if constexpr (WO) {
      const u32x2 aq = sl.aq[L];
#pragma unroll
      for (int jj = 0; jj < TPW; ++jj) Ot[jj] = add_aqk_u(Ot[jj], u[jj], aq);
      // O^T tile: token c, columns col0 + 16jj + 4g..+3
      Slot& slw = sm.slot[slot];
#pragma unroll
      for (int jj = 0; jj < TPW; ++jj) *reinterpret_cast<u32x2*>(&slw.vo[c][col0 + 16 * jj + 4 * g]) = pack4(Ot[jj]);
    }
    tiles_update<TPW>(S, u, kp, gc, sl, g, c);
    wg_store(&sm.done[slot][cw], lc);
    seen = __builtin_amdgcn_readfirstlane(peek);
    return true;
  };

  // The first pass's K chunks into the next segment (ext > 0), from this
  // block's end state S.  Each consumer then compares its columns with the
  // next segment's checkpoint, which the same wavefront of that segment's
  // block (same launch) has usually published by then, and leaves the result
  // for the second pass per 16-column block; where the checkpoint is not yet
  // published (that block has not run far enough), the comparison is left to
  // the second pass, for which these columns are stored in fix.  Whether S was
  // the next segment's true start state is not decided here: the second pass
  // reads this segment's M flags for that.  (A stale fix column of a block
  // found equal here can only match the checkpoint if it holds the same bits.)
  auto extend = [&](f32x4 (&S)[TPW][8], bool ok) {
    for (int e = 0; ok && e < ext; ++e) ok = step_s(nch + e, S, WithOut{});
    uint32_t* nsy = sg.sync + ((long long)(sidx + 1) * H + h) * 16;
    const int b0 = col0 / 16;  // this wavefront's first 16-column block
    uint32_t code = 3u;
    if (ok) {
      // the checkpoint's columns are read only once their flags are seen (a
      // branch on the flags' values) and with coherent loads, so they are the
      // ones stored before the flags
      bool ready = true;
#pragma unroll
      for (int jj = 0; jj < TPW; ++jj)
        ready = ready && (uint32_t)__builtin_amdgcn_readfirstlane((int)__hip_atomic_load(
                             &nsy[b0 + jj], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) == sg.epoch;
      if (ready)
        code = __builtin_amdgcn_ballot_w64(!same_bits_coherent<TPW>(S, sg.chk, fix_base, col0, g, c)) == 0 ? 1u : 2u;
    }
    if (code == 3u && ok) store_state<TPW>(S, sg.fix, nullptr, fix_base, col0, g, c);
    if (L == 0) {
#pragma unroll
      for (int jj = 0; jj < TPW; ++jj) nsy[8 + b0 + jj] = (sg.epoch << 2) | code;
    }
  };

  if constexpr (MODE == 2) {
    f32x4 S[TPW][8];
    // Start state of segment j >= 1 (merge): S_j = M_{j-1} S_{j-1} + R_{j-1}.
    // Walk back to the nearest segment i0 whose start state is stored as is:
    // segment 1 (S_1, from segment 0's block) or a segment after one whose M
    // is exactly zero (then S_i0 = R_{i0-1}); then apply the maps of
    // segments i0 .. j-1 in order.  With every M zero this is one load.
    auto seg_at = [&](int m) { return ((long long)(sidx - (j - m)) * H + h) * D * D; };
    auto nz_bits = [&](int m) {
      const int32_t* f = sg.mnz + ((long long)(sidx - (j - m)) * H + h) * (D / 16);
      uint32_t b = 0;
#pragma unroll
      for (int q = 0; q < D / 16; ++q) b |= (f[q] != 0 ? 1u : 0u) << q;
      return b;
    };
    int i0 = j;
    while (i0 >= 2 && nz_bits(i0 - 1) != 0) --i0;
    load_state<TPW>(S, i0 == 1 ? sg.S + seg_at(1) : sg.R + seg_at(i0 - 1), true, 0, col0, g, c);
    for (int m = i0; m < j; ++m) apply_map<TPW>(S, sg.M + seg_at(m), sg.R + seg_at(m), nz_bits(m), col0, g, c);
    int lc = 0;
    bool ok = true;
    const int lim = may_stop ? K : nch;
    // the checkpoint is loaded first: its latency hides behind the first chunks
    f32x4 Ck[TPW][8];
    if (may_stop) load_state<TPW>(Ck, sg.chk, true, seg_base, col0, g, c);
    for (; ok && lc < lim; ++lc) ok = step_s(lc, S, WithOut{});
    bool stopped = false;
    if (ok && may_stop) {
      uint32_t diff = 0;
#pragma unroll
      for (int jj = 0; jj < TPW; ++jj)
#pragma unroll
        for (int tt = 0; tt < 8; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i) diff |= __float_as_uint(S[jj][tt][i]) ^ __float_as_uint(Ck[jj][tt][i]);
      const bool same = __builtin_amdgcn_ballot_w64(diff != 0u) == 0;
      if (L == 0) atomicAdd(&sm.vote, same ? 1 : 0x100);
      int it = 0, v;
      while (true) {
        v = wg_load(&sm.vote);
        if ((v & 0xFF) + (v >> 8) == NCW) break;
        if (++it > SPIN_LIMIT) {
          if (L == 0) atomicOr(&t.counters[CNT_FLAGS], 0x200);
          ok = false;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      stopped = ok && v == NCW;
      if (stopped && cw == 0 && L == 0) atomicAdd(&t.counters[CNT_EARLY_STOPS], 1);
      for (; ok && !stopped && lc < nch; ++lc) ok = step_s(lc, S, WithOut{});
    }
    // the caller's final state, in its dtype and layout; stopped: the end
    // state is the first pass's R of this segment, which that pass has written
    // there already unless the final state may alias the initial state
    if (j == ns - 1 && p.final_state && !(stopped && p.final_early)) {
      if (stopped) load_state<TPW>(S, sg.R, true, seg_base, col0, g, c);
      float* dst32 = p.state_fp32 ? static_cast<float*>(p.final_state) : nullptr;
      uint16_t* dst16 = p.state_fp32 ? nullptr : static_cast<uint16_t*>(p.final_state);
      if (p.state_kv)
        store_state_kv<TPW>(S, dst32, dst16, state_base, col0, g, c);
      else
        store_state<TPW>(S, dst32, dst16, state_base, col0, g, c);
    }
  } else {
    // First pass (or a serial call): the state S from the initial state, or,
    // for a segment >= 1 (pre), R from a zero state together with M from the
    // identity (V = 0).  A column of M evolves on its own (U = -T' Kbar M
    // needs only that column), and a column that is exactly zero stays zero
    // (every product with it is zero and gamma_C is finite).  Once this
    // wavefront's columns of M have underflowed to zero they are no longer
    // computed or stored, and R goes on alone through the same step as S.
    f32x4 S[TPW][8];
    int lc = 0;
    bool ok = true;
    // a stored checkpoint's flags, once its coherent stores have completed (one
    // chunk later, so that the wait costs nothing)
    bool pub = false;
    auto publish = [&]() {
      if (!pub) return;
      pub = false;
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(0);  // every count zero: the stores are complete
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      if (L == 0) {
#pragma unroll
        for (int jj = 0; jj < TPW; ++jj)
          __hip_atomic_store(&sg.sync[((long long)sidx * H + h) * 16 + col0 / 16 + jj], sg.epoch, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
    };
    if (!pre) {
      if (p.state_kv && p.init_state)
        load_state_kv<TPW>(S, p.init_state, p.state_fp32, state_base, col0, g, c);
      else
        load_state<TPW>(S, p.init_state, p.state_fp32, state_base, col0, g, c);
    } else {
      f32x4 Ms[TPW][8];
      bool mzero = false;
#pragma unroll
      for (int jj = 0; jj < TPW; ++jj)
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) {
          S[jj][tt] = zero4();
          f32x4 x;
#pragma unroll
          for (int i = 0; i < 4; ++i) x[i] = (16 * tt + 4 * g + i == col0 + 16 * jj + c) ? 1.f : 0.f;
          Ms[jj][tt] = x;
        }
      // R and M, with R's output when wo is set (R updated as step_s does)
      auto step_rm = [&](int lc, auto wo) -> bool {
        constexpr bool WO = decltype(wo)::value;
        const int slot = lc % NSLOT;
        if (!wait_ready(slot, lc)) return false;
        const Slot& sl = sm.slot[slot];
        u32x4 kb[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) kb[s] = sl.kbf[s][L];
        const u32x4 tf = sl.tf[L];
        U16 ur[TPW], um[TPW];
#pragma unroll
        for (int jj = 0; jj < TPW; ++jj) {  // one R and one M tile at a time: bounded live range
          const u32x2 v = slot_v(sl, g, col0 + 16 * jj + c);
          u32x2 Sb[2][8];
          pack_tile(S[jj], Sb[0]);
          pack_tile(Ms[jj], Sb[1]);
          f32x4 Y[2];
          tiles_y<2>(Sb, kb, Y);
          ur[jj] = to_u16(tile_u(Y[0], tf, &v));
          um[jj] = to_u16(tile_u(Y[1], tf, nullptr), false);
          if constexpr (WO) {
            f32x4 Ot = zero4();
#pragma unroll
            for (int s = 0; s < 4; ++s) Ot = mfma_k32(cat(Sb[0][2 * s], Sb[0][2 * s + 1]), sl.qbf[s][L], Ot);
            Ot = add_aqk_u(Ot, ur[jj], sl.aq[L]);
            Slot& slw = sm.slot[slot];
            *reinterpret_cast<u32x2*>(&slw.vo[c][col0 + 16 * jj + 4 * g]) = pack4(Ot);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        const uint32_t bits = tiles_update2<TPW>(S, ur, Ms, um, sl, g, c);
        wg_store(&sm.done[slot][cw], lc);
        mzero = __builtin_amdgcn_ballot_w64((bits & 0x7FFFFFFFu) != 0u) == 0;
        return true;
      };
      const int k1 = min(nch, o_from);
      for (; ok && lc < k1 && !mzero; ++lc) ok = step_rm(lc, NoOut{});
      for (; ok && lc < k1; ++lc) ok = step_s(lc, S, NoOut{});
      if (ok && has_chk) {
        // published to the previous segment's block, which compares it at its
        // end: coherent stores, whose flags follow after the next chunk
        store_state_coherent<TPW>(S, sg.chk, seg_base, col0, g, c);
        pub = true;
      }
      for (; ok && lc < nch && !mzero; ++lc) {
        ok = step_rm(lc, WithOut{});
        publish();
      }
      // M is final here (it has underflowed to zero or seen every chunk)
      if (j < ns - 1) {  // the second pass's merge reads the maps of middle segments
        if (!mzero) store_state<TPW>(Ms, sg.M, nullptr, seg_base, col0, g, c);
        if (L == 0) {
#pragma unroll
          for (int jj = 0; jj < TPW; ++jj)
            sg.mnz[((long long)sidx * H + h) * (D / 16) + col0 / 16 + jj] = mzero ? 0 : 1;
        }
      }
    }
    for (; ok && lc < nch; ++lc) {
      ok = step_s(lc, S, WithOut{});
      publish();
    }
    // a sequence's last segment: its end state is the caller's final state,
    // from the initial state (segment 0) or, in a segment >= 1, if the second
    // pass finds its start state changes nothing (else that pass rewrites it)
    const bool write_final = j == ns - 1 && p.final_state && (!pre || p.final_early);
    if (pre && !(write_final && has_chk)) store_state<TPW>(S, sg.R, nullptr, seg_base, col0, g, c);
    if (write_final) {  // the caller's final state, in its dtype and layout
      float* dst32 = p.state_fp32 ? static_cast<float*>(p.final_state) : nullptr;
      uint16_t* dst16 = p.state_fp32 ? nullptr : static_cast<uint16_t*>(p.final_state);
      if (p.state_kv)
        store_state_kv<TPW>(S, dst32, dst16, state_base, col0, g, c);
      else
        store_state<TPW>(S, dst32, dst16, state_base, col0, g, c);
    } else if (!pre && j < ns - 1) {
      // segment 0's end state is S_1, where the second pass's merge starts
      // (slot sidx + 1).  The second pass stores nothing here: the next
      // segment's block may be reading its start state in that launch.
      store_state<TPW>(S, sg.S, nullptr, seg_base + (long long)H * D * D, col0, g, c);
    }
    if (ext > 0) extend(S, ok);  // into the next segment (see above)
  }
}

// One block per (segment, head) unit: block u runs head u % H of the
// segment in row u / H of the dispatch table (full-length segments first,
// so that the long units start first).  Units that exist (the segment count
// is known only on the device) take the first blocks and the rest exit at
// once: blocks are dealt to the XCDs in turn, and this keeps their shares of
// the work equal.
// MODE 0: whole sequences (serial plan).
// MODE 1: first pass of a segmented call: segment 0 of each sequence from the
// initial state, the others from a zero state.
// MODE 2: second pass of a segmented call: segments >= 1 from their start states.
#if KDA_CONSUMERS == 8
#define KDA_CHUNK_KERNEL kda_chunk_kernel
#define KDA_LAUNCH_CHUNKS launch_chunks
#elif KDA_CONSUMERS == 4
#define KDA_CHUNK_KERNEL kda_chunk_kernel_c4
#define KDA_LAUNCH_CHUNKS launch_chunks_c4
#else
#error "KDA_CONSUMERS must be 8 or 4"
#endif

template <int MODE>
__global__ __launch_bounds__(NTHREADS) void KDA_CHUNK_KERNEL(Problem p, Tables t, Seg sg) {
  __shared__ Smem sm;
  const int k = (int)blockIdx.x / p.H;
  const int h = (int)blockIdx.x - k * p.H;
  Unit u;
  if (t.fixed) {
    // fixed length: every block takes its unit from the tables' closed form
    // The first launch sets the counters before any block can add to one.  No
    // kernel reads the table rows of a fixed-length call, and none stores them
    // (kda_write_fixed_tables does, for inspection).
    if (MODE != 2 && blockIdx.x == 0 && threadIdx.x == 0) fixed_counters(p.N, t.fixed_T, sg.seg_chunks, t);
    int32_t row[8];
    if (!fixed_unit_row(p.N, t.fixed_T, sg.seg_chunks, k, row)) return;
    u = Unit{row[0], row[1], row[2], row[3], row[4], row[5], row[6], row[7]};
  } else {
    // the whole row in one read (rows past the live units hold -1); the grid
    // has one row of blocks per table row
    const int4 r0 = reinterpret_cast<const int4*>(t.unit_tab)[2 * k];
    const int4 r1 = reinterpret_cast<const int4*>(t.unit_tab)[2 * k + 1];
    if (r0.x < 0) return;
    u = Unit{r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
  }
  chunk_body<MODE>(sm, p, t, sg, u, h);
}

hipError_t KDA_LAUNCH_CHUNKS(const Problem& p, Tables t, const Seg& sg, int64_t max_segs, int phase, bool segmented,
                             hipStream_t st) {
  if (max_segs <= 0) return hipSuccess;
  if (segmented && phase != 0 && KDA_CONSUMERS != 8) return hipErrorInvalidValue;  // second pass: 8 consumers only
  const unsigned blocks = (unsigned)(max_segs * p.H);
  hipEvent_t e0, e1;
  stage_events(phase == 0 ? KDA_STAGE_RECUR0 : KDA_STAGE_RECUR1, &e0, &e1);
  if (!segmented)
    hipExtLaunchKernelGGL(KDA_CHUNK_KERNEL<0>, dim3(blocks), dim3(NTHREADS), 0, st, e0, e1, 0, p, t, sg);
  else if (phase == 0)
    hipExtLaunchKernelGGL(KDA_CHUNK_KERNEL<1>, dim3(blocks), dim3(NTHREADS), 0, st, e0, e1, 0, p, t, sg);
  else
    hipExtLaunchKernelGGL(KDA_CHUNK_KERNEL<KDA_CONSUMERS == 8 ? 2 : 1>, dim3(blocks), dim3(NTHREADS), 0, st, e0, e1, 0, p,
                          t, sg);
  return hipGetLastError();
}

}  // namespace kda
