// Inter-chunk recurrence ("K2" on the cuLA PR #106 page) and the segment
// pre-scan of the segment split ("pre_scan" on the same page).
//
// Per chunk, with S the K x V fp32 state entering the chunk:
//   U = Ut - W S;   O = Qbar S + Aqk U;   S <- Diag(gamma_C) S + Khat^T U
// Every map acts on the key dimension only, so the 128 value columns evolve
// independently: a workgroup of 4 wavefronts owns 128 columns, each wavefront
// 32 of them (two 16-column MFMA tiles), held as fp32 MFMA accumulators for
// the whole segment.  The accumulator layout doubles as the bf16 operand layout
// of the next chunk's products (see kda_internal.h), so the state never leaves
// registers between chunks.
//
// Roles (one kernel, one per-chunk state step, so every chain that should be
// bit-identical runs the same instructions):
//   RECUR  : the state with output; serial sequences, segment 0 from the
//            initial state, later segments from their merged start states.
//   PRE_M  : the transition M of a middle segment (start I, Ut taken as 0).
//   PRE_R  : the zero-start state R of a middle segment (start 0, no output).
// M and R are the exact affine map of the segment (the page keeps an exact M).
#include "kda_internal.h"

namespace kda {

namespace {

enum Role { RECUR = 0, PRE_M = 1, PRE_R = 2 };

constexpr int NTW = 2;  // 16-column tiles per wavefront

struct ChunkOps {
  u32x4 W[4];
  u32x4 Q[4];
  u32x2 Kh[8];
  u32x2 Kl[8];
  u32x2 Aqh, Aql;
  f32x4 Ut[NTW];
  f32x4 gC[8];
};

__device__ __forceinline__ void load_ops(ChunkOps& o, const uint8_t* __restrict__ r, int L, int g, int ct0,
                                         bool want_out, bool want_ut) {
#pragma unroll
  for (int s = 0; s < 4; ++s) o.W[s] = reinterpret_cast<const u32x4*>(r + REC_W)[s * 64 + L];
  if (want_out) {
#pragma unroll
    for (int s = 0; s < 4; ++s) o.Q[s] = reinterpret_cast<const u32x4*>(r + REC_Q)[s * 64 + L];
    o.Aqh = reinterpret_cast<const u32x2*>(r + REC_AQK_HI)[L];
    o.Aql = reinterpret_cast<const u32x2*>(r + REC_AQK_LO)[L];
  }
#pragma unroll
  for (int tt = 0; tt < 8; ++tt) {
    o.Kh[tt] = reinterpret_cast<const u32x2*>(r + REC_KH_HI)[tt * 64 + L];
    o.Kl[tt] = reinterpret_cast<const u32x2*>(r + REC_KH_LO)[tt * 64 + L];
  }
  if (want_ut) {
#pragma unroll
    for (int j = 0; j < NTW; ++j) o.Ut[j] = reinterpret_cast<const f32x4*>(r + REC_UT)[(ct0 + j) * 64 + L];
  }
#pragma unroll
  for (int tt = 0; tt < 8; ++tt) o.gC[tt] = reinterpret_cast<const f32x4*>(r + REC_GC)[4 * tt + g];
}

// One chunk of the recurrence for this wavefront's column tiles.
//   U = Ut - W S (bf16 W and S); U kept as a high/low pair
//   O^T = S^T Qbar^T + U^T Aqk^T     (Aqk and U as high/low pairs)
//   S <- Diag(gamma_C) S + Khat^T U  (Khat and U as high/low pairs)
// Every product is a 16x16x32 MFMA; the split products put both halves of a
// 16-token reduction into the 32-long K dimension, e.g.
//   [Khat_hi | Khat_hi] [U_hi ; U_lo] + [Khat_lo | Khat_lo] [U_hi ; U_lo].
__device__ __forceinline__ void chunk_step(f32x4 (&S)[8][NTW], const ChunkOps& op, bool want_out, bool want_ut,
                                           uint16_t* __restrict__ out_row, bool store) {
  u32x2 Sb[8][NTW];
#pragma unroll
  for (int tt = 0; tt < 8; ++tt)
#pragma unroll
    for (int jj = 0; jj < NTW; ++jj) Sb[tt][jj] = pack4(S[tt][jj]);

  u32x4 Uhl[NTW];
#pragma unroll
  for (int jj = 0; jj < NTW; ++jj) {
    f32x4 X = zero4();
#pragma unroll
    for (int s = 0; s < 4; ++s) X = mfma_k32(op.W[s], cat(Sb[2 * s][jj], Sb[2 * s + 1][jj]), X);
    const f32x4 U = want_ut ? op.Ut[jj] - X : -X;
    u32x2 uh, ul;
    split4(U, uh, ul);
    Uhl[jj] = cat(uh, ul);
  }

  if (want_out) {
#pragma unroll
    for (int jj = 0; jj < NTW; ++jj) {
      f32x4 Ot = zero4();
#pragma unroll
      for (int s = 0; s < 4; ++s) Ot = mfma_k32(cat(Sb[2 * s][jj], Sb[2 * s + 1][jj]), op.Q[s], Ot);
      Ot = mfma_k32(Uhl[jj], cat(op.Aqh, op.Aqh), Ot);
      Ot = mfma_k32(Uhl[jj], cat(op.Aql, op.Aql), Ot);
      if (store) *reinterpret_cast<u32x2*>(out_row + 16 * jj) = pack4(Ot);
    }
  }

#pragma unroll
  for (int tt = 0; tt < 8; ++tt)
#pragma unroll
    for (int jj = 0; jj < NTW; ++jj) {
      f32x4 acc = mfma_k32(cat(op.Kh[tt], op.Kh[tt]), Uhl[jj], S[tt][jj] * op.gC[tt]);
      S[tt][jj] = mfma_k32(cat(op.Kl[tt], op.Kl[tt]), Uhl[jj], acc);
    }
}

}  // namespace

__global__ __launch_bounds__(256) void kda_recur_kernel(Problem p, Tables t, const uint8_t* __restrict__ rec,
                                                        float* __restrict__ segM, float* __restrict__ segR,
                                                        float* __restrict__ segS, int phase) {
  const int sidx = blockIdx.x >> 1;
  const int half = blockIdx.x & 1;
  const int h = blockIdx.y;
  if (sidx >= t.counters[CNT_N_SEGS]) return;
  const int seq = t.seg_tab[4 * sidx + 0];
  const int cb = t.seg_tab[4 * sidx + 1];
  const int ce = t.seg_tab[4 * sidx + 2];
  const int j = t.seg_tab[4 * sidx + 3];
  const int ns = t.seq_seg_off[seq + 1] - t.seq_seg_off[seq];
  int role;
  if (phase == 0) {
    if (j == 0) {
      if (half) return;
      role = RECUR;
    } else if (j < ns - 1) {
      role = half ? PRE_R : PRE_M;
    } else {
      return;
    }
  } else {
    if (j == 0 || half) return;
    role = RECUR;
  }

  const int H = p.H;
  const int w = threadIdx.x >> 6;
  const int L = threadIdx.x & 63;
  const int g = L >> 4;
  const int c = L & 15;
  const int ct0 = NTW * w;  // first 16-column tile of this wavefront
  const long long state_base = ((long long)seq * H + h) * D * D;
  const long long seg_base = ((long long)sidx * H + h) * D * D;

  // ---- initial accumulators: S[16tt+4g+i][16(ct0+jj)+c] ----
  f32x4 S[8][NTW];
  if (role == RECUR) {
    const bool from_seg = (phase == 1);
    const void* src = from_seg ? (const void*)(segS + seg_base) : p.init_state;
    const bool f32 = from_seg || p.state_fp32;
    const long long base = from_seg ? 0 : state_base;
#pragma unroll
    for (int jj = 0; jj < NTW; ++jj) {
      const int col = 16 * (ct0 + jj) + c;
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        f32x4 x = zero4();
        if (src) {
          const long long off = base + (long long)col * D + 16 * tt + 4 * g;
          if (f32) {
            x = *reinterpret_cast<const f32x4*>(static_cast<const float*>(src) + off);
          } else {
            const u32x2 b = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(src) + off);
            x[0] = __uint_as_float(b.x << 16);
            x[1] = __uint_as_float(b.x & 0xFFFF0000u);
            x[2] = __uint_as_float(b.y << 16);
            x[3] = __uint_as_float(b.y & 0xFFFF0000u);
          }
        }
        S[tt][jj] = x;
      }
    }
  } else {
#pragma unroll
    for (int jj = 0; jj < NTW; ++jj) {
      const int col = 16 * (ct0 + jj) + c;
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        f32x4 x = zero4();
        if (role == PRE_M) {
#pragma unroll
          for (int i = 0; i < 4; ++i) x[i] = (16 * tt + 4 * g + i == col) ? 1.f : 0.f;
        }
        S[tt][jj] = x;
      }
    }
  }

  const bool want_out = (role == RECUR);
  const bool want_ut = (role != PRE_M);
  const int first_chunk = t.seq_chunk_off[seq];
  const long long seq_tok0 = t.seq_start[seq];
  const int seq_len = t.seq_len[seq];
  const long long rec_stride = (long long)H * REC_BYTES;
  const uint8_t* rbase = rec + (long long)h * REC_BYTES;
  // output element (token c of the chunk, columns 16*ct0 + 4g ..) for chunk ch
  auto out_row = [&](int ch) -> uint16_t* {
    const long long tok = seq_tok0 + (long long)C * (ch - first_chunk) + c;
    return p.out + (tok * H + h) * D + 16 * ct0 + 4 * g;
  };
  auto stores = [&](int ch) -> bool { return c < seq_len - C * (ch - first_chunk); };

  // two operand sets, loaded one chunk ahead of their use
  ChunkOps opA, opB;
  if (cb < ce) load_ops(opA, rbase + cb * rec_stride, L, g, ct0, want_out, want_ut);
  for (int ch = cb; ch < ce; ch += 2) {
    if (ch + 1 < ce) load_ops(opB, rbase + (ch + 1) * rec_stride, L, g, ct0, want_out, want_ut);
    chunk_step(S, opA, want_out, want_ut, want_out ? out_row(ch) : nullptr, want_out && stores(ch));
    if (ch + 1 >= ce) break;
    if (ch + 2 < ce) load_ops(opA, rbase + (ch + 2) * rec_stride, L, g, ct0, want_out, want_ut);
    chunk_step(S, opB, want_out, want_ut, want_out ? out_row(ch + 1) : nullptr, want_out && stores(ch + 1));
  }

  // ---- write back ----
  if (role == RECUR) {
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
      // start state of the next segment of this sequence (slot sidx + 1)
      dst32 = segS;
      base = seg_base + (long long)H * D * D;
    }
#pragma unroll
    for (int jj = 0; jj < NTW; ++jj) {
      const int col = 16 * (ct0 + jj) + c;
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const long long off = base + (long long)col * D + 16 * tt + 4 * g;
        if (dst32) *reinterpret_cast<f32x4*>(dst32 + off) = S[tt][jj];
        if (dst16) *reinterpret_cast<u32x2*>(dst16 + off) = pack4(S[tt][jj]);
      }
    }
  } else {
    float* dst = (role == PRE_M) ? segM : segR;
#pragma unroll
    for (int jj = 0; jj < NTW; ++jj) {
      const int col = 16 * (ct0 + jj) + c;
#pragma unroll
      for (int tt = 0; tt < 8; ++tt)
        *reinterpret_cast<f32x4*>(dst + seg_base + (long long)col * D + 16 * tt + 4 * g) = S[tt][jj];
    }
  }
}

hipError_t launch_recur(const Problem& p, Tables t, const uint8_t* rec, float* segM, float* segR, float* segS,
                        int64_t max_segs, int phase, hipStream_t st) {
  if (max_segs <= 0) return hipSuccess;
  hipLaunchKernelGGL(kda_recur_kernel, dim3((unsigned)(2 * max_segs), (unsigned)p.H), dim3(256), 0, st, p, t, rec,
                     segM, segR, segS, phase);
  return hipGetLastError();
}

}  // namespace kda
