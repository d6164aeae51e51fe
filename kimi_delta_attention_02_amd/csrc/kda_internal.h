// Internal definitions shared by the HIP kernels and the host library.
//
// MFMA lane layouts used throughout (wave64, lane L, g = L / 16, c = L % 16):
//   v_mfma_f32_16x16x32_bf16 : A[c][8g+e], B[8g+e][c] (e = 0..7), D[4g+i][c]
//   v_mfma_f32_16x16x16_f16  : A[c][4g+e], B[4g+e][c] (e = 0..3), D[4g+i][c]
//   v_mfma_f32_16x16x4_f32   : A[c][g],    B[g][c],                D[4g+i][c]
// A 16x16 fp32 accumulator tile therefore holds rows 4g..4g+3 of column c in
// lane L.  For the 16x16x32 MFMA over a K range made of two 16-row tiles
// (a, b), lane group g supplies rows {16a+4g+0..3, 16b+4g+0..3}: the reduction
// index is permuted, and every operand that meets the state uses the same
// permutation.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kda.h"

namespace kda {

constexpr int D = KDA_HEAD_DIM;  // K = V = 128
constexpr int C = KDA_CHUNK;     // 16 tokens per chunk

// ---- counters block ----
constexpr int CNT_N_CHUNKS = 0;
constexpr int CNT_N_SEGS = 1;
constexpr int CNT_FLAGS = 2;
constexpr int CNT_EARLY_STOPS = 3;  // (segment, head) pairs whose second pass stopped at the checkpoint
constexpr int CNT_SEG_CHUNKS = 4;   // segment length in use (0: serial)
constexpr int CNT_ORDER = 5;        // unit_tab order: 0 segment order, 1 longest first (see kda_index.hip)
constexpr int kLptMaxSeqs = 256;    // a serial varlen plan of at most this many sequences goes longest first

// Pointers into a carved workspace (device addresses).
struct Tables {
  int32_t* counters;
  int32_t* seq_start;
  int32_t* seq_len;
  int32_t* seq_chunk_off;
  int32_t* seq_seg_off;
  int32_t* chunk_tab;
  int32_t* seg_tab;
  int32_t* seq_full_off;
  int32_t* unit_tab;
  // A fixed-length call (no cu_seqlens) launches no index kernel: its first
  // chunk-kernel launch writes these tables from their closed form, and every
  // block finds its unit from that closed form.
  int fixed;       // 1: fixed length, fixed_T tokens per sequence; 0: varlen
  int fixed_T;
  int64_t max_chunks, max_segs;  // table capacities
};

struct Problem {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* g;
  const uint16_t* beta;
  uint16_t* out;
  const float* A_log;
  const float* dt_bias;
  const void* init_state;
  void* final_state;
  int state_fp32;
  int state_kv;  // caller's states are [N][H][K][V] (else [N][H][V][K])
  // final_state shares no byte with initial_state: a segmented call's first
  // pass may then write the final state of a sequence's last segment itself
  // (while segment 0's blocks may still be reading the initial state).
  int final_early;
  float scale;
  float lower_bound;
  int H;    // heads of v, g, beta, out and the states
  int Hqk;  // heads of q and k (divides H; head h reads q/k head h / (H / Hqk))
  int N;
  int64_t total_tokens;
};

// Segment buffers of a segmented call (all null when serial), [segment][head][v][k] fp32:
//   M, R : transition and zero-start state of segments >= 1 (first pass);
//   S    : state entering segment 1 of each sequence (segment 0's end state);
//          the second pass merges the later start states itself;
//   chk  : R after the first chk_chunks chunks of segments >= 1 (first pass);
//   fix  : the state after a segment's first chk_chunks chunks as the first
//          pass's block of the previous segment reached it (first pass);
//   mnz  : per (segment, head, 16-column block of M) 1 if nonzero, 0 if exactly zero;
//   sync : per (segment, head) 16 words: the checkpoint's publication by each
//          consumer wavefront (words 0..7, this call's epoch once stored) and the
//          previous segment's decision about it (word 8 epoch, word 9 code).
// epoch is a number no earlier call on the same workspace wrote (nonzero), so
// words left by an earlier call never pass for this call's.
struct Seg {
  float* M;
  float* R;
  float* S;
  float* chk;
  float* fix;
  int32_t* mnz;
  uint32_t* sync;
  uint32_t epoch;
  int chk_chunks;
  int seg_chunks;  // segment length in chunks of a fixed-length call (0: serial); a varlen call's is in unit_tab
};

// ---- launchers (host functions defined next to their kernels) ----
// Kernel timing for the profiling hook (kda_profile_enable): a launch site asks
// for an event pair for its stage before each launch.  While profiling is on it
// gets two events, which hipExtLaunchKernelGGL stamps with the kernel's own
// start and end; otherwise both stay null and the launch is a plain one.
void stage_events(int stage, hipEvent_t* start, hipEvent_t* stop);
hipError_t launch_index_fixed(int N, int L, int seg, Tables t, hipStream_t st);
// choose: the library chooses the plan (seg_chunks is the planned, shortest
// length; the tables may use a longer one, see seg_span); may_serial: the
// tables stay serial unless the lengths are skewed (kda_index.hip); K:
// chk_chunks
hipError_t launch_index(const int32_t* cu_seqlens, int N, int64_t T_row, int64_t total_tokens, int seg_chunks,
                        int H, int K, bool choose, bool may_serial, int64_t max_chunks, int64_t max_segs, Tables t,
                        hipStream_t st);
// producer/consumer chunk kernel: one launch per pass (phase 0: every segment,
// phase 1: segments >= 1 from their start states, merged in the same launch)
hipError_t launch_chunks(const Problem& p, Tables t, const Seg& sg, int64_t max_segs, int phase, bool segmented,
                         hipStream_t st);
// the same kernel with 4 consumer wavefronts of two state tiles each
hipError_t launch_chunks_c4(const Problem& p, Tables t, const Seg& sg, int64_t max_segs, int phase, bool segmented,
                            hipStream_t st);

}  // namespace kda

#ifdef __HIPCC__
namespace kda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16 with round to nearest even: one v_cvt_pk_bf16_f32 per pair.
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ u32x2 pack4(f32x4 x) {
  u32x2 r;
  r.x = pack2(x[0], x[1]);
  r.y = pack2(x[2], x[3]);
  return r;
}

// x0 = h0 + l0, x1 = h1 + l1 with h = bf16(x) (round to nearest even) and
// l = bf16(x - h), so x = h + l + O(2^-16 |x|): hi = (h0, h1), lo = (l0, l1) as
// packed bf16 pairs.  One rounding per pair for h, whose fp32 values are read
// back from the packed word.
__device__ __forceinline__ void split_pair(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  hi = pack2(x0, x1);
  lo = pack2(x0 - __uint_as_float(hi << 16), x1 - __uint_as_float(hi & 0xFFFF0000u));
}

// fp32 -> fp16 with round to nearest even: one v_cvt_pk_f16_f32 per pair.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint32_t pack2_f16(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

__device__ __forceinline__ u32x2 pack4_f16(f32x4 x) {
  u32x2 r;
  r.x = pack2_f16(x[0], x[1]);
  r.y = pack2_f16(x[2], x[3]);
  return r;
}

__device__ __forceinline__ void split4(f32x4 x, u32x2& hi, u32x2& lo) {
  uint32_t h0, l0, h1, l1;
  split_pair(x[0], x[1], h0, l0);
  split_pair(x[2], x[3], h1, l1);
  hi = u32x2{h0, h1};
  lo = u32x2{l0, l1};
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ u32x4 cat(u32x2 a, u32x2 b) {
  u32x4 r;
  r.x = a.x;
  r.y = a.y;
  r.z = b.x;
  r.w = b.y;
  return r;
}

__device__ __forceinline__ f32x4 mfma_k32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f16_k16(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f32_k4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() {
  f32x4 z = {0.f, 0.f, 0.f, 0.f};
  return z;
}

// ---- tables of a fixed-length call (N sequences of L tokens), closed form ----
// A sequence has nc = ceil(L/16) chunks and, split into segments of seg
// chunks (seg = 0: one segment, serial), ns = ceil(nc/seg) segments (1 when
// nc = 0) of which nf = floor(nc/seg) are full length.  Dispatch rank r
// (a row of unit_tab) holds, for r < N nf, full segment r % nf of sequence
// r / nf, and past that the shorter last segment of sequence r - N nf.
struct FixedShape {
  int nc, ns, nf;
};

__device__ __forceinline__ FixedShape fixed_shape(int L, int seg) {
  FixedShape s;
  s.nc = (L + 15) / 16;
  s.ns = seg > 0 ? (s.nc > 0 ? (s.nc + seg - 1) / seg : 1) : 1;
  s.nf = seg > 0 ? s.nc / seg : 1;
  return s;
}

// The unit_tab row of dispatch rank r; false past the live units.  (Table
// sizes are validated to fit int32 with room to spare, so 32-bit arithmetic
// suffices here.)
__device__ __forceinline__ bool fixed_unit_row(int N, int L, int seg, int r, int32_t row[8]) {
  const FixedShape s = fixed_shape(L, seg);
  const int n_full = N * s.nf;
  if (r >= N * s.ns) return false;
  const int sq = r < n_full ? r / s.nf : r - n_full;
  const int j = r < n_full ? r - sq * s.nf : s.ns - 1;
  const int first = sq * s.nc;
  int b = first, e = first + s.nc;
  if (seg > 0) {
    const int b0 = j * seg;
    b = first + min(b0, s.nc);
    e = first + min(b0 + min(seg, s.nc), s.nc);
  }
  row[0] = sq * s.ns + j;  // segment row
  row[1] = sq;
  row[2] = b;
  row[3] = e;
  row[4] = j;
  row[5] = sq * L;
  row[6] = L;
  row[7] = seg;
  return true;
}

// The counters of a fixed-length call (one thread).
__device__ __forceinline__ void fixed_counters(int N, int L, int seg, const Tables& t) {
  const FixedShape s = fixed_shape(L, seg);
  t.counters[CNT_N_CHUNKS] = N * s.nc;
  t.counters[CNT_N_SEGS] = N * s.ns;
  t.counters[CNT_FLAGS] = 0;
  t.counters[CNT_EARLY_STOPS] = 0;
  t.counters[CNT_SEG_CHUNKS] = seg;
  t.counters[CNT_ORDER] = 0;
}

// Every table row of a fixed-length call, rows tid, tid + nthr, ... (the same
// contents the varlen index kernels give for equal lengths).  Rows number
// less than 2^30; tid and nthr come clamped to that.
__device__ __forceinline__ void fixed_tables(int tid, int nthr, int N, int L, int seg, const Tables& t) {
  const FixedShape s = fixed_shape(L, seg);
  for (int i = tid; i <= N; i += nthr) {
    t.seq_start[i] = i * L;
    t.seq_chunk_off[i] = i * s.nc;
    t.seq_seg_off[i] = i * s.ns;
    t.seq_full_off[i] = i * s.nf;
    if (i < N) t.seq_len[i] = L;
  }
  const int n_chunks = N * s.nc;
  const int max_chunks = (int)t.max_chunks, max_segs = (int)t.max_segs;
  for (int r = tid; r < max_chunks; r += nthr) {
    const bool live = r < n_chunks;
    const int sq = live ? r / s.nc : -1;
    t.chunk_tab[2 * (long long)r] = sq;
    t.chunk_tab[2 * (long long)r + 1] = live ? r - sq * s.nc : -1;
  }
  for (int r = tid; r < max_segs; r += nthr) {
    int32_t row[8];
    const bool live = fixed_unit_row(N, L, seg, r, row);
    int32_t* u = t.unit_tab + 8 * (long long)r;
#pragma unroll
    for (int q = 0; q < 8; ++q) u[q] = live ? row[q] : -1;
    if (live) {
      // the segment of this rank into its row of seg_tab
      int32_t* sr = t.seg_tab + 4 * (long long)row[0];
      sr[0] = row[1];
      sr[1] = row[2];
      sr[2] = row[3];
      sr[3] = row[4];
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) t.seg_tab[4 * (long long)r + q] = -1;
    }
  }
}

// ---- segment length of a plan the library chooses ----
// The host plans the shortest segment length, which sizes the workspace: one
// that would give 256 (segment, head) units if every sequence split evenly.
// How the units of a length s then pack onto the chip depends on the
// sequence lengths (a sequence's last segment is shorter, a short sequence is
// one short unit) and on how the hardware places workgroups: it deals them to
// the 8 XCDs in turn and, inside an XCD, to its 4 shader engines in turn (8
// CUs each, one chunk-kernel workgroup per CU), in order, so that a workgroup
// whose engine has no free CU holds back every later one of its XCD, although
// another engine may have one free (seen in per-workgroup clock stamps).
// seg_span replays that placement for one XCD (H a multiple of 8, so that
// every XCD gets the same share) and returns the first pass's predicted span
// in chunk steps: a unit costs the chunks it runs plus a fixed start cost.
// The units come in dispatch-table order: every full-length segment in
// segment order, then the shorter ones (a sequence's last segment, or a
// sequence shorter than s), in segment order or, with desc, longest first.
// A full segment runs K chunks into the next one when that one is longer
// than K; a later segment of K chunks or fewer ends at once.  Sequence i has
// nc[i] chunks; cu holds 32 + kSpanMaxSeqs ints at stride STRIDE (the CUs of
// one XCD, engine-major, then the costs of the shorter segments).
constexpr int kSpanStartCost = 4;    // a unit's fixed start cost, in chunk steps (measured 2 to 7)
constexpr int kSpanCandidates = 64;  // lengths tried: seg .. seg + min(seg / 4, 63)
constexpr int kSpanMaxSeqs = 16;  // a power of two (the sorting network)
// The index kernel spends a few microseconds on the choice (a wavefront per
// order replays up to 64 placements per candidate); it makes it only for a
// planned length of at least this many chunks, whose first pass takes ~180 us
// or more.
constexpr int kSpanDeviceMinSeg = 128;

__host__ __device__ inline bool span_model_applies(int seg, int N, int H) {
  return seg > 0 && N >= 1 && N <= kSpanMaxSeqs && H % 8 == 0 && N * H <= 256;
}

__host__ __device__ inline int span_candidates(int seg) {
  const int q = seg / 4;
  return 1 + (q < kSpanCandidates - 1 ? q : kSpanCandidates - 1);
}

// q = n / s and r = n - q s for 0 <= n < 2^27 and s >= 1, exactly.  On the
// device, for s >= 128 (every length the model scores there), from a float
// estimate, off by at most one in that range, then corrected: the quarter-rate
// steps of a plain integer division weigh on the model's cost.  Elsewhere by
// plain division.
__host__ __device__ inline int span_div(int n, int s, int& r) {
#if defined(__HIP_DEVICE_COMPILE__)
  if (s < 128) {
    const int q = n / s;
    r = n - q * s;
    return q;
  }
  int q = (int)((float)n * __builtin_amdgcn_rcpf((float)s));
  r = n - q * s;
  if (r < 0) {
    q -= 1;
    r += s;
  }
  if (r >= s) {
    q += 1;
    r -= s;
  }
  return q;
#else
  const int q = n / s;
  r = n - q * s;
  return q;
#endif
}

// The first-pass cost, in chunks, of the shorter segment of a sequence split
// into f full segments of s chunks and rem more, or -1 when it has none: a
// sequence shorter than s is one unit of rem chunks (0 for an empty one); a
// later last segment of rem chunks runs them unless rem <= K.
__host__ __device__ inline int rest_cost_of(int f, int rem, int K) {
  if (f == 0) return rem;
  if (rem == 0) return -1;
  return rem > K ? rem : 0;
}

__host__ __device__ inline int rest_cost(int n, int s, int K) {
  int rem;
  const int f = span_div(n, s, rem);
  return rest_cost_of(f, rem, K);
}

template <int STRIDE>
__host__ __device__ inline int seg_span(int s, int N, const int* nc, int H, int K, bool desc, int* cu) {
  for (int k = 0; k < 32; ++k) cu[k * STRIDE] = 0;
  const int per = H / 8;  // workgroups of a unit's row per XCD
  int last = 0, span = 0, blk = 0, row = 0;
  // the k-th workgroup an engine receives (its CUs at e): the first 8 fill its
  // empty CUs at once, the later ones wait for the earliest free CU and start
  // no earlier than the workgroup dispatched before them
  auto on_engine = [&](int* e, int k, int cost) {
    if (k < 8) {
      e[k * STRIDE] = cost + kSpanStartCost;
      span = cost + kSpanStartCost > span ? cost + kSpanStartCost : span;
      return;
    }
    int best = e[0], bk = 0;
    for (int c = 1; c < 8; ++c) {
      const int v = e[c * STRIDE];
      if (v < best) {
        best = v;
        bk = c;
      }
    }
    const int st = best > last ? best : last;
    last = st;
    const int fin = st + cost + kSpanStartCost;
    e[bk * STRIDE] = fin;
    span = fin > span ? fin : span;
  };
  // A row's workgroups go to engines blk % 4, blk + 1, ...  Engines that
  // always receive the same work are replayed once: with 2 per row (H = 16)
  // even rows reach engines 0 and 1 and odd rows 2 and 3, so one engine stands
  // for each pair; with a multiple of 4 (H = 32, 64, ...) every row reaches all
  // four alike, per / 4 workgroups each.  Otherwise each workgroup is placed.
  auto place = [&](int cost) {
    if (per == 2) {
      on_engine(cu + (row & 1) * 8 * STRIDE, row >> 1, cost);
    } else if ((per & 3) == 0) {
      for (int m = 0; m < per / 4; ++m) on_engine(cu, row * (per / 4) + m, cost);
    } else {
      for (int m = 0; m < per; ++m, ++blk) on_engine(cu + (blk & 3) * 8 * STRIDE, blk >> 2, cost);
    }
    ++row;
  };
  int rc[kSpanMaxSeqs];  // each sequence's shorter segment (-1: none)
#pragma unroll
  for (int i = 0; i < kSpanMaxSeqs; ++i) rc[i] = -1;
  for (int i = 0; i < N; ++i) {
    int rem;
    const int f = span_div(nc[i], s, rem);
    for (int j = 0; j < f; ++j) {
      const int nn = j + 1 < f ? s : rem;  // the next segment's chunks
      place(s + (nn > K ? K : 0));
    }
    const int c = rest_cost_of(f, rem, K);
#pragma unroll
    for (int q = 0; q < kSpanMaxSeqs; ++q) rc[q] = q == i ? c : rc[q];  // static indices: registers
  }
  if (desc) {
    // longest first: rc sorted in descending order by a bitonic network (the
    // placement depends on the costs alone, so ties may change places)
#pragma unroll
    for (int k = 2; k <= kSpanMaxSeqs; k <<= 1)
#pragma unroll
      for (int j = k >> 1; j > 0; j >>= 1)
#pragma unroll
        for (int i = 0; i < kSpanMaxSeqs; ++i) {
          const int l = i ^ j;
          if (l > i) {
            const int a = rc[i], b = rc[l];
            const bool sw = (i & k) == 0 ? a < b : a > b;
            rc[i] = sw ? b : a;
            rc[l] = sw ? a : b;
          }
        }
  }
  // placed from cu's second part in a rolled loop (one copy of the placement code)
  int n_rest = 0;
#pragma unroll
  for (int i = 0; i < kSpanMaxSeqs; ++i)
    if (rc[i] >= 0) cu[(32 + n_rest++) * STRIDE] = rc[i];
  for (int i = 0; i < n_rest; ++i) place(cu[(32 + i) * STRIDE]);
  return span;
}

}  // namespace kda
#endif
