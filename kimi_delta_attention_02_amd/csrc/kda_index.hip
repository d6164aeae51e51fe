// Varlen chunk / segment index construction.
//
// Sequence boundaries come from cu_seqlens (varlen, B = 1) or from b*T (fixed
// length); chunks of 16 tokens never cross a sequence start, and a sequence is
// split into segments of `seg_chunks` chunks for the segment (pre-scan + merge)
// path.  Pages: "How FlashKDA Integrates with CUTLASS", section
// "Variable-Length Sequence Support" (prefix-sum offsets from cu_seqlens);
// cuLA PR #106 commit list (CHUNK = 16, segment split) and review thread
// (cu_seqlens and chunk_indices passed to the kernels).
//
// Free of host synchronisation, in one of three forms:
//  - fixed length (no cu_seqlens): every row has a closed form (sequence i
//    starts at i T, has ceil(T/16) chunks, ...; fixed_tables in
//    kda_internal.h): kda_fwd launches no index kernel and the chunk kernel's
//    blocks find their units from that closed form; kda_index_fixed writes
//    the rows out only for kda_write_fixed_tables (inspection and tests);
//  - up to FUSED_MAX_N sequences and FUSED_MAX_ROWS table rows: one launch of
//    kda_index_fused (one 1024-thread workgroup) that does both steps below,
//    the second from copies of the prefix sums in LDS;
//  - otherwise two launches:
//    1. kda_index_scan (one 1024-thread workgroup): clamps the offsets into a
//       non-decreasing sequence within [0, total], then prefix-sums the chunk,
//       segment and full-length segment counts.  Tables: seq_start[N+1],
//       seq_len[N], seq_chunk_off[N+1], seq_seg_off[N+1], seq_full_off[N+1],
//       counters {n_chunks, n_segs, flags, 0}.
//    2. kda_index_fill: one thread per table row; binary search of the prefix
//       sums gives chunk_tab[c] = (seq, chunk in seq) and
//       seg_tab[s] = (seq, first chunk, end chunk, segment in seq), and puts
//       segment s into the dispatch table unit_tab (full-length segments
//       first, then the shorter ones, so that the long units start first).
//       Rows past the live counts are -1.
// A unit_tab row is (segment, seq, first chunk, end chunk, segment in seq,
// sequence start token, sequence length, segment length): everything the
// chunk kernel needs to place its unit, in one 32-byte row, so that its first
// input loads wait for a single table read.
//
// Where the library chooses the plan (seg_chunks 0) and plans segments of at
// least kSpanDeviceMinSeg chunks, step 1 may lengthen the planned segment
// length once the sequence lengths are known: wavefronts 0 and 1 score up to
// 64 lengths from the planned one up, one per lane, with the placement model
// seg_span (kda_internal.h), wavefront 0 with the shorter segments in segment
// order and wavefront 1 with them longest first.  The best length and order
// are used for every table; the length is recorded in the counters and in
// every unit_tab row, the order in the counters.  The planned length sizes the
// workspace; a longer one needs fewer rows.
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int SCAN_THREADS = 1024;
constexpr int SCAN_WAVES = SCAN_THREADS / 64;
constexpr int FUSED_MAX_N = 4095;      // sequences the fused launch takes (LDS copies of the offsets)
constexpr int FUSED_MAX_ROWS = 16384;  // table rows it fills (16 per thread at most)

template <typename T, typename Op>
__device__ T block_inclusive_scan(T x, Op op, T identity, T* smem, T* block_total) {
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    T y = __shfl_up(x, o, 64);
    if (lane >= o) x = op(x, y);
  }
  if (lane == 63) smem[wid] = x;
  __syncthreads();
  if (wid == 0) {
    T w = lane < SCAN_WAVES ? smem[lane] : identity;
#pragma unroll
    for (int o = 1; o < SCAN_WAVES; o <<= 1) {
      T y = __shfl_up(w, o, 64);
      if (lane >= o) w = op(w, y);
    }
    if (lane < SCAN_WAVES) smem[lane] = w;
  }
  __syncthreads();
  T prefix = wid > 0 ? smem[wid - 1] : identity;
  *block_total = smem[SCAN_WAVES - 1];
  __syncthreads();
  return op(prefix, x);
}

struct MaxOp {
  __device__ long long operator()(long long a, long long b) const { return a > b ? a : b; }
};
struct AddOp {
  __device__ long long operator()(long long a, long long b) const { return a + b; }
};

}  // namespace

// Longest-first ranks of the N <= kLptMaxSeqs sequences into lpt_rank (LDS),
// one per thread: the key is the unit's first-pass chunks, that of the
// shorter segment for a segmented plan (-1: it has none); ties in sequence
// order.  coff: the chunk prefix sums (LDS or global, complete).
__device__ void lpt_ranks(const int* coff, int N, int seg, int K, int* lpt_key, int* lpt_rank) {
  if ((int)threadIdx.x < N) {
    const int n = coff[threadIdx.x + 1] - coff[threadIdx.x];
    lpt_key[threadIdx.x] = seg > 0 ? rest_cost(n, seg, K) : n;
  }
  __syncthreads();
  if ((int)threadIdx.x < N) {
    const int me = (int)threadIdx.x, mine = lpt_key[me];
    int rank = 0;
    for (int i = 0; i < N; ++i) {
      const int c = lpt_key[i];
      rank += c > mine || (c == mine && i < me);
    }
    lpt_rank[me] = rank;
  }
  __syncthreads();
}

// Clamped boundaries, lengths, chunk and segment prefix sums and the counters
// (step 1 of the header).  When sst/coff/soff are given (LDS, N + 1 entries
// each), the boundaries and the chunk and segment prefix sums are also kept
// there, and the lengths are computed from the LDS copy.
// Returns the segment length the tables use and sets desc to their order (1:
// longest first; the shorter segments of a segmented plan, every sequence of
// a serial one).  With may_serial (a call the
// automatic plan would keep serial, N*H >= 256 chains, whose workspace holds
// the segmented layout) the tables stay serial unless the longest sequence
// has more than 5/4 of seg_chunks: only then does splitting shorten the pass,
// whose serial span is at least the longest sequence's.  With choose set, span_cu (LDS,
// 2 x (32 + kSpanMaxSeqs) x 64 + kSpanMaxSeqs ints) and span_key (LDS, 2
// entries) serve the choice.
__device__ int index_scan_body(const int32_t* __restrict__ cu, int N, long long T_row, long long total,
                               int seg_chunks, int H, int K, bool choose, bool may_serial, Tables t,
                               long long* smem, int* flags,
                               int* sst, int* coff, int* soff, int* foff, int* span_cu,
                               unsigned long long* span_key, int& desc) {
  if (threadIdx.x == 0) *flags = 0;
  __syncthreads();
  // pass 1: boundaries b_i, i = 0..N (clamped running maximum of the offsets)
  long long carry = 0;
  for (int base = 0; base <= N; base += SCAN_THREADS) {
    const int i = base + (int)threadIdx.x;
    long long x = 0;
    if (i <= N) {
      if (cu) {
        x = cu[i];
        int f = 0;
        if (i == 0 && x != 0) f |= 1;
        if (i > 0 && x < (long long)cu[i - 1]) f |= 2;
        if (i == N && x != total) f |= 4;
        if (x < 0 || x > total) f |= 8;
        if (f) atomicOr(flags, f);
      } else {
        x = (long long)i * T_row;
      }
    }
    long long tot;
    long long run = block_inclusive_scan(x, MaxOp(), (long long)INT64_MIN, smem, &tot);
    run = run > carry ? run : carry;
    long long b = run < 0 ? 0 : (run > total ? total : run);
    if (i <= N) {
      t.seq_start[i] = (int32_t)b;
      if (sst) sst[i] = (int32_t)b;
    }
    carry = tot > carry ? tot : carry;
  }
  __threadfence_block();
  __syncthreads();
  // a split of N*H >= 256 chains leaves many shorter units, which run in
  // several rounds after the full segments: longest first packs them best
  desc = 0;
  if (may_serial && seg_chunks > 0) {
    long long max_nc = 0;
    for (int base = 0; base < N; base += SCAN_THREADS) {
      const int i = base + (int)threadIdx.x;
      long long nc = 0;
      if (i < N) {
        const long long len = sst ? (long long)sst[i + 1] - (long long)sst[i]
                                  : (long long)t.seq_start[i + 1] - (long long)t.seq_start[i];
        nc = (len + C - 1) / C;
      }
      long long tot;
      block_inclusive_scan(nc, MaxOp(), 0LL, smem, &tot);
      max_nc = tot > max_nc ? tot : max_nc;
    }
    if (4 * max_nc <= 5 * (long long)seg_chunks)
      seg_chunks = 0;
    else if (N <= kLptMaxSeqs)
      desc = 1;
  }
  // the segment length and order: lane s of wavefront w scores length
  // seg_chunks + s with the shorter segments in segment order (w = 0) or
  // longest first (w = 1); the least (span, length, order) wins
  if (choose && seg_chunks >= kSpanDeviceMinSeg && span_model_applies(seg_chunks, N, H)) {
    constexpr int kWaveInts = (32 + kSpanMaxSeqs) * 64;  // one wavefront's cu arrays, lane-interleaved
    int* nc = span_cu + 2 * kWaveInts;                     // chunks of each sequence
    if (threadIdx.x < N) {
      const int32_t* bnd = sst ? sst : t.seq_start;
      nc[threadIdx.x] = (bnd[threadIdx.x + 1] - bnd[threadIdx.x] + C - 1) / C;
    }
    __syncthreads();
    if (threadIdx.x < 128) {
      const int lane = (int)threadIdx.x & 63;
      const int w = (int)threadIdx.x >> 6;
      unsigned long long key = ~0ull;
      if (lane < span_candidates(seg_chunks)) {
        const int len = seg_chunks + lane;
        const int span = seg_span<64>(len, N, nc, H, K, w == 1, span_cu + w * kWaveInts + lane);
        key = ((unsigned long long)(unsigned)span << 32) | ((unsigned)len << 1) | (unsigned)w;
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const unsigned long long y = __shfl_xor(key, o, 64);
        key = y < key ? y : key;
      }
      if (lane == 0) span_key[w] = key;
    }
    __syncthreads();
    const unsigned long long k0 = span_key[0], k1 = span_key[1];
    const unsigned long long key = k0 < k1 ? k0 : k1;
    seg_chunks = (int)((key & 0xFFFFFFFFu) >> 1);
    desc = (int)(key & 1u);
  }
  // a serial varlen plan dispatches its sequences longest first (the chains
  // of a batch of N*H >= 256 then run in several rounds, which list scheduling
  // packs best longest first; below that every unit starts at once)
  if (seg_chunks == 0 && cu && N <= kLptMaxSeqs) desc = 1;
  // pass 2: lengths, chunk and segment counts, exclusive prefix sums
  long long c_carry = 0, s_carry = 0, f_carry = 0;
  if (threadIdx.x == 0) {
    t.seq_chunk_off[0] = 0;
    t.seq_seg_off[0] = 0;
    t.seq_full_off[0] = 0;
    if (coff) coff[0] = 0;
    if (soff) soff[0] = 0;
    if (foff) foff[0] = 0;
  }
  for (int base = 0; base < N; base += SCAN_THREADS) {
    const int i = base + (int)threadIdx.x;
    long long nc = 0, ns = 0, nf = 0;
    if (i < N) {
      const long long len = sst ? (long long)sst[i + 1] - (long long)sst[i]
                                : (long long)t.seq_start[i + 1] - (long long)t.seq_start[i];
      t.seq_len[i] = (int32_t)len;
      nc = (len + C - 1) / C;
      ns = seg_chunks > 0 ? (nc > 0 ? (nc + seg_chunks - 1) / seg_chunks : 1) : 1;
      nf = seg_chunks > 0 ? nc / seg_chunks : 1;  // serial: every sequence counts as full
    }
    long long ctot, stot, ftot;
    const long long ci = block_inclusive_scan(nc, AddOp(), 0LL, smem, &ctot);
    const long long si = block_inclusive_scan(ns, AddOp(), 0LL, smem, &stot);
    const long long fi = block_inclusive_scan(nf, AddOp(), 0LL, smem, &ftot);
    if (i < N) {
      t.seq_chunk_off[i + 1] = (int32_t)(c_carry + ci);
      t.seq_seg_off[i + 1] = (int32_t)(s_carry + si);
      t.seq_full_off[i + 1] = (int32_t)(f_carry + fi);
      if (coff) coff[i + 1] = (int32_t)(c_carry + ci);
      if (soff) soff[i + 1] = (int32_t)(s_carry + si);
      if (foff) foff[i + 1] = (int32_t)(f_carry + fi);
    }
    c_carry += ctot;
    s_carry += stot;
    f_carry += ftot;
  }
  if (threadIdx.x == 0) {
    t.counters[CNT_N_CHUNKS] = (int32_t)c_carry;
    t.counters[CNT_N_SEGS] = (int32_t)s_carry;
    t.counters[CNT_FLAGS] = *flags;
    t.counters[CNT_EARLY_STOPS] = 0;
    t.counters[CNT_SEG_CHUNKS] = seg_chunks;
    t.counters[CNT_ORDER] = desc;
  }
  return seg_chunks;
}


// largest j in [0, n) with off[j] <= x, given off[0] = 0 <= x and off non-decreasing
__device__ __forceinline__ int owner_of(const int32_t* off, int n, int x) {
  int lo = 0, hi = n;  // invariant: off[lo] <= x, answer in [lo, hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off[mid] <= x)
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}

// seg_tab row of segment idx of sequence sq, given its prefix sums
__device__ __forceinline__ void seg_row(int32_t* row, int sq, int idx, const int* coff, const int* soff,
                                        int seg_chunks) {
  const int j = idx - soff[sq];
  const int first = coff[sq];
  const int nc = coff[sq + 1] - first;
  int r1, r2;
  if (seg_chunks > 0) {
    const long long b0 = (long long)j * seg_chunks;
    const long long e0 = b0 + seg_chunks;
    r1 = first + (int)(b0 < nc ? b0 : nc);
    r2 = first + (int)(e0 < nc ? e0 : nc);
  } else {
    r1 = first;
    r2 = first + nc;
  }
  row[0] = sq;
  row[1] = r1;
  row[2] = r2;
  row[3] = j;
}

// Puts segment idx (seg_tab row `row`) into the dispatch table at its rank:
// the full-length segments in segment order, then the others (a sequence's
// shorter last segment, or a sequence shorter than seg) in segment order or,
// with desc, longest first by rest_cost (ties in segment order; desc is only
// chosen for at most kLptMaxSeqs sequences, so the count below is short).
// A serial plan (seg 0) has one unit per sequence: in sequence order, or with
// desc (at most kLptMaxSeqs sequences) longest first, ties in sequence order.
// lpt_rank, where given, holds each sequence's longest-first rank (that of its
// shorter segment, for a segmented plan); else the rank is counted here.
__device__ __forceinline__ void put_unit(int32_t* unit_tab, int idx, const int32_t* row, const int* coff,
                                         const int* soff, const int* foff, int N, int n_full, int seq_start,
                                         int seq_len, int seg, int K, int desc, const int* lpt_rank) {
  const int sq = row[0], j = row[3];
  const int full_here = foff[sq + 1] - foff[sq];
  if (seg == 0 && desc) {
    int rank = 0;
    if (lpt_rank) {
      rank = lpt_rank[sq];
    } else {
      const int mine = coff[sq + 1] - coff[sq];
      for (int i = 0; i < N; ++i) {
        const int c = coff[i + 1] - coff[i];
        rank += c > mine || (c == mine && i < sq);
      }
    }
    int32_t* u = unit_tab + 8 * rank;
    u[0] = idx;
    u[1] = row[0];
    u[2] = row[1];
    u[3] = row[2];
    u[4] = row[3];
    u[5] = seq_start;
    u[6] = seq_len;
    u[7] = 0;
    return;
  }
  int rest_rank = soff[sq] - foff[sq];  // shorter segments of the sequences before this one
  if (desc && j >= full_here && lpt_rank) {
    rest_rank = lpt_rank[sq];
  } else if (desc && j >= full_here) {
    const int mine = rest_cost(coff[sq + 1] - coff[sq], seg, K);
    rest_rank = 0;
    for (int i = 0; i < N; ++i) {
      const int c = rest_cost(coff[i + 1] - coff[i], seg, K);
      rest_rank += c > mine || (c == mine && i < sq);  // c = -1 (no shorter segment) never counts
    }
  }
  const int rank = j < full_here ? foff[sq] + j : n_full + rest_rank;
  int32_t* u = unit_tab + 8 * rank;
  u[0] = idx;
  u[1] = row[0];
  u[2] = row[1];
  u[3] = row[2];
  u[4] = row[3];
  u[5] = seq_start;
  u[6] = seq_len;
  u[7] = seg;
}

__global__ __launch_bounds__(SCAN_THREADS) void kda_index_scan(const int32_t* __restrict__ cu, int N, long long T_row,
                                                               long long total, int seg_chunks, int H, int K,
                                                               int choose, int may_serial, Tables t) {
  __shared__ long long smem[SCAN_WAVES];
  __shared__ int flags;
  __shared__ int span_cu[2 * (32 + kSpanMaxSeqs) * 64 + kSpanMaxSeqs];
  __shared__ unsigned long long span_key[2];
  __shared__ int lpt_key[kLptMaxSeqs], lpt_rank[kLptMaxSeqs];
  int desc;
  seg_chunks = index_scan_body(cu, N, T_row, total, seg_chunks, H, K, choose != 0, may_serial != 0, t, smem, &flags,
                               nullptr, nullptr, nullptr, nullptr, span_cu, span_key, desc);
  if (!desc) return;
  // the longest-first rows, one thread per sequence; kda_index_fill writes
  // the others (the prefix sums were stored by this workgroup above)
  __threadfence_block();
  __syncthreads();
  lpt_ranks(t.seq_chunk_off, N, seg_chunks, K, lpt_key, lpt_rank);
  const int sq = (int)threadIdx.x;
  if (sq < N) {
    const int ns = t.seq_seg_off[sq + 1] - t.seq_seg_off[sq];
    const int nf = t.seq_full_off[sq + 1] - t.seq_full_off[sq];
    if (seg_chunks == 0 || ns > nf) {  // a serial unit, or this sequence's shorter segment
      const int idx = t.seq_seg_off[sq + 1] - 1;
      int32_t row[4];
      seg_row(row, sq, idx, t.seq_chunk_off, t.seq_seg_off, seg_chunks);
      put_unit(t.unit_tab, idx, row, t.seq_chunk_off, t.seq_seg_off, t.seq_full_off, N, t.seq_full_off[N],
               t.seq_start[sq], t.seq_len[sq], seg_chunks, K, desc, lpt_rank);
    }
  }
}

__global__ __launch_bounds__(256) void kda_index_fill(int N, int K, long long max_chunks, long long max_segs,
                                                      Tables t) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int n_chunks = t.counters[CNT_N_CHUNKS];
  const int n_segs = t.counters[CNT_N_SEGS];
  const int seg_chunks = t.counters[CNT_SEG_CHUNKS];  // the length and order kda_index_scan chose
  const int desc = t.counters[CNT_ORDER];
  if (idx < max_chunks) {
    int a = -1, b = -1;
    if (idx < n_chunks) {
      // the owning sequence is the last one whose first chunk is <= idx
      a = owner_of(t.seq_chunk_off, N + 1, (int)idx);
      // skip empty sequences that share the same first chunk
      while (a + 1 <= N && t.seq_chunk_off[a + 1] <= (int)idx) ++a;
      b = (int)idx - t.seq_chunk_off[a];
    }
    t.chunk_tab[2 * idx] = a;
    t.chunk_tab[2 * idx + 1] = b;
  }
  if (idx < max_segs) {
    int32_t row[4] = {-1, -1, -1, -1};
    if (idx < n_segs) {
      int s = owner_of(t.seq_seg_off, N + 1, (int)idx);
      while (s + 1 <= N && t.seq_seg_off[s + 1] <= (int)idx) ++s;
      seg_row(row, s, (int)idx, t.seq_chunk_off, t.seq_seg_off, seg_chunks);
      // with desc, kda_index_scan wrote the longest-first rows (a serial
      // plan's, or the shorter segments)
      if (!desc || (seg_chunks > 0 && row[3] < t.seq_full_off[s + 1] - t.seq_full_off[s]))
        put_unit(t.unit_tab, (int)idx, row, t.seq_chunk_off, t.seq_seg_off, t.seq_full_off, N, t.seq_full_off[N],
                 t.seq_start[s], t.seq_len[s], seg_chunks, K, desc, nullptr);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) t.unit_tab[8 * idx + k] = -1;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) t.seg_tab[4 * idx + k] = row[k];
  }
}

// Both steps in one workgroup.  Thread t fills a contiguous range of table
// rows: one binary search in the LDS copy of the prefix sums for its first
// row, then a forward walk (the owner of consecutive rows never decreases).
__global__ __launch_bounds__(SCAN_THREADS) void kda_index_fused(const int32_t* __restrict__ cu, int N, long long T_row,
                                                                long long total, int seg_chunks, int H, int K,
                                                                int choose, int may_serial, int max_chunks,
                                                                int max_segs, Tables t) {
  __shared__ long long smem[SCAN_WAVES];
  __shared__ int flags;
  __shared__ int sst[FUSED_MAX_N + 1], coff[FUSED_MAX_N + 1], soff[FUSED_MAX_N + 1], foff[FUSED_MAX_N + 1];
  __shared__ int span_cu[2 * (32 + kSpanMaxSeqs) * 64 + kSpanMaxSeqs];
  __shared__ unsigned long long span_key[2];
  int desc;
  seg_chunks = index_scan_body(cu, N, T_row, total, seg_chunks, H, K, choose != 0, may_serial != 0, t, smem, &flags,
                               sst, coff, soff, foff, span_cu, span_key, desc);
  __syncthreads();
  // longest-first ranks, once per sequence (desc is set for at most
  // kLptMaxSeqs sequences): the key is the unit's first-pass chunks, that of
  // the shorter segment for a segmented plan (-1: it has none)
  __shared__ int lpt_key[kLptMaxSeqs], lpt_rank[kLptMaxSeqs];
  if (desc) lpt_ranks(coff, N, seg_chunks, K, lpt_key, lpt_rank);
  const int n_chunks = coff[N], n_segs = soff[N];
  {
    const int per = (max_chunks + SCAN_THREADS - 1) / SCAN_THREADS;
    const int r0 = (int)threadIdx.x * per;
    const int r1 = min(r0 + per, max_chunks);
    int a = r0 < n_chunks ? owner_of(coff, N + 1, r0) : 0;
    for (int r = r0; r < r1; ++r) {
      int x = -1, y = -1;
      if (r < n_chunks) {
        while (a + 1 <= N && coff[a + 1] <= r) ++a;  // also skips empty sequences
        x = a;
        y = r - coff[a];
      }
      t.chunk_tab[2 * r] = x;
      t.chunk_tab[2 * r + 1] = y;
    }
  }
  {
    const int per = (max_segs + SCAN_THREADS - 1) / SCAN_THREADS;
    const int r0 = (int)threadIdx.x * per;
    const int r1 = min(r0 + per, max_segs);
    int a = r0 < n_segs ? owner_of(soff, N + 1, r0) : 0;
    for (int r = r0; r < r1; ++r) {
      int32_t row[4] = {-1, -1, -1, -1};
      if (r < n_segs) {
        while (a + 1 <= N && soff[a + 1] <= r) ++a;
        seg_row(row, a, r, coff, soff, seg_chunks);
        put_unit(t.unit_tab, r, row, coff, soff, foff, N, foff[N], sst[a], sst[a + 1] - sst[a], seg_chunks, K, desc,
                 desc ? lpt_rank : nullptr);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) t.unit_tab[8 * r + k] = -1;
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) t.seg_tab[4 * r + k] = row[k];
    }
  }
}

// Every table of a fixed-length call (N sequences of T tokens) from its
// closed form, one thread per row; the rows kda_fwd's kernels compute
// without storing them.
__global__ __launch_bounds__(256) void kda_index_fixed(int N, int L, int seg, Tables t) {
  const int tid = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (tid == 0) fixed_counters(N, L, seg, t);
  fixed_tables(tid, (int)(gridDim.x * blockDim.x), N, L, seg, t);
}

hipError_t launch_index_fixed(int N, int L, int seg, Tables t, hipStream_t st) {
  long long rows = t.max_chunks > t.max_segs ? t.max_chunks : t.max_segs;
  if (rows < N + 1) rows = N + 1;
  long long blocks = (rows + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(kda_index_fixed, dim3((unsigned)blocks), dim3(256), 0, st, N, L, seg, t);
  return hipGetLastError();
}

hipError_t launch_index(const int32_t* cu_seqlens, int N, int64_t T_row, int64_t total_tokens, int seg_chunks,
                        int H, int K, bool choose, bool may_serial, int64_t max_chunks, int64_t max_segs, Tables t,
                        hipStream_t st) {
  if (!cu_seqlens) return hipSuccess;  // fixed length: written by the first chunk-kernel launch
  if (N <= FUSED_MAX_N && max_chunks <= FUSED_MAX_ROWS && max_segs <= FUSED_MAX_ROWS) {
    hipEvent_t e0, e1;
    stage_events(KDA_STAGE_INDEX, &e0, &e1);
    hipExtLaunchKernelGGL(kda_index_fused, dim3(1), dim3(SCAN_THREADS), 0, st, e0, e1, 0, cu_seqlens, N,
                          (long long)T_row, (long long)total_tokens, seg_chunks, H, K, (int)choose, (int)may_serial,
                          (int)max_chunks, (int)max_segs, t);
    return hipGetLastError();
  }
  hipEvent_t e0, e1;
  stage_events(KDA_STAGE_INDEX, &e0, &e1);
  hipExtLaunchKernelGGL(kda_index_scan, dim3(1), dim3(SCAN_THREADS), 0, st, e0, e1, 0, cu_seqlens, N,
                        (long long)T_row, (long long)total_tokens, seg_chunks, H, K, (int)choose, (int)may_serial, t);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long rows = max_chunks > max_segs ? max_chunks : max_segs;
  if (rows > 0) {
    const unsigned blocks = (unsigned)((rows + 255) / 256);
    stage_events(KDA_STAGE_INDEX, &e0, &e1);
    hipExtLaunchKernelGGL(kda_index_fill, dim3(blocks), dim3(256), 0, st, e0, e1, 0, N, K, (long long)max_chunks,
                          (long long)max_segs, t);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace kda
