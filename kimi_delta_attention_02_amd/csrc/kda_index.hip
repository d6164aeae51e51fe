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
// Two launches, both free of host synchronisation:
//  1. kda_index_scan (one 1024-thread workgroup): clamps the offsets into a
//     non-decreasing sequence within [0, total], then prefix-sums the chunk
//     and segment counts.  Tables: seq_start[N+1], seq_len[N],
//     seq_chunk_off[N+1], seq_seg_off[N+1], counters {n_chunks, n_segs, flags}.
//  2. kda_index_fill: one thread per table row; binary search of the prefix
//     sums gives chunk_tab[c] = (seq, chunk in seq) and
//     seg_tab[s] = (seq, first chunk, end chunk, segment in seq).  Rows past
//     the live counts are filled with -1.
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int SCAN_THREADS = 1024;
constexpr int SCAN_WAVES = SCAN_THREADS / 64;

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

__global__ __launch_bounds__(SCAN_THREADS) void kda_index_scan(const int32_t* __restrict__ cu, int N, long long T_row,
                                                               long long total, int seg_chunks, Tables t) {
  __shared__ long long smem[SCAN_WAVES];
  __shared__ int flags;
  if (threadIdx.x == 0) flags = 0;
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
        if (f) atomicOr(&flags, f);
      } else {
        x = (long long)i * T_row;
      }
    }
    long long tot;
    long long run = block_inclusive_scan(x, MaxOp(), (long long)INT64_MIN, smem, &tot);
    run = run > carry ? run : carry;
    long long b = run < 0 ? 0 : (run > total ? total : run);
    if (i <= N) t.seq_start[i] = (int32_t)b;
    carry = tot > carry ? tot : carry;
  }
  __threadfence_block();
  __syncthreads();
  // pass 2: lengths, chunk and segment counts, exclusive prefix sums
  long long c_carry = 0, s_carry = 0;
  if (threadIdx.x == 0) {
    t.seq_chunk_off[0] = 0;
    t.seq_seg_off[0] = 0;
  }
  for (int base = 0; base < N; base += SCAN_THREADS) {
    const int i = base + (int)threadIdx.x;
    long long nc = 0, ns = 0;
    if (i < N) {
      const long long len = (long long)t.seq_start[i + 1] - (long long)t.seq_start[i];
      t.seq_len[i] = (int32_t)len;
      nc = (len + C - 1) / C;
      ns = seg_chunks > 0 ? (nc > 0 ? (nc + seg_chunks - 1) / seg_chunks : 1) : 1;
    }
    long long ctot, stot;
    const long long ci = block_inclusive_scan(nc, AddOp(), 0LL, smem, &ctot);
    const long long si = block_inclusive_scan(ns, AddOp(), 0LL, smem, &stot);
    if (i < N) {
      t.seq_chunk_off[i + 1] = (int32_t)(c_carry + ci);
      t.seq_seg_off[i + 1] = (int32_t)(s_carry + si);
    }
    c_carry += ctot;
    s_carry += stot;
  }
  if (threadIdx.x == 0) {
    t.counters[CNT_N_CHUNKS] = (int32_t)c_carry;
    t.counters[CNT_N_SEGS] = (int32_t)s_carry;
    t.counters[CNT_FLAGS] = flags;
    t.counters[3] = 0;
  }
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

__global__ __launch_bounds__(256) void kda_index_fill(int N, int seg_chunks, long long max_chunks, long long max_segs,
                                                      Tables t) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int n_chunks = t.counters[CNT_N_CHUNKS];
  const int n_segs = t.counters[CNT_N_SEGS];
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
    int r0 = -1, r1 = -1, r2 = -1, r3 = -1;
    if (idx < n_segs) {
      int s = owner_of(t.seq_seg_off, N + 1, (int)idx);
      while (s + 1 <= N && t.seq_seg_off[s + 1] <= (int)idx) ++s;
      const int j = (int)idx - t.seq_seg_off[s];
      const int first = t.seq_chunk_off[s];
      const int nc = t.seq_chunk_off[s + 1] - first;
      r0 = s;
      r3 = j;
      if (seg_chunks > 0) {
        const long long b0 = (long long)j * seg_chunks;
        const long long e0 = b0 + seg_chunks;
        r1 = first + (int)(b0 < nc ? b0 : nc);
        r2 = first + (int)(e0 < nc ? e0 : nc);
      } else {
        r1 = first;
        r2 = first + nc;
      }
    }
    t.seg_tab[4 * idx + 0] = r0;
    t.seg_tab[4 * idx + 1] = r1;
    t.seg_tab[4 * idx + 2] = r2;
    t.seg_tab[4 * idx + 3] = r3;
  }
}

hipError_t launch_index(const int32_t* cu_seqlens, int N, int64_t T_row, int64_t total_tokens, int seg_chunks,
                        int64_t max_chunks, int64_t max_segs, Tables t, hipStream_t st) {
  hipLaunchKernelGGL(kda_index_scan, dim3(1), dim3(SCAN_THREADS), 0, st, cu_seqlens, N, (long long)T_row,
                     (long long)total_tokens, seg_chunks, t);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long rows = max_chunks > max_segs ? max_chunks : max_segs;
  if (rows > 0) {
    const unsigned blocks = (unsigned)((rows + 255) / 256);
    hipLaunchKernelGGL(kda_index_fill, dim3(blocks), dim3(256), 0, st, N, seg_chunks, (long long)max_chunks,
                       (long long)max_segs, t);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace kda
