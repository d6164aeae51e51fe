// Segment merge ("merge" on the cuLA PR #106 page: K1 once -> pre_scan ->
// merge -> segment K2).
//
// For every sequence with n >= 3 segments, the state entering segment i+1 is
// S_{i+1} = M_i S_i + R_i for i = 1 .. n-2, in fp32, where (M_i, R_i) is the
// exact affine map of middle segment i produced by the pre-scan and S_1 was
// written by the recurrence over segment 0.  Value columns are independent, so
// each workgroup owns 16 of them and walks the segments of its sequence in
// order; the products use v_mfma_f32_16x16x4_f32.  Column blocks of M_i that
// underflowed to exactly zero are skipped (the pre-scan flags them and does not
// store them); when all are zero S_{i+1} = R_i exactly: the merge writes nothing
// for that boundary and the segment pass starts from R_i.  That equality is what
// makes the segmented path reproduce the serial bits once the zero-start chain
// has converged.
//
// All matrices are stored transposed ([v][k], like the state tensors).
#include "kda_internal.h"

namespace kda {

namespace {
constexpr int SP = 17;  // LDS pitch of the 128 x 16 column block
}

__global__ __launch_bounds__(256) void kda_merge_kernel(Problem p, Tables t, const float* __restrict__ segM,
                                                        const float* __restrict__ segR, float* __restrict__ segS,
                                                        const int32_t* __restrict__ segMnz) {
  __shared__ float Sl[D * SP];
  const int seq = blockIdx.x;
  const int h = blockIdx.y;
  const int vb = blockIdx.z;  // 16-column block
  const int s0 = t.seq_seg_off[seq];
  const int ns = t.seq_seg_off[seq + 1] - s0;
  if (ns < 3) return;
  const int H = p.H;
  const int w = threadIdx.x >> 6;
  const int L = threadIdx.x & 63;
  const int g = L >> 4;
  const int c = L & 15;
  const int v = 16 * vb + c;
  const long long mat = (long long)D * D;

  // column block vb of a [v][k] matrix -> Sl[k][v - 16 vb]
  auto to_lds = [&](const float* src) {
    for (int e = threadIdx.x; e < D * 16; e += 256) {
      const int k = e & (D - 1);
      const int vv = e >> 7;
      Sl[k * SP + vv] = src[(long long)(16 * vb + vv) * D + k];
    }
  };

  // Sl holds S_i when `have` is true.  When M_i is zero, S_{i+1} = R_i: nothing
  // is computed or written, and the segment pass reads R_i as its start state.
  // The nonzero masks of 256 boundaries at a time are read in parallel first:
  // bit b set when the 16-row block b of the reduction index (columns of M) is
  // nonzero (the pre-scan leaves zero blocks unstored).
  __shared__ uint32_t nzl[256];
  bool have = false;
  for (int i = 1; i <= ns - 2; ++i) {
    if ((i - 1) % 256 == 0) {
      __syncthreads();
      const int ii = i + (int)threadIdx.x;
      uint32_t m = 0;
      if (ii <= ns - 2) {
        const int32_t* f = segMnz + ((long long)(s0 + ii) * H + h) * (D / 16);
#pragma unroll
        for (int b = 0; b < D / 16; ++b) m |= (f[b] != 0 ? 1u : 0u) << b;
      }
      nzl[threadIdx.x] = m;
      __syncthreads();
    }
    const uint32_t nz = nzl[(i - 1) % 256];
    const long long base = ((long long)(s0 + i) * H + h) * mat;
    if (nz == 0) {
      have = false;
      continue;
    }
    if (!have) {  // S_i: the recurrence's output for segment 0, or R_{i-1}
      to_lds(i == 1 ? segS + ((long long)(s0 + 1) * H + h) * mat
                    : segR + ((long long)(s0 + i - 1) * H + h) * mat);
      __syncthreads();
    }
    const float* Mt = segM + base;  // Mt[p][k] = M[k][p]
    const float* Rt = segR + base;
    f32x4 acc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int to = 2 * w + u;  // output row tile
      acc[u] = *reinterpret_cast<const f32x4*>(Rt + (long long)v * D + 16 * to + 4 * g);
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        if (!((nz >> tt) & 1u)) continue;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int pr = 16 * tt + 4 * g + ii;  // reduction index supplied by lane group g
          acc[u] = mfma_f32_k4(Mt[(long long)pr * D + 16 * to + c], Sl[pr * SP + c], acc[u]);
        }
      }
    }
    __syncthreads();
    float* dst = segS + ((long long)(s0 + i + 1) * H + h) * mat;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int to = 2 * w + u;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) Sl[(16 * to + 4 * g + ii) * SP + c] = acc[u][ii];
      *reinterpret_cast<f32x4*>(dst + (long long)v * D + 16 * to + 4 * g) = acc[u];
    }
    __syncthreads();
    have = true;
  }
}

hipError_t launch_merge(const Problem& p, Tables t, const Seg& sg, hipStream_t st) {
  if (p.N <= 0) return hipSuccess;
  hipEvent_t e0, e1;
  stage_events(KDA_STAGE_MERGE, &e0, &e1);
  hipExtLaunchKernelGGL(kda_merge_kernel, dim3((unsigned)p.N, (unsigned)p.H, D / 16), dim3(256), 0, st, e0, e1, 0,
                        p, t, (const float*)sg.M, (const float*)sg.R, sg.S, (const int32_t*)sg.mnz);
  return hipGetLastError();
}

}  // namespace kda
