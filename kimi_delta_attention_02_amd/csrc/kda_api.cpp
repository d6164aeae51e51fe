// Host side of the C ABI declared in include/kda.h: argument validation,
// segment planning, workspace carving and the launch sequence.
//
// Launch sequence of one kda_fwd call, all on the caller's stream, with no
// host synchronisation, allocation or device-to-host copy:
//   index scan + table fill (varlen; a fixed-length call has none: the first
//   chunk-kernel launch writes its tables, whose closed form every block uses)
//   -> chunk kernel, first pass: chunk prep fused with the recurrence of whole
//      sequences / first segments from the initial state, and of segments >= 1
//      from a zero state (their transitions M while nonzero, their output
//      after the first kCheckChunks chunks, a checkpoint of the state there)
//   [-> chunk kernel, second pass: each block merges its segment's start state
//      (S_j = M_{j-1} S_{j-1} + R_{j-1}, walking back only over nonzero M), then
//      redoes the first kCheckChunks chunks of segments >= 1 from it, continued
//      to the segment's end only where the state differs from the checkpoint]
// The bracketed part runs only when the plan splits sequences into segments.
// It follows the segment scheme on the cuLA PR #106 page (pre-scan, merge,
// segment recurrence), with three changes: chunk prep is recomputed in each
// pass from the inputs rather than stored once (a stored prep record is larger
// than the inputs it is computed from); the zero-start pass also produces the
// output, so that the second pass only redoes a segment's first chunks where
// the start state's influence has decayed to nothing in fp32 by then; and the
// merge runs inside the second pass, so a call whose maps M are all zero
// launches no merge at all.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kda_internal.h"

namespace {

thread_local std::string g_last_error;

int32_t fail(int32_t status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

constexpr int64_t kMaxTokens = (int64_t)INT32_MAX - 16;  // tables are int32
constexpr int kTargetUnits = 256;   // (segment, head) units the automatic plan aims for: one per CU
constexpr int kMinSegChunks = 16;   // shortest automatic segment (256 tokens)
constexpr int kCheckChunks = 4;     // chunks the second pass redoes before comparing with the checkpoint
constexpr int kSerialChains = 256;  // chains that already fill the chip without splitting
#ifndef KDA_WIDE_MIN_CHUNKS
#define KDA_WIDE_MIN_CHUNKS 128
#endif
constexpr int kWideMinChunks = KDA_WIDE_MIN_CHUNKS;  // units at least this long (on average) run the 4-consumer kernel

// ---- optional per-kernel event timing (benchmarks) ----
struct Profiler {
  bool on = false;     // kernel events
  bool host = false;   // host time of each forward call
  double host_us = 0.0;
  int64_t host_calls = 0;
  std::vector<hipEvent_t> pool;
  struct Rec {
    int stage;
    hipEvent_t a, b;
  };
  std::vector<Rec> recs;
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    // timing only: no system-scope fence (an L2 write-back and invalidate)
    // when the event is reached, which would lengthen the kernel it times
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
    return e;
  }
};
thread_local Profiler g_prof;

// Adds the host time from construction to destruction to the profiler while
// host timing is on (every return path of a forward call).
struct HostTimer {
  bool on;
  std::chrono::steady_clock::time_point t0;
  HostTimer() : on(g_prof.host) {
    if (on) t0 = std::chrono::steady_clock::now();
  }
  ~HostTimer() {
    if (!on) return;
    g_prof.host_us += std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t0).count();
    g_prof.host_calls += 1;
  }
};

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

int64_t max_chunks_for(int64_t total, int32_t N) {
  // sum_i ceil(len_i / 16) <= (sum_i len_i + 15 N) / 16 for lengths summing to total
  return (total + 15 * (int64_t)N) / kda::C;
}

// A number for each call, written into the sync words of its segments: words
// an earlier call left in a workspace then never match the current call's.
// Zero is skipped, since fresh memory often holds zeros.
uint32_t next_epoch() {
  static std::atomic<uint32_t> counter{0};
  uint32_t e = counter.fetch_add(1, std::memory_order_relaxed) + 1;
  if (e == 0) e = counter.fetch_add(1, std::memory_order_relaxed) + 1;
  return e;
}

// segment length in chunks (0 = serial); negative status on bad arguments
int32_t plan(int64_t total, int32_t H, int32_t N, int32_t cp_mode, int32_t seg_chunks) {
  if (total < 0 || total > kMaxTokens) return fail(KDA_ERR_INVALID_ARG, "total_tokens %lld out of range", (long long)total);
  if (H < 1 || H > 65535) return fail(KDA_ERR_INVALID_ARG, "num_heads %d out of range [1, 65535]", H);
  if (N < 1) return fail(KDA_ERR_INVALID_ARG, "num_seqs %d must be >= 1", N);
  if (cp_mode < KDA_CP_AUTO || cp_mode > KDA_CP_FORCE) return fail(KDA_ERR_INVALID_ARG, "cp_mode %d invalid", cp_mode);
  if (seg_chunks < 0) return fail(KDA_ERR_INVALID_ARG, "seg_chunks %d must be >= 0", seg_chunks);
  if (cp_mode == KDA_CP_OFF) return 0;
  if (seg_chunks > 0) return seg_chunks;
  // the work in chunks: ceil(total / 16), what equal-length sequences give
  // (the tables are sized for the worst split, max_chunks_for)
  const int64_t mc = (total + kda::C - 1) / kda::C;
  int64_t seg = (mc * H + kTargetUnits - 1) / kTargetUnits;
  if (seg < kMinSegChunks) seg = kMinSegChunks;
  if (cp_mode == KDA_CP_FORCE) return (int32_t)seg;
  // automatic: keep serial when the chains already fill the chip or the
  // sequences are too short for the pre-scan and merge to pay off
  if ((int64_t)N * H >= kSerialChains) return 0;
  if (mc < 8 * seg) return 0;
  return (int32_t)seg;
}

struct Layout {
  int64_t off[KDA_WS_NUM_OFFSETS];
  int32_t seg;
};

// The segment length of a fixed-length call (N sequences of T tokens): the
// planned one, or, where the library chooses the plan (choose), the length
// from seg .. seg + min(seg/4, 63) that the placement model seg_span predicts
// fastest (the varlen index kernel makes the same choice on the device).  The
// last shape's answer is kept per host thread.
int32_t fixed_seg(int32_t seg, int32_t N, int64_t T, int32_t H, bool choose) {
  if (!choose || !kda::span_model_applies(seg, N, H)) return seg;
  struct Memo {
    int32_t seg = -1, N = 0, H = 0, out = 0;
    int64_t T = -1;
  };
  thread_local Memo m;
  if (m.seg == seg && m.N == N && m.H == H && m.T == T) return m.out;
  int nc[kda::kSpanMaxSeqs];
  for (int32_t i = 0; i < N; ++i) nc[i] = (int)((T + kda::C - 1) / kda::C);
  int cu[32 + kda::kSpanMaxSeqs];
  int best = INT32_MAX;
  int32_t out = seg;
  for (int c = 0; c < kda::span_candidates(seg); ++c) {
    const int span = kda::seg_span<1>(seg + c, N, nc, H, kCheckChunks, false, cu);  // equal lengths: one order
    if (span < best) {
      best = span;
      out = seg + c;
    }
  }
  m.seg = seg;
  m.N = N;
  m.H = H;
  m.T = T;
  m.out = out;
  return out;
}

int32_t layout(int64_t total, int32_t H, int32_t N, int32_t cp_mode, int32_t seg_chunks, Layout* out) {
  const int32_t seg = plan(total, H, N, cp_mode, seg_chunks);
  if (seg < 0) return seg;
  const int64_t mc = max_chunks_for(total, N);
  const int64_t ms = seg > 0 ? mc / seg + N : N;
  if (mc > INT32_MAX / 2 || ms > INT32_MAX / 2 || ms * H > INT32_MAX)
    return fail(KDA_ERR_INVALID_ARG, "problem too large for the index tables");
  const int64_t A = KDA_WORKSPACE_ALIGN;
  int64_t o = 0;
  auto take = [&](int idx, int64_t bytes) {
    out->off[idx] = o;
    o = align_up(o + bytes, A);
  };
  take(KDA_WS_COUNTERS, 4 * 6);
  take(KDA_WS_SEQ_START, 4 * ((int64_t)N + 1));
  take(KDA_WS_SEQ_LEN, 4 * (int64_t)N);
  take(KDA_WS_SEQ_CHUNK_OFF, 4 * ((int64_t)N + 1));
  take(KDA_WS_SEQ_SEG_OFF, 4 * ((int64_t)N + 1));
  take(KDA_WS_CHUNK_TAB, 8 * mc);
  take(KDA_WS_SEG_TAB, 16 * ms);
  const int64_t seg_bytes = seg > 0 ? ms * H * (int64_t)kda::D * kda::D * 4 : 0;
  take(KDA_WS_SEG_M, seg_bytes);
  take(KDA_WS_SEG_R, seg_bytes);
  take(KDA_WS_SEG_S, seg_bytes);
  take(KDA_WS_SEG_MNZ, seg > 0 ? ms * H * (kda::D / 16) * 4 : 0);
  take(KDA_WS_SEG_CHK, seg_bytes);
  take(KDA_WS_SEQ_FULL_OFF, 4 * ((int64_t)N + 1));
  take(KDA_WS_UNIT_TAB, 32 * ms);
  take(KDA_WS_SEG_FIX, seg_bytes);
  take(KDA_WS_SEG_SYNC, seg > 0 ? ms * H * 16 * 4 : 0);
  out->off[KDA_WS_MAX_CHUNKS] = mc;
  out->off[KDA_WS_MAX_SEGS] = ms;
  out->off[KDA_WS_TOTAL] = o;
  out->seg = seg;
  return KDA_OK;
}

}  // namespace

namespace kda {

void stage_events(int stage, hipEvent_t* start, hipEvent_t* stop) {
  *start = *stop = nullptr;
  if (!g_prof.on) return;
  hipEvent_t a = g_prof.get();
  if (!a) return;
  hipEvent_t b = g_prof.get();
  if (!b) {
    g_prof.pool.push_back(a);
    return;
  }
  g_prof.recs.push_back({stage, a, b});
  *start = a;
  *stop = b;
}

}  // namespace kda

// Tables carved from a workspace of layout lay; fixed_T >= 0 marks a
// fixed-length call of that many tokens per sequence, -1 a varlen one.
kda::Tables carve_tables(uint8_t* ws, const Layout& lay, int64_t fixed_T) {
  kda::Tables t;
  t.counters = reinterpret_cast<int32_t*>(ws + lay.off[KDA_WS_COUNTERS]);
  t.seq_start = reinterpret_cast<int32_t*>(ws + lay.off[KDA_WS_SEQ_START]);
  t.seq_len = reinterpret_cast<int32_t*>(ws + lay.off[KDA_WS_SEQ_LEN]);
  t.seq_chunk_off = reinterpret_cast<int32_t*>(ws + lay.off[KDA_WS_SEQ_CHUNK_OFF]);
  t.seq_seg_off = reinterpret_cast<int32_t*>(ws + lay.off[KDA_WS_SEQ_SEG_OFF]);
  t.chunk_tab = reinterpret_cast<int32_t*>(ws + lay.off[KDA_WS_CHUNK_TAB]);
  t.seg_tab = reinterpret_cast<int32_t*>(ws + lay.off[KDA_WS_SEG_TAB]);
  t.seq_full_off = reinterpret_cast<int32_t*>(ws + lay.off[KDA_WS_SEQ_FULL_OFF]);
  t.unit_tab = reinterpret_cast<int32_t*>(ws + lay.off[KDA_WS_UNIT_TAB]);
  t.fixed = fixed_T >= 0;
  t.fixed_T = fixed_T >= 0 ? (int)fixed_T : 0;
  t.max_chunks = lay.off[KDA_WS_MAX_CHUNKS];
  t.max_segs = lay.off[KDA_WS_MAX_SEGS];
  return t;
}

namespace {

// The arguments of one forward call, as kda_fwd receives them.
struct FwdArgs {
  const void *q, *k, *v, *g, *beta;
  float scale;
  void* out;
  const float *A_log, *dt_bias;
  float lower_bound;
  const void* initial_state;
  void* final_state;
  int32_t state_dtype, state_layout;
  const int32_t* cu_seqlens;
  int32_t num_seqs, B;
  int64_t T;
  int32_t H, H_qk, D, cp_mode, seg_chunks;
};

struct Prepared {
  Layout lay;
  // A varlen call on the automatic plan that keeps N*H >= 256 chains serial
  // may split a sequence much longer than the others when its workspace also
  // holds the segmented layout (split_lay, that of KDA_CP_FORCE): the index
  // kernel then decides from the lengths (may_serial).
  Layout split_lay;
  bool can_split = false, may_serial = false;
  int32_t N = 0, H_qk = 0;
  int64_t total = 0;
  bool nothing = false;  // a valid call with nothing to launch
};

// Takes the segmented layout when a call that may split has room for it.
void choose_layout(Prepared* pr, int64_t room) {
  if (pr->can_split && room >= pr->split_lay.off[KDA_WS_TOTAL]) {
    pr->lay = pr->split_lay;
    pr->may_serial = true;
  }
}

// Every check of a forward call that needs no workspace, before any HIP call.
int32_t prepare(const FwdArgs& a, Prepared* pr) {
  if (a.D != kda::D) return fail(KDA_ERR_UNSUPPORTED, "head dimension %d unsupported (only 128)", a.D);
  if (a.B < 0 || a.T < 0) return fail(KDA_ERR_INVALID_ARG, "B=%d and T=%lld must be >= 0", a.B, (long long)a.T);
  if (a.H < 1) return fail(KDA_ERR_INVALID_ARG, "H=%d must be >= 1", a.H);
  const int32_t H_qk = a.H_qk == 0 ? a.H : a.H_qk;
  if (H_qk < 1 || H_qk > a.H || a.H % H_qk != 0)
    return fail(KDA_ERR_INVALID_ARG, "H_qk=%d must divide H=%d", H_qk, a.H);
  if (a.T > 0 && a.B > kMaxTokens / a.T) return fail(KDA_ERR_INVALID_ARG, "B*T too large");
  const int64_t total = (int64_t)a.B * a.T;
  if (!(a.lower_bound >= -5.0f && a.lower_bound <= 0.0f))
    return fail(KDA_ERR_INVALID_ARG, "lower_bound %g outside [-5, 0]", (double)a.lower_bound);
  if (!std::isfinite(a.scale)) return fail(KDA_ERR_INVALID_ARG, "scale must be finite");
  if (a.state_dtype != KDA_STATE_BF16 && a.state_dtype != KDA_STATE_FP32)
    return fail(KDA_ERR_INVALID_ARG, "state_dtype %d invalid", a.state_dtype);
  if (a.state_layout != KDA_STATE_VK && a.state_layout != KDA_STATE_KV)
    return fail(KDA_ERR_INVALID_ARG, "state_layout %d invalid", a.state_layout);
  int32_t N;
  if (a.cu_seqlens) {
    if (a.B != 1) return fail(KDA_ERR_INVALID_ARG, "cu_seqlens requires B == 1 (got B=%d)", a.B);
    if (a.num_seqs < 1) return fail(KDA_ERR_INVALID_ARG, "num_seqs %d must be >= 1 with cu_seqlens", a.num_seqs);
    N = a.num_seqs;
  } else {
    if (a.num_seqs != 0 && a.num_seqs != a.B)
      return fail(KDA_ERR_INVALID_ARG, "num_seqs %d must equal B=%d without cu_seqlens", a.num_seqs, a.B);
    N = a.B;
  }
  pr->N = N;
  pr->H_qk = H_qk;
  pr->total = total;
  if (N < 1) {
    // B == 0 without cu_seqlens: nothing to compute and no state to write
    pr->nothing = true;
    return KDA_OK;
  }
  if (total > 0 && (!a.q || !a.k || !a.v || !a.g || !a.beta || !a.out))
    return fail(KDA_ERR_INVALID_ARG, "q, k, v, g, beta and out must be non-NULL");
  if (!a.A_log || !a.dt_bias) return fail(KDA_ERR_INVALID_ARG, "A_log and dt_bias must be non-NULL");
  const int32_t st = layout(total, a.H, N, a.cp_mode, a.seg_chunks, &pr->lay);
  if (st != KDA_OK) return st;
  if (a.cu_seqlens && a.cp_mode == KDA_CP_AUTO && a.seg_chunks == 0 && pr->lay.seg == 0 &&
      (int64_t)N * a.H >= kSerialChains && layout(total, a.H, N, KDA_CP_FORCE, 0, &pr->split_lay) == KDA_OK) {
    // the automatic plan's other rule still holds: at least 8 segments of work
    const int64_t mc = (total + kda::C - 1) / kda::C;
    pr->can_split = mc >= 8 * (int64_t)pr->split_lay.seg;
  }
  pr->nothing = total == 0 && !a.final_state;
  return KDA_OK;
}

// Carves the workspace ws (already checked to hold pr.lay) and launches the
// call's kernels on stream s.
int32_t launch(const FwdArgs& a, const Prepared& pr, uint8_t* ws, hipStream_t s) {
  const Layout& lay = pr.lay;
  const kda::Tables t = carve_tables(ws, lay, a.cu_seqlens ? -1 : a.T);
  const bool cp = lay.seg > 0;
  kda::Seg sg;
  sg.M = cp ? reinterpret_cast<float*>(ws + lay.off[KDA_WS_SEG_M]) : nullptr;
  sg.R = cp ? reinterpret_cast<float*>(ws + lay.off[KDA_WS_SEG_R]) : nullptr;
  sg.S = cp ? reinterpret_cast<float*>(ws + lay.off[KDA_WS_SEG_S]) : nullptr;
  sg.chk = cp ? reinterpret_cast<float*>(ws + lay.off[KDA_WS_SEG_CHK]) : nullptr;
  sg.fix = cp ? reinterpret_cast<float*>(ws + lay.off[KDA_WS_SEG_FIX]) : nullptr;
  sg.mnz = cp ? reinterpret_cast<int32_t*>(ws + lay.off[KDA_WS_SEG_MNZ]) : nullptr;
  sg.sync = cp ? reinterpret_cast<uint32_t*>(ws + lay.off[KDA_WS_SEG_SYNC]) : nullptr;
  sg.epoch = next_epoch();
  sg.chk_chunks = cp ? kCheckChunks : 0;
  // where the library chooses the plan, the tables may use a longer segment
  // length than the planned one (fixed length: chosen here; varlen: by the
  // index kernel)
  const bool choose = a.seg_chunks == 0;
  sg.seg_chunks = cp ? (a.cu_seqlens ? (int)lay.seg : fixed_seg(lay.seg, pr.N, a.T, a.H, choose)) : 0;
  const int64_t mc = lay.off[KDA_WS_MAX_CHUNKS];
  const int64_t ms = lay.off[KDA_WS_MAX_SEGS];
  const int32_t N = pr.N;

  kda::Problem p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.g = static_cast<const uint16_t*>(a.g);
  p.beta = static_cast<const uint16_t*>(a.beta);
  p.out = static_cast<uint16_t*>(a.out);
  p.A_log = a.A_log;
  p.dt_bias = a.dt_bias;
  p.init_state = a.initial_state;
  p.final_state = a.final_state;
  p.state_fp32 = a.state_dtype == KDA_STATE_FP32;
  p.state_kv = a.state_layout == KDA_STATE_KV;
  {
    const uintptr_t bytes = (uintptr_t)N * (uintptr_t)a.H * kda::D * kda::D * (p.state_fp32 ? 4u : 2u);
    const uintptr_t f = (uintptr_t)a.final_state, i = (uintptr_t)a.initial_state;
    p.final_early = a.final_state && (!a.initial_state || f + bytes <= i || i + bytes <= f);
  }
  p.scale = a.scale;
  p.lower_bound = a.lower_bound;
  p.H = a.H;
  p.Hqk = pr.H_qk;
  p.N = N;
  p.total_tokens = pr.total;

  hipError_t e;
  e = kda::launch_index(a.cu_seqlens, N, a.T, pr.total, lay.seg, a.H, kCheckChunks, choose, pr.may_serial, mc, ms, t,
                        s);
  // Long units run their first (or only) pass with 4 consumer wavefronts of two
  // state tiles each, short ones with 8 of one tile (measured: 2-3 % faster
  // at 256-512 chunks per unit, 4 % slower at 36).  The second pass keeps 8:
  // it usually only compares, and where it redoes chunks the 4-consumer
  // kernel would spill.  Both give the same bits.
  const int64_t unit_chunks = lay.seg > 0 ? lay.seg : (N > 0 ? mc / N : 0);
  // A fixed-length call knows its unit count, N sequences of ns segments: its
  // grid has no idle rows, which would be dispatched only once a CU frees up,
  // after the busy blocks.  (A varlen call's count is known on the device
  // only; its grid covers the table's capacity.)
  int64_t rows = ms;
  if (!a.cu_seqlens) {
    const int64_t nc = (a.T + kda::C - 1) / kda::C;
    const int64_t sgc = sg.seg_chunks;
    const int64_t nsq = sgc > 0 ? (nc > 0 ? (nc + sgc - 1) / sgc : 1) : 1;
    rows = std::min(ms, (int64_t)N * nsq);
  }
  if (e == hipSuccess)
    e = unit_chunks >= kWideMinChunks ? kda::launch_chunks_c4(p, t, sg, rows, 0, cp, s)
                                      : kda::launch_chunks(p, t, sg, rows, 0, cp, s);
  if (cp && e == hipSuccess) e = kda::launch_chunks(p, t, sg, rows, 1, cp, s);
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(e));
  return KDA_OK;
}

// ---- scratch of the no-allocation entry point ----
// One array per GPU, held from the library's first use of that GPU until the
// process ends.  In host code `scratch` names a host-side stand-in, not the
// device memory: its device address is taken once per device with that device
// current (hipGetSymbolAddress) and only that address is used.
static __device__ __align__(256) uint8_t scratch[KDA_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
std::vector<uint8_t*> g_scratch_ptr;  // by device ordinal; null until first use there

// The device address of `scratch` on the device stream s runs on (the current
// device for the null stream).
int32_t scratch_for_stream(hipStream_t s, uint8_t** out) {
  int dev = -1;
  hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) return fail(KDA_ERR_HIP, "cannot find the stream's device: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if ((size_t)dev >= g_scratch_ptr.size()) g_scratch_ptr.resize((size_t)dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    void* p = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur >= 0 && cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess || !p)
      return fail(KDA_ERR_HIP, "hipGetSymbolAddress of the scratch array failed on device %d: %s", dev,
                  hipGetErrorString(e));
    if (reinterpret_cast<uintptr_t>(p) % KDA_WORKSPACE_ALIGN != 0)
      return fail(KDA_ERR_HIP, "scratch array on device %d is not %d-byte aligned", dev, KDA_WORKSPACE_ALIGN);
    g_scratch_ptr[dev] = static_cast<uint8_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return KDA_OK;
}

}  // namespace

extern "C" {

int32_t kda_plan_seg_chunks(int64_t total_tokens, int32_t num_heads, int32_t num_seqs, int32_t cp_mode,
                            int32_t seg_chunks) {
  return plan(total_tokens, num_heads, num_seqs, cp_mode, seg_chunks);
}

int32_t kda_fixed_seg_chunks(int32_t B, int64_t T, int32_t num_heads, int32_t cp_mode, int32_t seg_chunks) {
  g_last_error.clear();
  if (B < 1 || T < 0) return fail(KDA_ERR_INVALID_ARG, "B=%d must be >= 1 and T=%lld >= 0", B, (long long)T);
  if (T > 0 && B > kMaxTokens / T) return fail(KDA_ERR_INVALID_ARG, "B*T too large");
  const int32_t seg = plan((int64_t)B * T, num_heads, B, cp_mode, seg_chunks);
  if (seg < 0) return seg;
  return fixed_seg(seg, B, T, num_heads, seg_chunks == 0);
}

int32_t kda_varlen_seg_choice(const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads, int32_t cp_mode,
                              int32_t seg_chunks, int32_t* seg_out, int32_t* order_out) {
  g_last_error.clear();
  if (!seq_lens || !seg_out || !order_out)
    return fail(KDA_ERR_INVALID_ARG, "seq_lens, seg_out and order_out must be non-NULL");
  if (num_seqs < 1) return fail(KDA_ERR_INVALID_ARG, "num_seqs %d must be >= 1", num_seqs);
  int64_t total = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    if (seq_lens[i] < 0) return fail(KDA_ERR_INVALID_ARG, "seq_lens[%d] = %d is negative", i, seq_lens[i]);
    total += seq_lens[i];
  }
  int32_t seg = plan(total, num_heads, num_seqs, cp_mode, seg_chunks);
  if (seg < 0) return seg;
  *seg_out = seg;
  *order_out = 0;
  if (seg == 0 && cp_mode == KDA_CP_AUTO && seg_chunks == 0 && (int64_t)num_seqs * num_heads >= kSerialChains) {
    // the split of a skewed batch whose workspace holds the segmented layout
    const int32_t f = plan(total, num_heads, num_seqs, KDA_CP_FORCE, 0);
    const int64_t mc = (total + kda::C - 1) / kda::C;
    int64_t max_nc = 0;
    for (int32_t i = 0; i < num_seqs; ++i) max_nc = std::max<int64_t>(max_nc, (seq_lens[i] + kda::C - 1) / kda::C);
    if (f > 0 && mc >= 8 * (int64_t)f && 4 * max_nc > 5 * (int64_t)f) {
      seg = f;
      *order_out = num_seqs <= kda::kLptMaxSeqs ? 1 : 0;  // the shorter units longest first
    }
    *seg_out = seg;
  }
  if (seg == 0) {  // a serial varlen plan goes longest first up to kLptMaxSeqs sequences
    *order_out = num_seqs <= kda::kLptMaxSeqs ? 1 : 0;
    return KDA_OK;
  }
  // the index kernel's choice (kda_index.hip), replayed on the host
  if (seg_chunks != 0 || seg < kda::kSpanDeviceMinSeg || !kda::span_model_applies(seg, num_seqs, num_heads))
    return KDA_OK;
  int nc[kda::kSpanMaxSeqs];
  for (int32_t i = 0; i < num_seqs; ++i) nc[i] = (seq_lens[i] + kda::C - 1) / kda::C;
  int cu[32 + kda::kSpanMaxSeqs];
  unsigned long long best = ~0ull;
  for (int d = 0; d < 2; ++d)
    for (int c = 0; c < kda::span_candidates(seg); ++c) {
      const int span = kda::seg_span<1>(seg + c, num_seqs, nc, num_heads, kCheckChunks, d == 1, cu);
      const unsigned long long key =
          ((unsigned long long)(unsigned)span << 32) | ((unsigned)(seg + c) << 1) | (unsigned)d;
      best = key < best ? key : best;
    }
  *seg_out = (int32_t)((best & 0xFFFFFFFFu) >> 1);
  *order_out = (int32_t)(best & 1u);
  return KDA_OK;
}

size_t kda_get_workspace_size(int64_t total_tokens, int32_t num_heads, int32_t num_seqs, int32_t cp_mode,
                              int32_t seg_chunks) {
  Layout lay;
  if (layout(total_tokens, num_heads, num_seqs, cp_mode, seg_chunks, &lay) != KDA_OK) return 0;
  return (size_t)lay.off[KDA_WS_TOTAL];
}

int32_t kda_workspace_offsets(int64_t total_tokens, int32_t num_heads, int32_t num_seqs, int32_t cp_mode,
                              int32_t seg_chunks, int64_t* offs) {
  if (!offs) return fail(KDA_ERR_INVALID_ARG, "offs is NULL");
  Layout lay;
  const int32_t st = layout(total_tokens, num_heads, num_seqs, cp_mode, seg_chunks, &lay);
  if (st != KDA_OK) return st;
  std::memcpy(offs, lay.off, sizeof(lay.off));
  return KDA_OK;
}

int32_t kda_write_fixed_tables(int32_t B, int64_t T, int32_t H, int32_t cp_mode, int32_t seg_chunks, void* workspace,
                               size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (B < 1 || T < 0) return fail(KDA_ERR_INVALID_ARG, "B=%d must be >= 1 and T=%lld >= 0", B, (long long)T);
  if (T > 0 && B > kMaxTokens / T) return fail(KDA_ERR_INVALID_ARG, "B*T too large");
  Layout lay;
  const int32_t st = layout((int64_t)B * T, H, B, cp_mode, seg_chunks, &lay);
  if (st != KDA_OK) return st;
  if (!workspace) return fail(KDA_ERR_INVALID_ARG, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % KDA_WORKSPACE_ALIGN != 0)
    return fail(KDA_ERR_INVALID_ARG, "workspace must be %d-byte aligned", KDA_WORKSPACE_ALIGN);
  if ((int64_t)workspace_bytes < lay.off[KDA_WS_TOTAL])
    return fail(KDA_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, need %lld", workspace_bytes,
                (long long)lay.off[KDA_WS_TOTAL]);
  const kda::Tables t = carve_tables(static_cast<uint8_t*>(workspace), lay, T);
  const hipError_t e = kda::launch_index_fixed(B, (int)T, fixed_seg(lay.seg, B, T, H, seg_chunks == 0), t,
                                               static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(e));
  return KDA_OK;
}

int32_t kda_fwd(const void* q, const void* k, const void* v, const void* g, const void* beta, float scale, void* out,
                const float* A_log, const float* dt_bias, float lower_bound, const void* initial_state,
                void* final_state, int32_t state_dtype, int32_t state_layout, const int32_t* cu_seqlens,
                int32_t num_seqs, int32_t B,
                int64_t T, int32_t H, int32_t H_qk, int32_t D, void* workspace, size_t workspace_bytes, int32_t cp_mode,
                int32_t seg_chunks, void* stream) {
  HostTimer timer;
  g_last_error.clear();
  const FwdArgs a{q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state, final_state,
                  state_dtype, state_layout, cu_seqlens, num_seqs, B, T, H, H_qk, D, cp_mode, seg_chunks};
  Prepared pr;
  int32_t st = prepare(a, &pr);
  if (st != KDA_OK || pr.nothing) return st;
  if (!workspace) return fail(KDA_ERR_INVALID_ARG, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % KDA_WORKSPACE_ALIGN != 0)
    return fail(KDA_ERR_INVALID_ARG, "workspace must be %d-byte aligned", KDA_WORKSPACE_ALIGN);
  choose_layout(&pr, (int64_t)workspace_bytes);
  if ((int64_t)workspace_bytes < pr.lay.off[KDA_WS_TOTAL])
    return fail(KDA_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, need %lld", workspace_bytes,
                (long long)pr.lay.off[KDA_WS_TOTAL]);
  return launch(a, pr, static_cast<uint8_t*>(workspace), static_cast<hipStream_t>(stream));
}

int32_t kda_fwd_noalloc(const void* q, const void* k, const void* v, const void* g, const void* beta, float scale,
                        void* out, const float* A_log, const float* dt_bias, float lower_bound,
                        const void* initial_state, void* final_state, int32_t state_dtype, int32_t state_layout,
                        const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int64_t T, int32_t H, int32_t H_qk,
                        int32_t D, int32_t cp_mode, int32_t seg_chunks, void* stream) {
  HostTimer timer;
  g_last_error.clear();
  const FwdArgs a{q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state, final_state,
                  state_dtype, state_layout, cu_seqlens, num_seqs, B, T, H, H_qk, D, cp_mode, seg_chunks};
  Prepared pr;
  int32_t st = prepare(a, &pr);
  if (st != KDA_OK || pr.nothing) return st;
  choose_layout(&pr, (int64_t)KDA_NOALLOC_SCRATCH_BYTES);
  if (pr.lay.off[KDA_WS_TOTAL] > (int64_t)KDA_NOALLOC_SCRATCH_BYTES)
    return fail(KDA_ERR_WORKSPACE_TOO_SMALL,
                "this call needs %lld bytes of scratch, more than the %lld bytes the no-allocation entry point "
                "holds (a longer seg_chunks, or cp_mode off, needs less)",
                (long long)pr.lay.off[KDA_WS_TOTAL], (long long)KDA_NOALLOC_SCRATCH_BYTES);
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = nullptr;
  st = scratch_for_stream(s, &ws);
  if (st != KDA_OK) return st;
  return launch(a, pr, ws, s);
}

int32_t kda_profile_enable(int32_t enable) {
  g_prof.on = (enable & KDA_PROFILE_KERNELS) != 0;
  g_prof.host = (enable & KDA_PROFILE_HOST) != 0;
  return KDA_OK;
}

int32_t kda_profile_host(double* host_us, int64_t* calls) {
  if (host_us) *host_us = g_prof.host_us;
  if (calls) *calls = g_prof.host_calls;
  g_prof.host_us = 0.0;
  g_prof.host_calls = 0;
  return KDA_OK;
}

int32_t kda_profile_collect(double* stage_ms, int64_t* stage_calls, int32_t n_stages) {
  int32_t status = KDA_OK;
  for (auto& r : g_prof.recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
      status = fail(KDA_ERR_HIP, "event timing failed");
    } else if (r.stage < n_stages) {
      if (stage_ms) stage_ms[r.stage] += ms;
      if (stage_calls) stage_calls[r.stage] += 1;
    }
    g_prof.pool.push_back(r.a);
    g_prof.pool.push_back(r.b);
  }
  g_prof.recs.clear();
  return status;
}

const char* kda_strerror(int32_t status) {
  switch (status) {
    case KDA_OK: return "ok";
    case KDA_ERR_INVALID_ARG: return "invalid argument";
    case KDA_ERR_UNSUPPORTED: return "unsupported";
    case KDA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case KDA_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* kda_last_error(void) { return g_last_error.c_str(); }

const char* kda_version(void) { return "kda-mi355x 0.1.0 (gfx950)"; }

}  // extern "C"
