// C ABI of the KDA forward: argument checks, workspace carve-up, launches.
// Declarations and the contract of every entry point are in include/kda.h.
#include "kda.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "kda_launch.h"

namespace {

constexpr int64_t kChunkTokens = 64;

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

struct Carve {
  size_t info, table, seq_off, seq_order, rank_desc, passes, small_list, defer, flags, rec, total;
};

bool sizes_ok(const kda_problem_t* p, bool packed, int64_t* N, int64_t* n_chunk_ub) {
  if (!p) return false;
  if (p->batch < 1 || p->seqlen < 0 || p->heads < 1 || p->num_seqs < 0) return false;
  if (packed) {
    if (p->batch != 1 || p->num_seqs < 1) return false;
    *N = p->num_seqs;
    *n_chunk_ub = (p->seqlen + kChunkTokens - 1) / kChunkTokens + p->num_seqs;
  } else {
    if (p->num_seqs != 0 && p->num_seqs != p->batch) return false;
    *N = p->batch;
    *n_chunk_ub = p->batch * ((p->seqlen + kChunkTokens - 1) / kChunkTokens);
  }
  // grid limits: chunks and scan workgroups must fit the launch dimensions
  if (*n_chunk_ub * (int64_t)p->heads > 0x7fffffffLL || *N * (int64_t)p->heads * 8 > 0x7fffffffLL) return false;
  // int32 token offsets inside the packed table; 64-bit element offsets elsewhere
  if (packed && p->seqlen > 0x7fffffffLL) return false;
  return true;
}

bool dims_supported(const kda_problem_t* p) {
  return (p->dk == 64 || p->dk == 128) && (p->dv == 64 || p->dv == 128) &&
         (p->dtype == KDA_BF16 || p->dtype == KDA_F32);
}

Carve carve(const kda_problem_t* p, int64_t N, int64_t n_chunk_ub) {
  Carve c;
  c.info = 0;
  c.table = c.info + 256;
  c.seq_off = c.table + align256((size_t)n_chunk_ub * 16);
  c.seq_order = c.seq_off + align256((size_t)(N + 1) * 4);
  c.rank_desc = c.seq_order + align256((size_t)N * 4);
  c.passes = c.rank_desc + align256((size_t)N * 16);
  c.small_list = c.passes + align256((size_t)n_chunk_ub * 8);
  c.defer = c.small_list + align256((size_t)n_chunk_ub * 4);
  c.flags = c.defer + align256((size_t)n_chunk_ub * (size_t)p->heads * 4);
  c.rec = c.flags + align256((size_t)n_chunk_ub * (size_t)p->heads * 8 * 2);  // a flag per 64-column slice
  c.total = c.rec + (size_t)n_chunk_ub * (size_t)p->heads * kda::record_bytes(p->dk, p->dv);
  return c;
}

bool misaligned(const void* ptr) { return ptr && (reinterpret_cast<uintptr_t>(ptr) & 15u); }

bool overlap(const void* a, size_t an, const void* b, size_t bn) {
  if (!a || !b || an == 0 || bn == 0) return false;
  uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + bn && b0 < a0 + an;
}

// Compute units of the current device, queried once per device (a HIP attribute query
// on every call cost host time on the launch path).
int compute_units() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];  // 0 = not yet queried
  int dev = 0;
  hipGetDevice(&dev);
  if (dev >= 0 && dev < kMaxDevices) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (cus <= 0) cus = 256;
  if (dev >= 0 && dev < kMaxDevices) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Polls before a wait of the fused kernel gives up: KDA_SPIN_LIMIT=n (n >= 1) overrides the
// default (several times the whole chunk walk), which the tests use to force the failure
// path; 0 = default.
int spin_limit_override() {
  const char* env = std::getenv("KDA_SPIN_LIMIT");
  if (!env) return 0;
  const long v = std::atol(env);
  return v >= 1 ? (int)(v < (1L << 30) ? v : (1L << 30)) : 0;
}

// Byte offset of the control words inside the workspace's info block (256 bytes: the chunk
// map's counters come first): [0] flag value of the most recent launch, [1] flag value of a
// launch whose wait gave up, [2] launch counter of captured fused calls.
constexpr size_t kCtlOffset = 64;

// Value columns per state-scan workgroup.  A workgroup's step costs about the same for
// 16, 32 or 64 columns (it is bound by loading the chunk's factors), so the widest slice
// that still gives every compute unit a workgroup wins: fewer workgroups walk the chains
// in fewer rounds.  KDA_SCAN_SLICE=16|32|64 overrides.
int slice_width(const kda_problem_t* p, int64_t N) {
  const char* env = std::getenv("KDA_SCAN_SLICE");
  if (env) {
    int v = std::atoi(env);
    if ((v == 16 || v == 32 || v == 64) && v <= p->dv) return v;
  }
  const int64_t cus = compute_units();
  for (int v = 64; v > 16; v >>= 1)
    if (v <= p->dv && N * (int64_t)p->heads * (p->dv / v) >= cus) return v;
  return 16;
}

// Packed batches: the persistent state scan on one workgroup per compute unit (KDA_TASK_SCAN=0
// takes the one-workgroup-per-chain scan instead, KDA_TASK_SCAN=n >= 1 caps the workgroups at
// n: tuning, and tests of long per-workgroup walks and of a single queue), with sequences of at least
// KDA_LONG_CHUNKS chunks (rounded up to a power of two; default 4) taken one at a time from
// a cold start, on narrower value slices when their chains alone would not fill the
// compute units, and the shorter ones pipelined.
int task_scan_workgroups(bool packed) {
  if (!packed) return 0;
  const int cus = compute_units();
  const char* env = std::getenv("KDA_TASK_SCAN");
  if (!env) return cus;
  const int v = std::atoi(env);
  if (v <= 0) return 0;
  return v < cus ? v : cus;
}

int long_chunks() {
  const char* env = std::getenv("KDA_LONG_CHUNKS");
  if (!env) return 4;
  const int v = std::atoi(env);
  if (v <= 0) return 0;
  int p = 1;
  while (p < v && p < (1 << 30)) p <<= 1;  // rounded up to a power of two
  return p;
}

// KDA_LONG_SLICE=32|64: value columns of a long task of the persistent scan (tuning and
// tests); unset or anything else: the scan chooses.
int long_width() {
  const char* env = std::getenv("KDA_LONG_SLICE");
  const int v = env ? std::atoi(env) : 0;
  return v == 32 || v == 64 ? v : 0;
}

// Workgroups of the persistent chunk kernel: one per compute unit, or fewer when
// KDA_CHUNK_WGS=n (n >= 1) asks for it (tuning, and tests of long per-workgroup walks).
int chunk_workgroups() {
  int n = compute_units();
  const char* env = std::getenv("KDA_CHUNK_WGS");
  if (env) {
    const int v = std::atoi(env);
    if (v >= 1 && v < n) n = v;
  }
  return n;
}

// Fused forward (one kernel: chunk walk and scan side by side) for fixed-length rows when
// the chains are few: the scan then runs on 64-column slices in a quarter of the compute
// units or less and the chunk walk on the rest.  KDA_FUSED=0 turns it off.  Returns the
// number of chunk-walk workgroups, 0 for the two-kernel path.
int fused_producers(const kda_problem_t* p, int64_t N, bool packed) {
  const char* env = std::getenv("KDA_FUSED");
  if (env && env[0] == '0') return 0;
  if (packed || p->seqlen <= 0) return 0;
  const int64_t cus = compute_units();
  const int64_t chains = N * (int64_t)p->heads * (p->dv / 64);
  if (chains * 4 > cus) return 0;
  const int64_t walk = cus - chains;
  const int64_t cap = chunk_workgroups();  // KDA_CHUNK_WGS caps the chunk walk here too
  return (int)(walk < cap ? walk : cap);
}

// Fused: chunk-walk rounds that every workgroup of the launch takes (the scan workgroups one
// item per round before their chains start), KDA_FUSE_ROUNDS=n overrides (0: none).
int fuse_rounds() {
  const char* env = std::getenv("KDA_FUSE_ROUNDS");
  if (!env) return 1;
  const int v = std::atoi(env);
  return v < 0 ? 0 : (v > 64 ? 64 : v);
}

// Flag value of a fused call: a process-wide counter from a time-derived start, so that
// flags left by earlier calls (or uninitialised workspace) do not match.
uint64_t next_epoch() {
  static std::atomic<uint64_t> counter{
      (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count() * 0x9E3779B97F4A7C15ull | 1ull};
  return counter.fetch_add(2, std::memory_order_relaxed);
}

}  // namespace

extern "C" {

int kda_version(void) { return 104; }

kda_status_t kda_test_fill_lds(uint32_t bits, void* stream) {
  return kda::fill_lds(bits, static_cast<hipStream_t>(stream)) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

const char* kda_status_string(kda_status_t s) {
  switch (s) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_NULL: return "KDA_ERR_NULL: a required pointer is NULL";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: dk/dv must be 64 or 128, dtype bf16 or fp32";
    case KDA_ERR_BAD_ARG: return "KDA_ERR_BAD_ARG: inconsistent sizes, non-finite scale or bad cu_seqlens";
    case KDA_ERR_ALIGN: return "KDA_ERR_ALIGN: tensor pointers must be 16-byte aligned";
    case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace smaller than kda_fwd_workspace_size()";
    case KDA_ERR_ALIAS: return "KDA_ERR_ALIAS: out or ht overlaps an input";
    case KDA_ERR_HIP: return "KDA_ERR_HIP: a HIP launch failed";
    case KDA_ERR_TIMEOUT: return "KDA_ERR_TIMEOUT: a wait of the fused kernel gave up; its outputs hold NaN";
  }
  return "unknown kda_status_t";
}

size_t kda_fwd_workspace_size(const kda_problem_t* prob) {
  if (!prob || !dims_supported(prob)) return 0;
  int64_t N = 0, ub = 0;
  // the workspace depends only on sizes; packed mode is the one with num_seqs >= 1 and batch == 1
  // when the caller passes cu_seqlens, so size for the larger of the two readings
  bool fixed_ok = sizes_ok(prob, false, &N, &ub);
  size_t best = 0;
  if (fixed_ok) best = carve(prob, N, ub).total;
  int64_t N2 = 0, ub2 = 0;
  if (sizes_ok(prob, true, &N2, &ub2)) {
    size_t t2 = carve(prob, N2, ub2).total;
    if (t2 > best) best = t2;
  }
  return best;
}

}  // extern "C"

// The checks of kda_fwd_validate; `use_workspace` = false for kda_decode, which takes none.
static kda_status_t validate(const kda_problem_t* prob, const void* q, const void* k, const void* v,
                             const float* g, const void* beta, const float* h0, const int32_t* cu_seqlens,
                             float scale, const void* out, const float* ht, const void* workspace,
                             size_t workspace_bytes, bool use_workspace) {
  if (!prob) return KDA_ERR_NULL;
  if (!dims_supported(prob)) return KDA_ERR_UNSUPPORTED;
  const bool packed = cu_seqlens != nullptr;
  int64_t N = 0, ub = 0;
  if (!sizes_ok(prob, packed, &N, &ub)) return KDA_ERR_BAD_ARG;
  if (!std::isfinite(scale)) return KDA_ERR_BAD_ARG;
  const int64_t toks = prob->batch * prob->seqlen;
  if (toks > 0 && (!q || !k || !v || !g || !beta || !out)) return KDA_ERR_NULL;
  if (!use_workspace) {
    workspace = nullptr;
    workspace_bytes = 0;
  } else if (!workspace) {
    return KDA_ERR_NULL;
  }
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(g) || misaligned(beta) ||
      misaligned(h0) || misaligned(out) || misaligned(ht) || misaligned(workspace))
    return KDA_ERR_ALIGN;
  if (use_workspace && workspace_bytes < carve(prob, N, ub).total) return KDA_ERR_WORKSPACE;
  const size_t es = prob->dtype == KDA_BF16 ? 2 : 4;
  const size_t nqk = (size_t)toks * prob->heads * prob->dk;
  const size_t nv = (size_t)toks * prob->heads * prob->dv;
  const size_t nst = (size_t)N * prob->heads * prob->dk * prob->dv * 4;
  struct In { const void* p; size_t n; } ins[] = {
      {q, nqk * es}, {k, nqk * es}, {v, nv * es}, {g, nqk * 4}, {beta, (size_t)toks * prob->heads * es},
      {h0, h0 ? nst : 0}, {cu_seqlens, packed ? (size_t)(N + 1) * 4 : 0}, {workspace, workspace_bytes}};
  for (const In& in : ins) {
    if (overlap(out, nv * es, in.p, in.n)) return KDA_ERR_ALIAS;
    if (ht && in.p != h0 && overlap(ht, nst, in.p, in.n)) return KDA_ERR_ALIAS;
  }
  if (ht && h0 && ht != h0 && overlap(ht, nst, h0, nst)) return KDA_ERR_ALIAS;
  if (ht && overlap(ht, nst, out, nv * es)) return KDA_ERR_ALIAS;
  const char* env = std::getenv("KDA_VALIDATE_CU_SEQLENS");
  if (packed && env && env[0] == '1') {
    std::vector<int32_t> host((size_t)N + 1);
    if (hipMemcpy(host.data(), cu_seqlens, host.size() * 4, hipMemcpyDeviceToHost) != hipSuccess)
      return KDA_ERR_HIP;
    if (host[0] != 0 || host[N] != prob->seqlen) return KDA_ERR_BAD_ARG;
    for (int64_t i = 0; i < N; ++i)
      if (host[i + 1] < host[i]) return KDA_ERR_BAD_ARG;
  }
  return KDA_OK;
}

extern "C" {

kda_status_t kda_fwd_validate(const kda_problem_t* prob, const void* q, const void* k, const void* v,
                              const float* g, const void* beta, const float* h0,
                              const int32_t* cu_seqlens, float scale, const void* out, const float* ht,
                              const void* workspace, size_t workspace_bytes) {
  return validate(prob, q, k, v, g, beta, h0, cu_seqlens, scale, out, ht, workspace, workspace_bytes, true);
}

static kda_status_t forward(const kda_problem_t* prob, const void* q, const void* k, const void* v,
                            const float* g, const void* beta, const float* h0, const int32_t* cu_seqlens,
                            float scale, void* out, float* ht, void* workspace, size_t workspace_bytes,
                            void* stream, void* const* events) {
  kda_status_t st = kda_fwd_validate(prob, q, k, v, g, beta, h0, cu_seqlens, scale, out, ht, workspace,
                                     workspace_bytes);
  if (st != KDA_OK) return st;
  const bool packed = cu_seqlens != nullptr;
  int64_t N = 0, ub = 0;
  sizes_ok(prob, packed, &N, &ub);
  Carve c = carve(prob, N, ub);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  kda::ForwardPlan p;
  p.B = prob->batch;
  p.T = prob->seqlen;
  p.N = N;
  p.T_total = prob->batch * prob->seqlen;
  p.n_chunk_ub = ub;
  p.H = prob->heads;
  p.dk = prob->dk;
  p.dv = prob->dv;
  p.dtype = prob->dtype;
  p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta; p.h0 = h0; p.cu = cu_seqlens;
  p.scale = scale;
  p.out = out;
  p.ht = ht;
  p.info = reinterpret_cast<int32_t*>(ws + c.info);
  p.table = ws + c.table;
  p.seq_off = reinterpret_cast<int32_t*>(ws + c.seq_off);
  p.seq_order = reinterpret_cast<int32_t*>(ws + c.seq_order);
  p.rank_desc = ws + c.rank_desc;
  p.passes = ws + c.passes;
  p.small_list = reinterpret_cast<int32_t*>(ws + c.small_list);
  p.rec = ws + c.rec;
  p.defer = reinterpret_cast<int32_t*>(ws + c.defer);
  p.flags = reinterpret_cast<uint64_t*>(ws + c.flags);
  p.ctl = reinterpret_cast<uint64_t*>(ws + c.info + kCtlOffset);
  p.fuse_producers = fused_producers(prob, N, packed);
  p.epoch = p.fuse_producers > 0 ? next_epoch() : 0;
  p.spin_limit = spin_limit_override();
  p.fuse_rounds = p.fuse_producers > 0 ? fuse_rounds() : 0;
  p.captured = false;
  if (p.fuse_producers > 0) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(static_cast<hipStream_t>(stream), &cs) != hipSuccess) return KDA_ERR_HIP;
    p.captured = cs == hipStreamCaptureStatusActive;
  }
  p.slice = slice_width(prob, N);
  p.chunk_wgs = chunk_workgroups();
  p.task_scan = task_scan_workgroups(packed);
  p.long_chunks = long_chunks();
  p.long_width = long_width();
  for (int i = 0; i < 4; ++i) p.marks[i] = events ? static_cast<hipEvent_t>(events[i]) : nullptr;
  hipError_t e = kda::launch_forward(p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status_t kda_fwd(const kda_problem_t* prob, const void* q, const void* k, const void* v, const float* g,
                     const void* beta, const float* h0, const int32_t* cu_seqlens, float scale, void* out,
                     float* ht, void* workspace, size_t workspace_bytes, void* stream) {
  return forward(prob, q, k, v, g, beta, h0, cu_seqlens, scale, out, ht, workspace, workspace_bytes, stream,
                 nullptr);
}

kda_status_t kda_fwd_status(const void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace) return KDA_ERR_NULL;
  if (misaligned(workspace)) return KDA_ERR_ALIGN;
  if (workspace_bytes < 256) return KDA_ERR_WORKSPACE;
  if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return KDA_ERR_HIP;
  uint64_t ctl[2] = {0, 0};
  if (hipMemcpy(ctl, static_cast<const uint8_t*>(workspace) + kCtlOffset, sizeof(ctl), hipMemcpyDeviceToHost) !=
      hipSuccess)
    return KDA_ERR_HIP;
  // flag values are odd; the two-kernel path records 0 (it has no waits)
  return ((ctl[0] & 1u) && ctl[1] == ctl[0]) ? KDA_ERR_TIMEOUT : KDA_OK;
}

kda_status_t kda_decode(const kda_problem_t* prob, const void* q, const void* k, const void* v,
                        const float* g, const void* beta, const float* h0, const int32_t* cu_seqlens,
                        float scale, void* out, float* ht, void* stream) {
  kda_status_t st = validate(prob, q, k, v, g, beta, h0, cu_seqlens, scale, out, ht, nullptr, 0, false);
  if (st != KDA_OK) return st;
  int64_t N = 0, ub = 0;
  sizes_ok(prob, cu_seqlens != nullptr, &N, &ub);
  kda::ForwardPlan p{};
  p.B = prob->batch;
  p.T = prob->seqlen;
  p.N = N;
  p.T_total = prob->batch * prob->seqlen;
  p.H = prob->heads;
  p.dk = prob->dk;
  p.dv = prob->dv;
  p.dtype = prob->dtype;
  p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta; p.h0 = h0; p.cu = cu_seqlens;
  p.scale = scale;
  p.out = out;
  p.ht = ht;
  hipError_t e = kda::launch_recurrent(p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

// Backward workspace: chunk map (packed), then per (chunk, head) the chunk's factors and its
// state block (S0, Hn, dD, D; later the first gradient kernel's results).
struct BwdCarve {
  size_t info, table, seq_off, seq_order, fac, st, total;
};

static BwdCarve bwd_carve(const kda_problem_t* p, int64_t N, int64_t n_chunk_ub) {
  BwdCarve c;
  const size_t items = (size_t)n_chunk_ub * p->heads;
  c.info = 0;
  c.table = c.info + 256;
  c.seq_off = c.table + align256((size_t)n_chunk_ub * 16);
  c.seq_order = c.seq_off + align256((size_t)(N + 1) * 4);
  c.fac = c.seq_order + align256((size_t)N * 4);
  c.st = c.fac + align256(items * kda::chunk_bwd_factor_floats(p->dk, p->dv) * 4);
  c.total = c.st + align256(items * kda::chunk_bwd_state_floats(p->dk, p->dv) * 4);
  return c;
}

size_t kda_bwd_workspace_size(const kda_problem_t* prob) {
  if (!prob || !dims_supported(prob)) return 0;
  size_t best = 0;
  int64_t N = 0, ub = 0;
  if (sizes_ok(prob, false, &N, &ub)) best = bwd_carve(prob, N, ub).total;
  if (sizes_ok(prob, true, &N, &ub)) {
    const size_t t = bwd_carve(prob, N, ub).total;
    if (t > best) best = t;
  }
  return best;
}

kda_status_t kda_bwd(const kda_problem_t* prob, const void* q, const void* k, const void* v, const float* g,
                     const void* beta, const float* h0, const int32_t* cu_seqlens, float scale,
                     const void* dout, const float* dht, void* dq, void* dk, void* dv, float* dg, void* dbeta,
                     float* dh0, void* workspace, size_t workspace_bytes, void* stream) {
  if (!prob) return KDA_ERR_NULL;
  if (!dims_supported(prob)) return KDA_ERR_UNSUPPORTED;
  const bool packed = cu_seqlens != nullptr;
  int64_t N = 0, ub = 0;
  if (!sizes_ok(prob, packed, &N, &ub)) return KDA_ERR_BAD_ARG;
  if (!std::isfinite(scale)) return KDA_ERR_BAD_ARG;
  const int64_t toks = prob->batch * prob->seqlen;
  if (toks > 0 && (!q || !k || !v || !g || !beta || !dout || !dq || !dk || !dv || !dg || !dbeta))
    return KDA_ERR_NULL;
  if (!workspace) return KDA_ERR_NULL;
  const void* ptrs[] = {q, k, v, g, beta, h0, dout, dht, dq, dk, dv, dg, dbeta, dh0, workspace};
  for (const void* ptr : ptrs)
    if (misaligned(ptr)) return KDA_ERR_ALIGN;
  const BwdCarve c = bwd_carve(prob, N, ub);
  if (workspace_bytes < c.total) return KDA_ERR_WORKSPACE;
  const size_t es = prob->dtype == KDA_BF16 ? 2 : 4;
  const size_t nqk = (size_t)toks * prob->heads * prob->dk;
  const size_t nv = (size_t)toks * prob->heads * prob->dv;
  const size_t nst = (size_t)N * prob->heads * prob->dk * prob->dv * 4;
  struct Buf { const void* p; size_t n; };
  const Buf ins[] = {{q, nqk * es}, {k, nqk * es}, {v, nv * es}, {g, nqk * 4},
                     {beta, (size_t)toks * prob->heads * es}, {h0, h0 ? nst : 0},
                     {cu_seqlens, packed ? (size_t)(N + 1) * 4 : 0}, {dout, nv * es},
                     {dht, dht ? nst : 0}, {workspace, workspace_bytes}};
  const Buf outs[] = {{dq, nqk * es}, {dk, nqk * es}, {dv, nv * es}, {dg, nqk * 4},
                      {dbeta, (size_t)toks * prob->heads * es}, {dh0, dh0 ? nst : 0}};
  for (const Buf& o : outs) {
    for (const Buf& in : ins)
      if (overlap(o.p, o.n, in.p, in.n)) return KDA_ERR_ALIAS;
    for (const Buf& o2 : outs)
      if (&o2 != &o && overlap(o.p, o.n, o2.p, o2.n)) return KDA_ERR_ALIAS;
  }
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  kda::BackwardPlan p{};
  p.B = prob->batch; p.T = prob->seqlen; p.N = N; p.T_total = toks; p.n_chunk_ub = ub;
  p.H = prob->heads; p.dk = prob->dk; p.dv = prob->dv; p.dtype = prob->dtype;
  p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta; p.h0 = h0; p.cu = cu_seqlens; p.scale = scale;
  p.dout = dout; p.dht = dht;
  p.dq = dq; p.dk_ = dk; p.dv_ = dv; p.dg = dg; p.dbeta = dbeta; p.dh0 = dh0;
  p.info = reinterpret_cast<int32_t*>(ws + c.info);
  p.table = ws + c.table;
  p.seq_off = reinterpret_cast<int32_t*>(ws + c.seq_off);
  p.seq_order = reinterpret_cast<int32_t*>(ws + c.seq_order);
  p.cb_fac = reinterpret_cast<float*>(ws + c.fac);
  p.cb_st = reinterpret_cast<float*>(ws + c.st);
  hipError_t e = kda::launch_backward(p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status_t kda_fwd_timed(const kda_problem_t* prob, const void* q, const void* k, const void* v,
                           const float* g, const void* beta, const float* h0, const int32_t* cu_seqlens,
                           float scale, void* out, float* ht, void* workspace, size_t workspace_bytes,
                           void* stream, void* const* events) {
  return forward(prob, q, k, v, g, beta, h0, cu_seqlens, scale, out, ht, workspace, workspace_bytes, stream,
                 events);
}

}  // extern "C"
