// Kernel instantiations and launch sequence of the KDA forward (gfx950).
#include "kda_launch.h"

#include <atomic>
#include <cstdlib>
#include <mutex>
#include <utility>
#include <vector>

#include "kda_chunkmap.h"
#include "kda_prep.h"
#include "kda_scan.h"
#include "kda_scan_tasks.h"
#include "kda_fused.h"
#include "kda_recurrent.h"
#include "kda_chunk_bwd.h"

namespace kda {

size_t record_bytes(int dk, int dv) {
  if (dk == 64 && dv == 64) return Rec<64, 64>::BYTES;
  if (dk == 64 && dv == 128) return Rec<64, 128>::BYTES;
  if (dk == 128 && dv == 64) return Rec<128, 64>::BYTES;
  if (dk == 128 && dv == 128) return Rec<128, 128>::BYTES;
  return 0;
}

// Raises a kernel's dynamic LDS limit once per (kernel, device) (the attribute persists;
// setting it on every call cost host time on the launch path).
template <typename K>
static hipError_t allow_smem(K kern, size_t smem) {
  static std::mutex mu;
  static std::vector<std::pair<const void*, uint64_t>> done;  // kernel, bit set of devices
  const void* key = reinterpret_cast<const void*>(kern);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  std::lock_guard<std::mutex> lock(mu);
  for (const auto& d : done)
    if (d.first == key && (d.second & bit)) return hipSuccess;
  e = hipFuncSetAttribute(key, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  for (auto& d : done)
    if (d.first == key) {
      d.second |= bit;
      return hipSuccess;
    }
  done.emplace_back(key, bit);
  return hipSuccess;
}

// Test hook: with KDA_TEST_LDS_FILL=<32-bit pattern> set, every kernel of a call is preceded
// by a fill of the whole LDS of every compute unit with that pattern.  No kernel here may
// read an LDS word it has not written in the same launch (LDS keeps what the previous
// kernel on the compute unit left); a NaN or Inf pattern makes any such read visible in
// the outputs.
__global__ __launch_bounds__(1024) void lds_fill_kernel(uint32_t bits, uint32_t words) {
  extern __shared__ __align__(16) uint32_t lds_words[];
  volatile uint32_t* v = lds_words;  // stores the compiler must keep
  for (uint32_t i = threadIdx.x; i < words; i += blockDim.x) v[i] = bits;
}

hipError_t fill_lds(uint32_t bits, hipStream_t stream) {
  int dev = 0, bytes = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&bytes, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev)) != hipSuccess)
    return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  if (bytes <= 0 || cus <= 0) return hipErrorInvalidValue;
  if ((e = allow_smem(lds_fill_kernel, (size_t)bytes)) != hipSuccess) return e;
  hipLaunchKernelGGL(lds_fill_kernel, dim3((unsigned)(4 * cus)), dim3(1024), (size_t)bytes, stream, bits,
                     (uint32_t)(bytes / 4));
  return hipGetLastError();
}

static hipError_t stale_lds(hipStream_t stream) {
  const char* env = std::getenv("KDA_TEST_LDS_FILL");
  if (!env || !env[0]) return hipSuccess;
  return fill_lds((uint32_t)std::strtoul(env, nullptr, 0), stream);
}

static void mark(const ForwardPlan& p, int i, hipStream_t stream) {
  if (p.marks[i]) (void)hipEventRecord(p.marks[i], stream);
}

static PrepArgs prep_args(const ForwardPlan& p) {
  PrepArgs a;
  a.q = p.q; a.k = p.k; a.v = p.v; a.g = p.g; a.beta = p.beta; a.cu = p.cu;
  a.T = p.T; a.T_total = p.T_total; a.H = p.H;
  a.info = p.info;
  a.nc = p.cu ? 0 : (p.T + kChunk - 1) / kChunk;
  a.table = reinterpret_cast<const ChunkEntry*>(p.table);
  a.passes = reinterpret_cast<const int2*>(p.passes);
  a.rec = p.rec;
  a.defer = p.defer;
  return a;
}

static ScanArgs scan_args(const ForwardPlan& p) {
  ScanArgs a;
  a.h0 = p.h0; a.ht = p.ht; a.out = p.out; a.cu = p.cu;
  a.T = p.T; a.T_total = p.T_total; a.N = p.N; a.H = p.H; a.n_chunk_ub = p.n_chunk_ub;
  a.seq_off = p.seq_off; a.seq_order = p.seq_order; a.rec = p.rec; a.scale = p.scale;
  a.nc = p.cu ? 0 : (p.T + kChunk - 1) / kChunk;
  a.ctl = p.ctl;
  return a;
}

template <int DK, int DV, typename InT>
static hipError_t launch_prep(const ForwardPlan& p, hipStream_t stream) {
  const PrepArgs a = prep_args(p);
  const size_t smem = PrepSmem<DK, DV>::BYTES;
  auto kern = chunk_prep_kernel<DK, DV, InT>;
  hipError_t ea = allow_smem(kern, smem);
  if (ea != hipSuccess) return ea;
  // persistent workgroups, at most one per compute unit (the LDS footprint admits one)
  int64_t grid = p.chunk_wgs > 0 ? p.chunk_wgs : 256;
  const int64_t items = p.n_chunk_ub * (int64_t)p.H;
  if (grid > items) grid = items;
  if (hipError_t ep = stale_lds(stream); ep != hipSuccess) return ep;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kPrepThreads), smem, stream, a);
  return hipGetLastError();
}

template <int DK, int DV, int NV, typename OutT>
static hipError_t launch_scan_nv(const ForwardPlan& p, hipStream_t stream) {
  const ScanArgs a = scan_args(p);
  const size_t smem = ScanSmem<DK, DV, NV>::BYTES;
  auto kern = state_scan_kernel<DK, DV, NV, OutT>;
  const int64_t blocks = p.N * (int64_t)p.H * (DV / NV);
  if (hipError_t ep = stale_lds(stream); ep != hipSuccess) return ep;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kScanThreads), smem, stream, a);
  return hipGetLastError();
}

template <int DK, int DV, typename OutT>
static hipError_t launch_scan_tasks(const ForwardPlan& p, hipStream_t stream) {
  constexpr int NVL = DV < 32 ? DV : 32, NVW = DV < 64 ? DV : 64;
  ScanArgs a = scan_args(p);
  TaskArgs ta;
  ta.queue = p.info + 8;
  ta.n_long = p.info + 2;
  ta.rank_desc = reinterpret_cast<const int4*>(p.rank_desc);
  ta.long_width = p.long_width == NVL || p.long_width == NVW ? p.long_width : 0;
  const size_t smem = scan_tasks_smem<DK, DV, NVL, NVW>();
  auto kern = state_scan_tasks_kernel<DK, DV, NVL, NVW, OutT>;
  hipError_t ea = allow_smem(kern, smem);
  if (ea != hipSuccess) return ea;
  if (hipError_t ep = stale_lds(stream); ep != hipSuccess) return ep;
  hipLaunchKernelGGL(kern, dim3((unsigned)p.task_scan), dim3(kScanThreads), smem, stream, a, ta);
  return hipGetLastError();
}

template <int DK, int DV, typename OutT>
static hipError_t launch_scan(const ForwardPlan& p, hipStream_t stream) {
  if (p.cu && p.task_scan > 0) return launch_scan_tasks<DK, DV, OutT>(p, stream);
  switch (p.slice) {
    case 16: return launch_scan_nv<DK, DV, 16, OutT>(p, stream);
    case 32: return launch_scan_nv<DK, DV, 32, OutT>(p, stream);
    default: return launch_scan_nv<DK, DV, 64, OutT>(p, stream);
  }
}

template <int DK, int DV, typename InT>
static hipError_t launch_fused(const ForwardPlan& p, hipStream_t stream) {
  FuseArgs fz;
  fz.flags = p.flags;
  fz.epoch = p.epoch;
  fz.ctl = p.ctl;
  fz.dev_epoch = nullptr;
  fz.producers = p.fuse_producers;
  fz.scan_rounds = p.fuse_rounds;
  if (p.spin_limit > 0) {
    fz.spin_limit = p.spin_limit;
  } else {
    // a wait never needs longer than the whole chunk walk (about 10 us per item and
    // workgroup, a poll about 60 ns): allow several times that
    const int64_t per_wg = p.n_chunk_ub * (int64_t)p.H / p.fuse_producers + 2;
    const int64_t spins = per_wg * 1000;
    fz.spin_limit = (int32_t)(spins < (1 << 16) ? (1 << 16) : (spins > (1 << 30) ? (1 << 30) : spins));
  }
  if (p.captured) {
    // a replay of a captured launch keeps its arguments: the flag value is derived on the
    // device from a counter that this one-thread kernel advances before every replay
    hipLaunchKernelGGL(epoch_advance_kernel, dim3(1), dim3(64), 0, stream, p.ctl + 2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    fz.dev_epoch = p.ctl + 2;
  }
  const size_t s1 = PrepSmem<DK, DV>::BYTES, s2 = ScanSmem<DK, DV, 64>::BYTES;
  const size_t smem = s1 > s2 ? s1 : s2;
  auto kern = fused_fwd_kernel<DK, DV, InT>;
  hipError_t ea = allow_smem(kern, smem);
  if (ea != hipSuccess) return ea;
  const int64_t chains = p.N * (int64_t)p.H * (DV / 64);
  if (hipError_t ep = stale_lds(stream); ep != hipSuccess) return ep;
  hipLaunchKernelGGL(kern, dim3((unsigned)(p.fuse_producers + chains)), dim3(kPrepThreads), smem, stream,
                     prep_args(p), scan_args(p), fz);
  return hipGetLastError();
}

template <int DK, int DV>
static hipError_t launch_dkdv(const ForwardPlan& p, hipStream_t stream) {
  hipError_t e = hipSuccess;
  if (p.fuse_producers > 0) {
    e = (p.dtype == 0) ? launch_fused<DK, DV, uint16_t>(p, stream) : launch_fused<DK, DV, float>(p, stream);
    mark(p, 2, stream);
    mark(p, 3, stream);
    return e;
  }
  if (p.T_total > 0) {
    e = (p.dtype == 0) ? launch_prep<DK, DV, uint16_t>(p, stream) : launch_prep<DK, DV, float>(p, stream);
    if (e != hipSuccess) return e;
  }
  mark(p, 2, stream);
  e = (p.dtype == 0) ? launch_scan<DK, DV, uint16_t>(p, stream) : launch_scan<DK, DV, float>(p, stream);
  mark(p, 3, stream);
  return e;
}

hipError_t launch_forward(const ForwardPlan& p, hipStream_t stream) {
  if (p.N <= 0) return hipSuccess;
  mark(p, 0, stream);
  // packed sequences: chunk table, sequence offsets and order from cu_seqlens on the device;
  // fixed-length rows need none of it (the kernels derive every chunk from its index)
  if (p.cu) {
    if (hipError_t ep = stale_lds(stream); ep != hipSuccess) return ep;
    hipLaunchKernelGGL(chunk_map_kernel, dim3(1), dim3(kMapThreads), 0, stream, p.cu, p.T, p.N, p.n_chunk_ub,
                       p.info, reinterpret_cast<ChunkEntry*>(p.table), p.seq_off, p.seq_order,
                       reinterpret_cast<int4*>(p.rank_desc), p.long_chunks, reinterpret_cast<int2*>(p.passes),
                       p.small_list);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  mark(p, 1, stream);
  if (p.dk == 64 && p.dv == 64) return launch_dkdv<64, 64>(p, stream);
  if (p.dk == 64 && p.dv == 128) return launch_dkdv<64, 128>(p, stream);
  if (p.dk == 128 && p.dv == 64) return launch_dkdv<128, 64>(p, stream);
  return launch_dkdv<128, 128>(p, stream);
}

template <int DK, int DV, typename InT>
static hipError_t launch_recurrent_dkdv(const ForwardPlan& p, hipStream_t stream) {
  RecurrentArgs a;
  a.q = p.q; a.k = p.k; a.v = p.v; a.g = p.g; a.beta = p.beta; a.h0 = p.h0; a.cu = p.cu;
  a.ht = p.ht; a.out = p.out; a.T = p.T; a.N = p.N; a.H = p.H; a.scale = p.scale;
  a.waves = p.N * (int64_t)p.H * (DV / kRecCols);
  const int64_t per_block = kRecThreads / 64;
  const int64_t blocks = (a.waves + per_block - 1) / per_block;
  auto kern = recurrent_kernel<DK, DV, InT>;
  if (hipError_t ep = stale_lds(stream); ep != hipSuccess) return ep;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kRecThreads), 0, stream, a);
  return hipGetLastError();
}

template <int DK, int DV>
static hipError_t launch_recurrent_dt(const ForwardPlan& p, hipStream_t stream) {
  return p.dtype == 0 ? launch_recurrent_dkdv<DK, DV, uint16_t>(p, stream)
                      : launch_recurrent_dkdv<DK, DV, float>(p, stream);
}

hipError_t launch_recurrent(const ForwardPlan& p, hipStream_t stream) {
  if (p.N <= 0) return hipSuccess;
  if (p.dk == 64 && p.dv == 64) return launch_recurrent_dt<64, 64>(p, stream);
  if (p.dk == 64 && p.dv == 128) return launch_recurrent_dt<64, 128>(p, stream);
  if (p.dk == 128 && p.dv == 64) return launch_recurrent_dt<128, 64>(p, stream);
  return launch_recurrent_dt<128, 128>(p, stream);
}

template <int DK, int DV, typename InT>
static hipError_t launch_chunk_backward_t(const BackwardPlan& p, hipStream_t stream) {
  using WS = CbWs<DK, DV>;
  CbArgs a;
  a.q = p.q; a.k = p.k; a.v = p.v; a.g = p.g; a.beta = p.beta; a.h0 = p.h0;
  a.cu = p.cu;
  a.info = p.info;
  a.table = reinterpret_cast<const ChunkEntry*>(p.table);
  a.seq_off = p.seq_off;
  a.seq_order = p.seq_order;
  a.dout = p.dout; a.dht = p.dht;
  a.dq = p.dq; a.dk = p.dk_; a.dv = p.dv_; a.dg = p.dg; a.dbeta = p.dbeta; a.dh0 = p.dh0;
  const int64_t items = p.n_chunk_ub * (int64_t)p.H;
  float* f = p.cb_fac;
  a.W = f; f += (size_t)items * WS::W;
  a.U = f; f += (size_t)items * WS::U;
  a.KdT = f; f += (size_t)items * WS::KDT;
  a.QgT = f; f += (size_t)items * WS::QGT;
  a.PT = f; f += (size_t)items * WS::PT;
  a.L = f; f += (size_t)items * WS::L;
  a.TT = f; f += (size_t)items * WS::TT;
  a.eGn = f;
  a.st = p.cb_st;
  a.T = p.T; a.N = p.N; a.nc = p.cu ? 0 : (p.T + kChunk - 1) / kChunk;
  a.n_chunk_ub = p.n_chunk_ub;
  a.H = p.H; a.scale = p.scale;
  hipError_t e = hipSuccess;
  if (items > 0) {
    auto fac = cb_factor_kernel<DK, DV, InT>;
    const size_t smem = CbFacSmem<DK>::BYTES;
    if ((e = allow_smem(fac, smem)) != hipSuccess) return e;
    if (hipError_t ep = stale_lds(stream); ep != hipSuccess) return ep;
    hipLaunchKernelGGL(fac, dim3((unsigned)items), dim3(DK * 4), smem, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int64_t chains = p.N * (int64_t)p.H * (DV / 16);
  const size_t ssm = CbScanSmem<DK>::BYTES;
  auto sc = cb_state_scan_kernel<DK, DV, InT>;
  if ((e = allow_smem(sc, ssm)) != hipSuccess) return e;
  if (hipError_t ep = stale_lds(stream); ep != hipSuccess) return ep;
  hipLaunchKernelGGL(sc, dim3((unsigned)chains), dim3(DK * 4), ssm, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (items > 0) {
    auto ga = cb_grad_a_kernel<DK, DV, InT>;
    const size_t gsm = CbGradASmem<DK, DV>::BYTES;
    if ((e = allow_smem(ga, gsm)) != hipSuccess) return e;
    if (hipError_t ep = stale_lds(stream); ep != hipSuccess) return ep;
    hipLaunchKernelGGL(ga, dim3((unsigned)items), dim3(DK * 4), gsm, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    auto gb = cb_grad_b_kernel<DK, DV, InT>;
    const size_t smem = CbGradSmem<DK>::BYTES;
    if ((e = allow_smem(gb, smem)) != hipSuccess) return e;
    if (hipError_t ep = stale_lds(stream); ep != hipSuccess) return ep;
    hipLaunchKernelGGL(gb, dim3((unsigned)items), dim3(DK * 4), smem, stream, a);
    e = hipGetLastError();
  }
  return e;
}

template <int DK, int DV>
static hipError_t launch_backward_dt(const BackwardPlan& p, hipStream_t stream) {
  return p.dtype == 0 ? launch_chunk_backward_t<DK, DV, uint16_t>(p, stream)
                      : launch_chunk_backward_t<DK, DV, float>(p, stream);
}

size_t chunk_bwd_factor_floats(int dk, int dv) {
  if (dk == 64 && dv == 64) return CbWs<64, 64>::FACTOR_FLOATS;
  if (dk == 64 && dv == 128) return CbWs<64, 128>::FACTOR_FLOATS;
  if (dk == 128 && dv == 64) return CbWs<128, 64>::FACTOR_FLOATS;
  return CbWs<128, 128>::FACTOR_FLOATS;
}

size_t chunk_bwd_state_floats(int dk, int dv) {
  if (dk == 64 && dv == 64) return CbWs<64, 64>::SB;
  if (dk == 64 && dv == 128) return CbWs<64, 128>::SB;
  if (dk == 128 && dv == 64) return CbWs<128, 64>::SB;
  return CbWs<128, 128>::SB;
}

hipError_t launch_backward(const BackwardPlan& p, hipStream_t stream) {
  if (p.N <= 0) return hipSuccess;
  if (p.cu) {
    if (hipError_t ep = stale_lds(stream); ep != hipSuccess) return ep;
    hipLaunchKernelGGL(chunk_map_kernel, dim3(1), dim3(kMapThreads), 0, stream, p.cu, p.T, p.N, p.n_chunk_ub,
                       p.info, reinterpret_cast<ChunkEntry*>(p.table), p.seq_off, p.seq_order, nullptr, 0,
                       nullptr, nullptr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.dk == 64 && p.dv == 64) return launch_backward_dt<64, 64>(p, stream);
  if (p.dk == 64 && p.dv == 128) return launch_backward_dt<64, 128>(p, stream);
  if (p.dk == 128 && p.dv == 64) return launch_backward_dt<128, 64>(p, stream);
  return launch_backward_dt<128, 128>(p, stream);
}

}  // namespace kda
