// The fused forward kernel (fixed-length batches whose state-scan chains leave most of
// the compute units free): both roles of the two-kernel path in one launch, handing each
// chunk's record over through device-scope flags (kda_prep.h: chunk_walk; kda_scan.h:
// scan_chain).
#pragma once

#include "kda_prep.h"
#include "kda_scan.h"

namespace kda {

// Fused forward: workgroups 0 .. producers-1 walk the chunks (in the order the scan
// consumes them) and publish each record; the others first take the first `scan_rounds`
// rounds of items with them (publishing those records too, their deferred ones included),
// then each walk one (row, head, 64-column slice) chain, waiting for each record before
// loading it.  Every record is published by a workgroup before it waits on anything; the
// chunk workgroups never wait and have the lower block ids, so they are dispatched first.
template <int DK, int DV, typename InT>
__global__ __launch_bounds__(kPrepThreads, 1) void fused_fwd_kernel(PrepArgs pa, ScanArgs sa, FuseArgs fz) {
  static_assert(kPrepThreads == kScanThreads, "one block size for both roles");
  extern __shared__ __align__(16) uint8_t smem[];
  FuseArgs f = fz;
  f.epoch = launch_epoch(fz);
  const bool producer = (int)blockIdx.x < f.producers;
  if (producer || f.scan_rounds > 0)
    chunk_walk<DK, DV, InT, true>(pa, f, (int)blockIdx.x, f.producers, smem, (int)gridDim.x, f.scan_rounds);
  if (!producer) {
    __syncthreads();  // the chunk items' LDS is free
    scan_chain<DK, DV, 64, InT, true>(sa, f, (int64_t)blockIdx.x - f.producers,
                                      (int64_t)gridDim.x - f.producers, smem);
  }
}

}  // namespace kda
