// Host-side launch interface between the C ABI (kda_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

struct ForwardPlan {
  // sizes
  int64_t B, T, N, T_total, n_chunk_ub;
  int32_t H, dk, dv, dtype;  // dtype: 0 = bf16, 1 = fp32
  // tensors
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const void* beta;
  const float* h0;
  const int32_t* cu;
  float scale;
  void* out;
  float* ht;
  // workspace carve-up
  int32_t* info;
  void* table;
  int32_t* seq_off;
  int32_t* seq_order;
  void* rank_desc;  // packed: per rank of seq_order, {sequence, first chunk, first token, length}
  void* passes;     // packed: the chunk kernel's passes {chunk, partner chunk or -1}
  int32_t* small_list;  // packed: chunk map scratch (the chunks of at most 32 tokens)
  uint8_t* rec;
  int32_t* defer;  // per (chunk, head): the item needs the exact diagonal tiles (chunk kernel scratch)
  uint64_t* flags;        // per (chunk, head): record-ready flags of the fused kernel
  uint64_t epoch;         // this call's flag value (eager fused call) or salt (captured call)
  uint64_t* ctl;          // workspace control words: [0] last launch, [1] failed launch, [2] launch counter
  bool captured;          // the stream is capturing a graph: flag values come from the device counter
  int32_t spin_limit;     // polls before a fused-kernel wait gives up
  int32_t fuse_producers;  // > 0: one fused kernel, this many workgroups run the chunk walk
  int32_t fuse_rounds;     // fused: chunk-walk rounds shared by every workgroup (scan ones included)
  int32_t slice;  // value columns per scan workgroup (16, 32 or 64)
  int32_t task_scan;    // packed: > 0 runs the persistent state scan on this many workgroups
  int32_t long_chunks;  // packed: sequences of at least this many chunks form the long class (power of two; 0: none)
  int32_t long_width;   // packed: value columns of a long task (32 or 64; 0: chosen by the scan)
  int32_t chunk_wgs;  // workgroups of the persistent chunk kernel (>= 1)
  hipEvent_t marks[4];  // optional timing marks around the kernels (may be null)
};

// Bytes of one per-(chunk, head) record.
size_t record_bytes(int dk, int dv);

// Enqueue chunk map, chunk kernel and state scan on `stream`.
hipError_t launch_forward(const ForwardPlan& p, hipStream_t stream);

// Backward of the forward described by a ForwardPlan-like set of sizes (chunkwise form).
struct BackwardPlan {
  int64_t B, T, N, T_total, n_chunk_ub;
  int32_t H, dk, dv, dtype;
  const void* q; const void* k; const void* v; const float* g; const void* beta; const float* h0;
  const int32_t* cu;
  float scale;
  const void* dout; const float* dht;
  void* dq; void* dk_; void* dv_; float* dg; void* dbeta; float* dh0;
  // workspace
  int32_t* info; void* table; int32_t* seq_off; int32_t* seq_order;
  float* cb_fac;                                          // per (chunk, head): chunk_bwd_factor_floats
  float* cb_st;                                           // per (chunk, head): chunk_bwd_state_floats
};

// fp32 words per (chunk, head) item of the chunkwise backward: its factors and its state block.
size_t chunk_bwd_factor_floats(int dk, int dv);
size_t chunk_bwd_state_floats(int dk, int dv);

hipError_t launch_backward(const BackwardPlan& p, hipStream_t stream);

// Enqueue the token-by-token recurrent kernel on `stream` (uses the sizes, tensors and
// scale of `p`; no workspace).
hipError_t launch_recurrent(const ForwardPlan& p, hipStream_t stream);

// Fill the whole LDS of every compute unit with a 32-bit pattern (a test hook).
hipError_t fill_lds(uint32_t bits, hipStream_t stream);

}  // namespace kda
