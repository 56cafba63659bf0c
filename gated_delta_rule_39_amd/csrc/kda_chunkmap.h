// Chunk map: from the sequence boundaries to the table of 64-token chunks.
//
// Sequence boundaries are read from cu_seqlens on the device at run time and
// never assumed ("Kernel Design Agents (KDA) optimize Kimi Delta Attention
// (KDA)", section "03 - Reward hacking": hard-coded packed-sequence
// boundaries were one of the rejected shortcuts).  Chunks start at every
// sequence start, so a chunk never straddles two sequences; the last chunk of
// a sequence may be partial.
//
// Packed sequences only (fixed-length rows need no table: the kernels derive a
// chunk's row, index and length from its number).  One workgroup of 1024 threads
// builds:
//   info[0]           total number of chunks
//   table[c]          (sequence, valid length, index inside the sequence) of chunk c
//   seq_off[n]        first chunk of sequence n (exclusive prefix of chunk counts), seq_off[N] = total
//   seq_order[i]      sequences ordered by chunk count, longest first (buckets of
//                     powers of two), so the state scan starts its longest chains first
#pragma once

#include "kda_device.h"

namespace kda {

constexpr int kMapThreads = 1024;

__global__ __launch_bounds__(kMapThreads) void chunk_map_kernel(const int32_t* __restrict__ cu,
                                                                int64_t T, int64_t N,
                                                                int64_t n_chunk_ub,
                                                                int32_t* __restrict__ info,
                                                                ChunkEntry* __restrict__ table,
                                                                int32_t* __restrict__ seq_off,
                                                                int32_t* __restrict__ seq_order) {
  __shared__ int32_t scan[kMapThreads];
  __shared__ int32_t hist[34];
  __shared__ int32_t carry_s;
  const int tid = threadIdx.x;
  if (tid == 0) carry_s = 0;
  if (tid < 34) hist[tid] = 0;
  __syncthreads();

  // 1. chunk counts, exclusive prefix -> seq_off; bucket histogram
  for (int64_t base = 0; base < N; base += kMapThreads) {
    int64_t n = base + tid;
    int32_t cnt = 0;
    if (n < N) {
      int64_t L = seq_len(cu, T, n);
      int64_t c = (L + kChunk - 1) / kChunk;
      cnt = (int32_t)(c < n_chunk_ub ? c : n_chunk_ub);
      int b = cnt == 0 ? 0 : 32 - __clz(cnt);  // 1 + floor(log2(cnt))
      atomicAdd(&hist[b], 1);
    }
    scan[tid] = cnt;
    __syncthreads();
    for (int o = 1; o < kMapThreads; o <<= 1) {
      int32_t add = tid >= o ? scan[tid - o] : 0;
      __syncthreads();
      scan[tid] += add;
      __syncthreads();
    }
    int32_t carry = carry_s;
    if (n < N) seq_off[n] = carry + scan[tid] - cnt;
    __syncthreads();
    if (tid == kMapThreads - 1) carry_s = carry + scan[tid];
    __syncthreads();
  }
  int32_t total = carry_s;
  if (total > n_chunk_ub) total = (int32_t)n_chunk_ub;  // only on invalid cu_seqlens
  if (tid == 0) {
    info[0] = total;
    info[1] = (carry_s > n_chunk_ub) ? 1 : 0;
    seq_off[N] = carry_s;
  }
  __syncthreads();

  // 2. table: chunk c belongs to the last sequence n with seq_off[n] <= c
  for (int64_t c = tid; c < total; c += kMapThreads) {
    int64_t lo = 0, hi = N - 1;
    while (lo < hi) {
      int64_t mid = (lo + hi + 1) >> 1;
      if (seq_off[mid] <= c) lo = mid; else hi = mid - 1;
    }
    int64_t n = lo;
    int32_t idx = (int32_t)(c - seq_off[n]);
    int64_t L = seq_len(cu, T, n);
    int64_t rem = L - (int64_t)idx * kChunk;
    ChunkEntry e;
    e.seq = (int32_t)n;
    e.len = (int32_t)(rem < kChunk ? (rem > 0 ? rem : 0) : kChunk);
    e.idx = idx;
    e.pad = 0;
    table[c] = e;
  }

  // 3. longest-first order of sequences (bucket b = 1 + floor(log2(chunks)), descending)
  if (tid == 0) {
    int32_t run = 0;
    for (int b = 33; b >= 0; --b) {
      int32_t h = hist[b];
      hist[b] = run;
      run += h;
    }
  }
  __syncthreads();
  for (int64_t base = 0; base < N; base += kMapThreads) {
    int64_t n = base + tid;
    if (n < N) {
      int64_t L = seq_len(cu, T, n);
      int64_t c = (L + kChunk - 1) / kChunk;
      int32_t cnt = (int32_t)(c < n_chunk_ub ? c : n_chunk_ub);
      int b = cnt == 0 ? 0 : 32 - __clz(cnt);
      int32_t pos = atomicAdd(&hist[b], 1);
      seq_order[pos] = (int32_t)n;
    }
  }
}

}  // namespace kda
