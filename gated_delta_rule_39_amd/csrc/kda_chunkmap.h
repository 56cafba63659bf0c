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
//   seq_order[i]      sequences ordered by chunk count, longest first (four buckets per
//                     power of two), so the state scan starts its longest chains first
//   rank_desc[i]      (optional) {sequence, first chunk, first token, length} of seq_order[i]
//   info[2]           sequences of at least `long_chunks` chunks (a power of two, so they
//                     are exactly the first ones of seq_order); 0 when long_chunks is 0
//   info[8..15]       task counters of the persistent state scan, zeroed here
//   passes[p]         (optional) the chunk kernel's passes: {chunk, partner or -1}; a chunk of
//                     at most 32 tokens shares its 64-row pass with the next such chunk (rows
//                     0..31 and 32..63), every other chunk has a pass of its own;
//                     info[3] = number of passes (small_list[]: scratch, the short chunks in order)
#pragma once

#include "kda_device.h"

namespace kda {

constexpr int kMapThreads = 1024;
constexpr int kMapBuckets = 128;
// Batches of at most kMapLdsSeqs sequences keep their offsets, starts and lengths in LDS, and
// at most kMapLdsChunks chunks their lengths and the list of short chunks: the later steps
// then read what the earlier ones computed from LDS instead of through L2 (a binary search
// over the offsets is otherwise a chain of dependent global loads).  Larger batches use the
// global arrays.
constexpr int kMapLdsSeqs = 2048;
constexpr int kMapLdsChunks = 4096;

// Inclusive prefix sum over the workgroup's 1024 threads in thread order: a scan inside each
// wave, then the waves' totals through LDS (`wsum`, 16 words).  `total` gets the sum of all.
__device__ inline int32_t block_incl_scan(int32_t v, int32_t* wsum, int32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t x = __shfl_up(v, o, 64);
    if (lane >= o) v += x;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  int32_t off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kMapThreads / 64; ++w) {
    const int32_t x = wsum[w];
    off += w < wave ? x : 0;
    tot += x;
  }
  __syncthreads();  // wsum is free again
  total = tot;
  return v + off;
}

// Order bucket of a chunk count: 0 for none, else 1 + 4 floor(log2 c) + the next two bits
// of c (monotone in c; a power of two starts its bucket).
__device__ inline int order_bucket(int32_t c) {
  if (c <= 0) return 0;
  const int e = 31 - __clz(c);
  return 1 + 4 * e + ((int)(((uint32_t)c << 2) >> e) & 3);
}

__global__ __launch_bounds__(kMapThreads) void chunk_map_kernel(const int32_t* __restrict__ cu,
                                                                int64_t T, int64_t N,
                                                                int64_t n_chunk_ub,
                                                                int32_t* __restrict__ info,
                                                                ChunkEntry* __restrict__ table,
                                                                int32_t* __restrict__ seq_off,
                                                                int32_t* __restrict__ seq_order,
                                                                int4* __restrict__ rank_desc,
                                                                int32_t long_chunks,
                                                                int2* __restrict__ passes,
                                                                int32_t* __restrict__ small_list) {
  __shared__ int32_t hist[kMapBuckets];
  __shared__ int32_t wsum[kMapThreads / 64];
  __shared__ int32_t s_off[kMapLdsSeqs], s_start[kMapLdsSeqs], s_len[kMapLdsSeqs];
  __shared__ uint8_t s_clen[kMapLdsChunks];
  __shared__ int32_t s_small[kMapLdsChunks];
  const int tid = threadIdx.x;
  if (tid < kMapBuckets) hist[tid] = 0;
  __syncthreads();
  // packed offsets and lengths fit 31 bits (the host bounds the total tokens)
  const bool lds_seq = cu != nullptr && N <= kMapLdsSeqs;
  auto off_of = [&](int64_t m) { return lds_seq ? (int64_t)s_off[m] : (int64_t)seq_off[m]; };
  auto start_of = [&](int64_t m) { return lds_seq ? (int64_t)s_start[m] : seq_start(cu, T, m); };
  auto len_of = [&](int64_t m) { return lds_seq ? (int64_t)s_len[m] : seq_len(cu, T, m); };

  // 1. chunk counts, exclusive prefix -> seq_off; bucket histogram
  int32_t carry = 0;  // chunks of the sequences before this batch (the same in every thread)
  for (int64_t base = 0; base < N; base += kMapThreads) {
    int64_t n = base + tid;
    int32_t cnt = 0;
    if (n < N) {
      int64_t L = seq_len(cu, T, n);
      int64_t c = (L + kChunk - 1) / kChunk;
      cnt = (int32_t)(c < n_chunk_ub ? c : n_chunk_ub);
      atomicAdd(&hist[order_bucket(cnt)], 1);
      if (lds_seq) {
        s_start[n] = (int32_t)seq_start(cu, T, n);
        s_len[n] = (int32_t)L;
      }
    }
    int32_t batch;
    const int32_t incl = block_incl_scan(cnt, wsum, batch);
    if (n < N) {
      seq_off[n] = carry + incl - cnt;
      if (lds_seq) s_off[n] = carry + incl - cnt;
    }
    carry += batch;
  }
  int32_t total = carry;
  if (total > n_chunk_ub) total = (int32_t)n_chunk_ub;  // only on invalid cu_seqlens
  if (tid == 0) {
    info[0] = total;
    info[1] = (carry > n_chunk_ub) ? 1 : 0;
    seq_off[N] = carry;
  }
  if (tid < 8) info[8 + tid] = 0;
  __syncthreads();

  // 2. table: chunk c belongs to the last sequence n with seq_off[n] <= c
  const bool lds_chunks = total <= kMapLdsChunks;
  for (int64_t c = tid; c < total; c += kMapThreads) {
    int64_t lo = 0, hi = N - 1;
    while (lo < hi) {
      int64_t mid = (lo + hi + 1) >> 1;
      if (off_of(mid) <= c) lo = mid; else hi = mid - 1;
    }
    int64_t n = lo;
    int32_t idx = (int32_t)(c - off_of(n));
    int64_t L = len_of(n);
    int64_t rem = L - (int64_t)idx * kChunk;
    ChunkEntry e;
    e.seq = (int32_t)n;
    e.len = (int32_t)(rem < kChunk ? (rem > 0 ? rem : 0) : kChunk);
    e.idx = idx;
    e.pad = 0;
    table[c] = e;
    if (lds_chunks) s_clen[c] = (uint8_t)e.len;
  }

  // 3. longest-first order of sequences (order buckets, descending): each bucket's first
  //    position is the number of sequences in the buckets above it.  One wave scans the
  //    buckets from the top, two per lane.
  static_assert(kMapBuckets == 128, "two buckets per lane of one wave");
  if (tid < 64) {
    const int b1 = kMapBuckets - 1 - 2 * tid, b2 = b1 - 1;
    const int32_t c1 = hist[b1], c2 = hist[b2];
    int32_t incl = c1 + c2;
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t v = __shfl_up(incl, o, 64);
      if (tid >= o) incl += v;
    }
    const int32_t above = incl - c1 - c2;
    hist[b1] = above;
    hist[b2] = above + c1;
    // the long sequences are those of the buckets from long_chunks' on: the first position
    // of the bucket below it (read by the wave that wrote it, before the placements below)
    if (tid == 0) info[2] = long_chunks > 0 ? hist[order_bucket(long_chunks) - 1] : 0;
  }
  __syncthreads();
  for (int64_t base = 0; base < N; base += kMapThreads) {
    int64_t n = base + tid;
    if (n < N) {
      int64_t L = len_of(n);
      int64_t c = (L + kChunk - 1) / kChunk;
      int32_t cnt = (int32_t)(c < n_chunk_ub ? c : n_chunk_ub);
      int32_t pos = atomicAdd(&hist[order_bucket(cnt)], 1);
      seq_order[pos] = (int32_t)n;
      if (rank_desc) rank_desc[pos] = make_int4((int)n, (int)off_of(n), (int)start_of(n), (int)L);
    }
  }

  // 4. passes of the chunk kernel (the chunk table is complete: barriers since step 2).
  //    Rank of each short chunk among the short ones, then the pass heads (other chunks and
  //    short chunks of even rank) numbered in chunk order.
  if (!passes) return;
  __syncthreads();
  auto is_short = [&](int64_t c) { return c < total && (lds_chunks ? s_clen[c] : table[c].len) <= 32; };
  int32_t n_short = 0;
  for (int64_t base = 0; base < total; base += kMapThreads) {
    const int64_t c = base + tid;
    const int32_t f = is_short(c) ? 1 : 0;
    int32_t batch;
    const int32_t incl = block_incl_scan(f, wsum, batch);
    if (f) {
      if (lds_chunks) s_small[n_short + incl - 1] = (int32_t)c;
      else small_list[n_short + incl - 1] = (int32_t)c;
    }
    n_short += batch;
  }
  __syncthreads();  // small_list complete
  int32_t n_short_seen = 0, n_pass = 0;
  for (int64_t base = 0; base < total; base += kMapThreads) {
    const int64_t c = base + tid;
    const bool sh = is_short(c);
    int32_t shorts, heads;
    const int32_t rank = n_short_seen + block_incl_scan(sh ? 1 : 0, wsum, shorts) - 1;  // for short chunks
    const bool head = c < total && (!sh || (rank & 1) == 0);
    const int32_t hpos = block_incl_scan(head ? 1 : 0, wsum, heads);
    if (head) {
      const int32_t partner =
          (sh && rank + 1 < n_short) ? (lds_chunks ? s_small[rank + 1] : small_list[rank + 1]) : -1;
      passes[n_pass + hpos - 1] = make_int2((int32_t)c, partner);
    }
    n_short_seen += shorts;
    n_pass += heads;
  }
  if (tid == 0) info[3] = n_pass;
}

}  // namespace kda
