// Chunk kernel: everything about a 64-token chunk that does not depend on
// the recurrent state, for one (chunk, head) at a time per workgroup.
//
// The chunkwise form of the gated delta rule ("Autoresearch on Kimi Delta
// Attention", section "KDA in one minute": the state moves sequentially
// between blocks while the work inside a block becomes matrix products).
// Inside a chunk with incoming state S0 and G_t = sum_{s<=t} g_s (per key
// channel, from the chunk start):
//     L_ij   = sum_c khat_ic khat_jc exp(G_ic - G_jc)          (j < i)
//     Tinv   = (I + diag(beta) L)^-1                            (unit lower triangular)
//     W      = Tinv diag(beta) (Khat * exp(G))     U = Tinv diag(beta) V
//     Aqk_ij = sum_c qhat_ic khat_jc exp(G_ic - G_jc)          (j <= i)
// so that the scan kernel can finish the chunk with Delta = U - W S0,
// o = scale (Qhat*exp(G) S0 + Aqk Delta) and
// S_next = Diag(exp(G_last)) S0 + (Khat*exp(G_last-G))^T Delta.
//
// This kernel produces, per (chunk, head): the fragments of W, Qhat*exp(G),
// (Khat*exp(G_last-G))^T, Aqk, U (scaled by 2^ue), exp(G_last), max|v| and ue.
//
// Work split: a workgroup of 8 waves takes one (chunk, head) at a time; wave
// (w, hf) holds tokens 16w..16w+15 and one half (hf) of the key and value
// channels.  Channel-wise steps need no exchange; the two places that sum
// over all channels (the L2 norms and the Gram matrices) add the two halves'
// partial sums through LDS.  The workgroups are persistent: while one item is
// computed, the raw inputs of the next are already on their way into
// registers, so the HBM latency of the loads is hidden behind the arithmetic.
//
// Steps, each exact up to rounding for every legal input:
//  (a) Real L2 norms of q and k per token ("Kernel Design Agents (KDA)
//      optimize Kimi Delta Attention (KDA)", section "03 - Reward hacking":
//      a distribution constant in place of the norm was rejected).  Each
//      half's sum of squares is taken after an exact power-of-two rescale by
//      that half's largest entry, and the halves are brought to a common
//      exponent before they are added, so entries up to the bf16/fp32
//      maximum cannot overflow.
//  (a) In-chunk cumulative log-gate G, kept in fp32 and in log2 units
//      (the same section rejects an fp16 table of decays and decays formed
//      as ratios of cumulative powers that underflow past 126 bits).
//  (b) Gram matrices L and Aqk.  Every pair factor exp(G_i - G_j) is split
//      around a reference row r with j <= r <= i as exp(G_i - G_r) *
//      exp(G_r - G_j): both factors are <= 1, so nothing overflows at any
//      gate depth and underflow only drops terms below fp32 range.
//      Off-diagonal 16x16 tiles (fp16 MFMA) use the end of the column block
//      as r.  A diagonal tile uses its middle row as r, which puts the
//      factors in [exp(-D), exp(D)] with D the larger half-span of the tile's
//      decay; when D <= 80 nats on every channel of all four diagonal tiles
//      (checked per chunk and head) each tile is one fp32 MFMA product.
//      Otherwise the item is flagged and, once the workgroup has walked all
//      its items, redone by the exact variant, which uses per-4-token
//      column-group references plus exp(g) products inside each group, on
//      fp16 MFMA, exact at any depth.
//  (b) Tinv by blocked forward substitution in fp32 (16x16 diagonal blocks by
//      substitution, off-diagonal blocks by block products).
//  (b) W and U on fp16 MFMA from Tinv and the exchanged operand fragments.
//  Transposes (token-major operands of the token contractions) are MFMA
//  products with an identity matrix: the C fragment of X * I holds, lane for
//  lane, the operand fragment of X^T, exactly (fp16 values, fp32 sums).
//
// fp16 operands: every operand is bounded (|khat|,|qhat| <= 1, all decay
// factors <= 1, |Tinv| <= 1, |W| rows bounded) except V, which is rescaled
// by 2^ue so that max|v| < 2^12; then |U| <= 9 * 2^12 < 65504.  fp16 keeps
// 11 significant bits where bf16 keeps 8, which is what holds long-memory
// heads inside the accuracy budget.
#pragma once

#include "kda_device.h"

namespace kda {

constexpr int kPrepThreads = 512;  // 8 waves: 4 token blocks x 2 channel halves

template <int DK, int DV>
struct PrepSmem {
  static constexpr int KSK = DK / 32;
  static constexpr int NTK = DK / 16;
  static constexpr int NTV = DV / 16;
  static constexpr int LP = 68;  // pitch (floats) of 64x64 fp32 matrices
  static constexpr int ET_ROWS = 19;
  static constexpr size_t BTOT = 4 * DK * 4;
  static constexpr size_t YBF = 4 * KSK * 64 * 16;
  static constexpr size_t BWX = (size_t)NTK * 2 * 64 * 16;
  static constexpr size_t BUX = (size_t)NTV * 2 * 64 * 16;
  static_assert(YBF <= BWX, "column operands must not reach the Bu fragments");
  static constexpr size_t X_A = BTOT > YBF ? BTOT : YBF;
  static constexpr size_t X_BYTES = X_A > BWX + BUX ? X_A : BWX + BUX;
  static constexpr size_t MAT = 64 * LP * 4;
  static constexpr size_t ETB = (size_t)ET_ROWS * DK * 4;
  static constexpr size_t Z_BYTES = MAT > ETB ? MAT : ETB;
  static constexpr size_t X = 0;                  // btot -> column operands | Bu fragments -> Bw^T | Bu
  static constexpr size_t Y = X + X_BYTES;        // L (strict lower) + inverse temporaries (upper)
  static constexpr size_t Z = Y + MAT;            // decay-factor table -> Tinv
  static constexpr size_t GE = Z + Z_BYTES;       // G (log2 units) at the 16 group ends, then at token j* (x2)
  static constexpr size_t GP = GE + 18 * DK * 4;  // Gram partial tiles: [L | Aqk^T][block w][tile b][lane] x 4 fp32
  static constexpr size_t NRM = GP + 2 * 16 * 64 * 16;  // norm partials: [exp | sum][tensor 2][half 2][token 64]
  static constexpr size_t BETA = NRM + 2 * 2 * 2 * 64 * 4;
  static constexpr size_t RED = BETA + 64 * 4;    // [8] max |v| per wave, then the guard flag
  static constexpr size_t META = RED + 16 * 4;    // [64] per-item (first token lo, hi, valid tokens, -)
  static constexpr size_t BYTES = META + 64 * 16;
};

struct PrepArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const void* beta;
  const int32_t* cu;
  int64_t T;        // tokens per row (fixed) / total tokens (packed)
  int64_t T_total;  // total tokens in the flattened [B*T] order
  int32_t H;
  const int32_t* info;       // packed mode: info[0] = number of chunks
  const ChunkEntry* table;   // packed mode: the chunk table
  const int2* passes;        // packed mode: passes {chunk, partner or -1}; info[3] = their number
  int64_t nc;                // fixed-length mode (cu == NULL): chunks per row; no table is built
  uint8_t* rec;     // records [n_chunk_ub][H]
  int32_t* defer;   // [chunk * H + head]: 1 if the item needs the exact diagonal tiles (written for every item)
};

// Four consecutive input elements as loaded (bf16 pairs or fp32).
template <typename InT> struct Raw4;
template <> struct Raw4<uint16_t> { using T = uint2; };
template <> struct Raw4<float> { using T = float4; };

__device__ inline void unpack4(const uint2& r, float* o) {
  o[0] = __uint_as_float(r.x << 16);
  o[1] = __uint_as_float(r.x & 0xffff0000u);
  o[2] = __uint_as_float(r.y << 16);
  o[3] = __uint_as_float(r.y & 0xffff0000u);
}
__device__ inline void unpack4(const float4& r, float* o) { o[0] = r.x; o[1] = r.y; o[2] = r.z; o[3] = r.w; }
__device__ inline float unpack1(uint16_t b) { return bf16_to_f32(b); }
__device__ inline float unpack1(float b) { return b; }

// One lane's raw inputs of one (chunk, head): token 16w + t, channels of half hf,
// in groups of four at 16 j + 4 gq inside the half.
template <int DK, int DV, typename InT>
struct RawIn {
  static constexpr int KH = DK / 64;  // 32-wide key steps per half
  static constexpr int VH = DV / 64;  // 32-wide value steps per half
  using V4 = typename Raw4<InT>::T;
  V4 q[2 * KH], k[2 * KH], v[2 * VH];
  float4 g[2 * KH];
  InT beta;
  bool valid;
};

// The same inputs as fp32 (g in log2 units): x[4 j + r] is channel (half base) + 16 j + 4 gq + r.
template <int DK, int DV>
struct ItemIn {
  float q[DK / 8], k[DK / 8], g[DK / 8], v[DV / 8];
  float beta;
};

// Scalar-unit reads (through the constant cache, counted by lgkmcnt) of data that no
// kernel of this launch writes: the chunk table and cu_seqlens.  Read this way, the
// per-item metadata never waits behind the record stores on the vector-memory counter.
// Both need a wave-uniform address aligned to 4 bytes.
__device__ __forceinline__ uint32_t sload_u32(const void* p) {
  uint32_t r;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(r) : "s"(p) : "memory");
  return r;
}
__device__ __forceinline__ uint64_t sload_u64(const void* p) {
  uint64_t r;
  asm volatile("s_load_dwordx2 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(r) : "s"(p) : "memory");
  return r;
}
// Chunk c of a fixed-length batch: chunk c mod nc of row c / nc.
__device__ __forceinline__ ChunkEntry entry_fixed(const PrepArgs& a, int64_t c) {
  ChunkEntry e;
  const int64_t row = c / a.nc, idx = c - row * a.nc;
  const int64_t rem = a.T - idx * kChunk;
  e.seq = (int32_t)row;
  e.len = (int32_t)(rem < kChunk ? rem : kChunk);
  e.idx = (int32_t)idx;
  e.pad = 0;
  return e;
}
__device__ __forceinline__ ChunkEntry ld_entry(const ChunkEntry* p) {
  const uint64_t sl = sload_u64(p);
  ChunkEntry e;
  e.seq = (int32_t)(uint32_t)sl;
  e.len = (int32_t)(uint32_t)(sl >> 32);
  e.idx = (int32_t)sload_u32(reinterpret_cast<const int32_t*>(p) + 2);
  e.pad = 0;
  return e;
}

// Element offsets of one lane's inputs of an item (chunk, h).  Lanes past the chunk's
// end read token 0 instead (the kernel runs only when there are tokens) and are
// zeroed when unpacked.
struct RawAt {
  size_t rowk;  // q, k, g: token row + half base + 4 gq
  size_t rowv;  // v
  size_t bidx;  // beta
  bool valid;
};

// `start`: first token of the chunk in the flattened order, `len`: its valid tokens.  A pass
// of two chunks (`start2` >= 0): rows 32..63 are the second chunk's rows 0..31.
template <int DK, int DV>
__device__ __forceinline__ RawAt raw_at_tok(const PrepArgs& a, int64_t start, int len, int h,
                                            int64_t start2 = -1, int len2 = 0) {
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int w = wv & 3, hf = wv >> 2, l = tid & 63, t = l & 15, gq = l >> 4;
  const int i_loc = 16 * w + t;
  const bool second = start2 >= 0 && w >= 2;  // wave-uniform
  const int row = second ? i_loc - 32 : i_loc;
  const int64_t tok = (second ? start2 : start) + row;
  RawAt at;
  at.valid = (row < (second ? len2 : len)) && (tok >= 0) && (tok < a.T_total);
  const int64_t tk = at.valid ? tok : 0;
  at.rowk = ((size_t)tk * a.H + h) * DK + hf * (DK / 2) + 4 * gq;
  at.rowv = ((size_t)tk * a.H + h) * DV + hf * (DV / 2) + 4 * gq;
  at.bidx = (size_t)tk * a.H + h;
  return at;
}

template <int DK, int DV>
__device__ __forceinline__ RawAt raw_at(const PrepArgs& a, const ChunkEntry& ce, int h) {
  const int64_t s0 = a.cu ? (int64_t)(int32_t)sload_u32(a.cu + ce.seq) : (int64_t)ce.seq * a.T;
  return raw_at_tok<DK, DV>(a, s0 + (int64_t)ce.idx * kChunk, ce.len, h);
}

// Issues one group of an item's loads: 0 = q; 1 = k, beta; 2 = g; 3 = v.  The groups
// are issued at different points of the previous item: the vector-memory path takes
// each wave's load instructions one after the other, and a single burst from all eight
// waves would hold the last of them for over a thousand cycles.
template <int PART, int DK, int DV, typename InT>
__device__ __forceinline__ void load_part(RawIn<DK, DV, InT>& r, const PrepArgs& a, const RawAt& at) {
  using RI = RawIn<DK, DV, InT>;
  using V4 = typename RI::V4;
  if (PART == 0) {
    const InT* q = reinterpret_cast<const InT*>(a.q);
#pragma unroll
    for (int j = 0; j < 2 * RI::KH; ++j) r.q[j] = *reinterpret_cast<const V4*>(q + at.rowk + 16 * j);
    r.valid = at.valid;
  } else if (PART == 1) {
    const InT* k = reinterpret_cast<const InT*>(a.k);
#pragma unroll
    for (int j = 0; j < 2 * RI::KH; ++j) r.k[j] = *reinterpret_cast<const V4*>(k + at.rowk + 16 * j);
    r.beta = reinterpret_cast<const InT*>(a.beta)[at.bidx];
  } else if (PART == 2) {
#pragma unroll
    for (int j = 0; j < 2 * RI::KH; ++j) r.g[j] = *reinterpret_cast<const float4*>(a.g + at.rowk + 16 * j);
  } else {
    const InT* v = reinterpret_cast<const InT*>(a.v);
#pragma unroll
    for (int j = 0; j < 2 * RI::VH; ++j) r.v[j] = *reinterpret_cast<const V4*>(v + at.rowv + 16 * j);
  }
}

template <int DK, int DV, typename InT>
__device__ __forceinline__ void load_raw(RawIn<DK, DV, InT>& r, const PrepArgs& a, const ChunkEntry& ce, int h) {
  const RawAt at = raw_at<DK, DV>(a, ce, h);
  load_part<0>(r, a, at);
  load_part<1>(r, a, at);
  load_part<2>(r, a, at);
  load_part<3>(r, a, at);
}

template <int DK, int DV, typename InT>
__device__ __forceinline__ void unpack_raw(ItemIn<DK, DV>& in, const RawIn<DK, DV, InT>& r) {
  using RI = RawIn<DK, DV, InT>;
#pragma unroll
  for (int j = 0; j < 2 * RI::KH; ++j) {
    unpack4(r.q[j], in.q + 4 * j);
    unpack4(r.k[j], in.k + 4 * j);
    unpack4(r.g[j], in.g + 4 * j);
  }
#pragma unroll
  for (int j = 0; j < 2 * RI::VH; ++j) unpack4(r.v[j], in.v + 4 * j);
  in.beta = unpack1(r.beta);
#pragma unroll
  for (int e = 0; e < DK / 8; ++e) in.g[e] *= kLog2e;  // gates in log2 units
  // fresh definitions: later uses never wait on the vector-memory counter for them
#pragma unroll
  for (int e = 0; e < DK / 8; ++e) asm volatile("" : "+v"(in.q[e]), "+v"(in.k[e]), "+v"(in.g[e]));
#pragma unroll
  for (int e = 0; e < DV / 8; ++e) asm volatile("" : "+v"(in.v[e]));
  asm volatile("" : "+v"(in.beta));
  if (!r.valid) {
#pragma unroll
    for (int e = 0; e < DK / 8; ++e) in.q[e] = in.k[e] = in.g[e] = 0.f;
#pragma unroll
    for (int e = 0; e < DV / 8; ++e) in.v[e] = 0.f;
    in.beta = 0.f;
  }
}

// Decay-factor table rows (per key channel c, G in log2 units, Gend(p) = G at the end
// of 4-token group p, block w = tokens 16w..16w+15):
//   0..3    exp(Gprev(w))                  Gprev(w) = Gend(4w-1), Gprev(0) = 0
//   4..7    exp(Glast - Gnext(w))          Gnext(w) = Gend(4w+3)
//   8..10   exp(Gprev(w) - Gnext(b))       (b, w) = (0, 2), (0, 3), (1, 3)
//   11..14  exp(Gprev(w) - Gmid(w))        Gmid(w) = Gend(4w+1)   (>= 1, used under the guard)
//   15..18  exp(Gmid(w) - Gnext(w))        (>= 1, used under the guard)
constexpr float kGuardLog2 = 115.0f;  // 80 nats: half-span limit of the fp32 diagonal path
constexpr int kNoExp = -1000;         // exponent recorded for an all-zero half row

// Step J.. of the substitution for a unit lower-triangular 16x16 block (see its caller):
// x[r] += am[J] * (row J's x[r]), am = minus this lane's row of the strictly lower part.
template <int J>
__device__ __forceinline__ void subst_rows(float (&x)[4], const float (&am)[16]) {
  float b[4];  // all four broadcasts first: no VALU-to-DPP wait states between them and the FMAs
#pragma unroll
  for (int r = 0; r < 4; ++r) b[r] = row_bcast<J>(x[r]);
#pragma unroll
  for (int r = 0; r < 4; ++r) x[r] = fmaf(am[J], b[r], x[r]);
  if constexpr (J + 1 < 15) subst_rows<J + 1>(x, am);
}

// Record stores.  `present` = false: a part of the record that the chunk's length leaves
// empty (rec_rows_present), dropped by the buffer's range check: no bytes are written and
// the instruction stream is the same for every length.  WT (the fused kernel): device-scope
// stores (sc1), which write through the L2 of the compute die, so that once they complete the
// record is visible to the scan workgroups on every die; otherwise plain stores, kept in L2
// for the scan kernel.
template <bool WT, int BYTES, typename V>
__device__ __forceinline__ void rec_store(uint8_t* rec, size_t off, const V& v, bool present = true) {
  constexpr int aux = WT ? 16 : 0;
  // one resource per record; a missing part's offset lies past the record's range, so the
  // store is dropped
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(rec, 0, BYTES, kBufferFlags);
  const int o = (int)off + (present ? 0 : (1 << 30));
  if constexpr (sizeof(V) == 16) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(uint4_v, v), rs, o, 0, aux);
  } else if constexpr (sizeof(V) == 8) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(uint2_v, v), rs, o, 0, aux);
  } else {
    static_assert(sizeof(V) == 4, "record stores are 4, 8 or 16 bytes");
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rs, o, 0, aux);
  }
}

// Valid tokens of chunk c (1..64; fewer only in a sequence's last chunk).  Chunk numbers
// fit 31 bits (items are counted in int).
__device__ __forceinline__ int chunk_rows(const PrepArgs& a, int c) {
  if (a.cu) return (int)sload_u32(reinterpret_cast<const int32_t*>(a.table + c) + 1);
  const int nc = (int)a.nc, idx = c - (c / nc) * nc;
  const int64_t rem = a.T - (int64_t)idx * kChunk;
  return rem < kChunk ? (int)rem : kChunk;
}

// One (chunk, head) from its fp32 inputs.  EXACT = false: guarded fp32 diagonal tiles,
// the chunk is deferred when the guard fails.  EXACT = true: per-group references on
// every diagonal tile.  Every wave of the workgroup calls it (it holds barriers).
// `mid(1)`, `mid(2)` and `mid(3)` run right after barriers #1, #2 and #4 (the persistent kernel
// issues the next item's remaining loads there).
//
// Two chunks in one pass (`chunk2` >= 0, both of at most 32 tokens): rows 0..31 hold
// `chunk`, rows 32..63 hold `chunk2`.  The pass is then block diagonal in its two halves:
// the gate sum restarts at row 32, the Gram tiles across the halves are zero (so is Tinv
// across them), G_last and j* are taken per half, and each half goes to its own record
// (rows 0..31 there, the rest zero).
template <int DK, int DV, bool EXACT, bool WT, typename Mid>
__device__ __forceinline__ void prep_item(const PrepArgs& a, const int chunk, const int chunk2, const int h,
                                          ItemIn<DK, DV>& in, uint8_t* smem, Mid&& mid) {
  using R = Rec<DK, DV>;
  using SM = PrepSmem<DK, DV>;
  constexpr int KSK = DK / 32;   // contraction steps over key channels
  constexpr int KSV = DV / 32;
  constexpr int NTV = DV / 16;
  constexpr int KH = KSK / 2;    // key steps of one channel half
  constexpr int VH = KSV / 2;    // value steps of one channel half
  constexpr int NE = KH * 8;     // key channels held per lane
  constexpr int NEV = VH * 8;    // value channels held per lane
  constexpr int LP = SM::LP;

  float* btot = reinterpret_cast<float*>(smem + SM::X);            // [4][DK]
  f16x8* ybf = reinterpret_cast<f16x8*>(smem + SM::X);             // [4][KSK][64]
  uint8_t* bwx = smem + SM::X;                                     // [NTK][2][64] f16x8
  uint8_t* bux = smem + SM::X + SM::BWX;                           // [NTV][2][64] f16x8
  float* Lm = reinterpret_cast<float*>(smem + SM::Y);              // [64][LP]
  // K~^T halves on their way to one 16-byte record store per lane, in the L buffer (free
  // between barriers #3 and #5a): [hf][token block pair][pair half][j][lane] x f16x4
  f16x4* ktx = reinterpret_cast<f16x4*>(smem + SM::Y);
  static_assert(2 * 2 * 2 * (2 * (DK / 64)) * 64 * 8 <= SM::MAT, "K~^T exchange must fit the L buffer");
  float* et = reinterpret_cast<float*>(smem + SM::Z);              // [19][DK]
  float* Tm = reinterpret_cast<float*>(smem + SM::Z);              // [64][LP]
  float* gend = reinterpret_cast<float*>(smem + SM::GE);           // [16][DK]
  float* gpl = reinterpret_cast<float*>(smem + SM::GP);            // L partials [4][4][64][4]
  float* gpa = gpl + 16 * 64 * 4;                                  // Aqk^T partials [4][4][64][4]
  int* nrm_ex = reinterpret_cast<int*>(smem + SM::NRM);            // [2][2][64]
  float* nrm_ss = reinterpret_cast<float*>(smem + SM::NRM) + 256;  // [2][2][64]
  float* sbeta = reinterpret_cast<float*>(smem + SM::BETA);        // [64]
  float* red = reinterpret_cast<float*>(smem + SM::RED);           // [8]
  int* guard = reinterpret_cast<int*>(smem + SM::RED) + 8;

  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int w = wv & 3;          // token block
  const int hf = wv >> 2;        // channel half
  const int l = tid & 63;
  const int t = l & 15;
  const int gq = l >> 4;
  const int i_loc = 16 * w + t;  // this lane's token row inside the chunk
  const int cb = hf * (DK / 2);  // first key channel of the half
  const int sb = hf * KH;        // first key step of the half
  const bool paired = chunk2 >= 0;                 // workgroup-uniform
  const bool hi_half = paired && w >= 2;           // this wave's rows belong to chunk2
  uint8_t* rec = a.rec + ((size_t)chunk * a.H + h) * R::BYTES;
  uint8_t* rec2 = paired ? a.rec + ((size_t)chunk2 * a.H + h) * R::BYTES : rec;
  uint8_t* recw = hi_half ? rec2 : rec;            // this wave's record
  const int wr = hi_half ? w - 2 : w;              // this wave's row block there
  // valid tokens of this wave's chunk: the parts of its record past them are not stored.  The
  // fused kernel (fixed-length rows: at most one partial chunk per row) stores every part: its
  // walk bounds the launch, and the length lookup per item cost it more (about 1.5 %) than the
  // few empty parts it would drop (the scan may skip loading a part that was stored: it is zero)
  const int rows_w = WT ? kChunk : chunk_rows(a, hi_half ? chunk2 : chunk);

  // reads the lane's NE channels (of this half) of row `row` of a [*][DK] fp32 array in LDS
  auto lane_row = [&](const float* base, int row, float* out) {
    const float* p = base + row * DK + cb;
#pragma unroll
    for (int j = 0; j < 2 * KH; ++j) {
      const float4 r4 = *reinterpret_cast<const float4*>(p + 16 * j + 4 * gq);
      out[4 * j + 0] = r4.x; out[4 * j + 1] = r4.y; out[4 * j + 2] = r4.z; out[4 * j + 3] = r4.w;
    }
  };

  // reads the lane's 8 channels of (global) k-step s of row `row` (indices 8 s .. 8 s + 7)
  auto lane_step = [&](const float* base, int row, int s, float* out8) {
    const float* p = base + row * DK + 32 * s + 4 * gq;
    const float4 lo = *reinterpret_cast<const float4*>(p);
    const float4 hi = *reinterpret_cast<const float4*>(p + 16);
    out8[0] = lo.x; out8[1] = lo.y; out8[2] = lo.z; out8[3] = lo.w;
    out8[4] = hi.x; out8[5] = hi.y; out8[6] = hi.z; out8[7] = hi.w;
  };

  // ---------------- (a) norms, cumulative gate ----------------
  // Lane (token 16w + t, quarter gq) holds channels 32 (sb + s) + pi_index(gq, e) at index 8 s + e.
  float* xq = in.q;
  float* xk = in.k;
  float* G = in.g;
  float* xv = in.v;
  const float bt = in.beta;

  // half-row L2 norm partials (4 lanes share a token: lanes t, t+16, t+32, t+48); every
  // conditional store of this phase comes after all of its arithmetic, so the q, k, gate
  // and v chains form one block that the compiler can interleave
  auto half_norm = [&](float* x, int& ex) {
    float m = 0.f;
#pragma unroll
    for (int e = 0; e < NE; ++e) m = fmaxf(m, fabsf(x[e]));
    m = rows4_max(m);
    ex = (m > 0.f) ? ilogb_pos(m) : kNoExp;
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      x[e] = ldexpf(x[e], -ex);
      ss = fmaf(x[e], x[e], ss);
    }
    return rows4_sum(ss);
  };
  // both halves at the larger exponent, then x * 2^(ex - exm) / ||row||
  auto finish_norm = [&](float* x, int which, int ex, float ss) {
    const int ex_p = nrm_ex[(which * 2 + (hf ^ 1)) * 64 + i_loc];
    const float ss_p = nrm_ss[(which * 2 + (hf ^ 1)) * 64 + i_loc];
    const int exm = ex > ex_p ? ex : ex_p;
    const float tot = ldexpf(ss, 2 * (ex - exm)) + ldexpf(ss_p, 2 * (ex_p - exm));
    // tot >= 1 (the larger half's entries were scaled to [1, 2)): the hardware reciprocal
    // square root (about 1 ulp) is far inside the fp16 operand rounding that follows
    const float f = (tot > 0.f) ? ldexpf(__builtin_amdgcn_rsqf(tot), ex - exm) : 0.f;
#pragma unroll
    for (int e = 0; e < NE; ++e) x[e] *= f;
  };
  int exq, exk;
  const float ssq = half_norm(xq, exq);
  const float ssk = half_norm(xk, exk);

  // cumulative log2-gate inside the 16-token block (rows of 16 lanes), then block offsets
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    float x = G[e];
    x += row_shr<1>(x);
    x += row_shr<2>(x);
    x += row_shr<4>(x);
    x += row_shr<8>(x);
    G[e] = x;
  }
  float vm = 0.f;
#pragma unroll
  for (int e = 0; e < NEV; ++e) vm = fmaxf(vm, fabsf(xv[e]));
  vm = wave_max(vm);

  if (gq == 0) {
    nrm_ex[(0 * 2 + hf) * 64 + i_loc] = exq;
    nrm_ss[(0 * 2 + hf) * 64 + i_loc] = ssq;
    nrm_ex[(1 * 2 + hf) * 64 + i_loc] = exk;
    nrm_ss[(1 * 2 + hf) * 64 + i_loc] = ssk;
    if (hf == 0) sbeta[i_loc] = bt;
  }
  if (t == 15) {
#pragma unroll
    for (int j = 0; j < 2 * KH; ++j)
      *reinterpret_cast<float4*>(btot + w * DK + cb + 16 * j + 4 * gq) =
          make_float4(G[4 * j], G[4 * j + 1], G[4 * j + 2], G[4 * j + 3]);
  }
  if (l == 0) red[wv] = vm;
  if (tid == 0) *guard = 0;
  __syncthreads();  // #1: block totals, norm partials, max |v|
  mid(1);
  finish_norm(xq, 0, exq, ssq);
  finish_norm(xk, 1, exk, ssk);
#pragma unroll
  for (int j = 0; j < 2 * KH; ++j) {
    // totals of the earlier 16-token blocks, added in block order
    // (every row is read and the later ones masked, so this stays one block without branches)
    float4 off = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int b = 0; b < 3; ++b) {
      const float4 bt4 = *reinterpret_cast<const float4*>(btot + b * DK + cb + 16 * j + 4 * gq);
      const bool use = b < w && (!hi_half || b >= 2);  // a second chunk's sum starts at its row 0
      off.x += use ? bt4.x : 0.f; off.y += use ? bt4.y : 0.f;
      off.z += use ? bt4.z : 0.f; off.w += use ? bt4.w : 0.f;
    }
    G[4 * j + 0] += off.x; G[4 * j + 1] += off.y; G[4 * j + 2] += off.z; G[4 * j + 3] += off.w;
  }
  float vmax = red[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) vmax = fmaxf(vmax, red[i]);
  const int ue = (vmax > 0.f) ? 12 - (ilogb_pos(vmax) + 1) : 0;
  // beta v 2^ue rows in fp16 (|.| < 2^12)
  f16x8 vr[VH];
#pragma unroll
  for (int s = 0; s < VH; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) vr[s][e] = (_Float16)(bt * ldexpf(xv[8 * s + e], ue));
  if ((t & 3) == 3) {
#pragma unroll
    for (int j = 0; j < 2 * KH; ++j)
      *reinterpret_cast<float4*>(gend + (4 * w + (t >> 2)) * DK + cb + 16 * j + 4 * gq) =
          make_float4(G[4 * j], G[4 * j + 1], G[4 * j + 2], G[4 * j + 3]);
  }
  // j*: the last token with beta > 0 (-1: none).  Tokens after it write nothing (their
  // Delta rows are exactly zero), so the rows of the state-update operand
  // Khat*exp(G_last - G) are scaled by the largest factor that still multiplies a nonzero
  // Delta row, exp(G_last - G_j*) per channel: with deep decays and beta = 0 at the end of
  // a chunk, the entries that carry the new state would otherwise fall below fp16's range.
  // (two chunks in the pass: j* of each, the second's in gend row 17)
  const uint64_t bmask = __ballot(sbeta[l] > 0.f);
  const uint64_t bm1 = paired ? (bmask & 0xffffffffull) : bmask, bm2 = paired ? (bmask >> 32) : 0;
  const int jstar = bm1 ? 63 - __builtin_clzll(bm1) : -1;          // wave-uniform
  const int jstar2 = bm2 ? 32 + 63 - __builtin_clzll(bm2) : -1;    // wave-uniform
  const int jrow = hi_half ? jstar2 : jstar;                          // j* of this wave's chunk
  if (i_loc == jrow) {
#pragma unroll
    for (int j = 0; j < 2 * KH; ++j)
      *reinterpret_cast<float4*>(gend + (hi_half ? 17 : 16) * DK + cb + 16 * j + 4 * gq) =
          make_float4(G[4 * j], G[4 * j + 1], G[4 * j + 2], G[4 * j + 3]);
  }
  __syncthreads();  // #2: group-end gates visible, block totals and norm partials consumed
  mid(2);

  // decay-factor table and the guard of the fp32 diagonal path
  if (tid < DK) {
    const int c = tid;
    auto ge = [&](int p) { return p < 0 ? 0.f : gend[p * DK + c]; };
    // G_last of the chunk (of each chunk of a pair: end of row 31, end of row 63)
    const float glast = paired ? ge(7) : ge(15), glast2 = ge(15);
    // row exponent of Khat*exp(G_last - G): 2^-ec times every entry up to token j* stays
    // below 2 (|khat| <= 1, exp(G_last - G_j) <= exp(G_last - G_j*) for j <= j*)
    const int ec = jstar >= 0 ? max(-126, (int)floorf(glast - gend[16 * DK + c])) : 0;
    const int ec2 = jstar2 >= 0 ? max(-126, (int)floorf(glast2 - gend[17 * DK + c])) : 0;
    int bad = 0;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const bool second = paired && ww >= 2;  // a block of the pair's second chunk
      const float gp = (paired && ww == 2) ? 0.f : ge(4 * ww - 1), gn = ge(4 * ww + 3), gm = ge(4 * ww + 1);
      et[ww * DK + c] = exp2_hw(gp);
      et[(4 + ww) * DK + c] = exp2_hw((second ? glast2 : glast) - gn - (float)(second ? ec2 : ec));
      const float d1 = gp - gm, d2 = gm - gn;
      if (!(d1 <= kGuardLog2 && d2 <= kGuardLog2)) bad = 1;
      et[(11 + ww) * DK + c] = exp2_hw(fminf(d1, kGuardLog2));
      et[(15 + ww) * DK + c] = exp2_hw(fminf(d2, kGuardLog2));
    }
    et[8 * DK + c] = exp2_hw(ge(7) - ge(3));
    et[9 * DK + c] = exp2_hw(ge(11) - ge(3));
    et[10 * DK + c] = exp2_hw(ge(11) - ge(7));
    if (bad) atomicOr(guard, 1);
    rec_store<WT, R::BYTES>(rec, R::LAM + (size_t)c * 8, uint2_v{__float_as_uint(exp2_hw(glast)), (uint32_t)ec});
    if (paired)
      rec_store<WT, R::BYTES>(rec2, R::LAM + (size_t)c * 8, uint2_v{__float_as_uint(exp2_hw(glast2)), (uint32_t)ec2});
  }
  // operand bases: rows khat_i exp(G_i - Gprev(w)) and qhat_i exp(G_i - Gprev(w)),
  // columns khat_j exp(Gnext(w) - G_j); all factors <= 1
  float XB[NE], QB[NE], YC[NE];
  {
    float gp[NE], gn[NE];
    lane_row(gend, 4 * w + 3, gn);
    lane_row(gend, w > 0 ? 4 * w - 1 : 0, gp);  // read always, zero for a chunk's block 0: no branch
    const bool first_block = w == 0 || (paired && w == 2);
#pragma unroll
    for (int e = 0; e < NE; ++e) gp[e] = first_block ? 0.f : gp[e];
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const float fb = exp2_hw(G[e] - gp[e]);
      const float fc = exp2_hw(gn[e] - G[e]);
      XB[e] = xk[e] * fb;
      QB[e] = xq[e] * fb;
      YC[e] = xk[e] * fc;
    }
  }
  __syncthreads();  // #3: table and guard visible
  if (!EXACT) {
    // A diagonal tile spans more decay than the fp32 path covers: the item is flagged
    // and redone by the exact variant, which rewrites its record.  This variant still
    // runs to the end, so every item issues the same memory operations.
    if (tid == 0) {
      a.defer[(size_t)chunk * a.H + h] = *guard;
      if (paired) a.defer[(size_t)chunk2 * a.H + h] = *guard;
    }
  }

  // identity fragments: B[k][n] = 1 iff the channel of slot k is 16*hh + n of the step
  f16x8 ident[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      ident[hh][e] = (_Float16)(((t >> 2) == gq && e == 4 * hh + (t & 3)) ? 1.f : 0.f);

  // ---------------- outputs that need only G ----------------
  f16x8 bwr[KH];
  {
#pragma unroll
    for (int sl = 0; sl < KH; ++sl) {
      const int s = sb + sl;
      float eS[8], eE[8];
      lane_step(et, w, s, eS);
      lane_step(et, 4 + w, s, eE);
      f16x8 qf, kf, y;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qf[e] = (_Float16)(QB[8 * sl + e] * eS[e]);          // qhat exp(G)
        kf[e] = (_Float16)(i_loc <= jrow ? YC[8 * sl + e] * eE[e] : 0.f);  // khat exp(G_last - G) 2^-ec
        bwr[sl][e] = (_Float16)(bt * XB[8 * sl + e] * eS[e]); // beta khat exp(G)
        y[e] = (_Float16)YC[8 * sl + e];
      }
      rec_store<WT, R::BYTES>(recw, R::Q + ((size_t)(wr * KSK + s) * 64 + l) * 16, qf, rec_rows_present(rows_w, wr));
      // K~^T fragments: (K~ I) holds, per lane, key channel 16 ct + t at tokens 16 w + 4 gq + r,
      // ct = 2 s + hh.  The 16-byte record fragment of (ct, token pair w / 2) joins the halves of
      // token blocks 2 (w / 2) and 2 (w / 2) + 1: both go to LDS here, and after barrier #4 each
      // wave of the pair stores half of the pair's fragments whole (one 16-byte store per lane).
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const f32x4 c = mfma16(kf, ident[hh], zero4());
        const int j = 2 * sl + hh;
        f16x4 h4 = {(_Float16)c[0], (_Float16)c[1], (_Float16)c[2], (_Float16)c[3]};
        ktx[((((hf * 2 + (w >> 1)) * 2 + (w & 1)) * (2 * KH) + j) * 64) + l] = h4;
      }
      // column-side operands of the off-diagonal Gram tiles (reference = end of block w)
      ybf[(w * KSK + s) * 64 + l] = y;  // block 3's slot is never read (no branch around the store)
    }
    // Bu fragments (beta v 2^ue, rows = value channels, tokens in pi order)
#pragma unroll
    for (int svl = 0; svl < VH; ++svl) {
      const int sv = hf * VH + svl;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const f32x4 c = mfma16(vr[svl], ident[hh], zero4());
        f16x4 h4 = {(_Float16)c[0], (_Float16)c[1], (_Float16)c[2], (_Float16)c[3]};
        *reinterpret_cast<f16x4*>(bux + ((size_t)((2 * sv + hh) * 2 + (w >> 1)) * 64 + l) * 16 + (w & 1) * 8) = h4;
      }
    }
    if (tid == 0) {
      rec_store<WT, R::BYTES>(rec, R::HDR, vmax);
      rec_store<WT, R::BYTES>(rec, R::HDR + 4, ue);
      if (paired) {  // the pair's max |v| bounds both chunks; U of both uses the same ue
        rec_store<WT, R::BYTES>(rec2, R::HDR, vmax);
        rec_store<WT, R::BYTES>(rec2, R::HDR + 4, ue);
      }
    }
  }
  __syncthreads();  // #4: column operands visible
  mid(3);

  // whole K~^T fragments: this wave of the pair stores j = (w & 1) KH .. (w & 1) KH + KH - 1
#pragma unroll
  for (int jj = 0; jj < KH; ++jj) {
    const int j = (w & 1) * KH + jj;             // wave-uniform
    const int ct = 2 * (sb + (j >> 1)) + (j & 1);
    const f16x4 lo = ktx[((((hf * 2 + (w >> 1)) * 2 + 0) * (2 * KH) + j) * 64) + l];
    const f16x4 hi = ktx[((((hf * 2 + (w >> 1)) * 2 + 1) * (2 * KH) + j) * 64) + l];
    const f16x8 frag = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    // (a pair: token half w / 2 is a whole chunk, its record's first half)
    const int s2k = paired ? 0 : (w >> 1);
    rec_store<WT, R::BYTES>(recw, R::KT + ((size_t)(ct * 2 + s2k) * 64 + l) * 16, frag, rec_half_present(rows_w, s2k));
  }

  // ---------------- (b) Gram matrices L (row block w) and Aqk^T (column block w) ----------------
  // Partial sums over this half's channels.  offL[b]: L tile (w, b) and offA[b]: Aqk^T
  // tile (b, w) for b < w; dL, dA: the diagonal tiles.
  f32x4 offL[3], offA[3], dL = zero4(), dA = zero4();
#pragma unroll
  for (int b = 0; b < 3; ++b) { offL[b] = zero4(); offA[b] = zero4(); }

  // off-diagonal tiles (w, b), b < w: reference r = end of block b.
  // Row factor exp(G_i - Gnext(b)) = exp(G_i - Gprev(w)) * exp(Gprev(w) - Gnext(b)).
#pragma unroll
  for (int b = 0; b < 3; ++b) {
    if (b < w && !(hi_half && b < 2)) {  // tiles across a pair's two chunks stay zero
      const int trow = 8 + (b == 0 ? (w == 2 ? 0 : 1) : 2);
#pragma unroll
      for (int sl = 0; sl < KH; ++sl) {
        const int s = sb + sl;
        float fr[8];
        if (b == w - 1) {
#pragma unroll
          for (int e = 0; e < 8; ++e) fr[e] = 1.f;
        } else {
          lane_step(et, trow, s, fr);
        }
        f16x8 xk8, xq8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          xk8[e] = (_Float16)(XB[8 * sl + e] * fr[e]);
          xq8[e] = (_Float16)(QB[8 * sl + e] * fr[e]);
        }
        const f16x8 yb = ybf[(b * KSK + s) * 64 + l];
        offL[b] = mfma16(xk8, yb, offL[b]);
        offA[b] = mfma16(yb, xq8, offA[b]);
      }
    }
  }

  if (!EXACT) {
    // diagonal tile in one product around the tile's middle row m = 16w + 7:
    // rows exp(G_i - G_m) = exp(G_i - Gprev) exp(Gprev - G_m),
    // columns exp(G_m - G_j) = exp(Gnext - G_j) exp(G_m - Gnext).
    // Both half-span factors are >= 1; when every one of this wave's channels keeps
    // them <= 2^11 the operands fit fp16 (|.| <= 2^11) and the tile takes two fp16
    // MFMA steps, otherwise fp32 MFMA (factors up to the guard's 2^115).
    float er[KH][8], ec[KH][8];
    bool wide = false;
#pragma unroll
    for (int sl = 0; sl < KH; ++sl) {
      lane_step(et, 11 + w, sb + sl, er[sl]);
      lane_step(et, 15 + w, sb + sl, ec[sl]);
#pragma unroll
      for (int e = 0; e < 8; ++e) wide |= (er[sl][e] > 2048.f) | (ec[sl][e] > 2048.f);
    }
    if (__any(wide)) {
#pragma unroll
      for (int sl = 0; sl < KH; ++sl)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float xkr = XB[8 * sl + e] * er[sl][e], xqr = QB[8 * sl + e] * er[sl][e];
          const float ykc = YC[8 * sl + e] * ec[sl][e];
          dL = __builtin_amdgcn_mfma_f32_16x16x4f32(xkr, ykc, dL, 0, 0, 0);
          dA = __builtin_amdgcn_mfma_f32_16x16x4f32(ykc, xqr, dA, 0, 0, 0);
        }
    } else {
#pragma unroll
      for (int sl = 0; sl < KH; ++sl) {
        f16x8 xk8, xq8, yc8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          xk8[e] = (_Float16)(XB[8 * sl + e] * er[sl][e]);
          xq8[e] = (_Float16)(QB[8 * sl + e] * er[sl][e]);
          yc8[e] = (_Float16)(YC[8 * sl + e] * ec[sl][e]);
        }
        dL = mfma16(xk8, yc8, dL);
        dA = mfma16(yc8, xq8, dA);
      }
    }
    // keep L strictly below the diagonal and Aqk on and below it
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * gq + r;
      if (!(row > t)) dL[r] = 0.f;   // L tile: lane column j = t, row i
      if (!(row <= t)) dA[r] = 0.f;  // Aqk^T tile: lane column i = t, row j
    }
  } else {
    // exact at any gate depth: pairs in different 4-token groups use the end of the
    // column group as reference; pairs inside a group use products of exp(g)
    const int grp = t >> 2;
    float gown[NE];
    lane_row(gend, 4 * w + grp, gown);
    f16x8 yg[KH];  // khat_j * exp(Gend(group j) - G_j)
#pragma unroll
    for (int sl = 0; sl < KH; ++sl)
#pragma unroll
      for (int e = 0; e < 8; ++e) yg[sl][e] = (_Float16)(xk[8 * sl + e] * exp2_hw(gown[8 * sl + e] - G[8 * sl + e]));
#pragma unroll
    for (int qg = 0; qg < 3; ++qg) {
      float gr[NE];
      lane_row(gend, 4 * w + qg, gr);
      const bool col_in = (grp == qg);   // this lane's token as a column of group qg
      const bool row_in = (grp > qg);    // this lane's token as a row after group qg
#pragma unroll
      for (int sl = 0; sl < KH; ++sl) {
        f16x8 xk8, xq8, ym;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float f = row_in ? exp2_hw(G[8 * sl + e] - gr[8 * sl + e]) : 0.f;
          xk8[e] = (_Float16)(xk[8 * sl + e] * f);
          xq8[e] = (_Float16)(xq[8 * sl + e] * f);
          ym[e] = col_in ? yg[sl][e] : (_Float16)0.f;
        }
        dL = mfma16(xk8, ym, dL);
        dA = mfma16(ym, xq8, dA);
      }
    }
    f32x4 bandL[3], bandA[3];
#pragma unroll
    for (int d = 0; d < 3; ++d) { bandL[d] = zero4(); bandA[d] = zero4(); }
    float adiag = 0.f;
#pragma unroll
    for (int sl = 0; sl < KH; ++sl) {
      f16x8 kk;
      float al[8], p1[8], p2[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float gi = G[8 * sl + e];
        al[e] = exp2_hw(gi - row_shr<1>(gi));   // exp(g_i) (lane t-1 holds token i-1)
        kk[e] = (_Float16)xk[8 * sl + e];
        adiag = fmaf(xq[8 * sl + e], xk[8 * sl + e], adiag);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p1[e] = al[e] * row_shr<1>(al[e]);       // exp(G_i - G_{i-2})
        p2[e] = p1[e] * row_shr<2>(al[e]);       // exp(G_i - G_{i-3})
      }
      f16x8 k1, q1, k2, q2, k3, q3;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        k1[e] = (_Float16)(xk[8 * sl + e] * al[e]);
        q1[e] = (_Float16)(xq[8 * sl + e] * al[e]);
        k2[e] = (_Float16)(xk[8 * sl + e] * p1[e]);
        q2[e] = (_Float16)(xq[8 * sl + e] * p1[e]);
        k3[e] = (_Float16)(xk[8 * sl + e] * p2[e]);
        q3[e] = (_Float16)(xq[8 * sl + e] * p2[e]);
      }
      bandL[0] = mfma16(k1, kk, bandL[0]);
      bandL[1] = mfma16(k2, kk, bandL[1]);
      bandL[2] = mfma16(k3, kk, bandL[2]);
      bandA[0] = mfma16(kk, q1, bandA[0]);
      bandA[1] = mfma16(kk, q2, bandA[1]);
      bandA[2] = mfma16(kk, q3, bandA[2]);
    }
    adiag = rows4_sum(adiag);
    // L tile (w,w): lane (col j = t, rows 4gq + r); keep (i = j + d) inside j's group
    // Aqk^T tile (w,w): lane (col i = t, rows j = 4gq + r); keep (j = i - d) inside i's group
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * gq + r;
#pragma unroll
      for (int d = 1; d <= 3; ++d) {
        if (row == t + d && (row >> 2) == (t >> 2)) dL[r] += bandL[d - 1][r];
        if (row == t - d && (row >> 2) == (t >> 2)) dA[r] += bandA[d - 1][r];
      }
      if (row == t) dA[r] += adiag;
    }
  }

  // tile b (<= w) of this wave's row block of L, or of its column block of Aqk^T
  auto tileL = [&](int b) -> f32x4 {
    f32x4 x = dL;
#pragma unroll
    for (int bb = 0; bb < 3; ++bb) x = (bb == b && b < w) ? offL[bb] : x;
    return x;
  };
  auto tileA = [&](int b) -> f32x4 {
    f32x4 x = dA;
#pragma unroll
    for (int bb = 0; bb < 3; ++bb) x = (bb == b && b < w) ? offA[bb] : x;
    return x;
  };
  // The two halves' partial tiles meet in LDS: half 0 completes L, half 1 completes Aqk.
  // (tiles above block w are written too, into slots nobody reads: no branches here)
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    float* dst = (hf == 1 ? gpl : gpa) + ((w * 4 + b) * 64 + l) * 4;
    *reinterpret_cast<f32x4*>(dst) = (hf == 1) ? tileL(b) : tileA(b);
  }
  __syncthreads();  // #5a: partial tiles visible; every wave is past the column operands

  if (hf == 0) {
    // A = diag(beta) L into LDS (blocks (w, b <= w)).  The blocks above the diagonal get
    // values nobody reads before the doubling steps overwrite them (their scratch), so
    // every block is written without a branch.
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const f32x4 p = *reinterpret_cast<const f32x4*>(gpl + ((w * 4 + b) * 64 + l) * 4);
      const f32x4 own = tileL(b);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * w + 4 * gq + r;
        Lm[i * LP + 16 * b + t] = sbeta[i] * (own[r] + p[r]);
      }
    }
  } else {
    // Aqk A-fragments for row block w: slots (rows of Aqk^T tile (2 s2, w), rows of tile (2 s2 + 1, w))
    f32x4 full[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {  // zero above the diagonal (selected, not branched)
      const f32x4 p = *reinterpret_cast<const f32x4*>(gpa + ((w * 4 + b) * 64 + l) * 4);
      const f32x4 own = tileA(b);
#pragma unroll
      for (int r = 0; r < 4; ++r) full[b][r] = (b <= w) ? own[r] + p[r] : 0.f;
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      f16x8 f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        f[r] = (_Float16)full[2 * s2][r];
        f[4 + r] = (_Float16)full[2 * s2 + 1][r];
      }
      // a pair's second chunk: its columns are the pass's second half (s2 = 1), its record's first
      const int s2r = hi_half ? s2 ^ 1 : s2;
      // (row blocks 0 and 1 are zero in the second column half: not stored, never read)
      rec_store<WT, R::BYTES>(recw, R::A + ((size_t)(wr * 2 + s2r) * 64 + l) * 16, f,
                              rec_rows_present(rows_w, wr) && rec_half_present(rows_w, s2r) && (s2r == 0 || wr >= 2));
    }
  }
  // Bw^T fragments through identity products (rows = key channels, tokens in pi order)
#pragma unroll
  for (int sl = 0; sl < KH; ++sl)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int s = sb + sl;
      const f32x4 c = mfma16(bwr[sl], ident[hh], zero4());
      f16x4 h4 = {(_Float16)c[0], (_Float16)c[1], (_Float16)c[2], (_Float16)c[3]};
      *reinterpret_cast<f16x4*>(bwx + ((size_t)((2 * s + hh) * 2 + (w >> 1)) * 64 + l) * 16 + (w & 1) * 8) = h4;
    }
  __syncthreads();  // #5: L complete; table consumed

  // ---------------- (b) Tinv = (I + A)^-1, blocked ----------------
  if (hf == 0) {
    // diagonal block w by substitution, one whole wave: lane (row i = t, quarter gq) holds
    // Tinv[i][4 gq + r]; row j is final after the updates from rows 0..j-1 and is then
    // broadcast along each row of 16 lanes to the rows below it (A is zero on and above
    // the diagonal, so the other rows keep their values)
    const float* arow = Lm + (16 * w + t) * LP + 16 * w;
    float am[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 a4 = *reinterpret_cast<const float4*>(arow + 4 * q);
      am[4 * q + 0] = -a4.x; am[4 * q + 1] = -a4.y; am[4 * q + 2] = -a4.z; am[4 * q + 3] = -a4.w;
    }
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = (t == 4 * gq + r) ? 1.f : 0.f;
    subst_rows<0>(x, am);
    *reinterpret_cast<float4*>(Tm + (16 * w + t) * LP + 16 * w + 4 * gq) = make_float4(x[0], x[1], x[2], x[3]);
  }
  __syncthreads();  // #6
  // Off-diagonal blocks by doubling, on fp32 MFMA (16x16 blocks, D_a = Tinv_aa):
  //   inverse of a 32x32 half: [[D0, 0], [-D1 A10 D0, D1]]
  //   inverse of the whole:    [[T1, 0], [-T2 A21 T1, T2]]   (T1, T2 the half inverses,
  //                            A21 the lower-left 32x32 quarter of A)
  // with Y = A21 T1 formed first.  Y goes to the free upper blocks of the L buffer.
  {
    float* Y00 = Lm + 0 * LP + 16;   // Y blocks (row block, column block) of A21 T1
    float* Y01 = Lm + 0 * LP + 32;
    float* Y10 = Lm + 0 * LP + 48;
    float* Y11 = Lm + 16 * LP + 32;
    auto blk = [&](float* base, int rb, int cb2) { return base + 16 * rb * LP + 16 * cb2; };
    // c + Lf Rf with Lf read by rows from LDS and Rf either from LDS or a C-layout tile
    auto mm_lds = [&](const float* Lf, const float* Rf, f32x4 c) {
      const float4 lr = *reinterpret_cast<const float4*>(Lf + t * LP + 4 * gq);
      const float lv[4] = {lr.x, lr.y, lr.z, lr.w};
#pragma unroll
      for (int p = 0; p < 4; ++p) c = __builtin_amdgcn_mfma_f32_16x16x4f32(lv[p], Rf[(4 * gq + p) * LP + t], c, 0, 0, 0);
      return c;
    };
    auto mm_reg = [&](const float* Lf, const f32x4& Rc, f32x4 c) {
      const float4 lr = *reinterpret_cast<const float4*>(Lf + t * LP + 4 * gq);
      const float lv[4] = {lr.x, lr.y, lr.z, lr.w};
#pragma unroll
      for (int p = 0; p < 4; ++p) c = __builtin_amdgcn_mfma_f32_16x16x4f32(lv[p], Rc[p], c, 0, 0, 0);
      return c;
    };
    auto put = [&](float* dst, const f32x4& c, float sgn) {
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(4 * gq + r) * LP + t] = sgn * c[r];
    };
    f32x4 y = zero4();
    if (wv == 0) {         // T10 = -D1 A10 D0
      const f32x4 pq = mm_lds(blk(Lm, 1, 0), blk(Tm, 0, 0), zero4());
      put(blk(Tm, 1, 0), mm_reg(blk(Tm, 1, 1), pq, zero4()), -1.f);
    } else if (wv == 1) {  // T32 = -D3 A32 D2
      const f32x4 pq = mm_lds(blk(Lm, 3, 2), blk(Tm, 2, 2), zero4());
      put(blk(Tm, 3, 2), mm_reg(blk(Tm, 3, 3), pq, zero4()), -1.f);
    } else if (wv == 2) {  // Y01 = A21 D1
      put(Y01, mm_lds(blk(Lm, 2, 1), blk(Tm, 1, 1), zero4()), 1.f);
    } else if (wv == 3) {  // Y11 = A31 D1
      put(Y11, mm_lds(blk(Lm, 3, 1), blk(Tm, 1, 1), zero4()), 1.f);
    } else if (wv == 4) {  // Y00 = A20 D0 + A21 T10 (first term)
      y = mm_lds(blk(Lm, 2, 0), blk(Tm, 0, 0), zero4());
    } else if (wv == 5) {  // Y10 = A30 D0 + A31 T10 (first term)
      y = mm_lds(blk(Lm, 3, 0), blk(Tm, 0, 0), zero4());
    }
    __syncthreads();  // #7: T10, T32, Y01, Y11 visible
    if (wv == 4) put(Y00, mm_lds(blk(Lm, 2, 1), blk(Tm, 1, 0), y), 1.f);
    if (wv == 5) put(Y10, mm_lds(blk(Lm, 3, 1), blk(Tm, 1, 0), y), 1.f);
    __syncthreads();  // #8: Y complete
    // [T20 T21; T30 T31] = -[[D2, 0], [T32, D3]] Y
    if (wv == 0) put(blk(Tm, 2, 0), mm_lds(blk(Tm, 2, 2), Y00, zero4()), -1.f);
    if (wv == 1) put(blk(Tm, 2, 1), mm_lds(blk(Tm, 2, 2), Y01, zero4()), -1.f);
    if (wv == 2) put(blk(Tm, 3, 0), mm_lds(blk(Tm, 3, 3), Y10, mm_lds(blk(Tm, 3, 2), Y00, zero4())), -1.f);
    if (wv == 3) put(blk(Tm, 3, 1), mm_lds(blk(Tm, 3, 3), Y11, mm_lds(blk(Tm, 3, 2), Y01, zero4())), -1.f);
    __syncthreads();  // #9: Tinv complete
  }

  // ---------------- (b) W = Tinv Bw (as W^T tiles) and U = Tinv Bu ----------------
  {
    // Tinv row 16w + t at the tokens of the pi-ordered slots of step s
    f16x8 tf[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const float* trow = Tm + (16 * w + t) * LP + 32 * s + 4 * gq;
      const float4 lo = *reinterpret_cast<const float4*>(trow);
      const float4 hi = *reinterpret_cast<const float4*>(trow + 16);
      const bool klo = (2 * s <= w), khi = (2 * s + 1 <= w);
      tf[s][0] = (_Float16)(klo ? lo.x : 0.f); tf[s][1] = (_Float16)(klo ? lo.y : 0.f);
      tf[s][2] = (_Float16)(klo ? lo.z : 0.f); tf[s][3] = (_Float16)(klo ? lo.w : 0.f);
      tf[s][4] = (_Float16)(khi ? hi.x : 0.f); tf[s][5] = (_Float16)(khi ? hi.y : 0.f);
      tf[s][6] = (_Float16)(khi ? hi.z : 0.f); tf[s][7] = (_Float16)(khi ? hi.w : 0.f);
    }
#pragma unroll
    for (int skl = 0; skl < KH; ++skl) {
      const int sk = sb + skl;
      f32x4 c0 = zero4(), c1 = zero4();
#pragma unroll
      for (int s = 0; s < 2; ++s) {  // tf[1] is zero for blocks 0 and 1: no branch needed
        const f16x8 a0 = *reinterpret_cast<const f16x8*>(bwx + ((size_t)((2 * sk) * 2 + s) * 64 + l) * 16);
        const f16x8 a1 = *reinterpret_cast<const f16x8*>(bwx + ((size_t)((2 * sk + 1) * 2 + s) * 64 + l) * 16);
        c0 = mfma16(a0, tf[s], c0);
        c1 = mfma16(a1, tf[s], c1);
      }
      f16x8 wf = {(_Float16)c0[0], (_Float16)c0[1], (_Float16)c0[2], (_Float16)c0[3],
                  (_Float16)c1[0], (_Float16)c1[1], (_Float16)c1[2], (_Float16)c1[3]};
      rec_store<WT, R::BYTES>(recw, R::W + ((size_t)(wr * KSK + sk) * 64 + l) * 16, wf, rec_rows_present(rows_w, wr));
    }
#pragma unroll
    for (int ntl = 0; ntl < NTV / 2; ++ntl) {
      const int nt = hf * (NTV / 2) + ntl;
      f32x4 c = zero4();
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const f16x8 bfr = *reinterpret_cast<const f16x8*>(bux + ((size_t)(nt * 2 + s) * 64 + l) * 16);
        c = mfma16(tf[s], bfr, c);
      }
      f16x4 uf = {(_Float16)c[0], (_Float16)c[1], (_Float16)c[2], (_Float16)c[3]};
      rec_store<WT, R::BYTES>(recw, R::U + ((size_t)(wr * NTV + nt) * 64 + l) * 8, uf, rec_rows_present(rows_w, wr));
    }
  }
}

// Persistent workgroups walk the items x = chunk position * H + head slot, workgroup
// b taking x = b, b + grid, ...: the workgroups in flight read whole token rows (all
// heads) of q, k, v and g and write adjacent records.  Chunks go from the last to the
// first; the head of slot s at chunk position p is (s + p) mod H, so that a workgroup
// meets every head as it walks (items flagged for the exact pass, often whole heads,
// then spread evenly over the workgroups).  The next item's loads are issued as soon
// as the current item's inputs sit in registers.
//
// The loads of the next item are issued unconditionally (the last item re-reads its
// own inputs) and unpacked after the current item's record stores, so that on every
// path the same number of stores follows them: waiting for the loads then does not
// wait for the stores (one in-order counter covers both).
//
// After its walk, each workgroup redoes its own flagged items with the exact variant.
//
// FUSED (the chunk role of the fused forward kernel, fixed-length rows only): the walk
// goes in the order the scan consumes, every row's first chunk first, and each record is
// published (device-scope release, then its flag) as soon as it is final: right after
// its item, or after the exact pass for a flagged item.
//
// Schedule: workgroup wg takes items wg + j n_wg.  With `rounds` > 0 (the fused kernel) the
// first `rounds` rounds go over all n_all workgroups of the launch, the scan workgroups
// (wg >= n_wg) included, which walk only those rounds before their chains start (their
// chains would wait that long for the first records anyway); the later rounds go over the
// n_wg chunk workgroups.  4,096 items on 192 + 64 workgroups: one item each in the first
// round, then 20 more for each chunk workgroup (instead of 21 or 22).
template <int DK, int DV, typename InT, bool FUSED>
__device__ __forceinline__ void chunk_walk(const PrepArgs& a, const FuseArgs& fz, const int wg, const int n_wg,
                                           uint8_t* smem, const int n_all = 0, const int rounds = 0) {
  // items (fewer than 2^31), kept in scalar registers; packed batches walk the passes
  // (a pass: one chunk, or two chunks of at most 32 tokens)
  const int n_rows = (int)(a.T_total / (a.T > 0 ? a.T : 1));
  const int n_items = (a.cu ? (int)sload_u32(a.info + 3) : (int)(a.nc * n_rows)) * a.H;
  const int R = n_all > n_wg ? n_all : n_wg;
  auto item_of = [&](int j) { return j < rounds ? j * R + wg : rounds * R + wg + (j - rounds) * n_wg; };
  // this workgroup's items: item_of(0) .. item_of(n_own - 1)
  int n_own;
  {
    const int k1 = n_items > wg ? (n_items - wg + R - 1) / R : 0;  // shared rounds with an item
    if (wg >= n_wg || k1 < rounds) {
      n_own = k1 < rounds ? k1 : rounds;
    } else {
      const int rem = n_items - (rounds * R + wg);
      n_own = rounds + (rem > 0 ? (rem + n_wg - 1) / n_wg : 0);
    }
  }
  int it = wg;  // item_of(0)
  if (n_own <= 0) return;  // uniform for the workgroup
  auto entry = [&](int c) { return a.cu ? ld_entry(a.table + c) : entry_fixed(a, c); };
  // chunks from the last to the first: the records the scan reads first are written last
  // and are still in the caches (L2, MALL) when it starts.  Fused: position p holds chunk
  // p / rows of row p % rows.
  const int n_chunks = n_items / a.H;  // passes, for packed batches
  auto chunk_of = [&](int x) {
    const int pos = x / a.H;
    return FUSED ? (pos % n_rows) * (int)a.nc + pos / n_rows : n_chunks - 1 - pos;
  };
  // the chunks of item x's pass: {chunk, second chunk or -1}
  auto pass_of = [&](int x) {
    if (!a.cu) return make_int2(chunk_of(x), -1);
    const uint64_t pc = sload_u64(a.passes + chunk_of(x));
    return make_int2((int32_t)(uint32_t)pc, (int32_t)(uint32_t)(pc >> 32));
  };
  // every wave's record stores (written through at device scope) complete, then the flags
  // (device-scope stores), one per 64-column scan slice that reads the record
  constexpr int NSF = DV / 64;
  auto publish = [&](int chunk, int h, bool ready) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if ((int)threadIdx.x < NSF && ready)
      __hip_atomic_store(fz.flags + ((size_t)chunk * a.H + h) * NSF + threadIdx.x, fz.epoch, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  };
  auto head_of = [&](int x) { return (x % a.H + x / a.H) % a.H; };
  // Where the chunks of this workgroup's first 64 items start and how many tokens they
  // hold, staged in LDS (entry j: item blockIdx.x + j * gridDim.x) with one batch of
  // vector loads: the next item's input loads then never wait behind dependent scalar
  // metadata loads.  Later items (more than 64 per workgroup) read the tables.  Entry:
  // {first token lo, hi, valid tokens | second chunk's valid tokens << 16, second chunk's
  // first token or -1} (a second chunk exists in packed batches, whose token offsets fit
  // 31 bits).
  int4* meta = reinterpret_cast<int4*>(smem + PrepSmem<DK, DV>::META);
  auto start_of = [&](const ChunkEntry& e) { return seq_start(a.cu, a.T, e.seq) + (int64_t)e.idx * kChunk; };
  if (threadIdx.x < 64) {
    int4 m = make_int4(0, 0, 0, -1);
    if ((int)threadIdx.x < n_own) {
      const int item = item_of((int)threadIdx.x);
      int2 pc = make_int2(chunk_of(item), -1);
      if (a.cu) pc = a.passes[pc.x];
      const ChunkEntry e = a.cu ? a.table[pc.x] : entry_fixed(a, pc.x);
      const int64_t st = start_of(e);
      int len2 = 0, st2 = -1;
      if (pc.y >= 0) {
        const ChunkEntry e2 = a.table[pc.y];
        len2 = e2.len;
        st2 = (int32_t)start_of(e2);
      }
      m = make_int4((int32_t)(uint32_t)st, (int32_t)(st >> 32), e.len | (len2 << 16), st2);
    }
    meta[threadIdx.x] = m;
  }
  __syncthreads();
  auto at_of = [&](int j, int item) {
    if (j < 64) {
      const int4 m = meta[j];  // same address in every lane
      const uint32_t lo = __builtin_amdgcn_readfirstlane(m.x);
      const int32_t hi = __builtin_amdgcn_readfirstlane(m.y);
      const int lens = __builtin_amdgcn_readfirstlane(m.z);
      const int st2 = __builtin_amdgcn_readfirstlane(m.w);
      return raw_at_tok<DK, DV>(a, (int64_t)(((uint64_t)(uint32_t)hi << 32) | lo), lens & 0xffff, head_of(item),
                                st2, lens >> 16);
    }
    const int2 pc = pass_of(item);
    if (pc.y < 0) return raw_at<DK, DV>(a, entry(pc.x), head_of(item));
    const ChunkEntry e = entry(pc.x), e2 = entry(pc.y);
    return raw_at_tok<DK, DV>(a, start_of(e), e.len, head_of(item), start_of(e2), e2.len);
  };
  {
    RawIn<DK, DV, InT> raw;
    ItemIn<DK, DV> in;
    {
      const RawAt at = at_of(0, it);
      load_part<0>(raw, a, at);
      load_part<1>(raw, a, at);
      load_part<2>(raw, a, at);
      load_part<3>(raw, a, at);
    }
    unpack_raw(in, raw);
    for (int j = 0;; ++j) {
      const bool more = j + 1 < n_own;
      const int nx = __builtin_amdgcn_readfirstlane(more ? item_of(j + 1) : it);
      const RawAt at = at_of(more ? j + 1 : j, more ? nx : it);
      load_part<0>(raw, a, at);
      const int2 pc = pass_of(it);
      prep_item<DK, DV, false, FUSED>(a, pc.x, pc.y, head_of(it), in, smem, [&](int phase) {
        if (phase == 1) load_part<1>(raw, a, at);
        if (phase == 2) load_part<2>(raw, a, at);
        if (phase == 3) load_part<3>(raw, a, at);
      });
      if (FUSED) {
        // the guard flag of this item, before the next item resets it
        const bool deferred = *reinterpret_cast<volatile int*>(smem + PrepSmem<DK, DV>::RED + 32) != 0;
        unpack_raw(in, raw);
        publish(chunk_of(it), head_of(it), !deferred);  // its barrier also guards the LDS reuse
        if (!more) break;
      } else {
        unpack_raw(in, raw);
        if (!more) break;
        __syncthreads();  // LDS is rewritten by the next item
      }
      it = nx;
    }
  }
  __syncthreads();  // LDS is rewritten below; this workgroup's flags are visible to it

  // exact pass over this workgroup's flagged items, 64 items per batch of flag loads; each
  // flagged chunk of a pass is redone on its own
  const int lane = threadIdx.x & 63;
  for (int kb = 0; kb < n_own; kb += 64) {
    int f = 0;
    if (kb + lane < n_own) {
      const int x = item_of(kb + lane);
      const int2 pc = a.cu ? a.passes[chunk_of(x)] : make_int2(chunk_of(x), -1);
      f = a.defer[(size_t)pc.x * a.H + head_of(x)] != 0;  // both chunks of a pass share the flag
    }
    uint64_t bits = __ballot(f != 0);  // the same in every wave
    while (bits) {
      const int b = __builtin_ctzll(bits);
      bits &= bits - 1;
      const int x = __builtin_amdgcn_readfirstlane(item_of(kb + b));
      const int2 pc = pass_of(x);
      for (int k = 0; k < (pc.y >= 0 ? 2 : 1); ++k) {
        const int c = k ? pc.y : pc.x;
        RawIn<DK, DV, InT> raw;
        load_raw(raw, a, entry(c), head_of(x));
        ItemIn<DK, DV> in;
        unpack_raw(in, raw);
        prep_item<DK, DV, true, FUSED>(a, c, -1, head_of(x), in, smem, [](int) {});
        if (FUSED) {
          publish(c, head_of(x), true);
        } else {
          __syncthreads();  // LDS is rewritten by the next item
        }
      }
    }
  }
}

template <int DK, int DV, typename InT>
__global__ __launch_bounds__(kPrepThreads, 1) void chunk_prep_kernel(PrepArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  chunk_walk<DK, DV, InT, false>(a, FuseArgs{}, (int)blockIdx.x, (int)gridDim.x, smem);
}

}  // namespace kda
