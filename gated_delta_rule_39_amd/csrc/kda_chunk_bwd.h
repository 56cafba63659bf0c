// Backward pass of the gated delta rule in chunkwise form, on the fp32 matrix cores.
//
// "Autoresearch on Kimi Delta Attention" (phase "Parallelize the recurrence") replaces the
// token-by-token reverse walk by chunkwise transforms and a scan over chunks.  Per head and
// 64-token chunk, with G the in-chunk cumulative log-gate (rows are tokens), the forward
// step of the same page's section "KDA in one minute", unrolled over the chunk, reads
//     Kg = khat e^G,  Qg = qhat e^G,  Kd = khat e^(G_n - G)
//     L  = strictly lower part of (Kg)(khat e^-G)^T,  T = (I + diag(beta) L)^-1
//     W  = T diag(beta) Kg,  U = T diag(beta) V,  D = U - W S0
//     P  = lower part (diagonal included) of (Qg)(khat e^-G)^T
//     O  = scale (Qg S0 + P D),  S_n = diag(e^G_n) S0 + Kd^T D
// and its reverse-mode derivative, with Hn = dL/dS_n carried from the later chunks:
//     dD  = scale P^T dO + Kd Hn
//     dS0 = scale Qg^T dO + diag(e^G_n) Hn - W^T dD                      (the previous Hn)
//     dW  = -dD S0^T,  dX = T^T dW,  dY = T^T dD          (X = diag(beta) Kg, Y = diag(beta) V)
//     dA  = -(dX W^T + dY U^T) on the strictly lower part,  dL = diag(beta) dA
//     dbeta = rowsum(dA o L) + rowsum(dX o Kg) + rowsum(dY o V),  dv = beta dY
// then the backward of the two gated products L and P, the scalings of Kg, Qg, Kd and
// e^G_n, dg as the reverse cumulative sum of dG over the chunk, and dq, dk through the L2
// normalisation.
//
// Every product runs on v_mfma_f32_16x16x4f32 (fp32 operands and sums): the fp32
// gradients (dg, dh0) keep the precision of a scalar fp32 walk.  Five kernels:
//   cb_factor_kernel     per (chunk, head): unit q and k, G, the gated Grams L and P, T, W,
//                        U, Kd^T, Qg^T, e^G_n
//   cb_state_fwd_kernel  per (sequence, head, 16 value columns): the state at every chunk
//                        start (S0), walking the chunks forwards
//   cb_state_rev_kernel  per (sequence, head, 16 value columns): Hn of every chunk and dD,
//                        walking the chunks backwards; dh0
//   cb_grad_a_kernel     per (chunk, head): the products over value channels (dQg, dW, dKd,
//                        dP, D recomputed), dX, dY, dv, dA
//   cb_grad_b_kernel     per (chunk, head): the gated-product backward, dG and dg, dq, dk,
//                        dbeta
// The value columns of the state evolve independently in both scans, so a scan workgroup
// owns 16 columns and its four waves split the key rows; a step adds the waves' partial
// sums through LDS in a fixed order.  Results are deterministic.
//
// Gated products: M_ij = sum_c a_ic b_jc e^(G_ic - G_jc) over 16 x 16 token blocks is a
// matrix product of a e^(G - G_r) and b e^(G_r - G) for a reference row r.  Off-diagonal
// blocks take r between the two blocks, so both factors are at most 1.  A diagonal block
// takes its middle row, which keeps every factor within e^80 of 1 when the gate falls by at
// most 80 nats over either half of the block (checked per block); past that the block is
// summed element by element with one exponential per term.
//
// MFMA fragments (v_mfma_f32_16x16x4f32, lane l, r = l % 16, q = l / 16):
//   A (16 x 4): lane holds A[r][q];  B (4 x 16): B[q][r];  C (16 x 16): C[4q + i][r], i = 0..3.
// A product sums over its index in steps of 4; the kernels let step e of a 16-wide group
// stand for index 4q + e, so a C tile serves, without data movement, as the B operand of a
// product over its rows and as the (transposed) A operand of one.
#pragma once

#include "kda_recurrent_bwd.h"

namespace kda {

__device__ inline f32x4 mfma_f32(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ inline float cb_exp(float x) { return exp2_hw(x * kLog2e); }

// Buffer loads: a resource over one chunk's array (uniform, in scalar registers) and 32-bit
// byte offsets per lane.  Per-lane 64-bit addresses of loads inside the chunk loops would be
// strength-reduced into pointers that stay live across the loop; these offsets do not
// change with the chunk.  Loads past `bytes` return 0.
__device__ inline __amdgpu_buffer_rsrc_t cb_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kBufferFlags);
}
__device__ inline float cb_ld1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
__device__ inline float4 cb_ld4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const uint4_v v = __builtin_bit_cast(uint4_v, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}
// one element of the io dtype as fp32
__device__ inline float cb_ld_io(__amdgpu_buffer_rsrc_t r, uint32_t idx, const uint16_t*) {
  return bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, (int)(idx * 2), 0, 0));
}
__device__ inline float cb_ld_io(__amdgpu_buffer_rsrc_t r, uint32_t idx, const float*) {
  return cb_ld1(r, idx * 4);
}
// four consecutive elements of the io dtype as fp32
__device__ inline float4 cb_ld4_io(__amdgpu_buffer_rsrc_t r, uint32_t idx, const uint16_t*) {
  const uint2_v v = __builtin_bit_cast(uint2_v, __builtin_amdgcn_raw_buffer_load_b64(r, (int)(idx * 2), 0, 0));
  return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u), __uint_as_float(v.y << 16),
                     __uint_as_float(v.y & 0xffff0000u));
}
__device__ inline float4 cb_ld4_io(__amdgpu_buffer_rsrc_t r, uint32_t idx, const float*) { return cb_ld4(r, idx * 4); }

// Tile list of the lower 4 x 4 block triangle: diagonal blocks first, then by distance.
__device__ __host__ constexpr int cb_tile_i(int p) {
  return p < 4 ? p : p < 7 ? p - 3 : p < 9 ? p - 5 : 3;
}
__device__ __host__ constexpr int cb_tile_j(int p) {
  return p < 4 ? p : p < 7 ? p - 4 : p < 9 ? p - 7 : 0;
}

// Per-(chunk, head) workspace.  Item it = chunk * H + head.
template <int DK, int DV>
struct CbWs {
  static constexpr size_t W = 64 * DK;        // W [64][DK]
  static constexpr size_t U = 64 * DV;        // U [64][DV]
  static constexpr size_t KDT = DK * 64;      // Kd^T [DK][64]
  static constexpr size_t QGT = DK * 64;      // Qg^T [DK][64]
  static constexpr size_t PT = 64 * 64;       // P^T [64][64]
  static constexpr size_t L = 64 * 64;        // L [64][64]
  static constexpr size_t TT = 64 * 64;       // T^T [64][64]
  static constexpr size_t EGN = DK;           // e^G_n [DK]
  // State block: S0 [DK][DV], Hn [DK][DV], dD [64][DV]; cb_grad_a_kernel then reuses it for
  // its results (dQg^T, dKd^T, dX^T as C fragments [DK/16][4][64 lanes][4], dA and dP
  // [64][64], a partial dbeta [64] and a partial dG_n [DK]).
  static constexpr size_t S0 = 0;
  static constexpr size_t HN = DK * DV;
  static constexpr size_t DD = 2 * DK * DV;
  static constexpr size_t GQ = 0;
  static constexpr size_t GKD = DK * 64;
  static constexpr size_t GX = 2 * DK * 64;
  static constexpr size_t GA = 3 * DK * 64;
  static constexpr size_t GP = GA + 64 * 64;
  static constexpr size_t GB = GP + 64 * 64;
  static constexpr size_t GN = GB + 64;
  static constexpr size_t GEND = GN + DK;
  static constexpr size_t SB0 = DD + 64 * DV > GEND ? DD + 64 * DV : GEND;
  static constexpr size_t SB = (SB0 + 63) / 64 * 64;
  static constexpr size_t FACTOR_FLOATS = W + U + KDT + QGT + PT + L + TT + EGN;
};

struct CbArgs {
  const void* q; const void* k; const void* v; const float* g; const void* beta; const float* h0;
  const int32_t* cu;          // packed offsets (device) or NULL
  const int32_t* info;        // packed: info[0] = number of chunks
  const ChunkEntry* table;    // packed: chunk table
  const int32_t* seq_off;     // packed: first chunk of each sequence
  const void* dout; const float* dht;
  void* dq; void* dk; void* dv; float* dg; void* dbeta; float* dh0;
  float* W; float* U; float* KdT; float* QgT; float* PT; float* L; float* TT; float* eGn;
  float* st;                  // state blocks [items][SB]
  int64_t T, N, nc;           // tokens per row (fixed), sequences, chunks per row (fixed)
  int64_t n_chunk_ub;         // chunks the workspace holds
  int32_t H;
  float scale;
};

struct CbItem {
  int64_t tok0;  // first token of the chunk
  int32_t len;   // valid tokens (1..64)
};

__device__ inline bool cb_item(const CbArgs& a, int64_t c, CbItem& it) {
  if (a.cu) {
    if (c >= a.info[0]) return false;
    const ChunkEntry e = a.table[c];
    it.len = e.len;
    it.tok0 = (int64_t)a.cu[e.seq] + (int64_t)e.idx * kChunk;
  } else {
    const int64_t b = c / a.nc;
    const int64_t idx = c - b * a.nc;
    const int64_t rem = a.T - idx * kChunk;
    it.len = (int32_t)(rem < kChunk ? rem : kChunk);
    it.tok0 = b * a.T + idx * kChunk;
  }
  return true;
}

// Chunks of sequence n: first chunk and count.
__device__ inline void cb_chunks(const CbArgs& a, int64_t n, int64_t& c0, int64_t& cnt) {
  if (a.cu) {
    c0 = a.seq_off[n];
    int64_t c1 = a.seq_off[n + 1];
    if (c1 > a.n_chunk_ub) c1 = a.n_chunk_ub;  // only on invalid cu_seqlens
    if (c0 > c1) c0 = c1;
    cnt = c1 - c0;
  } else {
    c0 = n * a.nc;
    cnt = a.nc;
  }
}

// LDS rows of the chunk: unit q and unit k (rows past the chunk's end are zero), the
// in-chunk cumulative gate G (constant past the end), beta (zero past the end), and per
// token the norm data of q and k: |x| 2^-ex and ex, after the same exact power-of-two
// rescale as the forward kernels.  NT threads (256 or 512); row stride KS = DK + 4 floats.
template <int DK, typename InT, int NT = 256>
__device__ void cb_load_rows(const CbArgs& a, const CbItem& it, int h, float* kh, float* qh, float* G,
                             float* bs, float* nrm) {
  constexpr int KS = DK + 4;
  constexpr int TP = NT / 64;   // threads per token
  constexpr int CH = DK / TP;  // channels per thread
  const int tid = threadIdx.x;
  const int t = tid / TP, p = tid % TP;
  const bool valid = t < it.len;
  const int64_t row = (it.tok0 + t) * a.H + h;
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    float x[CH];
    if (valid) {
      const InT* src = reinterpret_cast<const InT*>(which ? a.k : a.q) + row * DK + p * CH;
#pragma unroll
      for (int c = 0; c < CH; c += 4) load4(src + c, x + c);
    } else {
#pragma unroll
      for (int c = 0; c < CH; ++c) x[c] = 0.f;
    }
    float m = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) m = fmaxf(m, fabsf(x[c]));
#pragma unroll
    for (int o = 1; o < TP; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
    const int ex = m > 0.f ? ilogb_pos(m) : 0;
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      x[c] = ldexpf(x[c], -ex);
      ss = fmaf(x[c], x[c], ss);
    }
#pragma unroll
    for (int o = 1; o < TP; o <<= 1) ss += __shfl_xor(ss, o);
    const float nv = sqrtf(ss);
    float* dst = (which ? kh : qh) + t * KS + p * CH;
#pragma unroll
    for (int c = 0; c < CH; c += 4) {
      float4 o;
      o.x = ss > 0.f ? x[c] / nv : 0.f;
      o.y = ss > 0.f ? x[c + 1] / nv : 0.f;
      o.z = ss > 0.f ? x[c + 2] / nv : 0.f;
      o.w = ss > 0.f ? x[c + 3] / nv : 0.f;
      *reinterpret_cast<float4*>(dst + c) = o;
    }
    if (nrm && p == 0) {
      nrm[which * 128 + t] = nv;
      nrm[which * 128 + 64 + t] = (float)ex;
    }
  }
  if (tid < 64) bs[tid] = tid < it.len ? load1(reinterpret_cast<const InT*>(a.beta) + (it.tok0 + tid) * a.H + h) : 0.f;
  // g: coalesced 16-byte loads of the chunk's rows into LDS (rows past the end are 0), then
  // the cumulative sum down each channel in PT parts of 64 / PT tokens, each part adding
  // the totals of the parts before it
  {
    constexpr int C4 = DK / 4;
    const auto gr = cb_rsrc(a.g + (it.tok0 * a.H + h) * DK, (uint32_t)(((it.len - 1) * a.H * DK + DK) * 4));
#pragma unroll
    for (int j = 0; j < 64 * C4 / NT; ++j) {
      const int e4 = tid + NT * j;
      const int t = e4 / C4, c4 = e4 - t * C4;
      const float4 v4 = cb_ld4(gr, (uint32_t)((t * a.H * DK + 4 * c4) * 4));
      *reinterpret_cast<float4*>(G + t * KS + 4 * c4) = v4;
    }
  }
  __syncthreads();
  {
    constexpr int PT = NT / DK, TL = 64 / PT;
    const int c = tid % DK, part = tid / DK;
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < TL; ++u) {
      acc += G[(part * TL + u) * KS + c];
      G[(part * TL + u) * KS + c] = acc;
    }
    __syncthreads();
    float carry = 0.f;
#pragma unroll
    for (int p = 0; p < PT - 1; ++p)
      if (p < part) carry += G[(p * TL + TL - 1) * KS + c];
    __syncthreads();
    if (part > 0) {
#pragma unroll
      for (int u = 0; u < TL; ++u) G[(part * TL + u) * KS + c] += carry;
    }
  }
}

// ---------------------------------------------------------------------------------------
// cb_factor_kernel

template <int DK>
struct CbFacSmem {
  static constexpr int KS = DK + 4;
  static constexpr size_t KH = 0;
  static constexpr size_t QH = KH + 64 * KS;
  static constexpr size_t G = QH + 64 * KS;
  static constexpr size_t L = G + 64 * KS;      // [64][64]
  static constexpr size_t P = L + 64 * 64;      // [64][64]
  static constexpr size_t TI = P + 64 * 64;     // [64][64]
  static constexpr size_t BETA = TI + 64 * 64;  // [64]
  static constexpr size_t BYTES = (BETA + 64) * 4;
};

// One 16 x 16 block (I >= J) of L (strictly lower) and P (lower) into LDS; one wave.
template <int DK>
__device__ void cb_gram_block(const float* kh, const float* qh, const float* G, int I, int J, float* Ls,
                              float* Ps) {
  constexpr int KS = DK + 4;
  const int l = threadIdx.x & 63, lr = l & 15, gq = l >> 4;
  const bool diag = I == J;
  const int ref = diag ? 16 * I + 8 : 16 * I;
  bool use_mfma = true;
  if (diag) {
    float sp = 0.f;
    for (int c = l; c < DK; c += 64) {
      const float gr = G[ref * KS + c];
      sp = fmaxf(sp, fmaxf(fabsf(G[16 * I * KS + c] - gr), fabsf(G[(16 * I + 15) * KS + c] - gr)));
    }
    use_mfma = !__any(sp > 80.f);
  }
  if (use_mfma) {
    const int ia = 16 * I + lr, jb = 16 * J + lr;
    f32x4 aL = zero4(), aP = zero4();
#pragma unroll 4
    for (int kt = 0; kt < DK / 16; ++kt) {
      const int cb = 16 * kt + 4 * gq;
      const float4 ka = *reinterpret_cast<const float4*>(kh + ia * KS + cb);
      const float4 qa = *reinterpret_cast<const float4*>(qh + ia * KS + cb);
      const float4 ga = *reinterpret_cast<const float4*>(G + ia * KS + cb);
      const float4 gr = *reinterpret_cast<const float4*>(G + ref * KS + cb);
      const float4 kb = *reinterpret_cast<const float4*>(kh + jb * KS + cb);
      const float4 gb = *reinterpret_cast<const float4*>(G + jb * KS + cb);
      const float ka_[4] = {ka.x, ka.y, ka.z, ka.w}, qa_[4] = {qa.x, qa.y, qa.z, qa.w};
      const float ga_[4] = {ga.x, ga.y, ga.z, ga.w}, gr_[4] = {gr.x, gr.y, gr.z, gr.w};
      const float kb_[4] = {kb.x, kb.y, kb.z, kb.w}, gb_[4] = {gb.x, gb.y, gb.z, gb.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float fa = cb_exp(ga_[e] - gr_[e]);
        const float b = kb_[e] * cb_exp(gr_[e] - gb_[e]);
        aL = mfma_f32(ka_[e] * fa, b, aL);
        aP = mfma_f32(qa_[e] * fa, b, aP);
      }
    }
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int i = 16 * I + 4 * gq + ii, j = 16 * J + lr;
      Ls[i * 64 + j] = (!diag || i > j) ? aL[ii] : 0.f;
      Ps[i * 64 + j] = (!diag || i >= j) ? aP[ii] : 0.f;
    }
  } else {
    // element by element: lane handles 4 (i, j) pairs of the block
#pragma unroll 1
    for (int qq = 0; qq < 4; ++qq) {
      const int pidx = l + 64 * qq;
      const int i = 16 * I + (pidx >> 4), j = 16 * I + (pidx & 15);
      float sL = 0.f, sP = 0.f;
      if (j <= i) {
#pragma unroll 4
        for (int c = 0; c < DK; ++c) {
          const float E = cb_exp(G[i * KS + c] - G[j * KS + c]);
          const float kj = kh[j * KS + c] * E;
          sL = fmaf(kh[i * KS + c], kj, sL);
          sP = fmaf(qh[i * KS + c], kj, sP);
        }
      }
      Ls[i * 64 + j] = j < i ? sL : 0.f;
      Ps[i * 64 + j] = j <= i ? sP : 0.f;
    }
  }
}

// DK / 16 waves (two per SIMD at DK = 128).
template <int DK, int DV, typename InT>
__global__ __launch_bounds__(DK * 4) void cb_factor_kernel(CbArgs a) {
  extern __shared__ __align__(16) float sm[];
  using S = CbFacSmem<DK>;
  using WS = CbWs<DK, DV>;
  constexpr int KS = S::KS;
  constexpr int NW = DK / 16, NT = DK * 4, NTK = DK / 16, NTV = DV / 16;
  const int64_t item = blockIdx.x;
  const int64_t c = item / a.H;
  const int h = (int)(item - c * a.H);
  CbItem it;
  if (!cb_item(a, c, it)) return;  // whole workgroup
  float* kh = sm + S::KH;
  float* qh = sm + S::QH;
  float* G = sm + S::G;
  float* Ls = sm + S::L;
  float* Ps = sm + S::P;
  float* Ts = sm + S::TI;
  float* bs = sm + S::BETA;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, gq = l >> 4;
  for (int i = tid; i < 3 * 64 * 64 / 4; i += NT)
    reinterpret_cast<float4*>(Ls)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  cb_load_rows<DK, InT, NT>(a, it, h, kh, qh, G, bs, nullptr);
  __syncthreads();

  // 1. gated Grams, 10 blocks over the waves
  for (int p = w; p < 10; p += NW) cb_gram_block<DK>(kh, qh, G, cb_tile_i(p), cb_tile_j(p), Ls, Ps);
  __syncthreads();

  // 2. T = (I + diag(beta) L)^-1: diagonal blocks by substitution (wave w: block w, lane
  // column lr), then the off-diagonal blocks by distance from the diagonal:
  // T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ, with A = diag(beta) L
  if (w < 4) {
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int gi = 16 * w + i;
      float s = i == lr ? 1.f : 0.f;
      const float bi = bs[gi];
#pragma unroll
      for (int kk = 0; kk < i; ++kk) s = fmaf(-bi * Ls[gi * 64 + 16 * w + kk], x[kk], s);
      x[i] = s;
    }
    if (gq == 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) Ts[(16 * w + i) * 64 + 16 * w + lr] = x[i];
    }
  }
  __syncthreads();
  for (int d = 1; d < 4; ++d) {
    if (w <= 3 - d) {
      const int J = w, I = w + d;
      f32x4 M = zero4();
      for (int K = J; K < I; ++K) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float av = bs[16 * I + lr] * Ls[(16 * I + lr) * 64 + 16 * K + 4 * gq + e];
          const float bv = Ts[(16 * K + 4 * gq + e) * 64 + 16 * J + lr];
          M = mfma_f32(av, bv, M);
        }
      }
      f32x4 R = zero4();
#pragma unroll
      for (int e = 0; e < 4; ++e) R = mfma_f32(Ts[(16 * I + lr) * 64 + 16 * I + 4 * gq + e], M[e], R);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) Ts[(16 * I + 4 * gq + ii) * 64 + 16 * J + lr] = -R[ii];
    }
    __syncthreads();
  }

  // 3. W = T X (X = diag(beta) khat e^G) and U = T Y (Y = diag(beta) V), 16-column tiles
  // over the waves (the key tiles of W, then the value tiles of U)
  float* Wo = a.W + item * WS::W;
  float* Uo = a.U + item * WS::U;
  for (int tile = w; tile < NTK + NTV; tile += NW) {
    const bool isw = tile < NTK;
    const int cc = 16 * (isw ? tile : tile - NTK) + lr;
    float X[4][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = 16 * kt + 4 * gq + e;
        if (isw) {
          X[kt][e] = bs[j] * kh[j * KS + cc] * cb_exp(G[j * KS + cc]);
        } else {
          X[kt][e] = j < it.len ? bs[j] * load1(reinterpret_cast<const InT*>(a.v) + ((it.tok0 + j) * a.H + h) * DV + cc)
                                : 0.f;
        }
      }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kt = 0; kt <= mt; ++kt) {
        const float4 tv = *reinterpret_cast<const float4*>(Ts + (16 * mt + lr) * 64 + 16 * kt + 4 * gq);
        acc = mfma_f32(tv.x, X[kt][0], acc);
        acc = mfma_f32(tv.y, X[kt][1], acc);
        acc = mfma_f32(tv.z, X[kt][2], acc);
        acc = mfma_f32(tv.w, X[kt][3], acc);
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        if (isw) {
          Wo[(16 * mt + 4 * gq + ii) * DK + cc] = acc[ii];
        } else {
          Uo[(16 * mt + 4 * gq + ii) * DV + cc] = acc[ii];
        }
      }
    }
  }

  // 4. Kd^T, Qg^T, e^G_n, P^T, L, T^T
  float* kdt = a.KdT + item * WS::KDT;
  float* qgt = a.QgT + item * WS::QGT;
  for (int idx = tid; idx < DK * 16; idx += NT) {
    const int cc = idx >> 4, t4 = (idx & 15) * 4;
    const float gn = G[63 * KS + cc];
    float kd[4], qg[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float gt = G[(t4 + u) * KS + cc];
      kd[u] = kh[(t4 + u) * KS + cc] * cb_exp(gn - gt);
      qg[u] = qh[(t4 + u) * KS + cc] * cb_exp(gt);
    }
    *reinterpret_cast<float4*>(kdt + cc * 64 + t4) = make_float4(kd[0], kd[1], kd[2], kd[3]);
    *reinterpret_cast<float4*>(qgt + cc * 64 + t4) = make_float4(qg[0], qg[1], qg[2], qg[3]);
  }
  if (tid < DK) a.eGn[item * WS::EGN + tid] = cb_exp(G[63 * KS + tid]);
  float* pt = a.PT + item * WS::PT;
  float* tt = a.TT + item * WS::TT;
  float* lo = a.L + item * WS::L;
  for (int idx = tid; idx < 64 * 16; idx += NT) {
    const int j = idx >> 4, i4 = (idx & 15) * 4;
    *reinterpret_cast<float4*>(pt + j * 64 + i4) =
        make_float4(Ps[i4 * 64 + j], Ps[(i4 + 1) * 64 + j], Ps[(i4 + 2) * 64 + j], Ps[(i4 + 3) * 64 + j]);
    *reinterpret_cast<float4*>(tt + j * 64 + i4) =
        make_float4(Ts[i4 * 64 + j], Ts[(i4 + 1) * 64 + j], Ts[(i4 + 2) * 64 + j], Ts[(i4 + 3) * 64 + j]);
    reinterpret_cast<float4*>(lo)[idx] = reinterpret_cast<const float4*>(Ls)[idx];
  }
}

// ---------------------------------------------------------------------------------------
// State scans.  Workgroup = (sequence, head, 16 value columns) with DK / 16 waves: wave w
// owns key rows [16 w, 16 w + 16) of the slice's state, one C tile.  A step adds the
// waves' partial sums over key rows through LDS (two buffers, one barrier per step); the
// next chunk's factors are loaded while the current chunk is processed.  When the count of
// (sequence, head) pairs is a multiple of 8, the slices of a pair run on one compute die
// (workgroups are dealt to the 8 dies in turn), where they share its L2.

// LDS of a scan workgroup: the waves' partial tiles [2 buffers][NW waves][4 token tiles][64]
// and the summed tiles [2 buffers][4 token tiles][64], f32x4.  A step writes its partials,
// waves 0..3 each add up one token tile (in wave order) after a barrier, and after a second
// barrier every wave reads the four sums.
template <int DK>
struct CbScanSmem {
  static constexpr int NW = DK / 16;
  static constexpr int PART = 0;
  static constexpr int SUM = 2 * NW * 4 * 64;  // in f32x4
  static constexpr size_t BYTES = (SUM + 2 * 4 * 64) * 16;
};

// Sum of the NW waves' partial tiles in wave order, every read issued before the adds.
template <int NW>
__device__ inline f32x4 cb_red_sum(const f32x4* part, int buf, int mt, int l) {
  f32x4 p[NW];
#pragma unroll
  for (int v = 0; v < NW; ++v) p[v] = part[((buf * NW + v) * 4 + mt) * 64 + l];
  f32x4 sum = p[0];
#pragma unroll
  for (int v = 1; v < NW; ++v) sum += p[v];
  return sum;
}

__device__ inline void cb_scan_slot(int64_t wg, int64_t pairs, int ns, int64_t& nh, int& s) {
  if ((pairs & 7) == 0) {
    const int64_t j = wg >> 3;
    nh = (wg & 7) + 8 * (j / ns);
    s = (int)(j % ns);
  } else {
    nh = wg / ns;
    s = (int)(wg % ns);
  }
}

// One chunk's operands of the forward scan for wave w (key rows 16 w ..).
struct CbFwdOps {
  float4 w[4];    // W[16 mt + lr][16 w + 4 gq + e]          A of W S
  float u[4];     // U[16 w + 4 gq + i][col] (waves 0..3)     C tile of U
  float4 kd[4];   // Kd^T[16 w + lr][16 mt + 4 gq + e]        A of Kd^T D
  float4 eg;      // e^G_n[16 w + 4 gq + i]
};

template <int DK, int DV>
__device__ inline void cb_fwd_load(const CbArgs& a, int64_t item, int w, int l, int col, CbFwdOps& o) {
  using WS = CbWs<DK, DV>;
  const unsigned lr = l & 15, gq = l >> 4;
  const auto Wr = cb_rsrc(a.W + item * WS::W, WS::W * 4);
  const auto Ur = cb_rsrc(a.U + item * WS::U, WS::U * 4);
  const auto Kr = cb_rsrc(a.KdT + item * WS::KDT, WS::KDT * 4);
  const auto Er = cb_rsrc(a.eGn + item * WS::EGN, WS::EGN * 4);
#pragma unroll
  for (unsigned mt = 0; mt < 4; ++mt) {
    o.w[mt] = cb_ld4(Wr, 4 * ((16 * mt + lr) * DK + 16 * w + 4 * gq));
    o.kd[mt] = cb_ld4(Kr, 4 * ((16 * w + lr) * 64 + 16 * mt + 4 * gq));
  }
  // waves 4.. read past the end of U (zeros): no branch around the loads
#pragma unroll
  for (unsigned ii = 0; ii < 4; ++ii) o.u[ii] = cb_ld1(Ur, 4 * ((16 * w + 4 * gq + ii) * DV + col));
  o.eg = cb_ld4(Er, 4 * (16 * w + 4 * gq));
}

// cb_state_fwd_kernel: S0 of every chunk.
template <int DK, int DV>
__global__ __launch_bounds__(DK * 4) void cb_state_fwd_kernel(CbArgs a) {
  using WS = CbWs<DK, DV>;
  using SM = CbScanSmem<DK>;
  constexpr int NW = DK / 16, NS = DV / 16;
  extern __shared__ __align__(16) f32x4 red[];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, gq = l >> 4;
  int64_t nh;
  int s;
  cb_scan_slot(blockIdx.x, a.N * a.H, NS, nh, s);
  const int h = (int)(nh % a.H);
  const int64_t n = nh / a.H;
  int64_t c0, cnt;
  cb_chunks(a, n, c0, cnt);
  const int col = 16 * s + lr;
  const int row0 = 16 * w + 4 * gq;
  f32x4 S;
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) S[ii] = a.h0 ? a.h0[((n * a.H + h) * DK + row0 + ii) * DV + col] : 0.f;
  // S0 of chunk i + 1 is stored at the end of step i, after the step's waits for its loads,
  // so no wait covers a store
  auto store_s0 = [&](int64_t i) {
    float* st = a.st + ((c0 + i) * a.H + h) * WS::SB;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) st[WS::S0 + (unsigned)((row0 + ii) * DV + col)] = S[ii];
  };
  auto step = [&](const CbFwdOps& o, int64_t i) {
    const int buf = (int)(i & 1);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 dp = zero4();
      dp = mfma_f32(o.w[mt].x, S[0], dp);
      dp = mfma_f32(o.w[mt].y, S[1], dp);
      dp = mfma_f32(o.w[mt].z, S[2], dp);
      dp = mfma_f32(o.w[mt].w, S[3], dp);
      red[SM::PART + ((buf * NW + w) * 4 + mt) * 64 + l] = dp;
    }
    __syncthreads();
    if (w < 4) {  // D = U - W S, token tile w
      const f32x4 sum = cb_red_sum<NW>(red + SM::PART, buf, w, l);
      f32x4 D;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) D[ii] = o.u[ii] - sum[ii];
      red[SM::SUM + (buf * 4 + w) * 64 + l] = D;
    }
    __syncthreads();
    f32x4 Dt[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) Dt[mt] = red[SM::SUM + (buf * 4 + mt) * 64 + l];
    f32x4 acc[2] = {f32x4{S[0] * o.eg.x, S[1] * o.eg.y, S[2] * o.eg.z, S[3] * o.eg.w}, zero4()};
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      acc[mt & 1] = mfma_f32(o.kd[mt].x, Dt[mt][0], acc[mt & 1]);
      acc[mt & 1] = mfma_f32(o.kd[mt].y, Dt[mt][1], acc[mt & 1]);
      acc[mt & 1] = mfma_f32(o.kd[mt].z, Dt[mt][2], acc[mt & 1]);
      acc[mt & 1] = mfma_f32(o.kd[mt].w, Dt[mt][3], acc[mt & 1]);
    }
    S = acc[0] + acc[1];
    if (i + 1 < cnt) store_s0(i + 1);
  };
  // the next chunk's loads are issued unconditionally (past the last chunk they reload the
  // last one), so the wait counts stay exact across the loop
  CbFwdOps A, B;
  auto load = [&](int64_t i, CbFwdOps& o) {
    cb_fwd_load<DK, DV>(a, (c0 + (i < cnt ? i : cnt - 1)) * a.H + h, w, l, col, o);
  };
  if (cnt > 0) {
    load(0, A);
    store_s0(0);
  }
  for (int64_t i = 0; i < cnt; i += 2) {
    load(i + 1, B);
    step(A, i);
    if (i + 1 >= cnt) break;
    load(i + 2, A);
    step(B, i + 1);
  }
}

// One chunk's operands of the reverse scan for wave w (key rows 16 w ..).  The terms that
// do not involve Hn (scale Qg^T dO on the wave's rows; scale P^T dO, split over the waves:
// token tile w % 4 of the contraction, output token tiles w / 4 + q NW / 4) are formed
// from their loads after the previous chunk's step, so only their results stay live.
template <int DK>
struct CbRevOps {
  static constexpr int MP = 16 / (DK / 16);
  float kd[4][4];   // Kd[16 mt + lr][16 w + 4 gq + e]           A of Kd Hn
  float wt[4][4];   // W[16 kt + 4 gq + e][16 w + lr]             A of W^T dD
  float4 eg;        // e^G_n[16 w + 4 gq + i]
  f32x4 qacc;       // scale Qg^T dO on the wave's rows
  f32x4 pp[MP];     // scale P^T dO, the wave's share
};
template <int DK>
struct CbRevRaw {
  static constexpr int MP = CbRevOps<DK>::MP;
  float4 qg[4];     // Qg^T[16 w + lr][16 kt + 4 gq + e]
  float4 pt[MP];    // P^T[16 mt + lr][16 (w % 4) + 4 gq + e]
  float dob[4][4];  // scale dO[16 kt + 4 gq + e][col]
};

template <int DK, int DV, typename InT>
__device__ inline void cb_rev_load(const CbArgs& a, int64_t item, int h, int64_t t0, int64_t len, int w, int l,
                                   int col, CbRevOps<DK>& o, CbRevRaw<DK>& r) {
  using WS = CbWs<DK, DV>;
  constexpr int NW = DK / 16;
  const unsigned lr = l & 15, gq = l >> 4;
  const auto Wr = cb_rsrc(a.W + item * WS::W, WS::W * 4);
  const auto Kr = cb_rsrc(a.KdT + item * WS::KDT, WS::KDT * 4);
  const auto Qr = cb_rsrc(a.QgT + item * WS::QGT, WS::QGT * 4);
  const auto Pr = cb_rsrc(a.PT + item * WS::PT, WS::PT * 4);
  const auto Er = cb_rsrc(a.eGn + item * WS::EGN, WS::EGN * 4);
  // the chunk's rows of dout for the slice's 16 columns; tokens past the chunk's end fall
  // outside the resource and read 0
  const unsigned tstride = (unsigned)a.H * DV;
  const auto Dr = cb_rsrc(reinterpret_cast<const InT*>(a.dout) + (t0 * a.H + h) * DV + (col & ~15),
                          (uint32_t)(((len - 1) * tstride + 16) * sizeof(InT)));
#pragma unroll
  for (unsigned m = 0; m < 4; ++m) {
    r.qg[m] = cb_ld4(Qr, 4 * ((16 * w + lr) * 64 + 16 * m + 4 * gq));
#pragma unroll
    for (unsigned e = 0; e < 4; ++e) {
      o.kd[m][e] = cb_ld1(Kr, 4 * ((16 * w + 4 * gq + e) * 64 + 16 * m + lr));
      o.wt[m][e] = cb_ld1(Wr, 4 * ((16 * m + 4 * gq + e) * DK + 16 * w + lr));
      const unsigned t = 16 * m + 4 * gq + e;
      r.dob[m][e] = a.scale * cb_ld_io(Dr, t * tstride + lr, (const InT*)nullptr);
    }
  }
#pragma unroll
  for (int q = 0; q < CbRevOps<DK>::MP; ++q) {
    const unsigned mt = (unsigned)(w >> 2) + q * (NW / 4);
    r.pt[q] = cb_ld4(Pr, 4 * ((16 * mt + lr) * 64 + 16 * (w & 3) + 4 * gq));
  }
  o.eg = cb_ld4(Er, 4 * (16 * w + 4 * gq));
}

template <int DK>
__device__ inline void cb_rev_finish(int w, CbRevOps<DK>& o, const CbRevRaw<DK>& r) {
  f32x4 q0 = zero4(), q1 = zero4();
#pragma unroll
  for (int kt = 0; kt < 4; kt += 2) {
    q0 = mfma_f32(r.qg[kt].x, r.dob[kt][0], q0);
    q1 = mfma_f32(r.qg[kt + 1].x, r.dob[kt + 1][0], q1);
    q0 = mfma_f32(r.qg[kt].y, r.dob[kt][1], q0);
    q1 = mfma_f32(r.qg[kt + 1].y, r.dob[kt + 1][1], q1);
    q0 = mfma_f32(r.qg[kt].z, r.dob[kt][2], q0);
    q1 = mfma_f32(r.qg[kt + 1].z, r.dob[kt + 1][2], q1);
    q0 = mfma_f32(r.qg[kt].w, r.dob[kt][3], q0);
    q1 = mfma_f32(r.qg[kt + 1].w, r.dob[kt + 1][3], q1);
  }
  o.qacc = q0 + q1;
  float db[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    db[e] = r.dob[0][e];
#pragma unroll
    for (int kt = 1; kt < 4; ++kt)
      if ((w & 3) == kt) db[e] = r.dob[kt][e];
  }
#pragma unroll
  for (int q = 0; q < CbRevOps<DK>::MP; ++q) {
    f32x4 pp = zero4();
    pp = mfma_f32(r.pt[q].x, db[0], pp);
    pp = mfma_f32(r.pt[q].y, db[1], pp);
    pp = mfma_f32(r.pt[q].z, db[2], pp);
    pp = mfma_f32(r.pt[q].w, db[3], pp);
    o.pp[q] = pp;
  }
}

// cb_state_rev_kernel: Hn and dD of every chunk, walking backwards; dh0.
template <int DK, int DV, typename InT>
__global__ __launch_bounds__(DK * 4) void cb_state_rev_kernel(CbArgs a) {
  using WS = CbWs<DK, DV>;
  using SM = CbScanSmem<DK>;
  constexpr int NW = DK / 16, NS = DV / 16, MP = CbRevOps<DK>::MP;
  extern __shared__ __align__(16) f32x4 red[];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, gq = l >> 4;
  int64_t nh;
  int s;
  cb_scan_slot(blockIdx.x, a.N * a.H, NS, nh, s);
  const int h = (int)(nh % a.H);
  const int64_t n = nh / a.H;
  int64_t c0, cnt;
  cb_chunks(a, n, c0, cnt);
  const int64_t seq0 = a.cu ? (int64_t)a.cu[n] : n * a.T;
  const int64_t seqlen = a.cu ? (int64_t)(a.cu[n + 1] - a.cu[n]) : a.T;
  const int col = 16 * s + lr;
  const int row0 = 16 * w + 4 * gq;
  f32x4 Hs;
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) Hs[ii] = a.dht ? a.dht[((n * a.H + h) * DK + row0 + ii) * DV + col] : 0.f;
  // Hn of chunk i - 1 is stored at the end of step i (see the forward scan)
  auto store_hn = [&](int64_t i) {
    float* st = a.st + ((c0 + i) * a.H + h) * WS::SB;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) st[WS::HN + (unsigned)((row0 + ii) * DV + col)] = Hs[ii];
  };
  auto step = [&](const CbRevOps<DK>& o, int64_t i) {
    float* st = a.st + ((c0 + i) * a.H + h) * WS::SB;
    const int buf = (int)(i & 1);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 dp = zero4();
#pragma unroll
      for (int e = 0; e < 4; ++e) dp = mfma_f32(o.kd[mt][e], Hs[e], dp);
#pragma unroll
      for (int q = 0; q < MP; ++q)
        if ((w >> 2) + q * (NW / 4) == mt) dp += o.pp[q];
      red[SM::PART + ((buf * NW + w) * 4 + mt) * 64 + l] = dp;
    }
    __syncthreads();
    if (w < 4) {  // dD, token tile w
      const f32x4 dD = cb_red_sum<NW>(red + SM::PART, buf, w, l);
      red[SM::SUM + (buf * 4 + w) * 64 + l] = dD;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) st[WS::DD + (unsigned)((16 * w + 4 * gq + ii) * DV + col)] = dD[ii];
    }
    __syncthreads();
    f32x4 acc0 = {Hs[0] * o.eg.x, Hs[1] * o.eg.y, Hs[2] * o.eg.z, Hs[3] * o.eg.w};
    f32x4 acc1 = o.qacc;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const f32x4 dD = red[SM::SUM + (buf * 4 + kt) * 64 + l];
      if (kt & 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc1 = mfma_f32(-o.wt[kt][e], dD[e], acc1);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc0 = mfma_f32(-o.wt[kt][e], dD[e], acc0);
      }
    }
    Hs = acc0 + acc1;
    if (i > 0) store_hn(i - 1);
  };
  CbRevOps<DK> A, B;
  CbRevRaw<DK> R;
  // as in the forward scan, loads past the first chunk reload it
  auto load = [&](int64_t i, CbRevOps<DK>& o) {
    if (i < 0) i = 0;
    const int64_t rem = seqlen - i * kChunk;
    cb_rev_load<DK, DV, InT>(a, (c0 + i) * a.H + h, h, seq0 + i * kChunk, rem < kChunk ? rem : kChunk, w, l, col,
                             o, R);
  };
  if (cnt > 0) {
    load(cnt - 1, A);
    store_hn(cnt - 1);
    cb_rev_finish<DK>(w, A, R);
  }
  for (int64_t i = cnt - 1; i >= 0; i -= 2) {
    load(i - 1, B);
    step(A, i);
    if (i < 1) break;
    cb_rev_finish<DK>(w, B, R);
    load(i - 2, A);
    step(B, i - 1);
    cb_rev_finish<DK>(w, A, R);
  }
  if (a.dh0) {
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) a.dh0[((n * a.H + h) * DK + row0 + ii) * DV + col] = Hs[ii];
  }
}

__device__ inline float f4_at(const float4& v, int e) { return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w; }

// ---------------------------------------------------------------------------------------
// cb_grad_a_kernel: per (chunk, head).  Wave w owns key tiles [w KR, (w+1) KR) and value
// tiles [w VR, (w+1) VR) of 16 channels.
//   D^T = U^T - S0^T W^T for its value tiles (into LDS as B fragments over value channels)
//   over all value channels: dQg^T = scale S0 dO^T, dW = -dD S0^T, dKd^T = Hn D^T (its key
//   tiles), dP = scale dO D^T (its share of the 10 lower tiles), rowsum(Hn o S0)
//   dX^T = dW^T T, dY^T = dD^T T, dv = beta dY, dA partial = -(dX W^T + dY U^T)
// The results go to the item's state block, whose S0, Hn and dD this workgroup alone reads,
// after a barrier that follows the last of those reads.

template <int DK, int DV, typename InT>
__global__ __launch_bounds__(256) void cb_grad_a_kernel(CbArgs a) {
  using WS = CbWs<DK, DV>;
  constexpr int NTK = DK / 16, NTV = DV / 16, KR = NTK / 4, VR = NTV / 4;
  constexpr int RED = NTV * 4 * 64 * 4 > 4 * 10 * 64 * 4 ? NTV * 4 * 64 * 4 : 4 * 10 * 64 * 4;
  __shared__ __align__(16) float sm[RED + 64 * 64 + 4 * 64];
  f32x4* DT = reinterpret_cast<f32x4*>(sm);   // [NTV][4][64]
  f32x4* red = reinterpret_cast<f32x4*>(sm);  // [4 waves][10 tiles][64], once DT is dead
  float* dAs = sm + RED;                       // [64][64]
  float* dyv = dAs + 64 * 64;                  // [4 waves][64]
  const int64_t item = blockIdx.x;
  const int64_t c = item / a.H;
  const int h = (int)(item - c * a.H);
  CbItem it;
  if (!cb_item(a, c, it)) return;  // whole workgroup
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, gq = l >> 4;
  float* st = a.st + item * WS::SB;
  const float* S0 = st + WS::S0;
  const float* Hn = st + WS::HN;
  const float* dD = st + WS::DD;
  const float* Wi = a.W + item * WS::W;
  const float* Ui = a.U + item * WS::U;
  const float* Ti = a.TT + item * WS::TT;
  const float* Li = a.L + item * WS::L;
  const float* Ei = a.eGn + item * WS::EGN;
  const InT* dO = reinterpret_cast<const InT*>(a.dout);
  const InT* V = reinterpret_cast<const InT*>(a.v);

  // the item's state block and the chunk's rows of dout: buffer resources, 32-bit offsets
  const auto Sr = cb_rsrc(st, WS::SB * 4);
  const auto Wr = cb_rsrc(Wi, WS::W * 4);
  const uint32_t tsd = (uint32_t)a.H * DV;  // token stride of dout, v (elements)
  const auto Or = cb_rsrc(dO + (it.tok0 * a.H + h) * DV, (uint32_t)(((it.len - 1) * tsd + DV) * sizeof(InT)));

  // 1. D^T for this wave's value tiles; the next key tile's operands load during the current one
  {
    struct Ops {
      float4 wv[4];    // W[16 nt + lr][16 kt + 4 gq + e]            B = W^T
      float s0[VR][4]; // S0[16 kt + 4 gq + e][16 (w VR + r) + lr]   A = -S0^T
    };
    auto load = [&](int kt, Ops& o) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) o.wv[nt] = cb_ld4(Wr, 4 * ((16 * nt + lr) * DK + 16 * kt + 4 * gq));
#pragma unroll
      for (int r = 0; r < VR; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o.s0[r][e] = cb_ld1(Sr, 4 * (WS::S0 + (16 * kt + 4 * gq + e) * DV + 16 * (w * VR + r) + lr));
    };
    f32x4 Dt[VR][4];
#pragma unroll
    for (int r = 0; r < VR; ++r)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const float4 u = *reinterpret_cast<const float4*>(Ui + (16 * nt + lr) * DV + 16 * (w * VR + r) + 4 * gq);
        Dt[r][nt] = f32x4{u.x, u.y, u.z, u.w};
      }
    auto work = [&](const Ops& o) {
#pragma unroll
      for (int r = 0; r < VR; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) Dt[r][nt] = mfma_f32(-o.s0[r][e], f4_at(o.wv[nt], e), Dt[r][nt]);
    };
    Ops A, B;
    load(0, A);
#pragma unroll 1
    for (int kt = 0; kt < NTK; kt += 2) {
      load(kt + 1, B);
      work(A);
      load(kt + 2 < NTK ? kt + 2 : kt + 1, A);
      work(B);
    }
#pragma unroll
    for (int r = 0; r < VR; ++r)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) DT[((w * VR + r) * 4 + nt) * 64 + l] = Dt[r][nt];
  }
  __syncthreads();

  // 2. products over the value channels, the next value tile's operands loading during the
  // current one
  f32x4 gQ[KR][4], gW[4][KR], gK[KR][4], gP[3];
  float gn[KR];
#pragma unroll
  for (int r = 0; r < KR; ++r) {
    gn[r] = 0.f;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) gQ[r][nt] = gW[nt][r] = gK[r][nt] = zero4();
  }
  gP[0] = gP[1] = gP[2] = zero4();
  int pI[3], pJ[3];
#pragma unroll
  for (int qq = 0; qq < 3; ++qq) {
    const int p = w + 4 * qq;
    pI[qq] = p < 10 ? cb_tile_i(p) : 0;
    pJ[qq] = p < 10 ? cb_tile_j(p) : 0;
  }
  const int np = w < 2 ? 3 : 2;
  struct Ops2 {
    float4 s0v[KR], hnv[KR];  // S0, Hn rows 16 (w KR + r) + lr, value channels 16 kt + 4 gq ..
    float4 ddv[4], dov[4];    // dD, dout rows 16 mt + lr (dout zero past the chunk's end)
  };
  auto load2 = [&](int kt, Ops2& o) {
#pragma unroll
    for (int r = 0; r < KR; ++r) {
      const uint32_t off = (16 * (w * KR + r) + lr) * DV + 16 * kt + 4 * gq;
      o.s0v[r] = cb_ld4(Sr, 4 * (WS::S0 + off));
      o.hnv[r] = cb_ld4(Sr, 4 * (WS::HN + off));
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      o.ddv[mt] = cb_ld4(Sr, 4 * (WS::DD + (16 * mt + lr) * DV + 16 * kt + 4 * gq));
      o.dov[mt] = cb_ld4_io(Or, (16 * mt + lr) * tsd + 16 * kt + 4 * gq, (const InT*)nullptr);
    }
  };
  auto work2 = [&](const Ops2& o, int kt) {
    f32x4 dtv[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) dtv[mt] = DT[(kt * 4 + mt) * 64 + l];
    // the wave's dP tiles: A rows of dout (token tile I), B fragments of D^T (token tile J)
    float4 pa[3];
    f32x4 pb[3];
#pragma unroll
    for (int qq = 0; qq < 3; ++qq) {
      pa[qq] = o.dov[0];
      pb[qq] = dtv[0];
#pragma unroll
      for (int mt = 1; mt < 4; ++mt) {
        if (pI[qq] == mt) pa[qq] = o.dov[mt];
        if (pJ[qq] == mt) pb[qq] = dtv[mt];
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
#pragma unroll
      for (int r = 0; r < KR; ++r) {
        const float sv = f4_at(o.s0v[r], e), hv = f4_at(o.hnv[r], e);
        gn[r] = fmaf(sv, hv, gn[r]);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          gQ[r][nt] = mfma_f32(sv, f4_at(o.dov[nt], e), gQ[r][nt]);
          gW[nt][r] = mfma_f32(f4_at(o.ddv[nt], e), sv, gW[nt][r]);
          gK[r][nt] = mfma_f32(hv, dtv[nt][e], gK[r][nt]);
        }
      }
#pragma unroll
      for (int qq = 0; qq < 3; ++qq)
        if (qq < np) gP[qq] = mfma_f32(f4_at(pa[qq], e), pb[qq][e], gP[qq]);
    }
  };
  {
    Ops2 A, B;
    load2(0, A);
#pragma unroll 1
    for (int kt = 0; kt < NTV; kt += 2) {
      load2(kt + 1, B);
      work2(A, kt);
      load2(kt + 2 < NTV ? kt + 2 : kt + 1, A);
      work2(B, kt + 1);
    }
  }
#pragma unroll
  for (int r = 0; r < KR; ++r) {
    gn[r] = rows4_sum(gn[r]);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      gQ[r][nt] *= a.scale;
      gW[nt][r] = -gW[nt][r];
    }
  }
#pragma unroll
  for (int qq = 0; qq < 3; ++qq) gP[qq] *= a.scale;

  // 3. dX^T = dW^T T, dY^T = dD^T T (T lower: token tile I >= J)
  f32x4 gX[KR][4], gY[VR][4];
#pragma unroll
  for (int J = 0; J < 4; ++J) {
#pragma unroll
    for (int r = 0; r < KR; ++r) gX[r][J] = zero4();
#pragma unroll
    for (int r = 0; r < VR; ++r) gY[r][J] = zero4();
#pragma unroll
    for (int I = J; I < 4; ++I) {
      const float4 tv = *reinterpret_cast<const float4*>(Ti + (16 * J + lr) * 64 + 16 * I + 4 * gq);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float te = f4_at(tv, e);
#pragma unroll
        for (int r = 0; r < KR; ++r) gX[r][J] = mfma_f32(gW[I][r][e], te, gX[r][J]);
#pragma unroll
        for (int r = 0; r < VR; ++r)
          gY[r][J] = mfma_f32(dD[(16 * I + 4 * gq + e) * DV + 16 * (w * VR + r) + lr], te, gY[r][J]);
      }
    }
  }
  // dv = beta dY; the dY o V part of dbeta
  {
    float dyp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      const int t = 16 * J + lr;
      const bool valid = t < it.len;
      const int64_t row = (it.tok0 + t) * a.H + h;
      const float bt = valid ? load1(reinterpret_cast<const InT*>(a.beta) + row) : 0.f;
#pragma unroll
      for (int r = 0; r < VR; ++r) {
        const int cv = 16 * (w * VR + r) + 4 * gq;
        float vv[4] = {0.f, 0.f, 0.f, 0.f};
        if (valid) load4(V + row * DV + cv, vv);
        float o[4];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          o[ii] = bt * gY[r][J][ii];
          dyp[J] = fmaf(gY[r][J][ii], vv[ii], dyp[J]);
        }
        if (valid) store4(reinterpret_cast<InT*>(a.dv) + row * DV + cv, o);
      }
    }
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      const float sum = rows4_sum(dyp[J]);
      if (gq == 0) dyv[w * 64 + 16 * J + lr] = sum;
    }
  }
  __syncthreads();  // every wave is past its last read of DT

  // 4. dA partial over this wave's key and value tiles, all 10 lower tiles
#pragma unroll
  for (int p = 0; p < 10; ++p) {
    const int I = cb_tile_i(p), J = cb_tile_j(p);
    f32x4 acc = zero4();
#pragma unroll
    for (int r = 0; r < KR; ++r) {
      const float4 wv = *reinterpret_cast<const float4*>(Wi + (16 * J + lr) * DK + 16 * (w * KR + r) + 4 * gq);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = mfma_f32(gX[r][I][e], f4_at(wv, e), acc);
    }
#pragma unroll
    for (int r = 0; r < VR; ++r) {
      const float4 uv = *reinterpret_cast<const float4*>(Ui + (16 * J + lr) * DV + 16 * (w * VR + r) + 4 * gq);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = mfma_f32(gY[r][I][e], f4_at(uv, e), acc);
    }
    red[(w * 10 + p) * 64 + l] = acc;
  }
  __syncthreads();  // all reads of S0, Hn and dD are complete: the state block is free

  // 5. results: dA (strictly lower, summed over the waves in order), dP, the fragments
#pragma unroll
  for (int qq = 0; qq < 3; ++qq) {
    const int p = w + 4 * qq;
    if (p >= 10) continue;
    const int I = cb_tile_i(p), J = cb_tile_j(p);
    const f32x4 sum = ((red[(0 * 10 + p) * 64 + l] + red[(1 * 10 + p) * 64 + l]) + red[(2 * 10 + p) * 64 + l]) +
                      red[(3 * 10 + p) * 64 + l];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int i = 16 * I + 4 * gq + ii, j = 16 * J + lr;
      const float va = (I > J || i > j) ? -sum[ii] : 0.f;
      const float vp = (I > J || i >= j) ? gP[qq][ii] : 0.f;
      dAs[i * 64 + j] = va;
      st[WS::GA + i * 64 + j] = va;
      st[WS::GP + i * 64 + j] = vp;
    }
  }
#pragma unroll
  for (int r = 0; r < KR; ++r) {
    const int kc = w * KR + r;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const size_t f = ((size_t)(kc * 4 + nt) * 64 + l) * 4;
      *reinterpret_cast<f32x4*>(st + WS::GQ + f) = gQ[r][nt];
      *reinterpret_cast<f32x4*>(st + WS::GKD + f) = gK[r][nt];
      *reinterpret_cast<f32x4*>(st + WS::GX + f) = gX[r][nt];
    }
    if (gq == 0) st[WS::GN + 16 * kc + lr] = Ei[16 * kc + lr] * gn[r];
  }
  __syncthreads();
  if (tid < 64) {
    const int t = tid;
    float s = 0.f;
    for (int j = 0; j < t; ++j) s = fmaf(dAs[t * 64 + j], Li[t * 64 + j], s);
    st[WS::GB + t] = s + ((dyv[t] + dyv[64 + t]) + dyv[128 + t]) + dyv[192 + t];
  }
}

// ---------------------------------------------------------------------------------------
// cb_grad_b_kernel: per (chunk, head).  Wave w owns key tiles [w KR, (w+1) KR) and every
// token; its gradients are held as C tiles over (key channel, token).

template <int DK>
struct CbGradSmem {
  static constexpr int KS = DK + 4;
  static constexpr int MS = 68;                   // row stride of dL, dP
  static constexpr size_t KH = 0;
  static constexpr size_t QH = KH + 64 * KS;
  static constexpr size_t G = QH + 64 * KS;
  static constexpr size_t DL = G + 64 * KS;       // [64][MS] diag(beta) dA; later dG [64][KS]
  static constexpr size_t DP = DL + 64 * MS;      // [64][MS]
  static constexpr int NW = DK / 16;             // waves
  static constexpr size_t NRM = DP + 64 * MS;     // [2][2][64]: per q, k: |x| 2^-ex, ex
  static constexpr size_t BETA = NRM + 256;       // [64]
  static constexpr size_t DOT = BETA + 64;        // [2][NW][64]
  static constexpr size_t DBP = DOT + 2 * NW * 64;  // [NW][64]
  static constexpr size_t DPD = DBP + NW * 64;    // [64] diagonal of dP
  static constexpr size_t BYTES = (DPD + 64) * 4;
  static_assert(64 * KS <= 2 * 64 * MS, "dG must fit the dL and dP rows");
};

template <int DK, int DV, typename InT>
__global__ __launch_bounds__(DK * 4) void cb_grad_b_kernel(CbArgs a) {
  extern __shared__ __align__(16) float sm[];
  using S = CbGradSmem<DK>;
  using WS = CbWs<DK, DV>;
  constexpr int KS = S::KS, MS = S::MS, NW = S::NW, NT = DK * 4;
  constexpr int KR = 1;
  const int64_t item = blockIdx.x;
  const int64_t c = item / a.H;
  const int h = (int)(item - c * a.H);
  CbItem it;
  if (!cb_item(a, c, it)) return;  // whole workgroup
  float* kh = sm + S::KH;
  float* qh = sm + S::QH;
  float* G = sm + S::G;
  float* dLs = sm + S::DL;
  float* dPs = sm + S::DP;
  float* nrm = sm + S::NRM;
  float* bs = sm + S::BETA;
  float* dots = sm + S::DOT;
  float* dbp = sm + S::DBP;
  float* dpd = sm + S::DPD;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, gq = l >> 4;
  const float* st = a.st + item * WS::SB;
  cb_load_rows<DK, InT, NT>(a, it, h, kh, qh, G, bs, nrm);
  __syncthreads();
  for (int idx = tid; idx < 64 * 16; idx += NT) {
    const int i = idx >> 4, j4 = (idx & 15) * 4;
    const float4 av = *reinterpret_cast<const float4*>(st + WS::GA + i * 64 + j4);
    const float4 pv = *reinterpret_cast<const float4*>(st + WS::GP + i * 64 + j4);
    const float bi = bs[i];
    float4 lo, po;
    lo.x = j4 < i ? bi * av.x : 0.f;
    lo.y = j4 + 1 < i ? bi * av.y : 0.f;
    lo.z = j4 + 2 < i ? bi * av.z : 0.f;
    lo.w = j4 + 3 < i ? bi * av.w : 0.f;
    // dP without its diagonal: a term i = j of P's backward adds qhat_i dP_ii khat_i to dG
    // through both factors with opposite signs; summed apart they would leave their rounding
    // in dg, so the diagonal's dq and dk terms are added directly and it stays out of dG
    po.x = j4 < i ? pv.x : 0.f;
    po.y = j4 + 1 < i ? pv.y : 0.f;
    po.z = j4 + 2 < i ? pv.z : 0.f;
    po.w = j4 + 3 < i ? pv.w : 0.f;
    if ((i >> 2) == (j4 >> 2)) dpd[i] = f4_at(pv, i & 3);
    *reinterpret_cast<float4*>(dLs + i * MS + j4) = lo;
    *reinterpret_cast<float4*>(dPs + i * MS + j4) = po;
  }
  __syncthreads();

  // dG here leaves out the terms of Kd: with them, dg would take sum_s dKd_s Kd_s at the last
  // row and subtract each dKd_s Kd_s at row s, a cancellation of order-1 terms where strong
  // decay makes dg small.  Their net part of dg_t, the sum over s < t, is added directly.
  f32x4 dkh[KR][4], dqh[KR][4], dG[KR][4];
  float kdk[KR][4][4], dbx[4] = {0.f, 0.f, 0.f, 0.f};

  // 1. the terms of the scalings: Kg (dX, with beta), Qg (dQg), Kd (dKd)
#pragma unroll
  for (int r = 0; r < KR; ++r) {
    const int kc = w * KR + r;
    const int cb = 16 * kc + 4 * gq;
    const float4 gn4 = *reinterpret_cast<const float4*>(G + 63 * KS + cb);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int t = 16 * nt + lr;
      const float bt = bs[t], pd = dpd[t];
      const size_t f = ((size_t)(kc * 4 + nt) * 64 + l) * 4;
      const f32x4 xg = *reinterpret_cast<const f32x4*>(st + WS::GX + f);
      const f32x4 qg = *reinterpret_cast<const f32x4*>(st + WS::GQ + f);
      const f32x4 kd = *reinterpret_cast<const f32x4*>(st + WS::GKD + f);
      const float4 g4 = *reinterpret_cast<const float4*>(G + t * KS + cb);
      const float4 k4 = *reinterpret_cast<const float4*>(kh + t * KS + cb);
      const float4 q4 = *reinterpret_cast<const float4*>(qh + t * KS + cb);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const float gt = f4_at(g4, ii), kt_ = f4_at(k4, ii), qt = f4_at(q4, ii);
        const float eg = cb_exp(gt), ed = cb_exp(f4_at(gn4, ii) - gt);
        const float xk = bt * xg[ii];
        const float kg = kt_ * eg, kdv = kt_ * ed;
        dkh[r][nt][ii] = fmaf(xk, eg, fmaf(kd[ii], ed, pd * qt));
        dqh[r][nt][ii] = fmaf(qg[ii], eg, pd * kt_);
        dG[r][nt][ii] = fmaf(xk, kg, qg[ii] * (qt * eg));
        kdk[r][nt][ii] = kd[ii] * kdv;
        dbx[nt] = fmaf(xg[ii], kg, dbx[nt]);
      }
    }
  }

  // 2. backward of the gated products, block by block
#pragma unroll
  for (int B = 0; B < 4; ++B) {
    // ra over key blocks J < B, reference row 16 B: outputs at tokens of block B
    if (B > 0) {
      const int ref = 16 * B;
      f32x4 aL[KR], aP[KR];
#pragma unroll
      for (int r = 0; r < KR; ++r) {
        aL[r] = aP[r] = zero4();
        const int cch = 16 * (w * KR + r) + lr;
        const float gr = G[ref * KS + cch];
        for (int J = 0; J < B; ++J) {
          const float4 bl = *reinterpret_cast<const float4*>(dLs + (16 * B + lr) * MS + 16 * J + 4 * gq);
          const float4 bp = *reinterpret_cast<const float4*>(dPs + (16 * B + lr) * MS + 16 * J + 4 * gq);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = 16 * J + 4 * gq + e;
            const float A = kh[j * KS + cch] * cb_exp(gr - G[j * KS + cch]);
            aL[r] = mfma_f32(A, f4_at(bl, e), aL[r]);
            aP[r] = mfma_f32(A, f4_at(bp, e), aP[r]);
          }
        }
      }
#pragma unroll
      for (int r = 0; r < KR; ++r)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int cch = 16 * (w * KR + r) + 4 * gq + ii, i = 16 * B + lr;
          const float f = cb_exp(G[i * KS + cch] - G[ref * KS + cch]);
          const float rL = aL[r][ii] * f, rP = aP[r][ii] * f;
          dkh[r][B][ii] += rL;
          dqh[r][B][ii] += rP;
          dG[r][B][ii] += kh[i * KS + cch] * rL + qh[i * KS + cch] * rP;
        }
    }
    // rb over query blocks I > B, reference row 16 B + 15: outputs at tokens of block B
    if (B < 3) {
      const int ref = 16 * B + 15;
      f32x4 bL[KR], bP[KR];
#pragma unroll
      for (int r = 0; r < KR; ++r) {
        bL[r] = bP[r] = zero4();
        const int cch = 16 * (w * KR + r) + lr;
        const float gr = G[ref * KS + cch];
        for (int I = B + 1; I < 4; ++I) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 16 * I + 4 * gq + e;
            const float f = cb_exp(G[i * KS + cch] - gr);
            bL[r] = mfma_f32(kh[i * KS + cch] * f, dLs[i * MS + 16 * B + lr], bL[r]);
            bP[r] = mfma_f32(qh[i * KS + cch] * f, dPs[i * MS + 16 * B + lr], bP[r]);
          }
        }
      }
#pragma unroll
      for (int r = 0; r < KR; ++r)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int cch = 16 * (w * KR + r) + 4 * gq + ii, j = 16 * B + lr;
          const float f = cb_exp(G[ref * KS + cch] - G[j * KS + cch]);
          const float rL = bL[r][ii] * f, rP = bP[r][ii] * f;
          dkh[r][B][ii] += rL + rP;
          dG[r][B][ii] -= kh[j * KS + cch] * (rL + rP);
        }
    }
    // diagonal block B: middle reference row when the gate's fall allows, else term by term
    {
      const int ref = 16 * B + 8;
      float sp = 0.f;
      for (int cc = l; cc < DK; cc += 64) {
        const float gr = G[ref * KS + cc];
        sp = fmaxf(sp, fmaxf(fabsf(G[16 * B * KS + cc] - gr), fabsf(G[(16 * B + 15) * KS + cc] - gr)));
      }
      if (!__any(sp > 80.f)) {
        f32x4 aL[KR], aP[KR], bL[KR], bP[KR];
#pragma unroll
        for (int r = 0; r < KR; ++r) {
          aL[r] = aP[r] = bL[r] = bP[r] = zero4();
          const int cch = 16 * (w * KR + r) + lr;
          const float gr = G[ref * KS + cch];
          const float4 bl = *reinterpret_cast<const float4*>(dLs + (16 * B + lr) * MS + 16 * B + 4 * gq);
          const float4 bp = *reinterpret_cast<const float4*>(dPs + (16 * B + lr) * MS + 16 * B + 4 * gq);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = 16 * B + 4 * gq + e;
            const float gj = G[j * KS + cch];
            const float A = kh[j * KS + cch] * cb_exp(gr - gj);
            aL[r] = mfma_f32(A, f4_at(bl, e), aL[r]);
            aP[r] = mfma_f32(A, f4_at(bp, e), aP[r]);
            const float f = cb_exp(gj - gr);
            bL[r] = mfma_f32(kh[j * KS + cch] * f, dLs[j * MS + 16 * B + lr], bL[r]);
            bP[r] = mfma_f32(qh[j * KS + cch] * f, dPs[j * MS + 16 * B + lr], bP[r]);
          }
        }
#pragma unroll
        for (int r = 0; r < KR; ++r)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int cch = 16 * (w * KR + r) + 4 * gq + ii, t = 16 * B + lr;
            const float dgr = G[t * KS + cch] - G[ref * KS + cch];
            const float fa = cb_exp(dgr), fb = cb_exp(-dgr);
            const float rL = aL[r][ii] * fa, rP = aP[r][ii] * fa;
            const float sL = bL[r][ii] * fb, sP = bP[r][ii] * fb;
            const float kt_ = kh[t * KS + cch];
            dkh[r][B][ii] += rL + sL + sP;
            dqh[r][B][ii] += rP;
            dG[r][B][ii] += kt_ * rL + qh[t * KS + cch] * rP - kt_ * (sL + sP);
          }
      } else {
#pragma unroll
        for (int r = 0; r < KR; ++r)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int cch = 16 * (w * KR + r) + 4 * gq + ii, t = 16 * B + lr;
            const float gt = G[t * KS + cch];
            float rL = 0.f, rP = 0.f, sL = 0.f, sP = 0.f;
#pragma unroll 1
            for (int u = 0; u < 16; ++u) {
              const int j = 16 * B + u;
              const float gj = G[j * KS + cch];
              if (j <= t) {
                const float kj = kh[j * KS + cch] * cb_exp(gt - gj);
                rL = fmaf(dLs[t * MS + j], kj, rL);
                rP = fmaf(dPs[t * MS + j], kj, rP);
              }
              if (j >= t) {
                const float E = cb_exp(gj - gt);
                sL = fmaf(dLs[j * MS + t], kh[j * KS + cch] * E, sL);
                sP = fmaf(dPs[j * MS + t], qh[j * KS + cch] * E, sP);
              }
            }
            const float kt_ = kh[t * KS + cch];
            dkh[r][B][ii] += rL + sL + sP;
            dqh[r][B][ii] += rP;
            dG[r][B][ii] += kt_ * rL + qh[t * KS + cch] * rP - kt_ * (sL + sP);
          }
      }
    }
  }

  // 3. the Kd terms of dg_t: sum over s < t of dKd_s Kd_s (exclusive prefix over tokens, in
  // each row of 16 lanes, carried across the token tiles)
#pragma unroll
  for (int r = 0; r < KR; ++r)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      float carry = 0.f;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const float x = kdk[r][nt][ii];
        float y = row_shr<1>(x);
        y += row_shr<1>(y);
        y += row_shr<2>(y);
        y += row_shr<4>(y);
        y += row_shr<8>(y);
        kdk[r][nt][ii] = carry + y;
        carry += row_bcast<15>(y + x);
      }
    }

  // 4. dq, dk through the normalisation; dbeta parts
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int t = 16 * nt + lr;
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int r = 0; r < KR; ++r) {
      const int cb = 16 * (w * KR + r) + 4 * gq;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        sq = fmaf(qh[t * KS + cb + ii], dqh[r][nt][ii], sq);
        sk = fmaf(kh[t * KS + cb + ii], dkh[r][nt][ii], sk);
      }
    }
    sq = rows4_sum(sq);
    sk = rows4_sum(sk);
    const float sb = rows4_sum(dbx[nt]);
    if (gq == 0) {
      dots[w * 64 + t] = sq;
      dots[NW * 64 + w * 64 + t] = sk;
      dbp[w * 64 + t] = sb;
    }
  }
  __syncthreads();  // dLs and dPs are free; dots complete
  float* gds = dLs;   // dG [64][KS]
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int t = 16 * nt + lr;
    const bool valid = t < it.len;
    const int64_t row = (it.tok0 + t) * a.H + h;
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      const float* xh = which ? kh : qh;
      const float* dsum = dots + which * NW * 64;
      float dot = dsum[t];
#pragma unroll
      for (int v = 1; v < NW; ++v) dot += dsum[v * 64 + t];
      const float nv = nrm[which * 128 + t];
      const int ex = (int)nrm[which * 128 + 64 + t];
#pragma unroll
      for (int r = 0; r < KR; ++r) {
        const int cb = 16 * (w * KR + r) + 4 * gq;
        float o[4];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const float dx = which ? dkh[r][nt][ii] : dqh[r][nt][ii];
          o[ii] = nv > 0.f ? ldexpf((dx - xh[t * KS + cb + ii] * dot) / nv, -ex) : 0.f;
        }
        if (valid) store4(reinterpret_cast<InT*>(which ? a.dk : a.dq) + row * DK + cb, o);
      }
    }
#pragma unroll
    for (int r = 0; r < KR; ++r) {
      const int cb = 16 * (w * KR + r) + 4 * gq;
      *reinterpret_cast<float4*>(gds + t * KS + cb) =
          make_float4(dG[r][nt][0], dG[r][nt][1], dG[r][nt][2], dG[r][nt][3]);
    }
  }
  __syncthreads();
  // 5. reverse cumulative sum of dG over the chunk (in place); dbeta
  if (tid < DK) {
    float acc = 0.f;
    for (int t = 63; t >= 0; --t) {
      acc += gds[t * KS + tid];
      gds[t * KS + tid] = acc;
    }
  }
  if (tid >= NT - 64 && tid - (NT - 64) < it.len) {
    const int t = tid - (NT - 64);
    float v = dbp[t];
#pragma unroll
    for (int u = 1; u < NW; ++u) v += dbp[u * 64 + t];
    store1(reinterpret_cast<InT*>(a.dbeta) + (it.tok0 + t) * a.H + h, st[WS::GB + t] + v);
  }
  __syncthreads();
  // 6. dg = that sum + the Kd prefix + e^G_n rowsum(Hn o S0)
#pragma unroll
  for (int r = 0; r < KR; ++r) {
    const int cb = 16 * (w * KR + r) + 4 * gq;
    const float4 gn = *reinterpret_cast<const float4*>(st + WS::GN + cb);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int t = 16 * nt + lr;
      if (t < it.len) {
        const float4 sv = *reinterpret_cast<const float4*>(gds + t * KS + cb);
        *reinterpret_cast<float4*>(a.dg + ((it.tok0 + t) * a.H + h) * DK + cb) =
            make_float4(sv.x + (kdk[r][nt][0] + gn.x), sv.y + (kdk[r][nt][1] + gn.y), sv.z + (kdk[r][nt][2] + gn.z),
                        sv.w + (kdk[r][nt][3] + gn.w));
      }
    }
  }
}

}  // namespace kda
