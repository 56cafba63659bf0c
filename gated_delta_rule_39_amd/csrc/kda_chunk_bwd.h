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
// gradients (dg, dh0) keep the precision of a scalar fp32 walk.  Four kernels:
//   cb_factor_kernel     per (chunk, head): unit q and k, G, the gated Grams L and P, T, W,
//                        U, Kd^T, Qg^T, e^G_n
//   cb_state_scan_kernel per (sequence, head, 16 value columns): the state at every chunk
//                        start (S0), walking the chunks forwards, and beside it Hn of every
//                        chunk and dD, walking them backwards; dh0
//   cb_grad_a_kernel     per (chunk, head): the products over value channels (dQg, dW, dKd,
//                        dP, D recomputed), dX, dY, dv, dA
//   cb_grad_b_kernel     per (chunk, head): the gated-product backward, dG and dg, dq, dk,
//                        dbeta
// The value columns of the state evolve independently in both scans, so a scan workgroup
// owns 16 columns and its waves split the key rows; a step adds the waves' partial sums
// through LDS in a fixed order.  Results are deterministic.
//
// Gated products: M_ij = sum_c a_ic b_jc e^(G_ic - G_jc) over 16 x 16 token blocks is a
// matrix product of a e^(G - G_r) and b e^(G_r - G) for a reference row r.  Off-diagonal
// blocks take r between the two blocks, so both factors are at most 1.  A diagonal block
// takes its middle row, which keeps every factor within e^40 of 1 when the gate falls by at
// most 40 nats over either half of the block (checked per block; products of such factors
// and unit-norm rows stay far from fp32 denormals); past that the block is summed element
// by element with one exponential per term.
//
// MFMA fragments (v_mfma_f32_16x16x4f32, lane l, r = l % 16, q = l / 16):
//   A (16 x 4): lane holds A[r][q];  B (4 x 16): B[q][r];  C (16 x 16): C[4q + i][r], i = 0..3.
// A product sums over its index in steps of 4; the kernels let step e of a 16-wide group
// stand for index 4q + e, so a C tile serves, without data movement, as the B operand of a
// product over its rows and as the (transposed) A operand of one.
#pragma once

#include "kda_device.h"

namespace kda {

__device__ inline f32x4 mfma_f32(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ inline float cb_exp(float x) { return exp2_hw(x * kLog2e); }

// Largest fall of the gate (nats) over either half of a diagonal 16 x 16 block for which the
// block's gated product runs on the matrix cores.
constexpr float kCbDiagSpan = 40.f;

__device__ inline float f4_at(const float4& v, int e) { return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w; }

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
// Position in that list of block (I, J), I >= J.
__device__ __host__ constexpr int cb_blk(int I, int J) {
  return I == J ? I : I - J == 1 ? 4 + J : I - J == 2 ? 7 + J : 9;
}

// Per-(chunk, head) workspace.  Item it = chunk * H + head.
template <int DK, int DV>
struct CbWs {
  static constexpr size_t W = 64 * DK;        // W [64][DK]
  static constexpr size_t U = 64 * DV;        // U [64][DV]
  static constexpr size_t KDT = DK * 64;      // Kd^T [DK][64]
  static constexpr size_t QGT = DK * 64;      // Qg^T [DK][64]
  // the lower triangular 64 x 64 factors keep their 10 lower 16 x 16 blocks, in the order
  // of cb_tile_i / cb_tile_j, each row-major
  static constexpr size_t PT = 10 * 256;      // P^T: block p holds (block (I, J) of P)^T
  static constexpr size_t L = 10 * 256;       // L: block p holds block (I, J) of L
  static constexpr size_t TT = 10 * 256;      // T^T: as P^T
  static constexpr size_t EGN = DK;           // e^G_n [DK]
  // State block: S0 [DK][DV], Hn [DK][DV], dD [64][DV], D [64][DV]; cb_grad_a_kernel then
  // reuses it for its results (dQg^T, dKd^T, dX^T as C fragments [DK/16][4][64 lanes][4],
  // dA and dP [64][64], a partial dbeta [64] and a partial dG_n [DK]).
  static constexpr size_t S0 = 0;
  static constexpr size_t HN = DK * DV;
  static constexpr size_t DD = 2 * DK * DV;
  static constexpr size_t DM = DD + 64 * DV;
  static constexpr size_t GQ = 0;
  static constexpr size_t GKD = DK * 64;
  static constexpr size_t GX = 2 * DK * 64;
  static constexpr size_t GA = 3 * DK * 64;
  static constexpr size_t GP = GA + 64 * 64;
  static constexpr size_t GB = GP + 64 * 64;
  static constexpr size_t GN = GB + 64;
  static constexpr size_t GEND = GN + DK;
  static constexpr size_t SB0 = DM + 64 * DV > GEND ? DM + 64 * DV : GEND;
  static constexpr size_t SB = (SB0 + 63) / 64 * 64;
  static constexpr size_t FACTOR_FLOATS = W + U + KDT + QGT + PT + L + TT + EGN;
};

struct CbArgs {
  const void* q; const void* k; const void* v; const float* g; const void* beta; const float* h0;
  const int32_t* cu;          // packed offsets (device) or NULL
  const int32_t* info;        // packed: info[0] = number of chunks
  const ChunkEntry* table;    // packed: chunk table
  const int32_t* seq_off;     // packed: first chunk of each sequence
  const int32_t* seq_order;   // packed: sequences, longest first
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
  constexpr int C4 = DK / 4;
  constexpr int GJ = 64 * C4 / NT;  // 16-byte pieces of g per thread
  const int tid = threadIdx.x;
  const int t = tid / TP, p = tid % TP;
  // every load first (rows past the chunk's end fall outside the resources and read 0)
  const uint32_t ts = (uint32_t)a.H * DK;  // token stride, elements
  const uint32_t rows = (uint32_t)((it.len - 1) * ts + DK);
  const int64_t base = (it.tok0 * a.H + h) * DK;
  const auto qr = cb_rsrc(reinterpret_cast<const InT*>(a.q) + base, rows * sizeof(InT));
  const auto kr = cb_rsrc(reinterpret_cast<const InT*>(a.k) + base, rows * sizeof(InT));
  const auto gr = cb_rsrc(a.g + base, rows * 4);
  float4 gv[GJ];
#pragma unroll
  for (int j = 0; j < GJ; ++j) {
    const int e4 = tid + NT * j;
    const int tt = e4 / C4, c4 = e4 - tt * C4;
    gv[j] = cb_ld4(gr, (uint32_t)((tt * ts + 4 * c4) * 4));
  }
  float xs[2][CH];
#pragma unroll
  for (int c = 0; c < CH; c += 4) {
    const float4 vq = cb_ld4_io(qr, t * ts + p * CH + c, (const InT*)nullptr);
    const float4 vk = cb_ld4_io(kr, t * ts + p * CH + c, (const InT*)nullptr);
    xs[0][c] = vq.x; xs[0][c + 1] = vq.y; xs[0][c + 2] = vq.z; xs[0][c + 3] = vq.w;
    xs[1][c] = vk.x; xs[1][c + 1] = vk.y; xs[1][c + 2] = vk.z; xs[1][c + 3] = vk.w;
  }
  float bv = 0.f;
  if (tid < 64) {
    const auto br = cb_rsrc(reinterpret_cast<const InT*>(a.beta) + it.tok0 * a.H + h,
                            (uint32_t)(((it.len - 1) * a.H + 1) * sizeof(InT)));
    bv = cb_ld_io(br, tid * a.H, (const InT*)nullptr);
  }
#pragma unroll
  for (int j = 0; j < GJ; ++j) {
    const int e4 = tid + NT * j;
    const int tt = e4 / C4, c4 = e4 - tt * C4;
    *reinterpret_cast<float4*>(G + tt * KS + 4 * c4) = gv[j];
  }
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    float* x = xs[which];
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
    const float inv = ss > 0.f ? 1.f / nv : 0.f;
    float* dst = (which ? kh : qh) + t * KS + p * CH;
#pragma unroll
    for (int c = 0; c < CH; c += 4)
      *reinterpret_cast<float4*>(dst + c) = make_float4(x[c] * inv, x[c + 1] * inv, x[c + 2] * inv, x[c + 3] * inv);
    if (nrm && p == 0) {
      nrm[which * 128 + t] = nv;
      nrm[which * 128 + 64 + t] = (float)ex;
    }
  }
  if (tid < 64) bs[tid] = bv;
  // the cumulative sum of g down each channel in PT parts of 64 / PT tokens, each part
  // adding the totals of the parts before it
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
    use_mfma = !__any(sp > kCbDiagSpan);
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
  const int tid = threadIdx.x, l = tid & 63, lr = l & 15, gq = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
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
  for (int idx = tid; idx < 10 * 64; idx += NT) {
    const int p = idx >> 6, r = (idx >> 2) & 15, c4 = (idx & 3) * 4;
    const int I = cb_tile_i(p), J = cb_tile_j(p);
    const int i0 = 16 * I, j0 = 16 * J;
    const size_t o = (size_t)p * 256 + r * 16 + c4;
    *reinterpret_cast<float4*>(lo + o) = *reinterpret_cast<const float4*>(Ls + (i0 + r) * 64 + j0 + c4);
    *reinterpret_cast<float4*>(pt + o) = make_float4(Ps[(i0 + c4) * 64 + j0 + r], Ps[(i0 + c4 + 1) * 64 + j0 + r],
                                                     Ps[(i0 + c4 + 2) * 64 + j0 + r], Ps[(i0 + c4 + 3) * 64 + j0 + r]);
    *reinterpret_cast<float4*>(tt + o) = make_float4(Ts[(i0 + c4) * 64 + j0 + r], Ts[(i0 + c4 + 1) * 64 + j0 + r],
                                                     Ts[(i0 + c4 + 2) * 64 + j0 + r], Ts[(i0 + c4 + 3) * 64 + j0 + r]);
  }
}

// ---------------------------------------------------------------------------------------
// cb_state_scan_kernel: the two scans over a sequence's chunks in one loop.  The forward
// scan (S0 of every chunk, walking up) and the reverse scan (Hn and dD of every chunk,
// walking down; dh0) do not depend on each other, so a workgroup walks both: step j is
// forward step j and reverse step cnt - 1 - j, and the two chains share its barriers, each
// one's matrix-core work filling the other's waits.
//
// Workgroup = (sequence, head, 16 value columns) with DK / 16 waves: wave w owns key rows
// [16 w, 16 w + 16) of both slices' states, one C tile each.  A step adds the waves' partial
// sums over key rows through LDS: the waves write their partials, then (after a barrier)
// four waves each add up one token tile of the forward D and four one of the reverse dD (in
// wave order), and after a second barrier every wave reads the sums.  The next chunks'
// factors are loaded while the current ones are processed.  When the count of (sequence,
// head) pairs is a multiple of 8, the slices of a pair run on one compute die (workgroups
// are dealt to the 8 dies in turn), where they share its L2.

template <int DK>
struct CbScanSmem {
  static constexpr int NW = DK / 16;
  static constexpr int PART = 0;                  // [2 buffers][NW][4 token tiles][64] f32x4
  static constexpr int SUM = 2 * NW * 4 * 64;     // [2 buffers][4 token tiles][64] f32x4
  static constexpr int ONE = SUM + 2 * 4 * 64;    // one scan's share, f32x4
  static constexpr size_t BYTES = (size_t)2 * ONE * 16;  // forward, then reverse
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

// Buffer resources over one chunk's factors.
template <int DK, int DV>
struct CbChunkRes {
  __amdgpu_buffer_rsrc_t W, U, K, Q, P, E;
  __device__ CbChunkRes(const CbArgs& a, int64_t item) {
    using WS = CbWs<DK, DV>;
    W = cb_rsrc(a.W + item * WS::W, WS::W * 4);
    U = cb_rsrc(a.U + item * WS::U, WS::U * 4);
    K = cb_rsrc(a.KdT + item * WS::KDT, WS::KDT * 4);
    Q = cb_rsrc(a.QgT + item * WS::QGT, WS::QGT * 4);
    P = cb_rsrc(a.PT + item * WS::PT, WS::PT * 4);
    E = cb_rsrc(a.eGn + item * WS::EGN, WS::EGN * 4);
  }
};

template <int DK, int DV, typename InT>
__global__ __launch_bounds__(DK * 4) void cb_state_scan_kernel(CbArgs a) {
  using WS = CbWs<DK, DV>;
  using SM = CbScanSmem<DK>;
  using Res = CbChunkRes<DK, DV>;
  constexpr int NW = DK / 16, NS = DV / 16;
  constexpr int MP = 16 / NW;  // output token tiles of the wave's share of P^T dO
  extern __shared__ __align__(16) f32x4 red[];
  f32x4* redF = red;
  f32x4* redR = red + SM::ONE;
  const int tid = threadIdx.x, l = tid & 63, lr = l & 15, gq = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  int64_t nh;
  int s;
  cb_scan_slot(blockIdx.x, a.N * a.H, NS, nh, s);
  const int h = (int)(nh % a.H);
  // packed sequences in the chunk map's order, longest first, so the longest chains start
  // first
  const int64_t n = a.cu ? (int64_t)a.seq_order[nh / a.H] : nh / a.H;
  int64_t c0, cnt;
  cb_chunks(a, n, c0, cnt);
  if (cnt == 0) {  // no chunks: dh0 = dht
    if (a.dh0) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int64_t o = ((n * a.H + h) * DK + 16 * w + 4 * gq + ii) * DV + 16 * s + lr;
        a.dh0[o] = a.dht ? a.dht[o] : 0.f;
      }
    }
    return;
  }
  const int64_t seq0 = a.cu ? (int64_t)a.cu[n] : n * a.T;
  const int64_t seqlen = a.cu ? (int64_t)(a.cu[n + 1] - a.cu[n]) : a.T;
  const int col = 16 * s + lr;
  const int row0 = 16 * w + 4 * gq;
  const int tw = w & 3;
  // which token tiles this wave sums: with 8 waves, waves 0..3 the forward ones and 4..7 the
  // reverse ones; with 4 waves, each both
  const bool sum_f = NW == 4 || w < 4, sum_r = NW == 4 || w >= 4;
  const unsigned tstride = (unsigned)a.H * DV;
  const unsigned ulr = lr, ugq = gq;

  // Operands, one buffer each, refilled for the next chunk as soon as the current values
  // are consumed (so each load has most of a step to arrive):
  float4 fw[4];    // forward: W[16 mt + lr][16 w + 4 gq + e]          A of W S
  float fu[4];     //          U[16 tw + 4 gq + i][col]                 C tile of U
  float4 fk[4];    //          Kd^T[16 w + lr][16 mt + 4 gq + e]       A of Kd^T D
  float4 fe;       //          e^G_n[16 w + 4 gq + i]
  float rk[4][4];  // reverse: Kd[16 mt + lr][16 w + 4 gq + e]          A of Kd Hn
  float rw[4][4];  //          W[16 kt + 4 gq + e][16 w + lr]            A of W^T dD
  float4 re;       //          e^G_n[16 w + 4 gq + i]
  float4 qg[4];    //          Qg^T[16 w + lr][16 kt + 4 gq + e]        A of Qg^T dO
  float4 pt[MP];   //          P^T[16 mt + lr][16 tw + 4 gq + e]        A of P^T dO
  float dob[4][4]; //          scale dO[16 kt + 4 gq + e][col]          B over the chunk's tokens
  f32x4 qacc, pp[MP];  // scale Qg^T dO on the wave's rows; the wave's share of scale P^T dO

  auto itemf = [&](int64_t i) { return (c0 + (i < cnt ? i : cnt - 1)) * a.H + h; };  // clamped
  auto itemr = [&](int64_t i) { return (c0 + (i > 0 ? i : 0)) * a.H + h; };
  auto load_fw = [&](const Res& r) {
#pragma unroll
    for (unsigned mt = 0; mt < 4; ++mt) fw[mt] = cb_ld4(r.W, 4 * ((16 * mt + ulr) * DK + 16 * w + 4 * ugq));
  };
  auto load_fu = [&](const Res& r) {
#pragma unroll
    for (unsigned ii = 0; ii < 4; ++ii) fu[ii] = cb_ld1(r.U, 4 * ((16 * tw + 4 * ugq + ii) * DV + col));
  };
  auto load_fk = [&](const Res& r) {
#pragma unroll
    for (unsigned mt = 0; mt < 4; ++mt) fk[mt] = cb_ld4(r.K, 4 * ((16 * w + ulr) * 64 + 16 * mt + 4 * ugq));
    fe = cb_ld4(r.E, 4 * (16 * w + 4 * ugq));
  };
  auto load_rk = [&](const Res& r) {
#pragma unroll
    for (unsigned m = 0; m < 4; ++m)
#pragma unroll
      for (unsigned e = 0; e < 4; ++e) rk[m][e] = cb_ld1(r.K, 4 * ((16 * w + 4 * ugq + e) * 64 + 16 * m + ulr));
  };
  auto load_rw = [&](const Res& r) {
#pragma unroll
    for (unsigned m = 0; m < 4; ++m)
#pragma unroll
      for (unsigned e = 0; e < 4; ++e) rw[m][e] = cb_ld1(r.W, 4 * ((16 * m + 4 * ugq + e) * DK + 16 * w + ulr));
    re = cb_ld4(r.E, 4 * (16 * w + 4 * ugq));
  };
  auto load_raw = [&](const Res& r, int64_t i) {
    if (i < 0) i = 0;
    const int64_t rem = seqlen - i * kChunk;
    const int64_t len = rem < kChunk ? rem : kChunk;
    // the chunk's rows of dout for the slice's 16 columns; tokens past the chunk's end fall
    // outside the resource and read 0
    const auto Dr = cb_rsrc(reinterpret_cast<const InT*>(a.dout) + ((seq0 + i * kChunk) * a.H + h) * DV + 16 * s,
                            (uint32_t)(((len - 1) * tstride + 16) * sizeof(InT)));
#pragma unroll
    for (unsigned m = 0; m < 4; ++m) {
      qg[m] = cb_ld4(r.Q, 4 * ((16 * w + ulr) * 64 + 16 * m + 4 * ugq));
#pragma unroll
      for (unsigned e = 0; e < 4; ++e)
        dob[m][e] = a.scale * cb_ld_io(Dr, (16 * m + 4 * ugq + e) * tstride + ulr, (const InT*)nullptr);
    }
#pragma unroll
    for (int q = 0; q < MP; ++q) {  // P^T[j][i] = 0 for token tile of i < that of j
      const int mt = (w >> 2) + q * (NW / 4);
      pt[q] = tw >= mt ? cb_ld4(r.P, 4 * (cb_blk(tw, mt) * 256 + ulr * 16 + 4 * ugq)) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto finish_raw = [&]() {  // qacc and pp of the chunk whose raw operands are loaded
    f32x4 q0 = zero4(), q1 = zero4();
#pragma unroll
    for (int kt = 0; kt < 4; kt += 2)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        q0 = mfma_f32(f4_at(qg[kt], e), dob[kt][e], q0);
        q1 = mfma_f32(f4_at(qg[kt + 1], e), dob[kt + 1][e], q1);
      }
    qacc = q0 + q1;
    float db[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      db[e] = dob[0][e];
#pragma unroll
      for (int kt = 1; kt < 4; ++kt)
        if (tw == kt) db[e] = dob[kt][e];
    }
#pragma unroll
    for (int q = 0; q < MP; ++q) {
      f32x4 p = zero4();
#pragma unroll
      for (int e = 0; e < 4; ++e) p = mfma_f32(f4_at(pt[q], e), db[e], p);
      pp[q] = p;
    }
  };

  f32x4 S, Hs;
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    S[ii] = a.h0 ? a.h0[((n * a.H + h) * DK + row0 + ii) * DV + col] : 0.f;
    Hs[ii] = a.dht ? a.dht[((n * a.H + h) * DK + row0 + ii) * DV + col] : 0.f;
  }
  auto store_s0 = [&](int64_t i) {
    float* st = a.st + ((c0 + i) * a.H + h) * WS::SB;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) st[WS::S0 + (unsigned)((row0 + ii) * DV + col)] = S[ii];
  };
  auto store_hn = [&](int64_t i) {
    float* st = a.st + ((c0 + i) * a.H + h) * WS::SB;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) st[WS::HN + (unsigned)((row0 + ii) * DV + col)] = Hs[ii];
  };
  {
    const Res rf(a, itemf(0)), rr(a, itemr(cnt - 1));
    load_fw(rf);
    load_fu(rf);
    load_fk(rf);
    load_rk(rr);
    load_rw(rr);
    load_raw(rr, cnt - 1);
    finish_raw();
  }
  store_s0(0);
  store_hn(cnt - 1);
  // step j: forward chunk j, reverse chunk cnt - 1 - j.  Loads past either end reload the
  // end chunk, so every step issues the same loads and the wait counts stay exact.
#pragma unroll 1
  for (int64_t j = 0; j < cnt; ++j) {
    const int64_t jr = cnt - 1 - j;
    const int buf = (int)(j & 1);
    const Res nf(a, itemf(j + 1)), nr(a, itemr(jr - 1));
    load_raw(nr, jr - 1);  // raw operands of the next reverse chunk: formed after this step
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 dp = zero4();
      dp = mfma_f32(fw[mt].x, S[0], dp);
      dp = mfma_f32(fw[mt].y, S[1], dp);
      dp = mfma_f32(fw[mt].z, S[2], dp);
      dp = mfma_f32(fw[mt].w, S[3], dp);
      redF[SM::PART + ((buf * NW + w) * 4 + mt) * 64 + l] = dp;
      f32x4 rp = zero4();
#pragma unroll
      for (int e = 0; e < 4; ++e) rp = mfma_f32(rk[mt][e], Hs[e], rp);
#pragma unroll
      for (int q = 0; q < MP; ++q)
        if ((w >> 2) + q * (NW / 4) == mt) rp += pp[q];
      redR[SM::PART + ((buf * NW + w) * 4 + mt) * 64 + l] = rp;
    }
    load_fw(nf);
    load_rk(nr);
    __syncthreads();
    if (sum_f) {  // D = U - W S0, token tile tw (kept for the gradient kernel)
      const f32x4 sum = cb_red_sum<NW>(redF + SM::PART, buf, tw, l);
      f32x4 D;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) D[ii] = fu[ii] - sum[ii];
      redF[SM::SUM + (buf * 4 + tw) * 64 + l] = D;
      float* st = a.st + ((c0 + j) * a.H + h) * WS::SB;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) st[WS::DM + (unsigned)((16 * tw + 4 * gq + ii) * DV + col)] = D[ii];
    }
    if (sum_r) {  // dD, token tile tw
      const f32x4 dD = cb_red_sum<NW>(redR + SM::PART, buf, tw, l);
      redR[SM::SUM + (buf * 4 + tw) * 64 + l] = dD;
      float* st = a.st + ((c0 + jr) * a.H + h) * WS::SB;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) st[WS::DD + (unsigned)((16 * tw + 4 * gq + ii) * DV + col)] = dD[ii];
    }
    load_fu(nf);
    __syncthreads();
    f32x4 fa[2] = {f32x4{S[0] * fe.x, S[1] * fe.y, S[2] * fe.z, S[3] * fe.w}, zero4()};
    f32x4 ra[2] = {f32x4{Hs[0] * re.x, Hs[1] * re.y, Hs[2] * re.z, Hs[3] * re.w}, qacc};
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const f32x4 Dt = redF[SM::SUM + (buf * 4 + mt) * 64 + l];
      const f32x4 dDt = redR[SM::SUM + (buf * 4 + mt) * 64 + l];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        fa[mt & 1] = mfma_f32(f4_at(fk[mt], e), Dt[e], fa[mt & 1]);
        ra[mt & 1] = mfma_f32(-rw[mt][e], dDt[e], ra[mt & 1]);
      }
    }
    S = fa[0] + fa[1];
    Hs = ra[0] + ra[1];
    load_fk(nf);
    load_rw(nr);
    if (j + 1 < cnt) store_s0(j + 1);
    if (jr > 0) store_hn(jr - 1);
    finish_raw();
  }
  if (a.dh0) {
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) a.dh0[((n * a.H + h) * DK + row0 + ii) * DV + col] = Hs[ii];
  }
}

// ---------------------------------------------------------------------------------------
// cb_grad_a_kernel: per (chunk, head), DK / 16 waves.  Wave w owns key tile w and value
// tiles [w VR, (w+1) VR) of 16 channels (with fewer value tiles than waves, waves 0.. own
// one each and the rest none).
//   over all value channels: dQg^T = scale S0 dO^T, dW = -dD S0^T, dKd^T = Hn D^T (its key
//   tile), dP = scale dO D^T (its share of the 10 lower tiles), rowsum(Hn o S0)
//   dX^T = dW^T T, dY^T = dD^T T, dv = beta dY, dA partial = -(dX W^T + dY U^T)
// The results go to the item's state block, whose S0, Hn and dD this workgroup alone reads,
// after a barrier that follows the last of those reads.

// LDS of cb_grad_a_kernel: the chunk's rows of dD, D and dout (fp32, rows padded to DV + 4
// floats so the 16 rows a fragment load touches fall in different banks), staged once for
// all waves; later the waves' dA partials in the same space; dA; the dY o V row sums.
template <int DK, int DV>
struct CbGradASmem {
  static constexpr int NW = DK / 16;
  static constexpr int RS = DV + 4;                 // staged row stride, floats
  static constexpr size_t DDS = 0;                  // dD [64][RS]
  static constexpr size_t DMS = DDS + 64 * RS;      // D [64][RS]
  static constexpr size_t DOS = DMS + 64 * RS;      // dout [64][RS]
  static constexpr size_t STAGE = DOS + 64 * RS;
  static constexpr size_t REDF = (size_t)NW * 10 * 64 * 4;  // dA partials [NW][10][64] f32x4, as floats
  static constexpr size_t DAS = (STAGE > REDF ? STAGE : REDF);  // dA [64][64]
  static constexpr size_t DYV = DAS + 64 * 64;      // [NW][64]
  static constexpr size_t BYTES = (DYV + NW * 64) * 4;
};

template <int DK, int DV, typename InT>
__global__ __launch_bounds__(DK * 4) void cb_grad_a_kernel(CbArgs a) {
  using WS = CbWs<DK, DV>;
  using SM = CbGradASmem<DK, DV>;
  constexpr int NW = DK / 16, NT = DK * 4, NTV = DV / 16, RS = SM::RS;
  constexpr int VR = NTV >= NW ? NTV / NW : 1;  // value tiles per wave
  constexpr int MAXP = (10 + NW - 1) / NW;      // lower tiles of dP per wave
  extern __shared__ __align__(16) float sm[];
  float* dDs = sm + SM::DDS;
  float* Dms = sm + SM::DMS;
  float* dOs = sm + SM::DOS;
  f32x4* red = reinterpret_cast<f32x4*>(sm);  // [NW][10][64], once the staged rows are dead
  float* dAs = sm + SM::DAS;                   // [64][64]
  float* dyv = sm + SM::DYV;                   // [NW][64]
  const int64_t item = blockIdx.x;
  const int64_t c = item / a.H;
  const int h = (int)(item - c * a.H);
  CbItem it;
  if (!cb_item(a, c, it)) return;  // whole workgroup
  const int tid = threadIdx.x, l = tid & 63, lr = l & 15, gq = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const bool vown = NTV >= NW || w < NTV;  // this wave owns value tiles
  const int vt0 = w * VR;                  // its first value tile
  float* st = a.st + item * WS::SB;
  const float* Wi = a.W + item * WS::W;
  const float* Ui = a.U + item * WS::U;
  const float* Ti = a.TT + item * WS::TT;
  const float* Li = a.L + item * WS::L;
  const float* Ei = a.eGn + item * WS::EGN;
  const InT* V = reinterpret_cast<const InT*>(a.v);
  // the item's state block and the chunk's rows of dout: buffer resources, 32-bit offsets
  const auto Sr = cb_rsrc(st, WS::SB * 4);
  const uint32_t tsd = (uint32_t)a.H * DV;  // token stride of dout, v (elements)
  const auto Or = cb_rsrc(reinterpret_cast<const InT*>(a.dout) + (it.tok0 * a.H + h) * DV,
                          (uint32_t)(((it.len - 1) * tsd + DV) * sizeof(InT)));

  // 0. stage dD, D and dout (zero past the chunk's end) in LDS
  {
    constexpr int C4 = DV / 4;
#pragma unroll
    for (int j = 0; j < 64 * C4 / NT; ++j) {
      const int e4 = tid + NT * j;
      const int t = e4 / C4, c4 = 4 * (e4 - t * C4);
      const float4 dd = cb_ld4(Sr, 4 * (WS::DD + t * DV + c4));
      const float4 dm = cb_ld4(Sr, 4 * (WS::DM + t * DV + c4));
      const float4 dz = cb_ld4_io(Or, t * tsd + c4, (const InT*)nullptr);
      *reinterpret_cast<float4*>(dDs + t * RS + c4) = dd;
      *reinterpret_cast<float4*>(Dms + t * RS + c4) = dm;
      *reinterpret_cast<float4*>(dOs + t * RS + c4) = dz;
    }
  }

  // 1. products over the value channels: S0 and Hn rows from HBM (two value tiles ahead),
  // dD, D and dout rows from LDS
  f32x4 gQ[4], gW[4], gK[4], gP[MAXP];
  float gn = 0.f;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) gQ[nt] = gW[nt] = gK[nt] = zero4();
  int pI[MAXP], pJ[MAXP];
#pragma unroll
  for (int qq = 0; qq < MAXP; ++qq) {
    const int p = w + NW * qq;
    gP[qq] = zero4();
    pI[qq] = p < 10 ? cb_tile_i(p) : 0;
    pJ[qq] = p < 10 ? cb_tile_j(p) : 0;
  }
  struct SH {
    float4 s0v, hnv;  // S0, Hn row 16 w + lr, value channels 16 kt + 4 gq ..
  };
  auto loadsh = [&](int kt, SH& o) {
    const int k = kt < NTV ? kt : NTV - 1;
    const uint32_t off = (16 * w + lr) * DV + 16 * k + 4 * gq;
    o.s0v = cb_ld4(Sr, 4 * (WS::S0 + off));
    o.hnv = cb_ld4(Sr, 4 * (WS::HN + off));
  };
  auto work = [&](const SH& o, int kt) {
    float4 ddv[4], dtv[4], dov[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int ro = (16 * mt + lr) * RS + 16 * kt + 4 * gq;
      ddv[mt] = *reinterpret_cast<const float4*>(dDs + ro);
      dtv[mt] = *reinterpret_cast<const float4*>(Dms + ro);
      dov[mt] = *reinterpret_cast<const float4*>(dOs + ro);
    }
    // the wave's dP tiles: A rows of dout (token tile I), B fragments of D^T (token tile J)
    float4 pa[MAXP], pb[MAXP];
#pragma unroll
    for (int qq = 0; qq < MAXP; ++qq) {
      pa[qq] = dov[0];
      pb[qq] = dtv[0];
#pragma unroll
      for (int mt = 1; mt < 4; ++mt) {
        if (pI[qq] == mt) pa[qq] = dov[mt];
        if (pJ[qq] == mt) pb[qq] = dtv[mt];
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float sv = f4_at(o.s0v, e), hv = f4_at(o.hnv, e);
      gn = fmaf(sv, hv, gn);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        gQ[nt] = mfma_f32(sv, f4_at(dov[nt], e), gQ[nt]);
        gW[nt] = mfma_f32(f4_at(ddv[nt], e), sv, gW[nt]);
        gK[nt] = mfma_f32(hv, f4_at(dtv[nt], e), gK[nt]);
      }
#pragma unroll
      for (int qq = 0; qq < MAXP; ++qq)
        if (w + NW * qq < 10) gP[qq] = mfma_f32(f4_at(pa[qq], e), f4_at(pb[qq], e), gP[qq]);
    }
  };
  {
    SH A, B, C;
    loadsh(0, A);
    loadsh(1, B);
    __syncthreads();  // staged rows complete
#pragma unroll 1
    for (int kt = 0; kt < NTV; kt += 3) {
      loadsh(kt + 2, C);
      work(A, kt);
      if (kt + 1 >= NTV) break;
      loadsh(kt + 3, A);
      work(B, kt + 1);
      if (kt + 2 >= NTV) break;
      loadsh(kt + 4, B);
      work(C, kt + 2);
    }
  }
  gn = rows4_sum(gn);
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    gQ[nt] *= a.scale;
    gW[nt] = -gW[nt];
  }
#pragma unroll
  for (int qq = 0; qq < MAXP; ++qq) gP[qq] *= a.scale;

  // 2. dX^T = dW^T T, dY^T = dD^T T (T lower: token tile I >= J)
  float4 tv[10];
#pragma unroll
  for (int p = 0; p < 10; ++p) tv[p] = *reinterpret_cast<const float4*>(Ti + p * 256 + lr * 16 + 4 * gq);
  f32x4 gX[4], gY[VR][4];
#pragma unroll
  for (int J = 0; J < 4; ++J) {
    gX[J] = zero4();
#pragma unroll
    for (int r = 0; r < VR; ++r) gY[r][J] = zero4();
#pragma unroll
    for (int I = J; I < 4; ++I) {
      const float4 t4 = tv[cb_blk(I, J)];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float te = f4_at(t4, e);
        gX[J] = mfma_f32(gW[I][e], te, gX[J]);
        if (vown) {
#pragma unroll
          for (int r = 0; r < VR; ++r)
            gY[r][J] = mfma_f32(dDs[(16 * I + 4 * gq + e) * RS + 16 * (vt0 + r) + lr], te, gY[r][J]);
        }
      }
    }
  }
  // operands of the dA products, loaded before the dv stores
  float4 wv[4], uv[VR][4];
#pragma unroll
  for (int J = 0; J < 4; ++J) {
    wv[J] = *reinterpret_cast<const float4*>(Wi + (16 * J + lr) * DK + 16 * w + 4 * gq);
#pragma unroll
    for (int r = 0; r < VR; ++r)
      uv[r][J] = vown ? *reinterpret_cast<const float4*>(Ui + (16 * J + lr) * DV + 16 * (vt0 + r) + 4 * gq)
                      : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  // dv = beta dY; the dY o V part of dbeta
  {
    float dyp[4] = {0.f, 0.f, 0.f, 0.f};
    if (vown) {
      float bt[4], vv[4][VR][4];
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        const int t = 16 * J + lr;
        const bool valid = t < it.len;
        const int64_t row = (it.tok0 + t) * a.H + h;
        bt[J] = valid ? load1(reinterpret_cast<const InT*>(a.beta) + row) : 0.f;
#pragma unroll
        for (int r = 0; r < VR; ++r) {
          vv[J][r][0] = vv[J][r][1] = vv[J][r][2] = vv[J][r][3] = 0.f;
          if (valid) load4(V + row * DV + 16 * (vt0 + r) + 4 * gq, vv[J][r]);
        }
      }
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        const int t = 16 * J + lr;
        const int64_t row = (it.tok0 + t) * a.H + h;
#pragma unroll
        for (int r = 0; r < VR; ++r) {
          float o[4];
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            o[ii] = bt[J] * gY[r][J][ii];
            dyp[J] = fmaf(gY[r][J][ii], vv[J][r][ii], dyp[J]);
          }
          if (t < it.len) store4(reinterpret_cast<InT*>(a.dv) + row * DV + 16 * (vt0 + r) + 4 * gq, o);
        }
      }
    }
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      const float sum = rows4_sum(dyp[J]);
      if (gq == 0) dyv[w * 64 + 16 * J + lr] = sum;
    }
  }
  __syncthreads();  // every wave is past its last read of the staged rows

  // 3. dA partial over this wave's key and value tiles, all 10 lower tiles
#pragma unroll
  for (int p = 0; p < 10; ++p) {
    const int I = cb_tile_i(p), J = cb_tile_j(p);
    f32x4 acc = zero4();
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = mfma_f32(gX[I][e], f4_at(wv[J], e), acc);
    if (vown) {
#pragma unroll
      for (int r = 0; r < VR; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = mfma_f32(gY[r][I][e], f4_at(uv[r][J], e), acc);
    }
    red[(w * 10 + p) * 64 + l] = acc;
  }
  __syncthreads();  // all reads of S0, Hn, dD and D are complete: the state block is free

  // 4. results: dA (strictly lower, summed over the waves in order), dP, the fragments
#pragma unroll
  for (int qq = 0; qq < MAXP; ++qq) {
    const int p = w + NW * qq;
    if (p >= 10) continue;
    const int I = cb_tile_i(p), J = cb_tile_j(p);
    f32x4 part[NW];
#pragma unroll
    for (int v = 0; v < NW; ++v) part[v] = red[(v * 10 + p) * 64 + l];
    f32x4 sum = part[0];
#pragma unroll
    for (int v = 1; v < NW; ++v) sum += part[v];
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
  for (int nt = 0; nt < 4; ++nt) {
    const size_t f = ((size_t)(w * 4 + nt) * 64 + l) * 4;
    *reinterpret_cast<f32x4*>(st + WS::GQ + f) = gQ[nt];
    *reinterpret_cast<f32x4*>(st + WS::GKD + f) = gK[nt];
    *reinterpret_cast<f32x4*>(st + WS::GX + f) = gX[nt];
  }
  if (gq == 0) st[WS::GN + 16 * w + lr] = Ei[16 * w + lr] * gn;
  __syncthreads();
  // the dA o L part of dbeta: row t of L (its lower blocks) against row t of dA
  if (tid < 64) {
    const int t = tid, I = t >> 4;
    float4 lv[4][4];
#pragma unroll
    for (int J = 0; J < 4; ++J)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        lv[J][q] = J <= I ? *reinterpret_cast<const float4*>(Li + cb_blk(I, J) * 256 + (t & 15) * 16 + 4 * q)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
    float s = 0.f;
#pragma unroll
    for (int J = 0; J < 4; ++J)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // only the lower blocks of dA are written: the others hold whatever an earlier
        // kernel left in LDS, so they are selected away, not multiplied by zero
        const float4 ar = *reinterpret_cast<const float4*>(dAs + t * 64 + 16 * J + 4 * q);
        const float4 av = J <= I ? ar : make_float4(0.f, 0.f, 0.f, 0.f);
        s = fmaf(av.x, lv[J][q].x, fmaf(av.y, lv[J][q].y, fmaf(av.z, lv[J][q].z, fmaf(av.w, lv[J][q].w, s))));
      }
    float y = dyv[t];
#pragma unroll
    for (int v = 1; v < NW; ++v) y += dyv[v * 64 + t];
    st[WS::GB + t] = s + y;
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
  const int tid = threadIdx.x, l = tid & 63, lr = l & 15, gq = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const float* st = a.st + item * WS::SB;
  constexpr int AJ = 64 * 16 / NT;  // 16-byte pieces of dA (and of dP) per thread
  float4 avs[AJ], pvs[AJ];          // loaded before the rows, written to LDS after them
#pragma unroll
  for (int j = 0; j < AJ; ++j) {
    const int idx = tid + NT * j, i = idx >> 4, j4 = (idx & 15) * 4;
    avs[j] = *reinterpret_cast<const float4*>(st + WS::GA + i * 64 + j4);
    pvs[j] = *reinterpret_cast<const float4*>(st + WS::GP + i * 64 + j4);
  }
  cb_load_rows<DK, InT, NT>(a, it, h, kh, qh, G, bs, nrm);
  __syncthreads();
#pragma unroll
  for (int jj = 0; jj < AJ; ++jj) {
    const int idx = tid + NT * jj;
    const int i = idx >> 4, j4 = (idx & 15) * 4;
    const float4 av = avs[jj];
    const float4 pv = pvs[jj];
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
      if (!__any(sp > kCbDiagSpan)) {
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
      const float inv = nv > 0.f ? 1.f / nv : 0.f;
      const int ex = (int)nrm[which * 128 + 64 + t];
#pragma unroll
      for (int r = 0; r < KR; ++r) {
        const int cb = 16 * (w * KR + r) + 4 * gq;
        float o[4];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const float dx = which ? dkh[r][nt][ii] : dqh[r][nt][ii];
          o[ii] = ldexpf((dx - xh[t * KS + cb + ii] * dot) * inv, -ex);
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
