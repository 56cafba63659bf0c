// Recurrent kernel: the gated delta rule evaluated token by token, for decode
// steps (one new token per sequence) and other short continuations.
//
// "Autoresearch on Kimi Delta Attention", section "KDA in one minute",
// describes one step of the memory: every key channel of the state forgets at
// its own rate, the state predicts the value for the new key, and only the
// difference between the actual and the predicted value is written back.
// Per head, with the state S (dk x dv, fp32) of the sequence:
//     a      = Diag(exp(g_t)) S                      (forget, per key channel)
//     delta  = v_t - a^T khat_t                      (actual minus predicted value)
//     S      = a + beta_t khat_t delta^T             (write the correction)
//     o_t    = scale S^T qhat_t = scale (a^T qhat_t + beta_t (qhat_t . khat_t) delta)
// which is (I - beta khat khat^T) Diag(exp(g)) S + beta khat v^T.  A step
// reads the whole state once and writes it once, so a decode batch is bound by
// HBM traffic on the state; the chunked forward pays a 64-token chunk per
// sequence for the same single token.
//
// Work split: the value columns of the state evolve independently (the step
// mixes key channels only), so one wave owns one (sequence, head, 32-column
// slice) and carries that slice in fp32 registers over the sequence's tokens.
// Lane (rg = l / 8, cg = l % 8) holds key channels rg*NR .. rg*NR + NR - 1 of
// columns 4 cg .. 4 cg + 3 of the slice: for every channel the eight lanes of
// a row group read one 128-byte segment of the state row.  Sums over key
// channels add the lanes' partial sums across the eight row groups (DPP row
// rotation and the gfx950 row swaps); there is no LDS and no barrier, and a
// workgroup is four independent waves.
//
// Norms: q and k are divided by their L2 norm after an exact power-of-two
// rescale by the largest entry (any finite bf16/fp32 magnitude), a zero vector
// stays zero.  Everything is fp32.
#pragma once

#include "kda_device.h"

namespace kda {

constexpr int kRecThreads = 256;  // four waves, each an independent column slice
#ifndef KDA_REC_COLS
#define KDA_REC_COLS 32
#endif
constexpr int kRecCols = KDA_REC_COLS;  // value columns per wave (16 or 32)

struct RecurrentArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const void* beta;
  const float* h0;
  const int32_t* cu;  // packed sequences (device), or NULL for B rows of T tokens
  float* ht;
  void* out;
  int64_t T;        // tokens per row (fixed) / total tokens (packed)
  int64_t N;        // sequences
  int32_t H;
  float scale;
  int64_t waves;    // N * H * (DV / kRecCols)
};

// Sum (max) over the row groups: the lanes with the same l % (COLS / 4), in every lane.
template <int COLS>
__device__ inline float rowgroups_sum(float x) {
  if (COLS == 16) x += row_ror<4>(x);
  return rows4_sum(x + row_ror<8>(x));
}
template <int COLS>
__device__ inline float rowgroups_max(float x) {
  if (COLS == 16) x = fmaxf(x, row_ror<4>(x));
  return rows4_max(fmaxf(x, row_ror<8>(x)));
}

// x / ||x||_2 over the whole key dimension, x held as NR channels per lane (the same
// channels in the eight lanes of a row group).
template <int COLS, int NR>
__device__ inline void normalise(float (&x)[NR]) {
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < NR; ++i) m = fmaxf(m, fabsf(x[i]));
  m = rowgroups_max<COLS>(m);
  const int ex = m > 0.f ? ilogb_pos(m) : 0;
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    x[i] = ldexpf(x[i], -ex);  // exact; the largest entry lands in [1, 2)
    ss = fmaf(x[i], x[i], ss);
  }
  ss = rowgroups_sum<COLS>(ss);
  const float inv = ss > 0.f ? 1.f / sqrtf(ss) : 0.f;
#pragma unroll
  for (int i = 0; i < NR; ++i) x[i] *= inv;
}

// State rows are touched once per call: non-temporal loads and stores (streaming hint).
__device__ inline void load_state4(const float* p, float* o) {
  const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  o[0] = x[0]; o[1] = x[1]; o[2] = x[2]; o[3] = x[3];
}
__device__ inline void store_state4(float* p, const float* v) {
  const f32x4 x = {v[0], v[1], v[2], v[3]};
  __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(p));
}

// One token's inputs as seen by one lane.
template <int NR>
struct TokIn {
  float q[NR], k[NR], g[NR], v[4], beta;
};

template <int DK, int DV, int NR, typename InT>
__device__ inline void load_token(TokIn<NR>& in, const RecurrentArgs& a, int64_t tok, int h, int r0, int col) {
  const size_t rk = ((size_t)tok * a.H + h) * DK + r0;
  const InT* q = reinterpret_cast<const InT*>(a.q) + rk;
  const InT* k = reinterpret_cast<const InT*>(a.k) + rk;
#pragma unroll
  for (int i = 0; i < NR; i += 4) {
    load4(q + i, in.q + i);
    load4(k + i, in.k + i);
    load4(a.g + rk + i, in.g + i);
  }
  load4(reinterpret_cast<const InT*>(a.v) + ((size_t)tok * a.H + h) * DV + col, in.v);
  in.beta = load1(reinterpret_cast<const InT*>(a.beta) + (size_t)tok * a.H + h);
}

template <int DK, int DV, typename InT>
__global__ __launch_bounds__(kRecThreads) void recurrent_kernel(RecurrentArgs a) {
  constexpr int CG = kRecCols / 4;  // column groups (lanes per row group)
  constexpr int NR = DK * CG / 64;  // key channels per lane
  constexpr int NS = DV / kRecCols;
  const int l = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kRecThreads / 64) + (threadIdx.x >> 6);
  if (wave >= a.waves) return;  // whole waves only; the kernel has no barrier
  const int slice = (int)(wave % NS);
  const int64_t nh = wave / NS;
  const int h = (int)(nh % a.H);
  const int64_t n = nh / a.H;
  const int cg = l % CG, rg = l / CG;
  const int r0 = rg * NR;                    // first key channel of the lane
  const int col = slice * kRecCols + 4 * cg;  // first value column of the lane

  // token range of the sequence (packed offsets clamped to [0, T], an empty or reversed
  // range is an empty sequence)
  int64_t t0 = n * a.T, t1 = t0 + a.T;
  if (a.cu) {
    t0 = a.cu[n];
    t1 = a.cu[n + 1];
    t0 = t0 < 0 ? 0 : (t0 > a.T ? a.T : t0);
    t1 = t1 < t0 ? t0 : (t1 > a.T ? a.T : t1);
  }

  const size_t sbase = ((size_t)n * a.H + h) * DK * DV;
  float S[NR][4];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    if (a.h0) {
      load_state4(a.h0 + sbase + (size_t)(r0 + i) * DV + col, S[i]);
    } else {
      S[i][0] = S[i][1] = S[i][2] = S[i][3] = 0.f;
    }
  }

  InT* out = reinterpret_cast<InT*>(a.out);
  TokIn<NR> cur;
  if (t0 < t1) load_token<DK, DV, NR, InT>(cur, a, t0, h, r0, col);
  for (int64_t tok = t0; tok < t1; ++tok) {
    // the next token's inputs are requested before this token's arithmetic
    TokIn<NR> nxt;
    load_token<DK, DV, NR, InT>(nxt, a, tok + 1 < t1 ? tok + 1 : tok, h, r0, col);

    normalise<kRecCols>(cur.q);
    normalise<kRecCols>(cur.k);
    float qk = 0.f;
#pragma unroll
    for (int i = 0; i < NR; ++i) qk = fmaf(cur.q[i], cur.k[i], qk);
    float p[4] = {0.f, 0.f, 0.f, 0.f}, r[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const float e = exp2_hw(cur.g[i] * kLog2e);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        S[i][j] *= e;
        p[j] = fmaf(cur.k[i], S[i][j], p[j]);
        r[j] = fmaf(cur.q[i], S[i][j], r[j]);
      }
    }
    qk = rowgroups_sum<kRecCols>(qk);
    float d[4], o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      d[j] = cur.v[j] - rowgroups_sum<kRecCols>(p[j]);
      o[j] = a.scale * fmaf(cur.beta * qk, d[j], rowgroups_sum<kRecCols>(r[j]));
    }
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const float bk = cur.beta * cur.k[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) S[i][j] = fmaf(bk, d[j], S[i][j]);
    }
    if (rg == 0) store4(out + ((size_t)tok * a.H + h) * DV + col, o);
    cur = nxt;
  }

  if (a.ht) {
#pragma unroll
    for (int i = 0; i < NR; ++i) store_state4(a.ht + sbase + (size_t)(r0 + i) * DV + col, S[i]);
  }
}

}  // namespace kda
