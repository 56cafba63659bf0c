// Backward pass of the gated delta rule, token by token (the recurrent form).
//
// "Autoresearch on Kimi Delta Attention" asks a training path for full gradients
// checked against an independent reference (stage "Frozen outside the loop") and
// runs the reverse recurrence over value tiles with the forward history produced
// in parallel instead of replayed serially (phase "Move the path into CUDA").
// Per head, with G = dL/dS_t carried backwards and the forward step of the same
// page's section "KDA in one minute" (a = Diag(exp g) S_{t-1},
// delta = v - a^T khat, S_t = a + beta khat delta^T, o_t = scale S_t^T qhat):
//     G     += scale qhat do^T
//     dqhat  = scale (a do + beta khat (delta . do))      (= scale S_t do)
//     u      = G^T khat              dv = beta u          dbeta = u . delta
//     dkhat  = beta (G delta - a u)
//     da     = G - beta khat u^T     dg = rowsum(a * da)   G <- Diag(exp g) da
// and dL/dh0 = G at the sequence start; dq, dk follow from dqhat, dkhat through
// the L2 normalisation (finish kernel).
//
// Work split: one workgroup per (sequence, head), one wave per 16-column slice of
// the state (the columns evolve independently, so the slices only meet in the
// per-row sums dqhat, dkhat, dg and the scalar dbeta, which they add through LDS in
// a fixed order: results are deterministic).  Slices are 16 columns wide, one wave
// each: lane (rg = l / 4, cg = l % 4) holds key channels rg*NR .. rg*NR + NR - 1 of the
// slice's columns 4 cg .. 4 cg + 3 (the narrow slice leaves room in registers for the
// next token's inputs and state, requested one token ahead in every walk).  The walk:
//   1. forward over the sequence, storing the slice's state at every 64-token
//      boundary (checkpoints, fp32, in the workspace);
//   2. backwards over the 64-token segments: from the segment's checkpoint the
//      forward is replayed into a per-workgroup scratch (the state before each of
//      the segment's tokens), then the segment's tokens are walked in reverse.
// Workgroups are persistent (one per compute unit at most), so the scratch is
// bounded by the grid, not by the number of sequences.
#pragma once

#include "kda_recurrent.h"

namespace kda {

constexpr int kBwdSeg = 64;  // tokens per checkpoint segment

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const void* beta;
  const float* h0;
  const int32_t* cu;      // packed offsets (device) or NULL
  const int32_t* seq_off; // packed: first 64-token segment of each sequence (chunk map), or NULL
  const void* dout;
  const float* dht;
  float* dqh;             // [tokens, H, DK] fp32: dL/dqhat (workspace)
  float* dkh;             // [tokens, H, DK] fp32: dL/dkhat (workspace)
  void* dv;               // [tokens, H, DV] io dtype
  float* dg;              // [tokens, H, DK]
  void* dbeta;            // [tokens, H] io dtype
  float* dh0;             // [N, H, DK, DV] or NULL
  float* ckpt;            // [segments, H, DK * DV] fp32
  float* scratch;         // [grid, kBwdSeg, DK * DV] fp32
  int64_t T, N, nc;       // tokens per row (fixed) / total (packed); sequences; fixed: segments per row
  int32_t H;
  float scale;
};

__device__ inline void store1(uint16_t* p, float x) { *p = (uint16_t)(pack_bf16x2(x, 0.f) & 0xffffu); }
__device__ inline void store1(float* p, float x) { *p = x; }

__device__ inline float wave_sum(float x) {
  x += row_ror<8>(x);
  x += row_ror<4>(x);
  x += row_ror<2>(x);
  x += row_ror<1>(x);
  return rows4_sum(x);
}

// Sum over the four lanes of a column quad (l ^ 1, l ^ 2: the lanes with the same l / 4),
// every lane gets the sum.
__device__ inline float quad_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));  // quad [1,0,3,2]
  return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));  // [2,3,0,1]
}

constexpr int kBwdCols = 16;  // value columns per wave (8 waves for dv = 128)

template <int DK, int DV, typename InT>
__global__ __launch_bounds__(512) void recurrent_bwd_kernel(BwdArgs a) {
  constexpr int NS = DV / kBwdCols;     // slices = waves
  constexpr int CG = kBwdCols / 4;      // 4 lanes per row group
  constexpr int NR = DK * CG / 64;      // key channels per lane
  constexpr int SLICE = DK * kBwdCols;  // floats of one slice's state
  // LDS: per slice and token parity, the row sums [dqhat | dkhat | dg] and dbeta
  __shared__ float part[2][NS][3 * DK + 4];
  const int l = threadIdx.x & 63;
  const int s = threadIdx.x >> 6;  // slice
  const int cg = l % CG, rg = l / CG;
  const int r0 = rg * NR;
  const int col = s * kBwdCols + 4 * cg;
  float* scratch = a.scratch + (size_t)blockIdx.x * kBwdSeg * DK * DV + (size_t)s * SLICE;
  const InT* dout = reinterpret_cast<const InT*>(a.dout);
  InT* dvo = reinterpret_cast<InT*>(a.dv);
  InT* dbo = reinterpret_cast<InT*>(a.dbeta);
  int par = 0;
  RecurrentArgs ra;  // the token loads of the forward recurrent kernel read these fields
  ra.q = a.q; ra.k = a.k; ra.v = a.v; ra.g = a.g; ra.beta = a.beta; ra.H = a.H;

  for (int64_t nh = blockIdx.x; nh < a.N * a.H; nh += gridDim.x) {
    const int h = (int)(nh % a.H);
    const int64_t n = nh / a.H;
    int64_t t0 = n * a.T, t1 = t0 + a.T, seg0 = n * a.nc;
    if (a.cu) {
      t0 = a.cu[n];
      t1 = a.cu[n + 1];
      t0 = t0 < 0 ? 0 : (t0 > a.T ? a.T : t0);
      t1 = t1 < t0 ? t0 : (t1 > a.T ? a.T : t1);
      seg0 = a.seq_off[n];
    }
    int64_t nseg = (t1 - t0 + kBwdSeg - 1) / kBwdSeg;
    if (a.cu) {
      // the checkpoints the chunk map set aside for this sequence (fewer only when
      // cu_seqlens breaks its precondition: the walk then stops there)
      const int64_t room = (int64_t)a.seq_off[n + 1] - seg0;
      nseg = nseg < room ? nseg : (room > 0 ? room : 0);
      t1 = t0 + nseg * kBwdSeg < t1 ? t0 + nseg * kBwdSeg : t1;
    }
    const size_t sbase = ((size_t)n * a.H + h) * DK * DV;
    auto ck = [&](int64_t seg) { return a.ckpt + (((size_t)(seg0 + seg) * a.H + h) * NS + s) * SLICE; };
    // slice state element (row r0 + i, columns col..col+3) in a lane-major block: float4 index i * 64 + l
    auto put = [&](float* base, const float (&S)[NR][4]) {
#pragma unroll
      for (int i = 0; i < NR; ++i)
        *reinterpret_cast<float4*>(base + ((size_t)i * 64 + l) * 4) = make_float4(S[i][0], S[i][1], S[i][2], S[i][3]);
    };
    auto get = [&](const float* base, float (&S)[NR][4]) {
#pragma unroll
      for (int i = 0; i < NR; ++i) load4(base + ((size_t)i * 64 + l) * 4, S[i]);
    };
    auto load = [&](TokIn<NR>& in, int64_t tok) { load_token<DK, DV, NR, InT>(in, ra, tok, h, r0, col); };
    // one forward step of the slice from already loaded inputs (as in the recurrent kernel,
    // without the output)
    auto fwd_step = [&](float (&S)[NR][4], TokIn<NR>& in) {
      normalise<kBwdCols>(in.k);
      float p[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const float e = exp2_hw(in.g[i] * kLog2e);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          S[i][j] *= e;
          p[j] = fmaf(in.k[i], S[i][j], p[j]);
        }
      }
      float d[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) d[j] = in.v[j] - rowgroups_sum<kBwdCols>(p[j]);
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const float bk = in.beta * in.k[i];
#pragma unroll
        for (int j = 0; j < 4; ++j) S[i][j] = fmaf(bk, d[j], S[i][j]);
      }
    };
    // forward over [ta, tb) from S; `at` stores the state before token t (or nothing)
    auto forward = [&](float (&S)[NR][4], int64_t ta, int64_t tb, auto&& at) {
      if (ta >= tb) return;
      TokIn<NR> cur;
      load(cur, ta);
      for (int64_t tok = ta; tok < tb; ++tok) {
        TokIn<NR> nxt;  // the next token's inputs are requested before this token's arithmetic
        load(nxt, tok + 1 < tb ? tok + 1 : tok);
        at(tok, S);
        fwd_step(S, cur);
        cur = nxt;
      }
    };

    // 1. forward with checkpoints
    {
      float S[NR][4];
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        if (a.h0) load4(a.h0 + sbase + (size_t)(r0 + i) * DV + col, S[i]);
        else S[i][0] = S[i][1] = S[i][2] = S[i][3] = 0.f;
      }
      forward(S, t0, t1, [&](int64_t tok, const float (&St)[NR][4]) {
        if ((tok - t0) % kBwdSeg == 0) put(ck((tok - t0) / kBwdSeg), St);
      });
    }

    // 2. backwards over the segments
    float G[NR][4];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      if (a.dht) load4(a.dht + sbase + (size_t)(r0 + i) * DV + col, G[i]);
      else G[i][0] = G[i][1] = G[i][2] = G[i][3] = 0.f;
    }
    for (int64_t seg = nseg - 1; seg >= 0; --seg) {
      const int64_t ts = t0 + seg * kBwdSeg;
      const int64_t te = ts + kBwdSeg < t1 ? ts + kBwdSeg : t1;
      {
        float S[NR][4];
        get(ck(seg), S);
        forward(S, ts, te, [&](int64_t tok, const float (&St)[NR][4]) {
          put(scratch + (size_t)(tok - ts) * DK * DV, St);
        });
      }
      // reverse walk; the next (earlier) token's inputs and state are requested one token ahead
      TokIn<NR> cur;
      float dov[4], An[NR][4];
      load(cur, te - 1);
      load4(dout + ((size_t)(te - 1) * a.H + h) * DV + col, dov);
      get(scratch + (size_t)(te - 1 - ts) * DK * DV, An);
      for (int64_t tok = te - 1; tok >= ts; --tok) {
        const int64_t pt = tok > ts ? tok - 1 : tok;
        float A[NR][4];  // S_{t-1}, then a
#pragma unroll
        for (int i = 0; i < NR; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) A[i][j] = An[i][j];
        TokIn<NR> nxt;
        float don[4];
        load(nxt, pt);
        load4(dout + ((size_t)pt * a.H + h) * DV + col, don);
        get(scratch + (size_t)(pt - ts) * DK * DV, An);
        TokIn<NR>& in = cur;
        normalise<kBwdCols>(in.q);
        normalise<kBwdCols>(in.k);
        float e[NR];
        float p[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NR; ++i) {
          e[i] = exp2_hw(in.g[i] * kLog2e);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            A[i][j] *= e[i];
            p[j] = fmaf(in.k[i], A[i][j], p[j]);
          }
        }
        float d[4];
        float ddo = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          d[j] = in.v[j] - rowgroups_sum<kBwdCols>(p[j]);
          ddo = fmaf(d[j], dov[j], ddo);
        }
        ddo = quad_sum(ddo);  // delta . do over the slice's columns
        // G += scale qhat do^T, then u = G^T khat
        float u[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NR; ++i) {
          const float sq = a.scale * in.q[i];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            G[i][j] = fmaf(sq, dov[j], G[i][j]);
            u[j] = fmaf(in.k[i], G[i][j], u[j]);
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) u[j] = rowgroups_sum<kBwdCols>(u[j]);
        float db = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) db = fmaf(u[j], d[j], db);
        db = quad_sum(db);
        // per-row partials over this lane's four columns, then over the quad
        float pq[NR], pk[NR], pg[NR];
#pragma unroll
        for (int i = 0; i < NR; ++i) {
          float aq = 0.f, gd = 0.f, au = 0.f, ag = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            aq = fmaf(A[i][j], dov[j], aq);
            gd = fmaf(G[i][j], d[j], gd);
            au = fmaf(A[i][j], u[j], au);
            const float da = G[i][j] - in.beta * in.k[i] * u[j];
            ag = fmaf(A[i][j], da, ag);
            G[i][j] = e[i] * da;  // dL/dS_{t-1}
          }
          pq[i] = quad_sum(aq);
          pk[i] = quad_sum(gd - au);
          pg[i] = quad_sum(ag);
        }
        // this slice's row sums to LDS (lanes cg == 0 hold the row group's totals)
        float* pp = part[par][s];
        if (cg == 0) {
#pragma unroll
          for (int i = 0; i < NR; ++i) {
            // dqhat = scale (a do + beta khat (delta . do)): per slice, summed over slices below
            pp[r0 + i] = a.scale * (pq[i] + in.beta * in.k[i] * ddo);
            pp[DK + r0 + i] = in.beta * pk[i];
            pp[2 * DK + r0 + i] = pg[i];
          }
        }
        if (l == 0) pp[3 * DK] = db;
        // dv for this slice's columns (complete: no other slice touches them)
        if (rg == 0) {
          float dvv[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) dvv[j] = in.beta * u[j];
          store4(dvo + ((size_t)tok * a.H + h) * DV + col, dvv);
        }
        __syncthreads();
        // the slices' sums in a fixed order
        {
          const size_t th = (size_t)tok * a.H + h;
          for (int idx = threadIdx.x; idx < 3 * DK + 1; idx += 64 * NS) {
            float acc = 0.f;
#pragma unroll
            for (int ss = 0; ss < NS; ++ss) acc += part[par][ss][idx];
            if (idx < DK) a.dqh[th * DK + idx] = acc;
            else if (idx < 2 * DK) a.dkh[th * DK + idx - DK] = acc;
            else if (idx < 3 * DK) a.dg[th * DK + idx - 2 * DK] = acc;
            else store1(dbo + th, acc);
          }
        }
        par ^= 1;  // the other buffer is written next: one barrier per token suffices
        cur = nxt;
#pragma unroll
        for (int j = 0; j < 4; ++j) dov[j] = don[j];
      }
    }
    if (a.dh0) {
#pragma unroll
      for (int i = 0; i < NR; ++i) store4(a.dh0 + sbase + (size_t)(r0 + i) * DV + col, G[i]);
    }
    __syncthreads();  // the next (sequence, head) rewrites LDS and scratch
  }
}

// dq, dk from dqhat, dkhat through the L2 normalisation: dx = (dxhat - xhat (xhat . dxhat)) / |x|
// (0 for a zero vector), one wave per (token, head), the norm taken after the same exact
// power-of-two rescale as in the forward kernels.
template <int DK, typename InT>
__global__ __launch_bounds__(256) void norm_bwd_kernel(const void* qv, const void* kv, const float* dqh,
                                                       const float* dkh, void* dqv, void* dkv, int64_t rows) {
  constexpr int PL = DK / 64;  // channels per lane
  const int l = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // whole waves, no barrier
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const InT* x = reinterpret_cast<const InT*>(which ? kv : qv) + row * DK + l * PL;
    const float* dxh = (which ? dkh : dqh) + row * DK + l * PL;
    InT* dx = reinterpret_cast<InT*>(which ? dkv : dqv) + row * DK + l * PL;
    float xv[PL], dh[PL];
#pragma unroll
    for (int c = 0; c < PL; ++c) {
      xv[c] = load1(x + c);
      dh[c] = dxh[c];
    }
    float m = 0.f;
#pragma unroll
    for (int c = 0; c < PL; ++c) m = fmaxf(m, fabsf(xv[c]));
    m = wave_max(m);
    const int ex = m > 0.f ? ilogb_pos(m) : 0;
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < PL; ++c) {
      xv[c] = ldexpf(xv[c], -ex);
      ss = fmaf(xv[c], xv[c], ss);
    }
    ss = wave_sum(ss);
    const float nrm = sqrtf(ss);  // |x| 2^-ex
    float dot = 0.f;
#pragma unroll
    for (int c = 0; c < PL; ++c) {
      xv[c] = ss > 0.f ? xv[c] / nrm : 0.f;  // xhat
      dot = fmaf(xv[c], dh[c], dot);
    }
    dot = wave_sum(dot);
#pragma unroll
    for (int c = 0; c < PL; ++c) {
      const float r = ss > 0.f ? ldexpf((dh[c] - xv[c] * dot) / nrm, -ex) : 0.f;
      store1(dx + c, r);
    }
  }
}

}  // namespace kda
