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
// Work split.  The value columns of the state evolve independently (a step mixes
// key channels only), so each (sequence, head) is cut into parts of 16 (or 32) value
// columns, one workgroup per part, and each of its eight waves owns WC = 2 (or 4)
// columns: lane l holds key channels l*NR .. l*NR + NR - 1 (NR = dk / 64) of those
// columns, so a lane carries 4 (or 8) state elements (dk = 128) and a step is short.
// Narrow parts give a few (sequence, head) pairs enough workgroups to fill the chip;
// wide ones do less work per column once there are workgroups enough.  Sums over key
// channels (per column) are wave sums; the per-row sums dqhat, dkhat, dg and the
// scalar dbeta add the eight waves' columns through LDS in a fixed order, and the
// parts' partial sums are added (again in a fixed order) by the finish kernel:
// results are deterministic.
//
// The walk, per part:
//   1. forward over the sequence, storing the part's state at the start of every
//      8-token segment (checkpoints, fp32, in the workspace) and every token's delta for
//      the part's columns;
//   2. backwards over the segments: the segment's forward is replayed from its
//      checkpoint into registers with the stored deltas (elementwise, no sums: the state
//      before each of its tokens, bitwise walk 1's), then its tokens are walked in
//      reverse.
// A pre-pass packs, per (token, head), [qhat | khat | exp(g) | beta] into one fp32 record.
// Each 8-token segment's records and the part's columns of v (walk 1) or of the stored
// deltas and dout (walk 2) are staged in LDS, the next segment's loads in flight while the
// current one is walked, so a step waits on LDS, never on HBM.
#pragma once

#include "kda_recurrent.h"

namespace kda {

constexpr int kBwdWaves = 8;                              // waves per workgroup
// value columns per wave: 2 or 4 (a template parameter of the kernel, chosen per call), so a
// workgroup (a part) owns kBwdWaves * 2 or * 4 value columns
constexpr int kBwdSeg = 8;                                // tokens per checkpoint segment
constexpr int kBwdThreads = 64 * kBwdWaves;

// The pre-pass record of one (token, head): qhat [DK], khat [DK], exp(g) [DK], beta, 3 zeros.
template <int DK>
struct BwdRec {
  static constexpr int FLOATS = 3 * DK + 4;
  static constexpr int U4 = FLOATS / 4;  // 16-byte units
};

struct BwdArgs {
  const float* rec;       // [tokens, H, 3 DK + 4] fp32 records (pre-pass)
  const void* v;
  const float* h0;
  const int32_t* cu;        // packed offsets (device) or NULL
  const int32_t* seq_off;   // packed: first 64-token chunk of each sequence (chunk map), or NULL
  const int32_t* seq_order; // packed: sequences longest first (chunk map), or NULL
  const void* dout;
  const float* dht;
  float* psum;            // [parts, tokens * H, 3 DK + 4] fp32: each part's row sums
                          // [dL/dqhat | dL/dkhat | dL/dg | dL/dbeta, 0, 0, 0]
  void* dv;               // [tokens, H, DV] io dtype
  float* dh0;             // [N, H, DK, DV] or NULL
  float* ckpt;            // [slots, H, parts, waves, 64 lanes, NR, 4] fp32
  float* delta;           // [tokens, H, DV] fp32: v - a^T khat of every token (walk 1)
  int64_t T, T_total, N;  // tokens per row (fixed) / total (packed); all tokens; sequences
  int64_t nc;             // fixed: 64-token chunks per row
  int64_t n_chunk_ub;     // 64-token chunks the workspace holds (8 checkpoint slots each)
  int32_t H;
  float scale;
};

__device__ inline void store1(uint16_t* p, float x) { *p = (uint16_t)(pack_bf16x2(x, 0.f) & 0xffffu); }
__device__ inline void store1(float* p, float x) { *p = x; }

// Row rotation written as a DPP move with a zero old value and bound_ctrl (the rotation
// reads a lane in every case, so the result is row_ror's): the compiler folds it into the
// add that consumes it (v_add_f32_dpp).
template <int N>
__device__ inline float row_ror_z(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + N, 0xF, 0xF, true));
}

__device__ inline float wave_sum(float x) {
  x += row_ror_z<8>(x);
  x += row_ror_z<4>(x);
  x += row_ror_z<2>(x);
  x += row_ror_z<1>(x);
  return rows4_sum(x);
}

// One segment's staged inputs in LDS, as 16-byte units copied unchanged from HBM:
//   [kBwdSeg records][kBwdSeg rows of V1][kBwdSeg rows of V2]
// V1 = the part's columns of v (walk 1, io dtype) or of the deltas (walk 2, fp32),
// V2 = the part's columns of dout (walk 2 only, io dtype).  Slot s of the staging loads
// is unit s.
template <int DK, typename InT, bool WALK2, int PC>
struct BwdStageMap {
  static constexpr int AR = BwdRec<DK>::U4;                               // units per record
  static constexpr int V1 = PC * (WALK2 ? 4 : (int)sizeof(InT)) / 16;    // units per V1 row
  static constexpr int V2 = WALK2 ? PC * (int)sizeof(InT) / 16 : 0;      // units per V2 row
  static constexpr int UNITS = kBwdSeg * (AR + V1 + V2);
  static constexpr int ROUNDS = (UNITS + kBwdThreads - 1) / kBwdThreads;
};
template <int DK>
constexpr int kBwdStageBytes = 16 * kBwdSeg * (BwdRec<DK>::U4 + 8 + 8);  // the largest map

// Request the inputs of tokens [ts, te) (0 < te - ts <= kBwdSeg) of head h, the part's value
// columns from c0.  Every slot is one unconditional 16-byte load whose address is chosen
// first, so no value merge waits on a load and the loads stay in flight until the commit
// (slots past te read token te - 1 and are never used).
template <int DK, int DV, typename InT, bool WALK2, int PC, int R>
__device__ inline void stage_issue(uint4_v (&r)[R], const BwdArgs& a, int64_t ts, int64_t te, int h, int c0) {
  using M = BwdStageMap<DK, InT, WALK2, PC>;
  static_assert(R == M::ROUNDS, "staging registers");
  const uint8_t* rec = reinterpret_cast<const uint8_t*>(a.rec);
  const uint8_t* v1 = WALK2 ? reinterpret_cast<const uint8_t*>(a.delta) : reinterpret_cast<const uint8_t*>(a.v);
  const uint8_t* v2 = reinterpret_cast<const uint8_t*>(a.dout);
  constexpr size_t E1 = WALK2 ? 4 : sizeof(InT);
  auto tok = [&](int u) { return ts + u < te ? ts + u : te - 1; };
#pragma unroll
  for (int rd = 0; rd < M::ROUNDS; ++rd) {
    const int s = (int)threadIdx.x + rd * kBwdThreads;
    const int s1 = s - kBwdSeg * M::AR;
    const int s2 = s1 - kBwdSeg * M::V1;
    const uint8_t* src;
    if (s1 < 0) {
      src = rec + (((size_t)tok(s / M::AR) * a.H + h) * M::AR + s % M::AR) * 16;
    } else if (s2 < 0) {
      src = v1 + (((size_t)tok(s1 / M::V1) * a.H + h) * DV + c0) * E1 + (size_t)(s1 % M::V1) * 16;
    } else {
      const int s2c = M::V2 > 0 ? s2 : 0;
      const int v2u = M::V2 > 0 ? M::V2 : 1;
      src = v2 + (((size_t)tok(s2c / v2u) * a.H + h) * DV + c0) * sizeof(InT) + (size_t)(s2c % v2u) * 16;
    }
    // slots past UNITS fall in the last region with an in-bounds address (clamped token,
    // unit index modulo the row): loaded unconditionally, never committed
    r[rd] = *reinterpret_cast<const uint4_v*>(src);
  }
}

template <int DK, typename InT, bool WALK2, int PC, int R>
__device__ inline void stage_commit(const uint4_v (&r)[R], uint8_t* st) {
  using M = BwdStageMap<DK, InT, WALK2, PC>;
  static_assert(R == M::ROUNDS, "staging registers");
#pragma unroll
  for (int rd = 0; rd < M::ROUNDS; ++rd) {
    const int s = (int)threadIdx.x + rd * kBwdThreads;
    if (s < M::UNITS) *reinterpret_cast<uint4_v*>(st + (size_t)s * 16) = r[rd];
  }
}

// WC (2 or 4) consecutive staged elements of a V row as fp32.
template <int WC>
__device__ inline void lds_cols(const uint8_t* p, bool bf16, float* o) {
  if constexpr (WC == 4) {
    if (bf16) {
      const uint2 x = *reinterpret_cast<const uint2*>(p);
      o[0] = __uint_as_float(x.x << 16); o[1] = __uint_as_float(x.x & 0xffff0000u);
      o[2] = __uint_as_float(x.y << 16); o[3] = __uint_as_float(x.y & 0xffff0000u);
    } else {
      const float4 x = *reinterpret_cast<const float4*>(p);
      o[0] = x.x; o[1] = x.y; o[2] = x.z; o[3] = x.w;
    }
  } else {
    if (bf16) {
      const uint32_t x = *reinterpret_cast<const uint32_t*>(p);
      o[0] = __uint_as_float(x << 16); o[1] = __uint_as_float(x & 0xffff0000u);
    } else {
      const float2 x = *reinterpret_cast<const float2*>(p);
      o[0] = x.x; o[1] = x.y;
    }
  }
}

// WC consecutive global elements (fp32 or bf16) as fp32, and back (bf16 rounds to nearest
// even).
template <int WC, typename T>
__device__ inline void gload_cols(const T* p, float* o) {
  if constexpr (WC == 4) {
    load4(p, o);
  } else if constexpr (sizeof(T) == 4) {
    const float2 x = *reinterpret_cast<const float2*>(p);
    o[0] = x.x; o[1] = x.y;
  } else {
    const uint32_t x = *reinterpret_cast<const uint32_t*>(p);
    o[0] = __uint_as_float(x << 16); o[1] = __uint_as_float(x & 0xffff0000u);
  }
}
template <int WC>
__device__ inline void gstore_cols(float* p, const float* x) {
  if constexpr (WC == 4) store4(p, x);
  else *reinterpret_cast<float2*>(p) = make_float2(x[0], x[1]);
}
template <int WC>
__device__ inline void gstore_cols(uint16_t* p, const float* x) {
  if constexpr (WC == 4) store4(p, x);
  else *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(x[0], x[1]);
}

// s_waitcnt vmcnt(0) as an instruction the compiler's wait tracking sees (gfx9 encoding:
// vmcnt 0, expcnt and lgkmcnt at their maxima): no vector-memory load is pending after it
// on any path, so a walk's loop never waits on loads issued before it.
__device__ inline void wait_vm_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int N>
__device__ inline void lds_read(const float* p, float (&o)[N]) {
  if constexpr (N == 2) {
    const float2 x = *reinterpret_cast<const float2*>(p);
    o[0] = x.x; o[1] = x.y;
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) o[i] = p[i];
  }
}

// Sums over the wave of N independent values, the reductions interleaved step by step so
// that each one's DPP and row-swap latencies overlap the others.
template <int N>
__device__ inline void wave_sums(float (&x)[N]) {
#pragma unroll
  for (int j = 0; j < N; ++j) x[j] += row_ror_z<8>(x[j]);
#pragma unroll
  for (int j = 0; j < N; ++j) x[j] += row_ror_z<4>(x[j]);
#pragma unroll
  for (int j = 0; j < N; ++j) x[j] += row_ror_z<2>(x[j]);
#pragma unroll
  for (int j = 0; j < N; ++j) x[j] += row_ror_z<1>(x[j]);
  uint32_t y[N][2];
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[j]), __float_as_uint(x[j]), false, false);
    y[j][0] = t[0];
    y[j][1] = t[1];
  }
#pragma unroll
  for (int j = 0; j < N; ++j) x[j] = __uint_as_float(y[j][0]) + __uint_as_float(y[j][1]);
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[j]), __float_as_uint(x[j]), false, false);
    y[j][0] = t[0];
    y[j][1] = t[1];
  }
#pragma unroll
  for (int j = 0; j < N; ++j) x[j] = __uint_as_float(y[j][0]) + __uint_as_float(y[j][1]);
}

template <int DK, int DV, typename InT, int WC>
__global__ __launch_bounds__(kBwdThreads) void recurrent_bwd_kernel(BwdArgs a) {
  static_assert(WC == 2 || WC == 4, "2 or 4 value columns per wave");
  constexpr int NR = DK / 64;                  // key channels per lane
  constexpr int PC = kBwdWaves * WC;           // value columns per workgroup (part)
  constexpr int PARTS = DV / PC;               // workgroups per (sequence, head)
  constexpr int CK = 64 * NR * WC;             // floats of one wave's share of a checkpoint
  constexpr bool BF = sizeof(InT) == 2;
  using M1 = BwdStageMap<DK, InT, false, PC>;
  using M2 = BwdStageMap<DK, InT, true, PC>;
  constexpr int RF = BwdRec<DK>::FLOATS;
  static_assert(DV % PC == 0 && DK % 64 == 0, "unsupported head dimensions");
  __shared__ __align__(16) uint8_t stage[2][kBwdStageBytes<DK>];
  // per token parity and wave: the wave's row sums [dqhat | dkhat | dg] and dbeta
  __shared__ float part[2][kBwdWaves][3 * DK + 1];
  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r0 = l * NR;            // first key channel of the lane
  const int wc = w * WC;            // first column of the wave inside the part
  const int pidx = (int)(blockIdx.x % PARTS);
  const int64_t nh = blockIdx.x / PARTS;
  const int h = (int)(nh % a.H);
  const int64_t n = a.cu ? (int64_t)a.seq_order[nh / a.H] : nh / a.H;
  const int c0 = pidx * PC;            // first column of the part
  const int col = c0 + wc;             // first column of the wave

  int64_t t0 = n * a.T, t1 = t0 + a.T, slot0 = n * a.nc * (kChunk / kBwdSeg);
  if (a.cu) {
    t0 = a.cu[n];
    t1 = a.cu[n + 1];
    t0 = t0 < 0 ? 0 : (t0 > a.T ? a.T : t0);
    t1 = t1 < t0 ? t0 : (t1 > a.T ? a.T : t1);
    slot0 = (int64_t)a.seq_off[n] * (kChunk / kBwdSeg);
  }
  int64_t nseg = (t1 - t0 + kBwdSeg - 1) / kBwdSeg;
  if (a.cu) {
    // the checkpoints the chunk map set aside for this sequence (fewer only when
    // cu_seqlens breaks its precondition: the walk then stops there)
    const int64_t end = (int64_t)a.seq_off[n + 1] < a.n_chunk_ub ? (int64_t)a.seq_off[n + 1] : a.n_chunk_ub;
    const int64_t room = (end - a.seq_off[n]) * (kChunk / kBwdSeg);
    nseg = nseg < room ? nseg : (room > 0 ? room : 0);
    t1 = t0 + nseg * kBwdSeg < t1 ? t0 + nseg * kBwdSeg : t1;
  }
  const size_t sbase = ((size_t)n * a.H + h) * DK * DV;
  auto ck = [&](int64_t seg) {
    return a.ckpt + ((((size_t)(slot0 + seg) * a.H + h) * PARTS + pidx) * kBwdWaves + w) * CK;
  };
  auto put = [&](float* base, const float (&S)[NR][WC]) {
#pragma unroll
    for (int i = 0; i < NR; ++i) gstore_cols<WC>(base + ((size_t)i * 64 + l) * WC, S[i]);
  };
  auto get = [&](const float* base, float (&S)[NR][WC]) {
#pragma unroll
    for (int i = 0; i < NR; ++i) gload_cols<WC>(base + ((size_t)i * 64 + l) * WC, S[i]);
  };
  auto seg_end = [&](int64_t ts) { return ts + kBwdSeg < t1 ? ts + kBwdSeg : t1; };
  // staged token u: its record, and the wave's four columns of V1 / V2
  auto srec = [&](const uint8_t* st, int u) { return reinterpret_cast<const float*>(st) + u * RF; };
  auto sv1 = [&](const uint8_t* st, int u, bool walk2, float* o) {
    const int v1u = walk2 ? M2::V1 : M1::V1;
    const size_t e1 = walk2 ? 4 : sizeof(InT);
    lds_cols<WC>(st + 16 * (kBwdSeg * M1::AR + u * v1u) + wc * e1, BF && !walk2, o);
  };
  auto sv2 = [&](const uint8_t* st, int u, float* o) {
    lds_cols<WC>(st + 16 * (kBwdSeg * (M2::AR + M2::V1) + u * M2::V2) + wc * sizeof(InT), BF, o);
  };

  // walk 1: one forward step of the lane's state from the staged token u; the token's
  // delta (v - a^T khat for the wave's columns) is stored for walk 2
  auto fwd_step = [&](float (&S)[NR][WC], const uint8_t* st, int u, int64_t tok) {
    const float* rc = srec(st, u);
    float ek[NR], kk[NR], vv[WC];
    lds_read<NR>(rc + 2 * DK + r0, ek);
    lds_read<NR>(rc + DK + r0, kk);
    sv1(st, u, false, vv);
    const float b = rc[3 * DK];
    float p[WC];
#pragma unroll
    for (int j = 0; j < WC; ++j) p[j] = 0.f;
#pragma unroll
    for (int i = 0; i < NR; ++i)
#pragma unroll
      for (int j = 0; j < WC; ++j) {
        S[i][j] *= ek[i];
        p[j] = fmaf(kk[i], S[i][j], p[j]);
      }
    wave_sums<WC>(p);
    float d[WC];
#pragma unroll
    for (int j = 0; j < WC; ++j) d[j] = vv[j] - p[j];
    if (l == 0) gstore_cols<WC>(a.delta + ((size_t)tok * a.H + h) * DV + col, d);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const float bk = b * kk[i];
#pragma unroll
      for (int j = 0; j < WC; ++j) S[i][j] = fmaf(bk, d[j], S[i][j]);
    }
  };
  // walk 2: the same step from the stored delta (elementwise: no sums over key channels,
  // and bitwise the state walk 1 had)
  auto replay_step = [&](float (&S)[NR][WC], const uint8_t* st, int u) {
    const float* rc = srec(st, u);
    float ek[NR], kk[NR], d[WC];
    lds_read<NR>(rc + 2 * DK + r0, ek);
    lds_read<NR>(rc + DK + r0, kk);
    sv1(st, u, true, d);
    const float b = rc[3 * DK];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const float bk = b * kk[i];
#pragma unroll
      for (int j = 0; j < WC; ++j) S[i][j] = fmaf(bk, d[j], S[i][j] * ek[i]);
    }
  };

  // 1. forward with a checkpoint at every segment start
  {
    uint4_v rg[M1::ROUNDS];
    float S[NR][WC];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      if (a.h0) gload_cols<WC>(a.h0 + sbase + (size_t)(r0 + i) * DV + col, S[i]);
      else
#pragma unroll
        for (int j = 0; j < WC; ++j) S[i][j] = 0.f;
    }
    if (nseg > 0) {
      stage_issue<DK, DV, InT, false, PC>(rg, a, t0, seg_end(t0), h, c0);
      stage_commit<DK, InT, false, PC>(rg, stage[0]);
    }
    wait_vm_loads();
    __syncthreads();
    for (int64_t k = 0; k < nseg; ++k) {
      const int64_t ts = t0 + k * kBwdSeg;
      const int len = (int)(seg_end(ts) - ts);
      if (k + 1 < nseg) stage_issue<DK, DV, InT, false, PC>(rg, a, ts + kBwdSeg, seg_end(ts + kBwdSeg), h, c0);
      put(ck(k), S);
      const uint8_t* st = stage[k & 1];
#pragma unroll
      for (int u = 0; u < kBwdSeg; ++u)
        if (u < len) fwd_step(S, st, u, ts + u);
      if (k + 1 < nseg) stage_commit<DK, InT, false, PC>(rg, stage[(k + 1) & 1]);
      __syncthreads();  // also orders walk 1's delta and checkpoint stores before walk 2 reads them
    }
  }

  // 2. backwards over the segments
  uint4_v rg[M2::ROUNDS];
  float G[NR][WC];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    if (a.dht) gload_cols<WC>(a.dht + sbase + (size_t)(r0 + i) * DV + col, G[i]);
    else
#pragma unroll
      for (int j = 0; j < WC; ++j) G[i][j] = 0.f;
  }
  InT* dvo = reinterpret_cast<InT*>(a.dv);
  const size_t pbase = (size_t)pidx * (size_t)a.T_total * a.H;
  int par = 0;
  float ckn[NR][WC];
  if (nseg > 0) {
    const int64_t ts = t0 + (nseg - 1) * kBwdSeg;
    stage_issue<DK, DV, InT, true, PC>(rg, a, ts, seg_end(ts), h, c0);
    stage_commit<DK, InT, true, PC>(rg, stage[(nseg - 1) & 1]);
    get(ck(nseg - 1), ckn);
  }
  wait_vm_loads();
  __syncthreads();
  for (int64_t k = nseg - 1; k >= 0; --k) {
    const int64_t ts = t0 + k * kBwdSeg;
    const int len = (int)(seg_end(ts) - ts);
    if (k > 0) stage_issue<DK, DV, InT, true, PC>(rg, a, ts - kBwdSeg, ts, h, c0);
    // St[u]: the state before token ts + u
    float St[kBwdSeg][NR][WC];
#pragma unroll
    for (int i = 0; i < NR; ++i)
#pragma unroll
      for (int j = 0; j < WC; ++j) St[0][i][j] = ckn[i][j];
    if (k > 0) get(ck(k - 1), ckn);  // the previous segment's checkpoint, one segment ahead
    const uint8_t* st = stage[k & 1];
#pragma unroll
    for (int u = 0; u + 1 < kBwdSeg; ++u) {
      if (u + 1 < len) {
#pragma unroll
        for (int i = 0; i < NR; ++i)
#pragma unroll
          for (int j = 0; j < WC; ++j) St[u + 1][i][j] = St[u][i][j];
        replay_step(St[u + 1], st, u);
      }
    }
#pragma unroll
    for (int u = kBwdSeg - 1; u >= 0; --u) {
      if (u >= len) continue;
      float (&A)[NR][WC] = St[u];  // S_{t-1}, then a
      const int64_t tok = ts + u;
      const float* rc = srec(st, u);
      float ek[NR], kk[NR], qq[NR], d[WC], dov[WC];
      lds_read<NR>(rc + 2 * DK + r0, ek);
      lds_read<NR>(rc + DK + r0, kk);
      lds_read<NR>(rc + r0, qq);
      sv1(st, u, true, d);
      sv2(st, u, dov);
      const float b = rc[3 * DK];
#pragma unroll
      for (int i = 0; i < NR; ++i)
#pragma unroll
        for (int j = 0; j < WC; ++j) A[i][j] *= ek[i];
      // G += scale qhat do^T, then u = G^T khat (column sums over the key channels)
      float uu[WC];
#pragma unroll
      for (int j = 0; j < WC; ++j) uu[j] = 0.f;
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const float sq = a.scale * qq[i];
#pragma unroll
        for (int j = 0; j < WC; ++j) {
          G[i][j] = fmaf(sq, dov[j], G[i][j]);
          uu[j] = fmaf(kk[i], G[i][j], uu[j]);
        }
      }
      wave_sums<WC>(uu);
      float ddo = 0.f, db = 0.f;  // delta . do and u . delta over the wave's columns
#pragma unroll
      for (int j = 0; j < WC; ++j) {
        ddo = fmaf(d[j], dov[j], ddo);
        db = fmaf(uu[j], d[j], db);
      }
      float* pp = part[par][w];
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        float aq = 0.f, gd = 0.f, au = 0.f, ag = 0.f;
        const float bk = b * kk[i];
#pragma unroll
        for (int j = 0; j < WC; ++j) {
          aq = fmaf(A[i][j], dov[j], aq);
          gd = fmaf(G[i][j], d[j], gd);
          au = fmaf(A[i][j], uu[j], au);
          const float da = G[i][j] - bk * uu[j];
          ag = fmaf(A[i][j], da, ag);
          G[i][j] = ek[i] * da;  // dL/dS_{t-1}
        }
        // dqhat = scale (a do + beta khat (delta . do)), dkhat = beta (G delta - a u), dg
        pp[r0 + i] = a.scale * (aq + bk * ddo);
        pp[DK + r0 + i] = b * (gd - au);
        pp[2 * DK + r0 + i] = ag;
      }
      const size_t th = (size_t)tok * a.H + h;
      if (l == 0) {
        pp[3 * DK] = db;
        // dv for the wave's columns (complete: no other wave or part touches them)
        float dvv[WC];
#pragma unroll
        for (int j = 0; j < WC; ++j) dvv[j] = b * uu[j];
        gstore_cols<WC>(dvo + th * DV + col, dvv);
      }
      __syncthreads();
      // the waves' sums in a fixed order: this part's share of the row sums, one
      // contiguous row per (token, head)
      for (int idx = tid; idx < 3 * DK + 1; idx += kBwdThreads) {
        float acc = 0.f;
#pragma unroll
        for (int ww = 0; ww < kBwdWaves; ++ww) acc += part[par][ww][idx];
        a.psum[(pbase + th) * (3 * DK + 4) + idx] = acc;
      }
      par ^= 1;  // the other buffer is written next: one barrier per token suffices
    }
    if (k > 0) stage_commit<DK, InT, true, PC>(rg, stage[(k - 1) & 1]);
    __syncthreads();
  }
  if (a.dh0) {
#pragma unroll
    for (int i = 0; i < NR; ++i) gstore_cols<WC>(a.dh0 + sbase + (size_t)(r0 + i) * DV + col, G[i]);
  }
}

// Pre-pass for the walks, one wave per (token, head): the record [qhat | khat | exp(g) |
// beta, 0, 0, 0], with x / |x| taken after the exact power-of-two rescale by the largest
// entry (as in the forward kernels; a zero vector stays zero).
template <int DK, typename InT>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const void* qv, const void* kv, const float* g,
                                                       const void* beta, float* rec, int64_t rows) {
  constexpr int PL = DK / 64;  // channels per lane
  const int l = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // whole waves, no barrier
  float* o = rec + row * BwdRec<DK>::FLOATS;
#pragma unroll
  for (int c = 0; c < PL; ++c) o[2 * DK + l * PL + c] = exp2_hw(g[row * DK + l * PL + c] * kLog2e);
  if (l < 4) o[3 * DK + l] = l == 0 ? load1(reinterpret_cast<const InT*>(beta) + row) : 0.f;
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const InT* x = reinterpret_cast<const InT*>(which ? kv : qv) + row * DK + l * PL;
    float xv[PL];
#pragma unroll
    for (int c = 0; c < PL; ++c) xv[c] = load1(x + c);
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
    const float inv = ss > 0.f ? 1.f / sqrtf(ss) : 0.f;
#pragma unroll
    for (int c = 0; c < PL; ++c) o[which * DK + l * PL + c] = xv[c] * inv;
  }
}

// Finish: the parts' row sums added in a fixed order (dg and dbeta written), then dq, dk
// from dqhat, dkhat through the L2 normalisation: dx = (dxhat - xhat (xhat . dxhat)) / |x|
// (0 for a zero vector), one wave per (token, head), the norm taken after the same exact
// power-of-two rescale as in the forward kernels.
template <int DK, typename InT>
__global__ __launch_bounds__(256) void bwd_finish_kernel(const void* qv, const void* kv, const float* psum,
                                                         int parts, int64_t rows, void* dqv, void* dkv,
                                                         float* dg, void* dbeta) {
  constexpr int PL = DK / 64;  // channels per lane
  constexpr int PR = 3 * DK + 4;
  const int l = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // whole waves, no barrier
  float sq[PL], sk[PL], sg[PL], sb = 0.f;
#pragma unroll
  for (int c = 0; c < PL; ++c) sq[c] = sk[c] = sg[c] = 0.f;
  for (int p = 0; p < parts; ++p) {
    const float* r = psum + ((size_t)p * rows + row) * PR + l * PL;
#pragma unroll
    for (int c = 0; c < PL; ++c) {
      sq[c] += r[c];
      sk[c] += r[DK + c];
      sg[c] += r[2 * DK + c];
    }
    if (l == 0) sb += psum[((size_t)p * rows + row) * PR + 3 * DK];
  }
#pragma unroll
  for (int c = 0; c < PL; ++c) dg[row * DK + l * PL + c] = sg[c];
  if (l == 0) store1(reinterpret_cast<InT*>(dbeta) + row, sb);
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const InT* x = reinterpret_cast<const InT*>(which ? kv : qv) + row * DK + l * PL;
    InT* dx = reinterpret_cast<InT*>(which ? dkv : dqv) + row * DK + l * PL;
    float xv[PL], dh[PL];
#pragma unroll
    for (int c = 0; c < PL; ++c) {
      xv[c] = load1(x + c);
      dh[c] = which ? sk[c] : sq[c];
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
