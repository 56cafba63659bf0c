// State-scan kernel: the sequential walk over a sequence's chunks, one
// workgroup per (sequence, head, slice of NV value columns).
//
// The value columns of the state evolve independently (the recurrence only
// mixes key channels), so a head's state is split into DV/NV column slices
// that walk their chunks in parallel ("Autoresearch on Kimi Delta
// Attention", section "The optimization trace": the recurrence split across
// value tiles to expose more independent work).  The state is carried in fp32
// registers for the whole walk; "Kernel Design Agents (KDA) optimize Kimi
// Delta Attention (KDA)", section "01 - Results", shows that a bf16 state
// compounds error along the sequence.  Per chunk (S0 = state at the chunk
// start, all products on fp16 MFMA with fp32 accumulation):
//     Delta  = U - W S0                                   (the corrected values)
//     o      = scale (Qhat*exp(G) S0 + Aqk Delta)         (chunk output, fused here)
//     S_next = Diag(exp(G_last)) S0 + (Khat*exp(G_last-G))^T Delta
// Boundaries come from the chunk table (built from cu_seqlens on the device);
// the walk never drops history.
//
// Work split (8 waves): waves 0..3 each own a 16-token block of the chunk: they
// hold that block's rows of W, Qhat*exp(G), Aqk and U, form its rows of Delta and
// of the output.  Waves 4..7 each own DK/4 key channels of the state: they hold
// the fp32 state rows and the matching rows of (Khat*exp(G_last-G))^T and
// exp(G_last), and form S_next.  Each chunk factor is read from memory once per
// workgroup.  Per chunk there are two barriers: A (Delta complete in LDS) and B
// (S_next complete in LDS); the fp16 state copy is double buffered because the
// token waves still read the chunk's S0 (for the output) while the key waves
// write the next one.
//
// fp16 range: the state is linear in (v, h0).  For beta in [0, 1], g <= 0 and
// unit keys, every column s of the state obeys ||s_t||^2 <= ||s_{t-1}||^2 + v_t^2,
// hence ||s_t|| <= B = sqrt(max_col ||h0_col||^2 + L vmax^2) over a sequence of
// length L, and |Delta| <= vmax + B.  The fp16 copies of S and Delta are taken
// after an exact power-of-two scale 2^es with 2^es B <= 2^14, so they stay
// below the fp16 maximum for every legal input; the fp32 state is unscaled.
#pragma once

#include "kda_device.h"

namespace kda {

constexpr int kScanThreads = 512;  // 4 token-block waves + 4 key-block waves
#ifndef KDA_SCAN_DEPTH
#define KDA_SCAN_DEPTH 3
#endif
// chunks of factors held in registers (prefetch distance + 1): three for 16-column slices;
// wider slices hold more state and output fragments, so their ring is two deep (no spills)
template <int NV>
constexpr int scan_depth() { return NV <= 16 ? KDA_SCAN_DEPTH : 2; }

struct ScanArgs {
  const float* h0;
  float* ht;
  void* out;
  const int32_t* cu;
  int64_t T;
  int64_t T_total;
  int64_t N;
  int32_t H;
  int64_t n_chunk_ub;
  const int32_t* seq_off;    // packed mode: first chunk of each sequence
  const int32_t* seq_order;  // packed mode: sequences, longest first
  int64_t nc;                // fixed-length mode (cu == NULL): chunks per row
  const uint8_t* rec;
  float scale;
  uint64_t* ctl;  // workspace control words ([0]: flag value of the most recent launch; 0 here)
};

template <int DK, int DV, int NV>
struct ScanSmem {
  static constexpr int KSK = DK / 32;
  static constexpr int NT = NV / 16;
  static constexpr size_t SBUF = (size_t)KSK * NT * 64 * 16;      // fp16 S0 fragments [KSK][NT][64] f16x8
  static constexpr size_t SB = 0;                                  // two S0 buffers (chunk parity)
  static constexpr size_t DB = SB + 2 * SBUF;                      // Delta fragments [2][NT][64] f16x8
  static constexpr size_t CN = DB + (size_t)2 * NT * 64 * 16;      // column norm partials [4][NV]
  static constexpr size_t RED = CN + 4 * NV * 4;                   // [8]
  static constexpr size_t FAIL = RED + 8 * 4;                      // fused: a token wave's wait gave up
  static constexpr size_t BYTES = FAIL + 16;
};

// Chunk factors of one token-block wave: rows 16 i .. 16 i + 15 of W, Qhat*exp(G),
// Aqk (A fragments) and the wave's slice of U (C-layout tiles).
template <int DK, int NV>
struct TokRegs {
  static constexpr int KSK = DK / 32;
  static constexpr int NT = NV / 16;
  f16x8 wf[KSK];
  f16x8 qf[KSK];
  f16x8 af[2];
  f16x4 uf[NT];
  int ue;
  float vmax;  // max |v| of the chunk (read only by the fused kernel)
};

// Chunk factors of one key-block wave: its row tiles of (Khat*exp(G_last-G))^T
// (A fragments over the chunk's tokens) and exp(G_last), one value per lane: lane
// (t, gq) holds channel 16 ct + 4 gq + (t & 3), and row broadcasts inside each row of
// 16 lanes hand every lane its four C-layout rows 16 ct + 4 gq + r (a float4 per lane
// would load each value sixteen times).
template <int DK>
struct KeyRegs {
  static constexpr int TPK = DK / 64;  // 16-row tiles per key wave
  f16x8 kt[TPK][2];
  float lam[TPK];
  int ec[TPK];  // row exponents of K~^T (the rows were scaled by 2^-ec)
  float vmax;  // max |v| of the chunk (read only by the fused kernel)
};

// The loads of a chunk's factors are issued in groups spread over the previous chunk's
// step, so that the eight waves never queue all of them on the vector-memory path at
// once.  Token waves: 0 = W, 1 = Qhat*exp(G), 2 = Aqk, U and ue (or 3 = U and ue, 4 = Aqk,
// for a walk that reuses its slot and so requests each factor after its last use).  Requesting
// U together with W instead (the next Delta needs both) was slower: the walk's loads then
// bunch at the start of the step.  Key
// waves: 0 = K~^T, 1 = exp(G_last).  `rows`: the chunk's valid tokens (0 past a walk's
// end); the parts of the record past them are not fetched and read as zeros.
template <int PART, int DK, int DV, int NV, bool FUSED = false>
__device__ __forceinline__ void load_tok(TokRegs<DK, NV>& c, const uint8_t* rec, int rows, int i, int l, int slice) {
  using R = Rec<DK, DV>;
  using TR = TokRegs<DK, NV>;
  const int nb = rec_rows_present(rows, i) ? (int)R::BYTES : 0;  // row block i
  if (PART == 0) {
#pragma unroll
    for (int s = 0; s < TR::KSK; ++s)
      c.wf[s] = rec_load<f16x8, FUSED>(rec, nb, R::W + ((size_t)(i * TR::KSK + s) * 64 + l) * 16);
  } else if (PART == 1) {
#pragma unroll
    for (int s = 0; s < TR::KSK; ++s)
      c.qf[s] = rec_load<f16x8, FUSED>(rec, nb, R::Q + ((size_t)(i * TR::KSK + s) * 64 + l) * 16);
  } else {
    if (PART == 2 || PART == 4) {
      // Aqk is lower triangular: token blocks 0 and 1 have nothing in the second 32-token
      // half of the columns (never stored), which reads as zeros
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
        c.af[s2] = rec_load<f16x8, FUSED>(rec, rec_half_present(rows, s2) && (s2 == 0 || i >= 2) ? nb : 0,
                                          R::A + ((size_t)(i * 2 + s2) * 64 + l) * 16);
    }
    if (PART == 2 || PART == 3) {
      const int nh = rows > 0 ? (int)R::BYTES : 0;
#pragma unroll
      for (int nt = 0; nt < TR::NT; ++nt)
        c.uf[nt] = rec_load<f16x4, FUSED>(rec, nb, R::U + ((size_t)(i * R::NTV + slice * TR::NT + nt) * 64 + l) * 8);
      c.ue = rec_load<int32_t, FUSED>(rec, nh, R::HDR + 4);
      if (FUSED) c.vmax = rec_load<float, true>(rec, nh, R::HDR);
    }
  }
}

template <int PART, int DK, int DV, bool FUSED = false>
__device__ __forceinline__ void load_key(KeyRegs<DK>& c, const uint8_t* rec, int rows, int m, int l) {
  using R = Rec<DK, DV>;
  using KR = KeyRegs<DK>;
  const int gq = l >> 4;
  const int nh = rows > 0 ? (int)R::BYTES : 0;
  if (FUSED && PART == 0) c.vmax = rec_load<float, true>(rec, nh, R::HDR);
#pragma unroll
  for (int p = 0; p < KR::TPK; ++p) {
    const int ct = KR::TPK * m + p;
    if (PART == 0) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
        c.kt[p][s2] = rec_load<f16x8, FUSED>(rec, rec_half_present(rows, s2) ? (int)R::BYTES : 0,
                                             R::KT + ((size_t)(ct * 2 + s2) * 64 + l) * 16);
    } else {
      const uint2_v le = rec_load<uint2_v, FUSED>(rec, nh, R::LAM + (size_t)(16 * ct + 4 * gq + (l & 3)) * 8);
      c.lam[p] = __uint_as_float(le[0]);
      c.ec[p] = (int)le[1];
    }
  }
}

// Exponent es of the fp16 state and Delta copies for a bound B^2 = b2 on the state's
// column norms (2^es B <= 2^14).
__device__ inline int copy_exponent(double b2) {
  int es = 0;
  if (b2 > 0.0 && b2 < 1e300) es = 14 - (ilogb(sqrt(b2)) + 1);
  return es < -250 ? -250 : (es > 250 ? 250 : es);
}

// One scan workgroup's walk of the chain (sequence n, head h, value slice `slice`), with a
// ring of DEPTH chunks of factors in registers.  FUSED: the chunk records are produced while
// the chain walks them (the fused forward kernel): each chunk's ready flag is awaited
// before its factors are loaded, and the copy exponent follows the running bound over the
// chunks walked so far instead of the whole sequence's.  `mark` (one workgroup per launch)
// records the launch in the workspace's control word.
template <int DK, int DV, int NV, typename OutT, bool FUSED, int DEPTH = scan_depth<NV>()>
__device__ __forceinline__ void scan_walk(const ScanArgs& a, const FuseArgs& fz, const int64_t n, const int h,
                                          const int slice, const bool mark, uint8_t* smem) {
  using R = Rec<DK, DV>;
  using SM = ScanSmem<DK, DV, NV>;
  using TR = TokRegs<DK, NV>;
  using KR = KeyRegs<DK>;
  constexpr int KSK = DK / 32;
  constexpr int TPK = DK / 64;
  constexpr int NT = NV / 16;
  constexpr int kScanDepth = DEPTH;
  static_assert(!FUSED || kScanDepth == 2, "the fused walk reads the next chunk's header from the ring");

  uint8_t* sbb = smem + SM::SB;
  uint8_t* db = smem + SM::DB;
  float* cn = reinterpret_cast<float*>(smem + SM::CN);
  float* red = reinterpret_cast<float*>(smem + SM::RED);
  volatile int* tok_failed = reinterpret_cast<volatile int*>(smem + SM::FAIL);

  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l = tid & 63, t = l & 15, gq = l >> 4;
  const bool tok_wave = wv < 4;
  const int i = wv & 3;  // token block (tok_wave) or key block (otherwise)
  int64_t c0 = a.cu ? (int64_t)a.seq_off[n] : n * a.nc;
  int64_t c1 = a.cu ? (int64_t)a.seq_off[n + 1] : (n + 1) * a.nc;
  if (c1 > a.n_chunk_ub) c1 = a.n_chunk_ub;  // only on invalid cu_seqlens
  if (c0 > c1) c0 = c1;
  const int64_t L = seq_len(a.cu, a.T, n);
  const int64_t s0 = seq_start(a.cu, a.T, n);
  const int col0 = slice * NV;
  const size_t sbase = ((size_t)n * a.H + h) * DK * DV;

  // fp32 state rows of a key wave (C layout: lane holds rows 16 ct + 4 gq + r of
  // column col0 + 16 nt + t, ct = TPK * i + p)
  float S[TPK][NT][4];
#pragma unroll
  for (int p = 0; p < TPK; ++p)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * (TPK * i + p) + 4 * gq + r;
        S[p][nt][r] = (!tok_wave && a.h0) ? a.h0[sbase + (size_t)row * DV + col0 + 16 * nt + t] : 0.f;
      }

  // power-of-two scale of the fp16 copies from the bound B (see the file comment)
  float vm = 0.f;
  if (!FUSED) {
    for (int64_t c = c0 + tid; c < c1; c += kScanThreads)
      vm = fmaxf(vm, reinterpret_cast<const float*>(a.rec + ((size_t)c * a.H + h) * R::BYTES + R::HDR)[0]);
  }
  vm = wave_max(vm);
  if (l == 0) red[wv] = vm;
  if (tid == 0) {
    *tok_failed = 0;
    // the most recent launch on this workspace (kda_fwd_status): this launch's flag value,
    // or 0 for the two-kernel path (which has no waits)
    if (FUSED) __hip_atomic_store(fz.ctl, fz.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else if (a.ctl && mark) __hip_atomic_store(a.ctl, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (!tok_wave) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float ss = 0.f;
#pragma unroll
      for (int p = 0; p < TPK; ++p)
#pragma unroll
        for (int r = 0; r < 4; ++r) ss = fmaf(S[p][nt][r], S[p][nt][r], ss);
      ss = rows4_sum(ss);
      if (gq == 0) cn[i * NV + 16 * nt + t] = ss;
    }
  }
  __syncthreads();
  // the largest column norm: one column per lane (the same sums as a loop over columns)
  const int jc = l < NV ? l : 0;
  const float cmax = wave_max(l < NV ? cn[jc] + cn[NV + jc] + cn[2 * NV + jc] + cn[3 * NV + jc] : 0.f);
  float vmax = red[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) vmax = fmaxf(vmax, red[j]);
  int es = copy_exponent((double)cmax + (double)L * (double)vmax * (double)vmax);
  // fused: running maximum of max|v| over the chunks walked so far, and the bound at the
  // end of chunk c (the state's column norms after t tokens are at most cmax + t vmax^2)
  float vrun = 0.f;
  auto es_at = [&](int64_t c, float vmax_c) {
    vrun = fmaxf(vrun, vmax_c);
    const int64_t toks = (c - c0 + 1) * kChunk < L ? (c - c0 + 1) * kChunk : L;
    return copy_exponent((double)cmax + (double)toks * (double)vrun * (double)vrun);
  };
  // fused: wait until chunk c's record is complete.  The wait is bounded: a flag that
  // never comes ends it, marks the launch as failed in the workspace's error word, and this
  // wave waits for no later chunk.  A key wave's state rows become NaN at that point (so do
  // all later outputs, which read the state); a token wave's failure is noted in LDS and
  // turns the final state NaN at the end.  The flag is read one step ahead (`pre`), so a
  // record that is already published costs no round trip.
  uint64_t pre = 0;
  bool failed = false;  // wave-uniform: a wait of this wave gave up
  // the flag of chunk c for this slice (the chunk walk writes one per slice)
  constexpr int NSF = DV / NV;
  auto flag_of = [&](int64_t c) { return fz.flags + ((size_t)c * a.H + h) * NSF + slice; };
  // The look-ahead poll is issued every step (past the walk's end it reads the last chunk's
  // flag, which is not used) at an address offset by a zero the compiler cannot see through:
  // its value then stays in a vector register until the next step reads it, instead of being
  // moved to a scalar register right after the load, which waited for every load of the wave
  // still in flight (the ring's prefetch of the next chunk) at each step.
  int vzero;
  asm volatile("v_mov_b32 %0, 0" : "=v"(vzero));
  auto prepoll = [&](int64_t c) {
    if (FUSED) {
      const int64_t cc = c < c1 ? c : c1 - 1;
      pre = __hip_atomic_load(flag_of(cc) + vzero, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  auto await_chunk = [&](int64_t c) {
    if (FUSED && c < c1) {
      const uint64_t* fl = flag_of(c);
      const uint64_t pu = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(pre >> 32)) << 32) |
                          (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)pre);
      if (pu != fz.epoch && !failed) {
        int spins = 0;
        while (__hip_atomic_load(fl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != fz.epoch && spins < fz.spin_limit) {
          __builtin_amdgcn_s_sleep(2);
          ++spins;
        }
        if (__any(spins >= fz.spin_limit)) {
          failed = true;
          if (l == 0) {
            __hip_atomic_store(fz.ctl + 1, fz.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (tok_wave) *tok_failed = 1;
          }
          // a key wave's state rows become NaN here and stay NaN (they only enter products)
#pragma unroll
          for (int p = 0; p < TPK; ++p)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
              for (int r = 0; r < 4; ++r) S[p][nt][r] = __builtin_nanf("");
        }
      }
      pre = 0;
      asm volatile("" ::: "memory");  // the record's loads stay after the wait
    }
  };

  // fp16 S0 fragments of k-step s, column tile nt: slot half (ct & 1) of [(ct / 2) * NT + nt]
  auto write_state = [&](int buf) {
    uint8_t* sb = sbb + (size_t)buf * SM::SBUF;
#pragma unroll
    for (int p = 0; p < TPK; ++p) {
      const int ct = TPK * i + p;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f16x4 f;
#pragma unroll
        for (int r = 0; r < 4; ++r) f[r] = (_Float16)ldexpf(S[p][nt][r], es);
        *reinterpret_cast<f16x4*>(sb + (((size_t)(ct >> 1) * NT + nt) * 64 + l) * 16 + (ct & 1) * 8) = f;
      }
    }
  };
  if (!FUSED) {
    if (!tok_wave) write_state(0);
    __syncthreads();  // S0 of the first chunk visible
  }

  OutT* out = reinterpret_cast<OutT*>(a.out);
  const float oscale = a.scale;
  auto rec_of = [&](int64_t c) {
    const int64_t cc = c < c1 ? c : c1 - 1;  // past the end: the last chunk again (loaded, never used)
    return a.rec + ((size_t)cc * a.H + h) * R::BYTES;
  };
  // valid tokens of chunk c (only a sequence's last chunk has fewer than 64); 0 past the end
  auto rows_of = [&](int64_t c) {
    const int64_t rem = L - (c - c0) * kChunk;
    return c >= c1 ? 0 : (rem < kChunk ? (int)rem : kChunk);
  };

  if (tok_wave) {
    // ---- token block i: Delta rows, then the output rows ----
    auto step = [&](const TR& cur, TR& nxt, const uint8_t* nrec, int nrows, int64_t c) {
      if (FUSED) {
        es = es_at(c, cur.vmax);
        await_chunk(c + kScanDepth - 1);
        prepoll(c + kScanDepth);
      }
      load_tok<0, DK, DV, NV, FUSED>(nxt, nrec, nrows, i, l, slice);
      const f16x8* sb = reinterpret_cast<const f16x8*>(sbb + (size_t)((c - c0) & 1) * SM::SBUF);
      // all S0 fragments at once, so that the MFMA chains below never wait on LDS one by one
      f16x8 sf[KSK][NT];
#pragma unroll
      for (int s = 0; s < KSK; ++s)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) sf[s][nt] = sb[(s * NT + nt) * 64 + l];
      // Delta = U 2^(es - ue) - W S0 (rows 16 i.., C layout: lane column = value column)
      f32x4 d[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) d[nt] = zero4();
#pragma unroll
      for (int s = 0; s < KSK; ++s)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) d[nt] = mfma16(cur.wf[s], sf[s][nt], d[nt]);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f16x4 df;
#pragma unroll
        for (int r = 0; r < 4; ++r) df[r] = (_Float16)(ldexpf((float)cur.uf[nt][r], es - cur.ue) - d[nt][r]);
        *reinterpret_cast<f16x4*>(db + (((size_t)(i >> 1) * NT + nt) * 64 + l) * 16 + (i & 1) * 8) = df;
      }
      load_tok<1, DK, DV, NV, FUSED>(nxt, nrec, nrows, i, l, slice);
      // o^T, inter-chunk part: S0^T (Qhat exp(G))^T
      f32x4 o[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) o[nt] = zero4();
#pragma unroll
      for (int s = 0; s < KSK; ++s)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) o[nt] = mfma16(sf[s][nt], cur.qf[s], o[nt]);
      __syncthreads();  // A: Delta complete
      load_tok<2, DK, DV, NV, FUSED>(nxt, nrec, nrows, i, l, slice);
      // o^T, intra-chunk part: Delta^T Aqk^T; then 4 consecutive value columns per lane
      f16x8 dfr[2][NT];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          dfr[s2][nt] = *reinterpret_cast<const f16x8*>(db + (((size_t)s2 * NT + nt) * 64 + l) * 16);
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) o[nt] = mfma16(dfr[s2][nt], cur.af[s2], o[nt]);
      const int64_t idx = c - c0;
      const int64_t rem = L - idx * kChunk;
      const int len = rem < kChunk ? (int)rem : kChunk;
      const int i_loc = 16 * i + t;
      const int64_t tok = s0 + idx * kChunk + i_loc;
      if (i_loc < len && tok >= 0 && tok < a.T_total) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          float v4[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v4[r] = ldexpf(o[nt][r], -es) * oscale;
          store4(out + ((size_t)tok * a.H + h) * DV + col0 + 16 * nt + 4 * gq, v4);
        }
      }
      __syncthreads();  // B: next S0 complete
    };
    // Ring of kScanDepth register buffers: the factors of chunk c + kScanDepth - 1 are
    // requested while chunk c is processed (the HBM latency spans several steps).
    if (FUSED && c0 >= c1) __syncthreads();  // the first-state barrier of the key waves
    if (c0 < c1) {
      TR buf[kScanDepth];
#pragma unroll
      for (int j = 0; j < kScanDepth - 1; ++j) {
        await_chunk(c0 + j);
        load_tok<0, DK, DV, NV, FUSED>(buf[j], rec_of(c0 + j), rows_of(c0 + j), i, l, slice);
        load_tok<1, DK, DV, NV, FUSED>(buf[j], rec_of(c0 + j), rows_of(c0 + j), i, l, slice);
        load_tok<2, DK, DV, NV, FUSED>(buf[j], rec_of(c0 + j), rows_of(c0 + j), i, l, slice);
      }
      if (FUSED) __syncthreads();  // S0 of the first chunk visible
      // whole groups of kScanDepth steps (no conditional step: the compiler's memory-counter
      // waits then stay exact across iterations), then the remaining steps
      int64_t c = c0;
      for (; c + kScanDepth <= c1; c += kScanDepth) {
#pragma unroll
        for (int j = 0; j < kScanDepth; ++j)
          step(buf[j], buf[(j + kScanDepth - 1) % kScanDepth], rec_of(c + j + kScanDepth - 1),
               rows_of(c + j + kScanDepth - 1), c + j);
      }
#pragma unroll
      for (int j = 0; j < kScanDepth - 1; ++j)
        if (c + j < c1)
          step(buf[j], buf[(j + kScanDepth - 1) % kScanDepth], rec_of(c + j + kScanDepth - 1),
               rows_of(c + j + kScanDepth - 1), c + j);
    }
  } else {
    // ---- key block i: S_next = Diag(exp(G_last)) S0 + K~^T Delta ----
    auto step = [&](const KR& cur, KR& nxt, const uint8_t* nrec, int nrows, int64_t c) {
      if (FUSED) {
        await_chunk(c + kScanDepth - 1);
        prepoll(c + kScanDepth);
      }
      load_key<0, DK, DV, FUSED>(nxt, nrec, nrows, i, l);
      __syncthreads();  // A: Delta complete
      f16x8 dfr[2][NT];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          dfr[s2][nt] = *reinterpret_cast<const f16x8*>(db + (((size_t)s2 * NT + nt) * 64 + l) * 16);
#pragma unroll
      for (int p = 0; p < TPK; ++p) {
        const float lam[4] = {row_bcast<0>(cur.lam[p]), row_bcast<1>(cur.lam[p]), row_bcast<2>(cur.lam[p]),
                              row_bcast<3>(cur.lam[p])};  // rows 16 ct + 4 gq + r
        const float ecf = __int_as_float(cur.ec[p]);
        const int ue4[4] = {__float_as_int(row_bcast<0>(ecf)) - es, __float_as_int(row_bcast<1>(ecf)) - es,
                            __float_as_int(row_bcast<2>(ecf)) - es, __float_as_int(row_bcast<3>(ecf)) - es};
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          f32x4 u = zero4();
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) u = mfma16(cur.kt[p][s2], dfr[s2][nt], u);
#pragma unroll
          for (int r = 0; r < 4; ++r) S[p][nt][r] = fmaf(lam[r], S[p][nt][r], ldexpf(u[r], ue4[r]));
        }
      }

      load_key<1, DK, DV, FUSED>(nxt, nrec, nrows, i, l);
      // the next chunk's copy exponent (the same value its token waves derive)
      if (FUSED && c + 1 < c1) es = es_at(c + 1, nxt.vmax);
      write_state((int)((c - c0 + 1) & 1));
      __syncthreads();  // B: next S0 complete
    };
    if (FUSED && c0 >= c1) {
      write_state(0);
      __syncthreads();  // the first-state barrier
    }
    if (c0 < c1) {
      KR buf[kScanDepth];
#pragma unroll
      for (int j = 0; j < kScanDepth - 1; ++j) {
        await_chunk(c0 + j);
        load_key<0, DK, DV, FUSED>(buf[j], rec_of(c0 + j), rows_of(c0 + j), i, l);
        load_key<1, DK, DV, FUSED>(buf[j], rec_of(c0 + j), rows_of(c0 + j), i, l);
      }
      if (FUSED) {
        es = es_at(c0, buf[0].vmax);
        write_state(0);
        __syncthreads();  // S0 of the first chunk visible
      }
      int64_t c = c0;
      for (; c + kScanDepth <= c1; c += kScanDepth) {
#pragma unroll
        for (int j = 0; j < kScanDepth; ++j)
          step(buf[j], buf[(j + kScanDepth - 1) % kScanDepth], rec_of(c + j + kScanDepth - 1),
               rows_of(c + j + kScanDepth - 1), c + j);
      }
#pragma unroll
      for (int j = 0; j < kScanDepth - 1; ++j)
        if (c + j < c1)
          step(buf[j], buf[(j + kScanDepth - 1) % kScanDepth], rec_of(c + j + kScanDepth - 1),
               rows_of(c + j + kScanDepth - 1), c + j);
    }
    if (a.ht) {
      // (fused) a token wave's wait gave up: the final state is not valid (every wave is past
      // the last barrier B, so the note is visible)
      const bool poison = FUSED && *tok_failed != 0;
#pragma unroll
      for (int p = 0; p < TPK; ++p)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = 16 * (TPK * i + p) + 4 * gq + r;
            a.ht[sbase + (size_t)row * DV + col0 + 16 * nt + t] = poison ? __builtin_nanf("") : S[p][nt][r];
          }
    }
  }
}

// One scan workgroup: chain `bid` of `nblk` (one per (sequence, head, slice)).
template <int DK, int DV, int NV, typename OutT, bool FUSED>
__device__ __forceinline__ void scan_chain(const ScanArgs& a, const FuseArgs& fz, const int64_t bid,
                                           const int64_t nblk, uint8_t* smem) {
  constexpr int NS = DV / NV;
  // Workgroups are dispatched round-robin over the 8 XCDs (block id mod 8).  The NS
  // slices of one (sequence, head) share every chunk factor except U, so they are
  // mapped to block ids with equal residue mod 8: one XCD's L2 serves all of them.
  int64_t chain, slice_l;
  if (nblk % (8 * NS) == 0) {
    const int64_t xcd = bid & 7, k = bid >> 3;
    slice_l = k % NS;
    chain = (k / NS) * 8 + xcd;
  } else {
    slice_l = bid % NS;
    chain = bid / NS;
  }
  const int h = (int)(chain % a.H);
  const int64_t n = a.cu ? (int64_t)a.seq_order[chain / a.H] : chain / a.H;
  scan_walk<DK, DV, NV, OutT, FUSED>(a, fz, n, h, (int)slice_l, bid == 0, smem);
}

template <int DK, int DV, int NV, typename OutT>
__global__ __launch_bounds__(kScanThreads) void state_scan_kernel(ScanArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  scan_chain<DK, DV, NV, OutT, false>(a, FuseArgs{}, blockIdx.x, gridDim.x, smem);
}

}  // namespace kda
