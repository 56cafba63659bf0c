// Persistent state scan for packed batches: the per-chunk step of state_scan_kernel
// (kda_scan.h), walked by one resident workgroup per compute unit that takes (sequence,
// head, value slice) tasks from a queue.
//
// Why: in a batch of many short sequences a one-shot workgroup per chain spends most of
// its life waiting: for its initial state rows, for the maxima of its chunk headers, for
// its first chunk's factors, and only then steps once or twice; and each of the value
// slices of a (sequence, head) pays that again.
//
// Two classes of sequences ("Autoresearch on Kimi Delta Attention", section "The
// optimization trace": the recurrence split across value tiles to expose more independent
// work):
//  * long (at least `long_chunks` chunks; the first ones of the longest-first order): one
//    task at a time, walked by scan_walk from a cold start, on NVW-column slices; when
//    those chains would leave compute units idle, on the narrower NVL-column slices: a
//    step of a narrow slice is shorter, so the longest chain, which bounds the launch,
//    ends sooner.
//  * short (fewer chunks): one task per (sequence, head), all value columns, walked in
//    64-column halves inside each step (so the registers stay those of a 64-column slice
//    while the per-task costs and the chunk factors the halves share are paid once);
//    pipelined: the next task's initial state, header maxima and first chunk are requested
//    while the current one walks, so those latencies run under its steps.  The factors
//    ring is one chunk deep (each step requests the next chunk into the slot it walks,
//    each part after its last use): that leaves the registers for the next task's state.
//    Task ids are taken two ahead (only short tasks are ever held that way, so no task
//    waits behind a long one).
//
// Queues: one counter per XCD (block id mod 8 is the XCD a workgroup runs on); the
// (sequence, head) pairs are dealt to the queues round-robin, and all slices of a pair sit
// in one queue, so one XCD's L2 serves the chunk factors the slices share.  A queue hands
// out its long tasks first, then its short ones.
#pragma once

#include "kda_scan.h"

namespace kda {
template <int V>
struct IntC {
  static constexpr int value = V;
};

constexpr int kQueueSlots = 8;
typedef int32_t int4_v __attribute__((ext_vector_type(4)));  // task counters in the workspace info block (one per XCD)

struct TaskArgs {
  int32_t* queue;          // kQueueSlots counters, zeroed by the chunk map before the launch
  const int32_t* n_long;   // sequences of at least long_chunks chunks (the first ones of seq_order)
  const int4* rank_desc;   // per rank of seq_order: {sequence, first chunk, first token, length}
  int32_t long_width;      // value columns of a long task: NVL, NVW, or 0 (chosen here)
};

// Task u of queue x among the (sequence, head) pairs [p_lo, p_hi) with p = x (mod nq),
// `slices` tasks per pair: its pair and slice, or false past the queue's end.
// (32-bit: the host bounds (sequences x heads x 8) below 2^31.)  nq is 1 or 8, slices a
// power of two.
__device__ __forceinline__ bool queue_task(int u, int slices, int x, int nq, int p_lo, int p_hi, int& p,
                                           int& slice) {
  if (u < 0) return false;
  const int first = p_lo + ((x - p_lo) & (nq - 1));
  const int cnt = p_hi > first ? (p_hi - first + nq - 1) / nq : 0;
  if (u >= cnt * slices) return false;
  p = first + nq * (u / slices);
  slice = u & (slices - 1);
  return true;
}

// Queue request whose result is waited for only where it is read.  A fetch-add at an address
// the compiler can prove uniform is rewritten into one wave-wide atomic whose result is
// broadcast at once, which would hold the wave for the round trip right there; the
// address is therefore offset by a register value the compiler cannot see through (0).
__device__ __forceinline__ int queue_request(int32_t* ctr) {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return __hip_atomic_fetch_add(ctr + z, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct ScanTask {
  bool ok;  // a task of the class being walked
  int h, slice, rank;
  int64_t n, c0, c1, L, s0;
};

// Shared by both classes: queue geometry and the id hand-off.
struct QueueCtx {
  int32_t* ctr;        // this workgroup's queue counter
  int x, nq;           // queue index and number of queues
  int long_pairs;      // pairs of the long class (p < long_pairs)
  int pairs;           // all pairs
  int long_tasks;      // long tasks of this queue (its ids below this are long tasks)
  int long_slices;     // value slices per long pair (DV / NVL or DV / NVW)
  int32_t* qs;         // LDS slots: [0] the published id, [1] a workgroup-wide id, [4..7] a descriptor
};

// The queue position (class check, pair, slice) of id u; `NS_` slices per pair.
__device__ __forceinline__ ScanTask task_ids(const ScanArgs& a, const QueueCtx& q, int u, bool is_long, int ns) {
  ScanTask k;
  int p = 0, sl = 0;
  k.ok = is_long ? queue_task(u, ns, q.x, q.nq, 0, q.long_pairs, p, sl)
                 : queue_task(u - q.long_tasks, ns, q.x, q.nq, q.long_pairs, q.pairs, p, sl);
  const int hh = (int)a.H;
  k.rank = p / hh;
  k.h = p - k.rank * hh;
  k.slice = sl;
  k.n = k.c0 = k.c1 = k.L = k.s0 = 0;
  return k;
}

// The sequence fields of task k from its rank descriptor d (wave-uniform values).
__device__ __forceinline__ void task_fields(const ScanArgs& a, ScanTask& k, const int4_v d) {
  if (!k.ok) return;
  k.n = __builtin_amdgcn_readfirstlane(d[0]);
  int64_t c0 = __builtin_amdgcn_readfirstlane(d[1]);
  k.s0 = __builtin_amdgcn_readfirstlane(d[2]);
  k.L = __builtin_amdgcn_readfirstlane(d[3]);
  int64_t cnt = (k.L + kChunk - 1) / kChunk;
  if (cnt > a.n_chunk_ub) cnt = a.n_chunk_ub;
  int64_t c1 = c0 + cnt;
  if (c1 > a.n_chunk_ub) c1 = a.n_chunk_ub;  // only on invalid cu_seqlens
  if (c0 > c1) c0 = c1;
  k.c0 = c0;
  k.c1 = c1;
}

// Walk the short tasks (all DV columns of a (sequence, head), in 64-column halves) from id
// `u_cur` on until the queue runs dry.  `pending` (lane 0 of wave 0) holds the request for
// the id after u_cur.
template <int DK, int DV, typename OutT>
__device__ __forceinline__ void scan_short_tasks(const ScanArgs& a, const QueueCtx& q, const int4* rank_desc,
                                                 int u_cur, int pending, uint8_t* smem) {
  constexpr int NV = DV;
  using R = Rec<DK, DV>;
  using SM = ScanSmem<DK, DV, NV>;
  using TR = TokRegs<DK, NV>;
  using KR = KeyRegs<DK>;
  constexpr int KSK = DK / 32;
  constexpr int TPK = DK / 64;
  constexpr int NT = NV / 16;   // 16-column tiles of the task
  constexpr int NH = NV / 64;   // 64-column halves
  constexpr int NS = 1;         // one task per (sequence, head)
  constexpr size_t STAGE = (SM::BYTES + 15) & ~(size_t)15;  // the key waves' state stage

  uint8_t* sbb = smem + SM::SB;
  uint8_t* db = smem + SM::DB;
  float* cn = reinterpret_cast<float*>(smem + SM::CN);
  float* red = reinterpret_cast<float*>(smem + SM::RED);

  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l = tid & 63, t = l & 15, gq = l >> 4;
  const bool tok_wave = wv < 4;
  const int i = wv & 3;  // token block (tok_wave) or key block (otherwise)

  ScanTask cur = task_ids(a, q, u_cur, false, NS);
  if (!cur.ok) return;
  task_fields(a, cur, reinterpret_cast<const int4_v*>(rank_desc)[cur.rank]);

  auto hdr_of = [&](int64_t c, int h) __attribute__((always_inline)) {
    return reinterpret_cast<const float*>(a.rec + ((size_t)c * a.H + h) * R::BYTES + R::HDR);
  };
  // record of virtual chunk v of the stream "this task's chunks, then the next task's"
  auto vrec = [&](int64_t v, const ScanTask& k, const ScanTask& nx, bool nx_ok, int& sl, int& rows)
                  __attribute__((always_inline)) {
    int64_t c, rem;
    int hh;
    const int64_t nk = k.c1 - k.c0;
    if (v < nk) {
      c = k.c0 + v; rem = k.L - v * kChunk; hh = k.h; sl = k.slice;
    } else if (nx_ok) {
      const int64_t w = v - nk, nn = nx.c1 - nx.c0, j = w < nn ? w : nn - 1;
      c = nx.c0 + j; rem = nx.L - j * kChunk; hh = nx.h; sl = nx.slice;
    } else {
      c = k.c1 - 1; rem = 0; hh = k.h; sl = k.slice;  // past the end: nothing is fetched
    }
    if (c < 0) c = 0;
    rows = rem <= 0 ? 0 : (rem < kChunk ? (int)rem : kChunk);
    return a.rec + ((size_t)c * a.H + hh) * R::BYTES;
  };

  OutT* out = reinterpret_cast<OutT*>(a.out);
  const float oscale = a.scale;

  // The two roles run their own task loops (their ring registers are then never live at
  // the same time) with the same sequence of barriers: 0 (norms, maxima and the published
  // id visible), 1 (S0 of the first chunk visible), then A and B of every step.
  //
  // Ids and descriptors: lane 0 of wave 0 holds the id after the next one (`pending`, its
  // request made at the previous boundary) and, once the request has returned (in the
  // first step of a task), that task's rank descriptor; at a boundary it publishes both in
  // LDS, so every wave decodes the next task from LDS alone (no vector-memory wait in the
  // boundary, where the counter would hold it behind the previous task's stores).
  int4_v pend_desc = {0, 0, 0, 0};
  auto fetch_desc = [&](int u) __attribute__((always_inline)) {
    const ScanTask k = task_ids(a, q, u, false, NS);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int4*>(rank_desc + (k.ok ? k.rank : 0)), 0, 16, kBufferFlags);
    return __builtin_bit_cast(int4_v, __builtin_amdgcn_raw_buffer_load_b128(rs, 0, 0, 0));
  };
  if (tid == 0) pend_desc = fetch_desc(pending);
  int4_v* qdesc = reinterpret_cast<int4_v*>(q.qs + 4);

  // After barrier 0, in both roles: the copy exponent from the LDS partials, then the next
  // task from the published id and descriptor.
  auto after_barrier0 = [&](const ScanTask& k, ScanTask& nx, int& es_out) __attribute__((always_inline)) {
    // the largest column norm: columns l and l + 64 per lane (the same sums as a loop over
    // columns)
    float cm = 0.f;
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      const int j = 64 * hh + l;
      cm = fmaxf(cm, cn[j] + cn[NV + j] + cn[2 * NV + j] + cn[3 * NV + j]);
    }
    const float cmax = wave_max(cm);
    float vmax = red[0];
#pragma unroll
    for (int jj = 1; jj < 8; ++jj) vmax = fmaxf(vmax, red[jj]);
    es_out = copy_exponent((double)cmax + (double)k.L * (double)vmax * (double)vmax);
    const int u_nxt = __builtin_amdgcn_readfirstlane(*q.qs);
    const int4_v nd = *qdesc;
    if (tid == 0) pending = queue_request(q.ctr);
    nx = task_ids(a, q, u_nxt, false, NS);
    task_fields(a, nx, nd);
  };
  // boundary start: publish the next task (lane 0 of wave 0)
  auto publish = [&]() __attribute__((always_inline)) {
    if (tid == 0) {
      *q.qs = pending;
      *qdesc = pend_desc;
    }
  };

  bool have_pre = false;  // the current task's initial state / header maxima were prefetched
  bool ring_ok = false;   // the ring slot holds the current task's first chunk

  if (tok_wave) {
    // ---- token block i: Delta rows, then the output rows ----
    TR tb[1];
    float hv = 0.f;  // header maxima max|v| of up to 256 chunks of a task (one per lane)
    auto load_hdr = [&](const ScanTask& k) __attribute__((always_inline)) {
      int64_t c = k.c0 + 64 * i + l;
      if (c >= k.c1) c = k.c1 > k.c0 ? k.c1 - 1 : 0;  // loaded, masked at the boundary
      hv = *hdr_of(c, k.h);
    };
    for (;;) {
      publish();
      if (!have_pre) load_hdr(cur);
      float vm = (cur.c0 + 64 * i + l < cur.c1) ? hv : 0.f;
      for (int64_t c = cur.c0 + 256 + tid; c < cur.c1; c += 256) vm = fmaxf(vm, *hdr_of(c, cur.h));
      vm = wave_max(vm);
      if (l == 0) red[wv] = vm;
      __syncthreads();  // 0
      int es;
      ScanTask nxt;
      after_barrier0(cur, nxt, es);
      const int64_t nk = cur.c1 - cur.c0;
      if (!ring_ok && nk > 0) {
        int sl, nr;
        const uint8_t* r0 = vrec(0, cur, nxt, false, sl, nr);
        load_tok<0, DK, DV, NV>(tb[0], r0, nr, i, l, sl);
        load_tok<1, DK, DV, NV>(tb[0], r0, nr, i, l, sl);
        load_tok<2, DK, DV, NV>(tb[0], r0, nr, i, l, sl);
      }
      __syncthreads();  // 1
      const bool nx_pre = nxt.ok && nxt.c1 > nxt.c0;  // the ring may run on into the next task
      if (nxt.ok) load_hdr(nxt);  // under this task's steps

      // Delta for both halves before barrier A (the key waves wait for it); the output rows
      // after it, half by half (S0 stays in its buffer until the step after)
      auto step = [&](const TR& c_, TR& n_, const uint8_t* nrec, int nsl, int nr, int64_t k, auto same, auto first)
                      __attribute__((always_inline)) {
        constexpr bool SAME = decltype(same)::value != 0;
        if (!SAME) load_tok<0, DK, DV, NV>(n_, nrec, nr, i, l, nsl);
        const f16x8* sb = reinterpret_cast<const f16x8*>(sbb + (size_t)(k & 1) * SM::SBUF);
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
          f16x8 sf[KSK][4];
#pragma unroll
          for (int s = 0; s < KSK; ++s)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) sf[s][nt] = sb[(s * NT + 4 * hh + nt) * 64 + l];
          f32x4 d[4];
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) d[nt] = zero4();
#pragma unroll
          for (int s = 0; s < KSK; ++s)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) d[nt] = mfma16(c_.wf[s], sf[s][nt], d[nt]);
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) {
            f16x4 df;
#pragma unroll
            for (int r = 0; r < 4; ++r)
              df[r] = (_Float16)(ldexpf((float)c_.uf[4 * hh + nt][r], es - c_.ue) - d[nt][r]);
            *reinterpret_cast<f16x4*>(db + (((size_t)(i >> 1) * NT + 4 * hh + nt) * 64 + l) * 16 + (i & 1) * 8) = df;
          }
        }
        // the descriptor of the id held in reserve (its request has returned by now)
        if (decltype(first)::value && tid == 0) pend_desc = fetch_desc(pending);
        if (SAME) {
          load_tok<0, DK, DV, NV>(n_, nrec, nr, i, l, nsl);  // W, U and ue are spent
          load_tok<3, DK, DV, NV>(n_, nrec, nr, i, l, nsl);
        } else {
          load_tok<1, DK, DV, NV>(n_, nrec, nr, i, l, nsl);
        }
        __syncthreads();  // A: Delta complete
        if (!SAME) load_tok<2, DK, DV, NV>(n_, nrec, nr, i, l, nsl);
        const int64_t rem = cur.L - k * kChunk;
        const int len = rem < kChunk ? (int)rem : kChunk;
        const int i_loc = 16 * i + t;
        const int64_t tok = cur.s0 + k * kChunk + i_loc;
        const bool row_ok = i_loc < len && tok >= 0 && tok < a.T_total;
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
          // o^T = S0^T (Qhat exp(G))^T + Delta^T Aqk^T, columns of half hh
          f16x8 sf[KSK][4];
#pragma unroll
          for (int s = 0; s < KSK; ++s)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) sf[s][nt] = sb[(s * NT + 4 * hh + nt) * 64 + l];
          f32x4 o[4];
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) o[nt] = zero4();
#pragma unroll
          for (int s = 0; s < KSK; ++s)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) o[nt] = mfma16(sf[s][nt], c_.qf[s], o[nt]);
          f16x8 dfr[2][4];
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
              dfr[s2][nt] = *reinterpret_cast<const f16x8*>(db + (((size_t)s2 * NT + 4 * hh + nt) * 64 + l) * 16);
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) o[nt] = mfma16(dfr[s2][nt], c_.af[s2], o[nt]);
          if (row_ok) {
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
              float v4[4];
#pragma unroll
              for (int r = 0; r < 4; ++r) v4[r] = ldexpf(o[nt][r], -es) * oscale;
              store4_nt(out + ((size_t)tok * a.H + cur.h) * DV + 64 * hh + 16 * nt + 4 * gq, v4);
            }
          }
        }
        if (SAME) {
          load_tok<1, DK, DV, NV>(n_, nrec, nr, i, l, nsl);
          load_tok<4, DK, DV, NV>(n_, nrec, nr, i, l, nsl);
        }
        __syncthreads();  // B: next S0 complete
      };
      // one slot: each step requests the next chunk (the next task's first after the last
      // step) into the slot it walks, each part after its last use
      // the first step on its own: a loop's memory-counter waits are set for its later
      // iterations and would make this one wait for the prefetches issued just before it
      auto walk_step = [&](int64_t k, auto first) __attribute__((always_inline)) {
        int sl, nr;
        const uint8_t* n1 = vrec(k + 1, cur, nxt, nx_pre, sl, nr);
        step(tb[0], tb[0], n1, sl, nr, k, IntC<1>{}, first);
      };
      if (nk > 0) walk_step(0, IntC<1>{});
      else if (tid == 0) pend_desc = fetch_desc(pending);
      for (int64_t k = 1; k < nk; ++k) walk_step(k, IntC<0>{});
      // the next task's first chunk sits in slot 0 when this task walked at least one step
      // and the next one has a chunk
      ring_ok = nk > 0 && nx_pre;
      have_pre = nxt.ok;
      if (!nxt.ok) return;
      cur = nxt;
    }
  } else {
    // ---- key block i: S_next = Diag(exp(G_last)) S0 + K~^T Delta ----
    KR kb[1];
    float S[TPK][NT][4];   // fp32 state rows (C layout, as in scan_walk)
    // The wave's RW state rows move between memory and S as 16-byte row pieces (piece
    // f = 64 j + l: row f / (DV / 4), columns 4 (f % (DV / 4)) ..): 16 loads or stores per
    // lane instead of 64 single words, which would fill the memory counter.  The C layout
    // is taken from and given to this wave's own rows of a padded LDS stage (row pitch
    // DV + 4 words: the 16 rows of a read or write fall in distinct banks); a wave's LDS
    // operations complete in order, so no barrier is involved.
    constexpr int RW = DK / 4;
    constexpr int SP = DV + 4;
    constexpr int PCS = RW * DV / 256;
    float4 Sv[PCS];  // the next task's initial rows, in flight
    constexpr int LPR = DV / 4;   // lanes per row of pieces
    constexpr int RPJ = 64 / LPR;  // rows per piece index j
    // piece j of lane l: memory offset 256 j + 4 l words from the wave's first row; stage
    // offset RPJ SP j + (l / LPR) SP + 4 (l % LPR)
    float* stage = reinterpret_cast<float*>(smem + STAGE) + (size_t)i * RW * SP;
    float* stage_l = stage + (l / LPR) * SP + 4 * (l % LPR);
    auto load_state = [&](const ScanTask& k) __attribute__((always_inline)) {
      if (a.h0) {
        const float* src = a.h0 + ((size_t)k.n * a.H + k.h) * DK * DV + (size_t)RW * i * DV + 4 * l;
#pragma unroll
        for (int j = 0; j < PCS; ++j) {
          const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + 256 * j));
          Sv[j] = make_float4(v[0], v[1], v[2], v[3]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < PCS; ++j) Sv[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    };
    auto unpack_state = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < PCS; ++j) *reinterpret_cast<float4*>(stage_l + RPJ * SP * j) = Sv[j];
#pragma unroll
      for (int p = 0; p < TPK; ++p)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r) S[p][nt][r] = stage[(16 * p + 4 * gq + r) * SP + 16 * nt + t];
    };
    auto store_state = [&](const ScanTask& k) __attribute__((always_inline)) {
#pragma unroll
      for (int p = 0; p < TPK; ++p)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r) stage[(16 * p + 4 * gq + r) * SP + 16 * nt + t] = S[p][nt][r];
      float* dst = a.ht + ((size_t)k.n * a.H + k.h) * DK * DV + (size_t)RW * i * DV + 4 * l;
#pragma unroll
      for (int j = 0; j < PCS; ++j)
        __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(stage_l + RPJ * SP * j),
                                    reinterpret_cast<f32x4*>(dst + 256 * j));
    };
    for (;;) {
      if (!have_pre) load_state(cur);
      unpack_state();
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
      if (l == 0) red[wv] = 0.f;
      __syncthreads();  // 0
      int es;
      ScanTask nxt;
      after_barrier0(cur, nxt, es);
      const int64_t nk = cur.c1 - cur.c0;
      if (!ring_ok && nk > 0) {
        int sl, nr;
        const uint8_t* r0 = vrec(0, cur, nxt, false, sl, nr);
        load_key<0, DK, DV>(kb[0], r0, nr, i, l);
        load_key<1, DK, DV>(kb[0], r0, nr, i, l);
      }
      auto write_state = [&](int buf) __attribute__((always_inline)) {
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
      write_state(0);
      __syncthreads();  // 1
      const bool nx_pre = nxt.ok && nxt.c1 > nxt.c0;
      if (nxt.ok) load_state(nxt);  // under this task's steps

      auto step = [&](const KR& c_, KR& n_, const uint8_t* nrec, int nr, int64_t k, auto same)
                      __attribute__((always_inline)) {
        constexpr bool SAME = decltype(same)::value != 0;
        if (!SAME) load_key<0, DK, DV>(n_, nrec, nr, i, l);
        __syncthreads();  // A: Delta complete

        float lam[TPK][4];
        int ue4[TPK][4];
#pragma unroll
        for (int p = 0; p < TPK; ++p) {
          lam[p][0] = row_bcast<0>(c_.lam[p]); lam[p][1] = row_bcast<1>(c_.lam[p]);
          lam[p][2] = row_bcast<2>(c_.lam[p]); lam[p][3] = row_bcast<3>(c_.lam[p]);
          const float ecf = __int_as_float(c_.ec[p]);
          ue4[p][0] = __float_as_int(row_bcast<0>(ecf)) - es; ue4[p][1] = __float_as_int(row_bcast<1>(ecf)) - es;
          ue4[p][2] = __float_as_int(row_bcast<2>(ecf)) - es; ue4[p][3] = __float_as_int(row_bcast<3>(ecf)) - es;
        }
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
          f16x8 dfr[2][4];
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
              dfr[s2][nt] = *reinterpret_cast<const f16x8*>(db + (((size_t)s2 * NT + 4 * hh + nt) * 64 + l) * 16);
#pragma unroll
          for (int p = 0; p < TPK; ++p)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
              f32x4 u = zero4();
#pragma unroll
              for (int s2 = 0; s2 < 2; ++s2) u = mfma16(c_.kt[p][s2], dfr[s2][nt], u);
#pragma unroll
              for (int r = 0; r < 4; ++r)
                S[p][4 * hh + nt][r] = fmaf(lam[p][r], S[p][4 * hh + nt][r], ldexpf(u[r], ue4[p][r]));
            }
        }
        if (SAME) load_key<0, DK, DV>(n_, nrec, nr, i, l);
        load_key<1, DK, DV>(n_, nrec, nr, i, l);
        write_state((int)((k + 1) & 1));
        __syncthreads();  // B: next S0 complete
      };
      auto walk_step = [&](int64_t k) __attribute__((always_inline)) {
        int sl, nr;
        const uint8_t* n1 = vrec(k + 1, cur, nxt, nx_pre, sl, nr);
        step(kb[0], kb[0], n1, nr, k, IntC<1>{});
      };
      if (nk > 0) walk_step(0);  // on its own, as in the token role
      for (int64_t k = 1; k < nk; ++k) walk_step(k);
      if (a.ht) store_state(cur);
      ring_ok = nk > 0 && nx_pre;
      have_pre = nxt.ok;
      if (!nxt.ok) return;
      cur = nxt;
    }
  }
}

// Dynamic LDS of the kernel below: the largest of its three scan layouts (the short one with
// the key waves' state stage), then the id slots.
template <int DK, int DV, int NVL, int NVW>
constexpr size_t scan_tasks_smem() {
  constexpr size_t A = ScanSmem<DK, DV, NVL>::BYTES, B = ScanSmem<DK, DV, NVW>::BYTES;
  constexpr size_t C = ((ScanSmem<DK, DV, DV>::BYTES + 15) & ~(size_t)15) + (size_t)DK * (DV + 4) * 4;
  constexpr size_t M = A > B ? (A > C ? A : C) : (B > C ? B : C);
  return ((M + 15) & ~(size_t)15) + 32;
}

// One resident workgroup per compute unit (gridDim.x of them): long tasks one at a time,
// then short tasks pipelined, each from this workgroup's queue.
template <int DK, int DV, int NVL, int NVW, typename OutT>
__global__ __launch_bounds__(kScanThreads) void state_scan_tasks_kernel(ScanArgs a, TaskArgs ta) {
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr int DL = 2;  // ring depth of the narrow long walk (three deep spills)
  constexpr size_t SMB = scan_tasks_smem<DK, DV, NVL, NVW>() - 32;  // the id slots follow
  int32_t* qs = reinterpret_cast<int32_t*>(smem + ((SMB + 15) & ~(size_t)15));
  QueueCtx q;
  q.nq = gridDim.x >= kQueueSlots ? kQueueSlots : 1;
  q.x = (int)(blockIdx.x % q.nq);
  q.ctr = ta.queue + q.x;
  q.pairs = (int)(a.N * a.H);
  // narrow slices for the long class only when its chains on wide slices would leave
  // compute units without a task
  const int lp = *ta.n_long * (int)a.H;
  const bool narrow = ta.long_width ? ta.long_width == NVL : (int64_t)lp * (DV / NVW) < (int64_t)gridDim.x;
  q.long_pairs = lp;
  q.long_slices = narrow ? DV / NVL : DV / NVW;
  const int lcnt = lp > q.x ? (lp - q.x + q.nq - 1) / q.nq : 0;
  q.long_tasks = lcnt * q.long_slices;
  q.qs = qs;
  const int tid = threadIdx.x;

  // long tasks: one id at a time
  bool mark = blockIdx.x == 0;
  int u;
  for (;;) {
    if (tid == 0) qs[1] = __hip_atomic_fetch_add(q.ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    u = __builtin_amdgcn_readfirstlane(qs[1]);
    const ScanTask k = task_ids(a, q, u, true, q.long_slices);
    if (!k.ok) break;
    const int64_t n = a.seq_order[k.rank];
    if (narrow) scan_walk<DK, DV, NVL, OutT, false, DL>(a, FuseArgs{}, n, k.h, k.slice, mark, smem);
    else scan_walk<DK, DV, NVW, OutT, false>(a, FuseArgs{}, n, k.h, k.slice, mark, smem);
    mark = false;
  }
  if (mark && tid == 0 && a.ctl)
    __hip_atomic_store(a.ctl, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // no waits in this path
  // short tasks: `u` is the first one (or past the queue's end); request the one after it
  int pending = 0;
  if (tid == 0) pending = queue_request(q.ctr);
  scan_short_tasks<DK, DV, OutT>(a, q, ta.rank_desc, u, pending, smem);
}

}  // namespace kda
