// Device-side building blocks shared by the KDA forward kernels (gfx950).
//
// Fragment conventions (v_mfma_f32_16x16x32_f16, one wave of 64 lanes, lane l):
//   A operand (16 x 32):  lane l holds A[l % 16][8 * (l / 16) + 0..7]
//   B operand (32 x 16):  lane l holds B[8 * (l / 16) + 0..7][l % 16]
//   C/D       (16 x 16):  lane l holds C[4 * (l / 16) + 0..3][l % 16]
// A 32-wide contraction step is free to use any order of its 32 indices as
// long as both operands agree.  The kernels use the order pi below, under
// which the C fragments of two stacked 16-row tiles are, lane for lane and
// without any data movement, the operand fragment of the next contraction:
//   slot 8*gq + e  (gq = l/16, e = 0..7)  <->  index 16*(e/4) + 4*gq + (e%4)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 64;      // tokens per chunk
constexpr float kLog2e = 1.4426950408889634f;

// Index (within a 32-wide step) that slot e of lane-quarter gq stands for.
__device__ __host__ constexpr int pi_index(int gq, int e) { return 16 * (e >> 2) + 4 * gq + (e & 3); }

__device__ inline f32x4 mfma16(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ inline f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// 2^x on the hardware exp unit (x <= 126 everywhere it is used: finite results).
__device__ inline float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Shift a value D lanes up inside each row of 16 lanes; lanes with no source get 0.
template <int D>
__device__ inline float row_shr(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + D, 0xF, 0xF, true));
}

// Lane N of each row of 16 lanes, broadcast to the whole row (DPP row_newbcast).
// Every lane is written, so no old value is needed.
template <int N>
__device__ inline float row_bcast(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x150 + N, 0xF, 0xF, false));
}

// floor(log2(x)) of a finite x > 0, denormals included (v_frexp_exp_i32_f32; the library
// ilogbf goes through double precision).
__device__ inline int ilogb_pos(float x) { return __builtin_amdgcn_frexp_expf(x) - 1; }

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Two fp32 -> bf16 conversions in one instruction (v_cvt_pk_bf16_f32: round to nearest
// even under the default rounding mode; NaN stays NaN), low half = a.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Load four consecutive elements (bf16 or fp32) as fp32.
__device__ inline void load4(const uint16_t* p, float* o) {
  uint2 r = *reinterpret_cast<const uint2*>(p);
  o[0] = __uint_as_float(r.x << 16);
  o[1] = __uint_as_float(r.x & 0xffff0000u);
  o[2] = __uint_as_float(r.y << 16);
  o[3] = __uint_as_float(r.y & 0xffff0000u);
}
__device__ inline void load4(const float* p, float* o) {
  float4 r = *reinterpret_cast<const float4*>(p);
  o[0] = r.x; o[1] = r.y; o[2] = r.z; o[3] = r.w;
}
__device__ inline float load1(const uint16_t* p) { return bf16_to_f32(*p); }
__device__ inline float load1(const float* p) { return *p; }

// Store four consecutive elements from fp32 (bf16 rounds to nearest even).
__device__ inline void store4(uint16_t* p, const float* x) {
  uint2 r;
  r.x = pack_bf16x2(x[0], x[1]);
  r.y = pack_bf16x2(x[2], x[3]);
  *reinterpret_cast<uint2*>(p) = r;
}
__device__ inline void store4(float* p, const float* x) {
  *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
}
// The same, as streaming stores (outputs that no kernel of the call reads again)
__device__ inline void store4_nt(uint16_t* p, const float* x) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 r = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
  __builtin_nontemporal_store(r, reinterpret_cast<u32x2*>(p));
}
__device__ inline void store4_nt(float* p, const float* x) {
  __builtin_nontemporal_store(f32x4{x[0], x[1], x[2], x[3]}, reinterpret_cast<f32x4*>(p));
}
__device__ inline void store1(uint16_t* p, float x) { *p = (uint16_t)(pack_bf16x2(x, 0.f) & 0xffffu); }
__device__ inline void store1(float* p, float x) { *p = x; }

// Reductions across the four rows of 16 lanes (lanes t, t + 16, t + 32, t + 48), the result
// in every lane, through the gfx950 row swaps (v_permlane16_swap: odd rows of the first
// operand with even rows of the second; v_permlane32_swap: upper half of the first with lower
// half of the second).  With both operands equal, the two results hold a lane's own row and
// its partner row, so their sum (max) is the pairwise sum (max); VALU latency, where a
// shuffle through ds_bpermute waits on the LDS.  Sums add in the same pairs as a butterfly.
__device__ inline float rows4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ inline float rows4_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Row rotation by N lanes inside each row of 16 (DPP row_ror), every lane written.
template <int N>
__device__ inline float row_ror(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x120 + N, 0xF, 0xF, false));
}

__device__ inline float wave_max(float x) {
  x = fmaxf(x, row_ror<8>(x));
  x = fmaxf(x, row_ror<4>(x));
  x = fmaxf(x, row_ror<2>(x));
  x = fmaxf(x, row_ror<1>(x));
  return rows4_max(x);
}

// Per 64-token chunk and head, the chunk factors handed from the chunk kernel
// to the state-scan kernel.  Every fragment block is stored lane-major so a
// wave moves it with one 16-byte (or 8-byte) access per lane.
template <int DK, int DV>
struct Rec {
  static constexpr int KSK = DK / 32;  // contraction steps over key channels
  static constexpr int NTK = DK / 16;  // 16-row tiles of key channels
  static constexpr int NTV = DV / 16;  // 16-column tiles of value channels
  // W: A fragments of W [64 x DK], [row block 4][KSK][lane 64] x f16x8 (channels in pi order)
  static constexpr size_t W = 0;
  // Q: A fragments of qhat * exp(G), same layout as W
  static constexpr size_t Q = W + 64 * DK * 2;
  // KT: A fragments of (khat * exp(G_last - G))^T [DK x 64], [NTK][2][lane] x f16x8 (tokens in pi order)
  static constexpr size_t KT = Q + 64 * DK * 2;
  // A: A fragments of the masked intra-chunk attention [64 x 64], [row block 4][2][lane] x f16x8
  static constexpr size_t A = KT + 64 * DK * 2;
  // U: C-layout tiles of U * 2^ue [64 x DV], [row block 4][NTV][lane] x f16x4
  static constexpr size_t U = A + 64 * 64 * 2;
  // LAM: per key channel c, { float exp(G_last), int ec } [DK]: ec <= 0 is the exponent by
  // which row c of Khat*exp(G_last-G) was scaled (by 2^-ec) before its fp16 rounding
  static constexpr size_t LAM = U + 64 * DV * 2;
  // HDR: { float vmax (max |v| over the chunk), int ue (U scale exponent), pad, pad }
  static constexpr size_t HDR = LAM + DK * 8;
  static constexpr size_t BYTES = (HDR + 16 + 255) / 256 * 256;
};

// The parts of a record that hold data for a chunk of `rows` valid tokens.  Tokens past the
// chunk's end would give zero rows of W, Qhat exp(G), U and Aqk and zero token columns of
// K~^T and Aqk, so those parts are neither stored nor loaded: a load of a missing part
// returns zeros.  Row block b (tokens 16 b .. 16 b + 15) of W, Qhat exp(G), U and Aqk;
// token half s2 (32 s2 .. 32 s2 + 31: pi stays inside a 32-wide step) of K~^T and Aqk; the
// per-channel and header words of any chunk.  rows = 0 (a load past the end of a walk, never
// used) fetches nothing.
__device__ __forceinline__ bool rec_rows_present(int rows, int b) { return 16 * b < rows; }
__device__ __forceinline__ bool rec_half_present(int rows, int s2) { return 32 * s2 < rows; }

// Raw buffer resources (record stores and loads): dword 3 with a 32-bit data format, byte
// offsets, no swizzle; accesses past num_records are dropped (loads return zeros).  A missing
// part of a record is accessed through a resource with num_records = 0, so the instruction
// stream (and the memory-counter waits the compiler derives from it) is the same for every
// chunk length.
constexpr int kBufferFlags = 0x00020000;
typedef uint32_t uint4_v __attribute__((ext_vector_type(4)));
typedef uint32_t uint2_v __attribute__((ext_vector_type(2)));

// Record loads of `bytes` (the record's size, or 0 for a missing part).  COHERENT (the scan
// role of the fused kernel): device-scope (sc1) loads, which see records that another compute
// die wrote through; otherwise plain loads.
template <typename V, bool COHERENT>
__device__ __forceinline__ V rec_load(const uint8_t* rec, int bytes, size_t off) {
  constexpr int aux = COHERENT ? 16 : 0;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(rec), 0, bytes, kBufferFlags);
  if constexpr (sizeof(V) == 16) {
    return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, aux));
  } else if constexpr (sizeof(V) == 8) {
    return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b64(rs, (int)off, 0, aux));
  } else {
    static_assert(sizeof(V) == 4, "record loads are 4, 8 or 16 bytes");
    return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b32(rs, (int)off, 0, aux));
  }
}

// Hand-off between the two roles of the fused forward kernel: the chunk workgroups
// publish each (chunk, head) record by writing the launch's flag value into its flags (one
// per 64-column scan slice) once the record's stores have completed, the scan workgroups
// wait for their flag before loading the record.  Records and flags move only through
// device-scope (sc1) stores and loads, which are coherent across the compute dies without
// L2 write-backs or invalidations.
//
// Every launch has its own flag value, so flags left by earlier launches (or an
// uninitialised workspace) never match and nothing needs clearing.  An eager call takes a
// fresh value from a process-wide host counter.  A call captured into a graph would replay
// the captured value, so there the value is derived on the device: a one-thread kernel
// captured just before the fused kernel advances a counter in the workspace, and every
// workgroup mixes the counter with the captured salt.
//
// Waits are bounded.  A wave whose wait gives up stores the launch's flag value into the
// workspace's error word (kda_fwd_status reports it) and stops waiting; its chain's final
// state is written as NaN, and a key wave's state rows become NaN at once, so the outputs
// after that point (which read the state) are NaN too.  No index or address is ever
// derived from a record's contents, so reading a record that is not complete is harmless.
struct FuseArgs {
  uint64_t* flags;            // [chunk * H + head][DV / 64]
  uint64_t epoch;             // eager call: the flag value; captured call: the salt
  const uint64_t* dev_epoch;  // captured call: the counter advanced before each launch; else null
  uint64_t* ctl;              // [0] flag value of the most recent launch, [1] value of a failed one
  int32_t producers;          // workgroups 0 .. producers-1 run the chunk walk, the rest the scan
  int32_t spin_limit;         // polls (about 130 cycles each) before a wait gives up
  int32_t scan_rounds;        // chunk-walk rounds every workgroup takes (scan ones before their chains)
};

// The flag value of this launch (the same in every workgroup: the counter is written by
// the kernel before it on the stream).  Always odd, so zeroed memory never matches.
__device__ inline uint64_t launch_epoch(const FuseArgs& fz) {
  if (!fz.dev_epoch) return fz.epoch;
  const uint64_t d = __hip_atomic_load(fz.dev_epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return (d * 0x9E3779B97F4A7C15ull + fz.epoch) | 1ull;
}

// Advances the per-workspace launch counter of captured fused calls (one thread).
__global__ void epoch_advance_kernel(uint64_t* dev_epoch) {
  if (threadIdx.x == 0) {
    const uint64_t d = __hip_atomic_load(dev_epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(dev_epoch, d + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// One entry of the chunk table.
struct ChunkEntry {
  int32_t seq;   // sequence index
  int32_t len;   // valid tokens in this chunk (1..64)
  int32_t idx;   // chunk index inside its sequence
  int32_t pad;
};

// Token offset of sequence n (packed: cu[n]; fixed-length: n * T).
__device__ inline int64_t seq_start(const int32_t* cu, int64_t T, int64_t n) {
  return cu ? (int64_t)cu[n] : n * T;
}
__device__ inline int64_t seq_len(const int32_t* cu, int64_t T, int64_t n) {
  if (!cu) return T;
  int64_t L = (int64_t)cu[n + 1] - (int64_t)cu[n];
  return L > 0 ? L : 0;
}

}  // namespace kda
