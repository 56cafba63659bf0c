/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention forward.
 *
 * The operation.  Per head and per sequence, with a dk x dv state S:
 *
 *     S_t = (I - beta_t khat_t khat_t^T) Diag(exp(g_t)) S_{t-1} + beta_t khat_t v_t^T
 *     o_t = scale * S_t^T qhat_t
 *
 * qhat = q/||q||_2 and khat = k/||k||_2 (a zero vector stays zero), g is a
 * natural-log gate with one value per key channel (it scales the rows of S),
 * beta is one scalar per (token, head), and o_t is read after token t's
 * update.  "Autoresearch on Kimi Delta Attention", section "KDA in one
 * minute", describes this memory in words (fixed-size state, read the
 * prediction, write only the correction, per-channel forgetting) and points
 * to the chunkwise form that turns most of the work into matrix products;
 * "Kernel Design Agents (KDA) optimize Kimi Delta Attention (KDA)", sections
 * "01 - Results" and "03 - Reward hacking", fix the interface this header
 * serves: a forward pass over fixed-length and packed variable-length
 * (cu_seqlens) batches, with an initial state in and the final state out,
 * real Q/K L2 norms, boundaries read from cu_seqlens at run time, 64-token
 * chunks, and a recurrent state that must not be kept in bf16.
 *
 * Conventions for every entry point:
 *   - Tensors are row-major and contiguous; every tensor pointer is 16-byte
 *     aligned.  All tensor pointers are DEVICE pointers; `prob` is a host
 *     pointer.  The library never allocates memory: the caller owns every
 *     buffer, including the workspace.
 *   - Errors are reported as kda_status_t; nothing is printed and nothing is
 *     thrown.  A failed call enqueues no work.
 *   - kda_fwd enqueues its kernels on `stream` and returns without waiting
 *     for them.  It keeps no pointer after that work completes, holds no
 *     global state beyond a process-wide call counter (atomic) and per-device
 *     caches of the compute-unit count and kernel attributes, and may be
 *     called from several host threads at once; two calls that run at the
 *     same time need separate workspaces.  The enqueued work is safe to capture
 *     in a HIP graph and replay (no memset nodes; a captured fused call also
 *     captures a one-thread kernel that advances a launch counter in the
 *     workspace, so every replay has its own hand-off flag value).
 *   - Results are deterministic: the same inputs on the same GPU and build
 *     give bitwise-equal out and ht.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dtype of q, k, v, beta and out (g, h0 and ht are always fp32). */
typedef enum { KDA_BF16 = 0, KDA_F32 = 1 } kda_dtype_t;

typedef enum {
  KDA_OK = 0,
  KDA_ERR_NULL = 1,        /* a required pointer is NULL */
  KDA_ERR_UNSUPPORTED = 2, /* dk/dv not in {64,128} or an unknown dtype */
  KDA_ERR_BAD_ARG = 3,     /* negative or inconsistent sizes, non-finite scale, bad cu_seqlens */
  KDA_ERR_ALIGN = 4,       /* a tensor pointer is not 16-byte aligned */
  KDA_ERR_WORKSPACE = 5,   /* workspace smaller than kda_fwd_workspace_size() */
  KDA_ERR_ALIAS = 6,       /* out or ht overlaps an input (ht == h0 exactly is allowed) */
  KDA_ERR_HIP = 7,         /* a HIP launch reported an error */
  KDA_ERR_TIMEOUT = 8      /* (kda_fwd_status) a wait of the fused kernel gave up */
} kda_status_t;

/*
 * Problem sizes.
 *   Fixed-length mode (cu_seqlens == NULL): `batch` sequences of `seqlen`
 *     tokens each; num_seqs must be 0 or equal to batch.
 *   Packed mode (cu_seqlens != NULL): batch == 1, `seqlen` is the total
 *     number of tokens and `num_seqs` >= 1 the number of packed sequences.
 *   Limits (KDA_ERR_BAD_ARG beyond them): (64-token chunks) x heads and
 *   8 x sequences x heads below 2^31; packed seqlen below 2^31.
 */
typedef struct {
  int64_t batch;    /* B */
  int64_t seqlen;   /* T (per row; total tokens in packed mode) */
  int64_t num_seqs; /* N */
  int32_t heads;    /* H >= 1 */
  int32_t dk;       /* key/query head size: 64 or 128 */
  int32_t dv;       /* value head size: 64 or 128 */
  int32_t dtype;    /* kda_dtype_t */
} kda_problem_t;

/*
 * Bytes of device workspace kda_fwd needs for `prob` (0 on an invalid
 * problem).  The workspace holds the chunk table and, per 64-token chunk and
 * head, the chunk's factors (the WY factors W and U, the decayed queries and
 * keys, the masked intra-chunk attention and the chunk decay) and a ready
 * flag.  Its contents are scratch: nothing in it needs initialising (flags are
 * compared with a per-launch value).  The only state that outlives a call is
 * the outcome word that kda_fwd_status reads.  The chunkwise form whose
 * per-chunk factors these are is the one "Autoresearch on Kimi Delta
 * Attention", section "KDA in one minute", points to (matrix products inside
 * a chunk, the state carried between chunks).
 */
size_t kda_fwd_workspace_size(const kda_problem_t* prob);

/*
 * Checks everything kda_fwd checks on the host, without touching the GPU:
 * sizes, dtype, NULL pointers, alignment, workspace size and overlaps.  With
 * the environment variable KDA_VALIDATE_CU_SEQLENS=1 it also copies
 * cu_seqlens to the host (a synchronising copy) and checks cu[0] == 0,
 * non-decreasing offsets and cu[N] == seqlen (KDA_ERR_BAD_ARG otherwise;
 * kda_fwd then enqueues nothing).  Arguments as for kda_fwd.  This is the
 * legal-input side of the contract: "Kernel Design Agents (KDA) optimize Kimi
 * Delta Attention (KDA)", section "04 - Hardening" (a strict specification of
 * the legal inputs, on each of which the kernels must be correct).
 */
kda_status_t kda_fwd_validate(const kda_problem_t* prob, const void* q, const void* k,
                              const void* v, const float* g, const void* beta, const float* h0,
                              const int32_t* cu_seqlens, float scale, const void* out,
                              const float* ht, const void* workspace, size_t workspace_bytes);

/*
 * KDA forward pass: the operation at the top of this header, over the batches
 * that "Kernel Design Agents (KDA) optimize Kimi Delta Attention (KDA)",
 * section "01 - Results", benchmarks (fixed-length and packed varlen, initial
 * and final state).
 *
 *   q, k        [B, T, H, dk]  dtype        queries and keys (any finite magnitude;
 *                                           normalised inside the kernels)
 *   v           [B, T, H, dv]  dtype        values
 *   g           [B, T, H, dk]  fp32         log-gate, finite and <= 0
 *   beta        [B, T, H]      dtype        write strength in [0, 1]
 *   h0          [N, H, dk, dv] fp32         initial state, or NULL for zeros
 *   cu_seqlens  [N + 1]        int32        packed-sequence token offsets (device),
 *                                           or NULL for fixed-length rows; cu[0] = 0,
 *                                           non-decreasing, cu[N] = T; empty sequences
 *                                           are allowed and return ht = h0
 *   scale                      host float   output scale (1/sqrt(dk) is the usual value)
 *   out         [B, T, H, dv]  dtype        output (written)
 *   ht          [N, H, dk, dv] fp32         final state (written), or NULL; may be
 *                                           exactly h0 for an in-place state update
 *   workspace   workspace_bytes             device scratch, >= kda_fwd_workspace_size()
 *   stream                                  hipStream_t to enqueue on (NULL = default)
 *
 * Inputs outside the stated domain (g > 0, beta outside [0, 1], non-finite
 * values) get no accuracy guarantee but never make the kernels read or write
 * out of bounds.  cu_seqlens is read on the device; its validity is the
 * caller's precondition (see kda_fwd_validate).
 *
 * Kernels.  Fixed-length batches with few (row, head) chains -- rows x heads x
 * dv/64 at most a quarter of the compute units -- run as one persistent
 * kernel in which most workgroups compute the chunk factors and the others
 * walk the chains as the factors appear; other batches run the chunk kernel
 * and then the state scan (packed batches after a small chunk-map kernel).
 *
 * Tuning (read at every call; results are the same up to rounding):
 *   KDA_FUSED=0              never use the single fused kernel
 *   KDA_SCAN_SLICE=16|32|64  value columns per state-scan workgroup of the two-kernel
 *                            path (default: the widest that still gives every compute
 *                            unit a workgroup)
 *   KDA_CHUNK_WGS=n          at most n workgroups compute chunk factors (default: one
 *                            per compute unit, minus the chain workgroups when fused)
 *   KDA_FUSE_ROUNDS=n        fused kernel: rounds of chunk items that the chain
 *                            workgroups take too, before their chains start (default 1;
 *                            0..64; the results are the same bits for every n)
 *   KDA_SPIN_LIMIT=n         polls before a wait of the fused kernel gives up (default:
 *                            several times the whole chunk walk); a small n forces the
 *                            failure path that kda_fwd_status reports
 */
kda_status_t kda_fwd(const kda_problem_t* prob, const void* q, const void* k, const void* v,
                     const float* g, const void* beta, const float* h0,
                     const int32_t* cu_seqlens, float scale, void* out, float* ht,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Outcome of the most recent kda_fwd call on `workspace`.  Waits inside the
 * fused kernel are bounded; one that gives up (its spin limit ran out before
 * the awaited chunk factors were published) writes NaN into the outputs and
 * final-state entries it would have produced and records the launch's flag
 * value in the workspace.  This call synchronises `stream`, copies that word
 * to the host and returns KDA_ERR_TIMEOUT if the most recent launch on the
 * workspace failed this way, KDA_OK otherwise (also for calls that took the
 * two-kernel path, which has no waits).  A failed launch captured in a graph
 * is reported again by each replay that fails.  KDA_ERR_NULL / KDA_ERR_ALIGN /
 * KDA_ERR_WORKSPACE for a bad workspace argument (at least 256 bytes).
 * "Kernel Design Agents (KDA) optimize Kimi Delta Attention (KDA)", section
 * "04 - Hardening", asks for correctness on every legal input: a result the
 * kernel could not finish must not pass silently.
 */
kda_status_t kda_fwd_status(const void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_fwd with timing marks for profiling: identical work, plus hipEventRecord
 * of events[0] before the chunk map, events[1] after it, events[2] after the
 * chunk kernel (including its pass over chunks whose in-chunk decay exceeds the
 * fast path's range) and events[3] after the state scan, all on `stream`
 * (fused kernel: events[2] and events[3] both after it).
 * `events` is a host array of 4 hipEvent_t handles created by the caller (NULL
 * entries are skipped); the elapsed time between consecutive marks is the
 * duration of each kernel.  Errors as for kda_fwd.
 */
kda_status_t kda_fwd_timed(const kda_problem_t* prob, const void* q, const void* k, const void* v,
                           const float* g, const void* beta, const float* h0,
                           const int32_t* cu_seqlens, float scale, void* out, float* ht,
                           void* workspace, size_t workspace_bytes, void* stream,
                           void* const* events);

/*
 * kda_fwd without a workspace argument, for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that forbid
 * allocation).  The workspace is a static device array of
 * KDA_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on until
 * the process ends; the call itself allocates nothing.  Problems whose
 * kda_fwd_workspace_size exceeds that size are rejected with KDA_ERR_WORKSPACE
 * before anything is enqueued (64 MiB: 8,192 tokens of up to 6 heads at
 * dk = dv = 128, i.e. up to 894 pairs of a 64-token chunk and a head).  All calls on
 * one GPU share its array: two calls that overlap in time on the same GPU (other
 * streams, other host threads) race and give wrong results; calls ordered on
 * one stream do not.  Arguments, results and the other errors as for kda_fwd.
 * A wait of the fused kernel that gives up still writes NaN into the affected
 * outputs; kda_fwd_status does not see this array.
 */
#define KDA_NOALLOC_SCRATCH_BYTES (64u << 20)
kda_status_t kda_fwd_noalloc(const kda_problem_t* prob, const void* q, const void* k, const void* v,
                             const float* g, const void* beta, const float* h0,
                             const int32_t* cu_seqlens, float scale, void* out, float* ht, void* stream);

/*
 * The same forward evaluated token by token, for decode steps (one new token
 * per sequence, seqlen == 1) and other short continuations of many sequences.
 * It is the step that "Autoresearch on Kimi Delta Attention", section "KDA in
 * one minute", describes (per-channel forgetting, read the prediction, write
 * the correction), applied once per token:
 *
 *     a = Diag(exp(g_t)) S,  delta = v_t - a^T khat_t,  S = a + beta_t khat_t delta^T,
 *     o_t = scale * S^T qhat_t
 *
 * Arguments, shapes, dtypes, modes (fixed-length rows or cu_seqlens), the
 * initial/final state convention (h0 NULL = zeros, ht NULL = not written,
 * ht == h0 for an in-place update, empty sequences return ht = h0), alignment,
 * aliasing rules and errors are those of kda_fwd; there is no workspace.  The
 * state is read from HBM once and written once per call and carried in fp32
 * registers in between; every step is fp32.  Each token costs O(dk * dv) per
 * (sequence, head) with no parallelism along the sequence, so long prompts
 * belong to kda_fwd; results agree with kda_fwd up to rounding.
 */
kda_status_t kda_decode(const kda_problem_t* prob, const void* q, const void* k, const void* v,
                        const float* g, const void* beta, const float* h0,
                        const int32_t* cu_seqlens, float scale, void* out, float* ht, void* stream);

/*
 * Backward pass: the gradients of a kda_fwd call.  "Autoresearch on Kimi Delta
 * Attention" (stage "Frozen outside the loop": full gradients against an
 * independent reference; phase "Parallelize the recurrence": chunkwise transforms
 * and a scan over chunks instead of the token-by-token reverse walk) fixes what it
 * must return and the form it takes.
 *
 *   q, k, v, g, beta, h0, cu_seqlens, scale   the forward's inputs, as for kda_fwd
 *   dout        [B, T, H, dv]  dtype   dL/dout
 *   dht         [N, H, dk, dv] fp32    dL/dht, or NULL for zero
 *   dq, dk      [B, T, H, dk]  dtype   dL/dq, dL/dk (through the L2 normalisation;
 *                                      zero for a zero q or k vector)
 *   dv          [B, T, H, dv]  dtype   dL/dv
 *   dg          [B, T, H, dk]  fp32    dL/dg
 *   dbeta       [B, T, H]      dtype   dL/dbeta
 *   dh0         [N, H, dk, dv] fp32    dL/dh0 (also when h0 is NULL, i.e. zero), or NULL
 *   workspace   >= kda_bwd_workspace_size(prob) bytes of device scratch
 *
 * Chunkwise, per 64-token chunk and head, with every product on the fp32 matrix cores:
 * a first kernel forms the chunk's factors (the gated Grams, the inverse of
 * I + diag(beta) L, W, U); one kernel walks each (sequence, head, 16 value columns)
 * forwards for the state at every chunk start and backwards for dL/dS at every chunk
 * end; two kernels then form each chunk's gradients.  The workspace holds per (chunk,
 * head) the factors (about 162 KB at dk = dv = 128) and a state block (S0, dL/dS and two
 * 64 x dv matrices, 192 KB): 1.47 GB for 8,192 tokens of 32 heads.  With cu_seqlens the
 * chunk count is bounded by T / 64 + N (the offsets stay on the device), so packed
 * batches size for that bound.  Conventions (stream, no allocation, errors, alignment)
 * as for kda_fwd; outputs must not overlap any input, the workspace or each other.
 * Results are deterministic.
 */
size_t kda_bwd_workspace_size(const kda_problem_t* prob);
kda_status_t kda_bwd(const kda_problem_t* prob, const void* q, const void* k, const void* v,
                     const float* g, const void* beta, const float* h0, const int32_t* cu_seqlens,
                     float scale, const void* dout, const float* dht, void* dq, void* dk, void* dv,
                     float* dg, void* dbeta, float* dh0, void* workspace, size_t workspace_bytes,
                     void* stream);

/* Test hook, not part of the method: fills the whole LDS of every compute unit with the
 * 32-bit pattern `bits`, asynchronously on `stream` (a HIP stream, NULL for the default
 * stream).  LDS keeps what the previous kernel on a compute unit left there, and no kernel
 * of this library may read an LDS word it has not written in the same launch; a call made
 * right after this fill with a NaN or Inf pattern shows any such read in its outputs.
 * With the environment variable KDA_TEST_LDS_FILL set to a pattern (decimal or 0x hex),
 * every kernel that kda_fwd, kda_decode and kda_bwd launch is preceded by this fill.
 * Returns KDA_ERR_HIP when the launch fails. */
kda_status_t kda_test_fill_lds(uint32_t bits, void* stream);

/* Human-readable name of a status code (static string). */
const char* kda_status_string(kda_status_t status);

/* Library version as major*10000 + minor*100 + patch. */
int kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
