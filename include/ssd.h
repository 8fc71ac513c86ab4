/*
 * ssd.h - C ABI of the MI355X (gfx950) SSD chunked forward pass.
 *
 * The operation is the Mamba-2 structured-state-space-duality forward pass
 * (page "State Space Duality and Mamba-2", sections "The Mathematical Bridge"
 * and "The SSD Block Decomposition Algorithm"):
 *
 *     a_t = exp(dt_t * A_h)                       scalar decay per token/head
 *     h_t = a_t * h_{t-1} + dt_t * x_t B_t^T      state, P x N per head
 *     y_t = h_t C_t + D_h * x_t
 *
 * equivalently Y = ((C B^T) o L) (dt x) + D x with the 1-semiseparable decay
 * mask L_ij = prod_{k=j+1..i} a_k (i >= j), evaluated blockwise: the sequence
 * is cut into chunks of chunk_size tokens; each chunk's diagonal block is a
 * masked quadratic product, and chunks are connected through the N x P state
 * (chunk-state contraction, inter-chunk scan, state projection onto the next
 * chunk's outputs).  Long rows are cut into sequence-parallel splits whose
 * length is chosen independently of chunk_size (page "GPU Hierarchy Meets
 * Structured Matrices", abstract: split-sequence algorithm); splits are joined
 * by an affine scan of their boundary states (page "Parallel Scan and
 * Hardware-Aware SSM Kernels", section "The scan").
 *
 * Document packing: where seq_idx changes between tokens t-1 and t the state
 * is reset (a_t is masked to 0), so no information flows across a document
 * boundary (page "Parallel Scan and Hardware-Aware SSM Kernels", section
 * "When it breaks").
 *
 * Layouts: every tensor is dense and row-major, no strides.
 *   x, y          [batch, seqlen, nheads, headdim]   io dtype
 *   dt            [batch, seqlen, nheads]            fp32, > 0 (post-softplus)
 *   A             [nheads]                           fp32, <= 0
 *   B, C          [batch, seqlen, ngroups, dstate]   io dtype
 *   D             [nheads]                           fp32 (nullable: no skip)
 *   seq_idx       [batch, seqlen]                    int32 (nullable: 1 doc/row)
 *   init_states,
 *   final_states  [batch, nheads, headdim, dstate]   fp32 (nullable)
 * Head h reads B/C group h / (nheads / ngroups) (grouped-query SSM, page
 * "State Space Duality and Mamba-2", section "Architectural Scaling").
 * init_states feeds only the first document of each row; final_states is the
 * state after the row's last token.
 *
 * Ownership and threading: the caller allocates every device buffer,
 * including the workspace; the library allocates no device memory and keeps
 * no mutable global state except a per-device cache of the compute-unit
 * count.  Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 * stream), reentrant, and make no implicit synchronisation.  Concurrent calls
 * must not share a workspace.
 *
 * Planning: the split plan (and so the workspace size) depends on the
 * compute-unit count of the device that `stream` belongs to (the current
 * device for the NULL stream); the *_workspace_bytes and ssd_plan_* queries,
 * which take no stream, plan for the current device.
 *
 * Errors: every argument is validated on the host before any kernel is
 * launched; the only HIP calls made before that are the planner's queries of
 * the stream's device and of its compute-unit count.  On failure the call
 * returns a status, launches nothing and records a message readable with
 * ssd_last_error() (thread-local).  A failed launch returns SSD_ERR_HIP.
 * Device-side faults surface at the caller's next synchronisation.  NaN or
 * Inf inputs propagate; the hot path does not check values.
 *
 * Supported set (anything else returns SSD_ERR_UNSUPPORTED):
 *   chunk_size in {64, 128, 256}; headdim in {16, 32, 64, 128};
 *   dstate in {16, 32, 64, 128}; nheads % ngroups == 0; seqlen >= 1;
 *   batch >= 1; x, B, C, y 16-byte aligned; every fp32 buffer 4-byte aligned
 *   and init/final states 16-byte aligned.
 */
#ifndef SSD_MI355X_H
#define SSD_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SSD_OK = 0,
    SSD_ERR_NULL = 1,         /* a required pointer is NULL               */
    SSD_ERR_SHAPE = 2,        /* a size is < 1 or sizes are inconsistent  */
    SSD_ERR_UNSUPPORTED = 3,  /* outside the supported set above          */
    SSD_ERR_ALIGN = 4,        /* a pointer is not aligned as required     */
    SSD_ERR_WORKSPACE = 5,    /* workspace NULL or smaller than required  */
    SSD_ERR_HIP = 6           /* a HIP runtime call or launch failed      */
} ssd_status_t;

typedef enum {
    SSD_F32 = 0,   /* x, B, C, y in fp32; fp32 arithmetic throughout          */
    SSD_BF16 = 1,  /* x, B, C, y in bf16; bf16 MFMA with fp32 accumulation    */
    SSD_DTYPE_RANGE_ = 0x7fffffff  /* not a dtype: makes every non-negative int
                                      a valid value of the type, so that an
                                      unknown one is rejected, not undefined */
} ssd_dtype_t;

typedef struct {
    int64_t batch, seqlen, nheads, headdim, dstate, ngroups;
} ssd_shape_t;

/* Test/benchmark options.  Zero-initialise for the defaults. */
typedef struct {
    int64_t split_len;   /* tokens per sequence-parallel split: 0 = planner's
                            choice, else a positive multiple of chunk_size   */
    int64_t flags;       /* SSD_OPT_* bits                                    */
    int64_t headdim_block; /* headdim columns per workgroup: 0 = planner's
                            choice, else a power of two >= 16 dividing
                            headdim whose tiles fit the LDS (bf16 io only;
                            fp32 io takes 0 or headdim)                     */
    int64_t reserved[5]; /* must be zero                                      */
} ssd_options_t;

/* flags: the workspace already holds the per-group operands (C_c B_c^T blocks
 * and token-transposed B) of exactly these B and C, shape and chunk size,
 * written by an earlier bf16 call on the same stream with the same workspace;
 * skip recomputing them.  Only the head kernels run.  Meaningful for bf16 io
 * (ignored for fp32).  The caller guarantees that B and C are unchanged; the
 * library cannot check it. */
#define SSD_OPT_REUSE_GROUP_OPERANDS 1

/* flags (segsum ablation, for tests and benchmarks): evaluate the
 * intra-chunk decay mask by the direct segsum (each entry its own running
 * sum) or by the diff segsum (difference of the chunk's prefix sums) instead
 * of the hierarchy-aware one (page "GPU Hierarchy Meets Structured Matrices",
 * abstract, compares the three).  At most one.  fp32 io: any shape.  bf16
 * io: the head kernel's output path masks every C B^T block element by
 * element instead of applying the rank-one factors; chunk_size 256, dstate 64
 * or 128 and a headdim block of 32 or 64 only (SSD_ERR_UNSUPPORTED
 * otherwise).  The chunk states and the decays of the state projection are
 * the hierarchy-aware ones in every case. */
#define SSD_OPT_SEGSUM_DIRECT 2
#define SSD_OPT_SEGSUM_DIFF 4

/* Bytes of device workspace ssd_fwd needs for this problem (16-byte aligned
 * pointer required).  Returns 0 when no workspace is needed, and also for an
 * invalid problem (ssd_fwd then reports the error).  The workspace holds,
 * each part rounded up to 256 bytes:
 *   - bf16 io, first: the per-group C B^T blocks of every chunk (the lower
 *     triangle of C_c B_c^T in 16 x 32-token blocks, 1 KiB each,
 *     (Q/32)(Q/32+1) blocks per chunk), B token-transposed and C in operand
 *     order, i.e. batch * ngroups * nchunks * (1024 (Q/32)(Q/32+1) +
 *     2 Q dstate) bytes + batch * ngroups * nchunks * 2 Q max(dstate, 32)
 *     bytes (C; dstate 16 is padded to 32 columns);
 *   - then, with more than one sequence split: the splits' states and
 *     decays, 4 * batch * nheads * nsplits * (headdim * dstate + 1) bytes.
 * Every byte the kernels read is written earlier in the same call, so the
 * workspace needs no clearing.  Only the per-group operands survive a bf16
 * call (for SSD_OPT_REUSE_GROUP_OPERANDS; their offsets depend on the shape
 * and chunk size only); everything else is scratch. */
size_t ssd_fwd_workspace_bytes(const ssd_shape_t *shape, int64_t chunk_size,
                               ssd_dtype_t io);

/* The forward pass.  x, dt, A, B, C, y are required; D, seq_idx, init_states
 * and final_states may be NULL.  The workspace may be NULL when
 * ssd_fwd_workspace_bytes() returns 0. */
ssd_status_t ssd_fwd(const ssd_shape_t *shape, ssd_dtype_t io,
                     const void *x, const float *dt, const float *A,
                     const void *B, const void *C, const float *D,
                     const int32_t *seq_idx, int64_t chunk_size,
                     const float *init_states,
                     void *y, float *final_states,
                     void *workspace, size_t workspace_bytes, void *stream);

/* ssd_fwd with options (tests and benchmarks: forced split length). */
size_t ssd_fwd_ex_workspace_bytes(const ssd_shape_t *shape, int64_t chunk_size,
                                  ssd_dtype_t io, const ssd_options_t *opts);
ssd_status_t ssd_fwd_ex(const ssd_shape_t *shape, ssd_dtype_t io,
                        const void *x, const float *dt, const float *A,
                        const void *B, const void *C, const float *D,
                        const int32_t *seq_idx, int64_t chunk_size,
                        const float *init_states,
                        void *y, float *final_states,
                        void *workspace, size_t workspace_bytes,
                        const ssd_options_t *opts, void *stream);

/* Fused prologue and epilogue of ssd_fwd_fused: the lightweight element-wise
 * work on either side of the scan, done inside its kernels so that neither dt
 * nor y makes an extra round trip through memory (page "NVIDIA Accelerates
 * Mamba-2 Forward Kernel with CUDA Tile": the forward pass carries
 * element-wise gating ("What CUDA Tile Is and Why It Suits Writing Mamba-2
 * Kernels") and the gating that follows the scan is fused into its kernel
 * ("From Python DSL to Production-Grade Kernels")).  The pages do not spell
 * the two maps out; they are Mamba-2's:
 *   dt_t  = clamp(softplus(dt_raw_t + dt_bias_h), dt_min, dt_max)
 *   out_t = (y_t + D_h x_t) * silu(z_t),   silu(z) = z / (1 + e^-z)
 * where each step applies only when enabled: dt_bias NULL = no bias,
 * dt_softplus 0 = no softplus, dt_clamp 0 = no clamp, z NULL = no gate.
 * Zero-initialise for none of them (then ssd_fwd_fused is ssd_fwd_ex).
 * final_states is the state of the recurrence (the gate acts on the output
 * only).  With io = SSD_BF16 the gate multiplies the bf16-rounded y, and
 * the product is rounded to bf16 again. */
typedef struct {
    const float *dt_bias;   /* [nheads] fp32, 4-byte aligned, nullable          */
    const void *z;          /* [batch, seqlen, nheads, headdim] io dtype,
                               16-byte aligned, nullable                        */
    int32_t dt_softplus;    /* nonzero: softplus after the bias                 */
    int32_t dt_clamp;       /* nonzero: clamp to [dt_min, dt_max] (finite,
                               dt_min <= dt_max, else SSD_ERR_UNSUPPORTED)      */
    float dt_min, dt_max;
    int64_t reserved[4];    /* must be zero                                     */
} ssd_fused_t;

/* ssd_fwd_ex with the fused prologue/epilogue above; dt holds the raw values
 * (dt_raw) when any of bias, softplus or clamp is enabled, and the step sizes
 * must come out > 0.  fused may be NULL.  Workspace as ssd_fwd_ex. */
ssd_status_t ssd_fwd_fused(const ssd_shape_t *shape, ssd_dtype_t io,
                           const void *x, const float *dt, const float *A,
                           const void *B, const void *C, const float *D,
                           const int32_t *seq_idx, int64_t chunk_size,
                           const float *init_states,
                           void *y, float *final_states,
                           const ssd_fused_t *fused,
                           void *workspace, size_t workspace_bytes,
                           const ssd_options_t *opts, void *stream);

/* The split length (tokens) the planner would use; 0 for an invalid problem. */
int64_t ssd_plan_split_len(const ssd_shape_t *shape, int64_t chunk_size,
                           ssd_dtype_t io);

/* The headdim columns per workgroup the planner would use (the whole head
 * unless the tiles do not fit the LDS, or halved when that alone gives every
 * CU a workgroup); 0 for an invalid problem. */
int64_t ssd_plan_headdim_block(const ssd_shape_t *shape, int64_t chunk_size,
                               ssd_dtype_t io);

/* Debug export of the decay mask exactly as the forward kernels build it
 * (page "GPU Hierarchy Meets Structured Matrices", abstract: hierarchy-aware
 * segsum; page "State Space Duality and Mamba-2", definition of L).  Writes
 * fp32 L_out[batch][nheads][chunk_count][chunk_size][chunk_size] for chunks
 * [chunk_begin, chunk_begin + chunk_count): L[i][j] = prod_{k=j+1..i} a_k for
 * j <= i, 0 above the diagonal, 0 across a document boundary, 0 for tokens
 * past the end of the row.  Only x-independent inputs are needed.  dstate,
 * headdim and ngroups in `shape` are validated but unused. */
ssd_status_t ssd_debug_chunk_mask(const ssd_shape_t *shape, const float *dt,
                                  const float *A, const int32_t *seq_idx,
                                  int64_t chunk_size, int64_t chunk_begin,
                                  int64_t chunk_count, float *L_out,
                                  void *stream);

/* Segsum evaluations of the decay mask (page "GPU Hierarchy Meets Structured
 * Matrices", abstract): the forward kernels use the hierarchy-aware one; the
 * other two exist for the comparison the page makes. */
#define SSD_SEGSUM_HIERARCHY 0 /* nested sub-block sums, rank-one off-diagonal factors */
#define SSD_SEGSUM_DIRECT 1    /* each entry its own running sum (dense direct segsum) */
#define SSD_SEGSUM_DIFF 2      /* difference of chunk prefix sums (diff segsum)      */

/* ssd_debug_chunk_mask with a choice of segsum evaluation.  L_out (as above)
 * and sums_out (fp32 [batch][nheads][chunk_count], the sum of each chunk's
 * mask entries) may each be NULL, not both; with L_out NULL the mask is
 * evaluated but not written (for timing the evaluation alone).  An unknown
 * variant returns SSD_ERR_UNSUPPORTED. */
ssd_status_t ssd_debug_chunk_mask_ex(const ssd_shape_t *shape, const float *dt,
                                     const float *A, const int32_t *seq_idx,
                                     int64_t chunk_size, int64_t chunk_begin,
                                     int64_t chunk_count, int32_t variant,
                                     float *L_out, float *sums_out,
                                     void *stream);

/* One decode step (single token) of the recurrence of page "State Space
 * Duality and Mamba-2" ("The Mathematical Bridge"), per (batch row, head h):
 *   a = exp(dt A_h);  state <- a state + dt x B^T;  y = state C + D_h x,
 * i.e. what ssd_fwd computes for one more token given its final_states.
 * shape->seqlen must be 1.  x, y: [batch][nheads][headdim]; dt: [batch][nheads]
 * fp32; B, C: [batch][ngroups][dstate]; A, D: [nheads] fp32 (D nullable);
 * x, B, C, y in the io dtype (aligned to its size).  state:
 * [batch][nheads][headdim][dstate] fp32, 16-byte aligned, updated in place
 * (the caller zeroes it to start a new sequence).  headdim and dstate in
 * {16, 32, 64, 128}; no workspace. */
ssd_status_t ssd_decode_step(const ssd_shape_t *shape, ssd_dtype_t io,
                             const void *x, const float *dt, const float *A,
                             const void *B, const void *C, const float *D,
                             float *state, void *y, void *stream);

/* ssd_decode_step with the fused dt map and output gate of ssd_fused_t (the
 * same maps as ssd_fwd_fused): dt holds the raw value when bias, softplus or
 * clamp is enabled; fused->z, if set, is [batch][nheads][headdim] in the io
 * dtype, aligned to its element size, and y becomes (state C + D_h x) *
 * silu(z).  fused may be NULL (then this is ssd_decode_step). */
ssd_status_t ssd_decode_step_fused(const ssd_shape_t *shape, ssd_dtype_t io,
                                   const void *x, const float *dt, const float *A,
                                   const void *B, const void *C, const float *D,
                                   float *state, void *y, const ssd_fused_t *fused,
                                   void *stream);

/* Backward pass: the gradients of J = <dy, y> + <dfinal, final_states> with
 * respect to every input of ssd_fwd (same shapes and layouts, no fused
 * prologue/epilogue), i.e. what training needs from this layer.  The method
 * differentiates the chunked decomposition of page "State Space Duality and
 * Mamba-2" ("The SSD Block Decomposition Algorithm"): one pass per (batch
 * row, head) walks the 64-token chunks in order and writes every
 * chunk-entering state, then one reverse walk over the chunks per (batch
 * row, head) carries the adjoint of the state in fp32.  fp32 inputs:
 * every product on fp32 MFMA tiles.  bf16 inputs: every product on bf16 MFMA
 * with fp32 accumulation; the masked products take their fp32 operand
 * rounded to bf16, the products with a carried state (adjoint or state) take
 * that fp32 operand as a sum of two bf16 parts (about 16 bits kept).
 *   dy [b, L, H, P] io dtype, 16-byte aligned; dfinal [b, H, P, N] fp32 or NULL;
 *   outputs, all fp32: dx [b, L, H, P], ddt [b, L, H], dA [H], dB and dC
 *   [b, L, G, N], dD [H] (NULL exactly when D is NULL), dinit [b, H, P, N]
 *   (NULL, or the gradient of init_states, which must then be given).
 * Supported set and errors as ssd_fwd (chunk 64 internally); the workspace
 * (ssd_bwd_workspace_bytes, 16-byte aligned, queried with the device that
 * will run the call current: its size depends on the compute-unit count)
 * holds the entering states, 4 b H ceil(L / 64) P N bytes when L > 64, then
 * 8 b L H N + 16 b H bytes, then, when the (batch row, head) walks of the
 * last round are split in two, 4 P N bytes for each of them (at most half the
 * compute units), each part rounded up to 256 bytes; nothing in it survives
 * the call, and nothing is read from it before the call writes it.
 * Repeatability: every gradient is the same bit for bit on every call with
 * the same inputs (each sum, over the waves of a workgroup, the chunks, the
 * heads of a group and the batch rows, is taken in a fixed order). */
size_t ssd_bwd_workspace_bytes(const ssd_shape_t *shape, ssd_dtype_t io);
ssd_status_t ssd_bwd(const ssd_shape_t *shape, ssd_dtype_t io,
                     const void *x, const float *dt, const float *A,
                     const void *B, const void *C, const float *D,
                     const int32_t *seq_idx, const float *init_states,
                     const void *dy, const float *dfinal,
                     float *dx, float *ddt, float *dA, float *dB, float *dC,
                     float *dD, float *dinit,
                     void *workspace, size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): ssd_fwd
 * with its workspace taken from a fixed array of SSD_NOALLOC_WORKSPACE_BYTES
 * that the library holds in the memory of each GPU it runs on, from its first
 * use until the process ends (its device address is looked up once per
 * device).  The caller still passes inputs and outputs.  A problem whose
 * workspace (ssd_fwd_workspace_bytes) exceeds the array returns
 * SSD_ERR_WORKSPACE and launches nothing; no call allocates or frees memory.
 * Every call on a GPU uses that GPU's one array: calls that overlap on one
 * GPU (other streams, other threads) race and must be serialised by the
 * caller.  The array needs no clearing between calls (every byte read is
 * written earlier in the same call).  Otherwise as ssd_fwd. */
#define SSD_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)
ssd_status_t ssd_fwd_noalloc(const ssd_shape_t *shape, ssd_dtype_t io,
                             const void *x, const float *dt, const float *A,
                             const void *B, const void *C, const float *D,
                             const int32_t *seq_idx, int64_t chunk_size,
                             const float *init_states,
                             void *y, float *final_states, void *stream);

/* ---- Debug exports (tests only) ---------------------------------------
 *
 * Segsum factor records.  The hierarchy-aware segsum (page "GPU Hierarchy
 * Meets Structured Matrices", abstract) reduces each chunk of each head to
 * per-token and per-sub-block factors (16-token sub-blocks): one record of
 * ssd_segsum_record_words(chunk_size) 32-bit words per (batch row, head,
 * chunk), records ordered [batch][nheads][nchunks], each holding
 *   d[Q]       log2-decay dt_t A_h log2(e) (0 past the end of the row)
 *   dt[Q]      dt_t (0 past the end)
 *   wd[Q]      W_t dt_t, W_t the decay from t to the end of its sub-block
 *   last1[Q]   int32: 1 + the last reset position <= t inside t's sub-block, 0 if none
 *   Tb[Q/16]   whole-sub-block decay (0 if a reset lies inside)
 *   blast1[Q/16]  int32: 1 + the last reset position inside the sub-block, 0 if none
 *   Tp[Q/32]   Tb[2m] Tb[2m+1]
 * All decays are exp2 of nested sequential sums of non-positive terms.  0 for
 * an invalid chunk size. */
int64_t ssd_segsum_record_words(int64_t chunk_size);

/* The factors as the mask export (ssd_debug_chunk_mask) builds them, with
 * sequential per-token sums: out holds batch * nheads * nchunks records.
 * Validation and errors as ssd_debug_chunk_mask; at most 65535 chunks. */
ssd_status_t ssd_debug_segsum_factors(const ssd_shape_t *shape, const float *dt,
                                      const float *A, const int32_t *seq_idx,
                                      int64_t chunk_size, float *out, void *stream);

/* ssd_fwd_ex (bf16 io only) that also writes the factors exactly as the bf16
 * head kernel builds them for its own use (row-shift sums across the lanes of
 * a wave): out holds batch * nheads * nchunks records.  y and final_states
 * are computed as by ssd_fwd_ex. */
ssd_status_t ssd_debug_fwd_segsum_factors(const ssd_shape_t *shape, ssd_dtype_t io,
                                          const void *x, const float *dt, const float *A,
                                          const void *B, const void *C, const float *D,
                                          const int32_t *seq_idx, int64_t chunk_size,
                                          const float *init_states,
                                          void *y, float *final_states,
                                          void *workspace, size_t workspace_bytes,
                                          const ssd_options_t *opts, float *out,
                                          void *stream);

/* Exhaustive check of the device's exp2 (the only exponential the decay
 * factors use; their [0, 1] range and monotonicity rest on it, page "GPU
 * Hierarchy Meets Structured Matrices", abstract) over the fp32 bit patterns
 * [first_bits, first_bits + count), which must lie in [0x80000000,
 * 0xff800000] (-0 down to -inf).  counts: device array of 3 * nthreads
 * uint32; thread t writes, for its share of the patterns, the number of
 * increases of exp2 as the argument decreases, of values above 1, and of
 * values below 0 or NaN.  nthreads in [1, 2^24]. */
ssd_status_t ssd_debug_exp2_probe(uint32_t first_bits, uint32_t count, uint32_t *counts,
                                  uint32_t nthreads, void *stream);

const char *ssd_status_str(ssd_status_t status);

/* Detail of the last failure on the calling thread ("" if none). */
const char *ssd_last_error(void);

/* Library version string. */
const char *ssd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSD_MI355X_H */
