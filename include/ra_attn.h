/*
 * ra_attn.h -- C ABI of libra_attn.so: RotateAttention INT4 FlashAttention
 * forward for 3D-RoPE video diffusion transformers, on AMD Instinct MI355X
 * (gfx950).
 *
 * The operation (page: "RotateAttention: RoPE-Aware Rotation and Range
 * Rectification for INT4 Quantized Attention in Video Generation",
 * pith.science review of arXiv 2607.02584):
 *   1. 3D RoPE over frame / height / width head-dim segments (Sec. 3, Fig. 2);
 *   2. a RoPE-aware 2x2 orthogonal rotation of Q and K: Interleaved (merged
 *      into the RoPE angles) or Half (dim i with dim i + L/2 inside each
 *      segment of length L, H2 blocks) (Sec. 4.1, Fig. 3);
 *   3. symmetric INT4 Q and K per (batch, head, 64-token block), symmetric
 *      INT4 V per (batch, head, channel) (abstract);
 *   4. online-softmax attention over 64-key steps, with the normalised P
 *      mapped onto the whole signed INT4 range, code = round(15 p) - 8
 *      (Sec. 4.2), and INT4 P x V;
 *   5. a bf16 full-precision path for the accuracy-sensitive denoising steps
 *      and DiT blocks (Sec. 5.1), selected per call.
 *
 * Conventions
 *   * q, k, v, o are device pointers to [B, N, H, D] tensors, contiguous,
 *     D fastest; N = F * H_grid * W tokens in (f, h, w) row-major order
 *     (w fastest).  Input dtype bf16 or f32; output dtype f32 or bf16.
 *   * All device pointers must be 16-byte aligned.
 *   * The caller owns q, k, v, o and the workspace; the library never frees
 *     them.  A plan owns only its tables: the RoPE cos/sin tables and the
 *     byte table of the P map (host copy, plus one small device copy per
 *     GPU, made by ra_plan_create on the device current then and by
 *     ra_plan_upload on any other).  The forward entry points
 *     (ra_attn_fwd, ra_attn_prologue, ra_attn_main, ra_attn_fwd_simple once
 *     its plan exists) allocate nothing and never synchronise with the
 *     host, so they may be captured into a HIP graph.
 *   * Every entry point validates its arguments before enqueueing anything and
 *     returns a status; on failure nothing is enqueued and
 *     ra_last_error_message() (thread-local) says why.  Work is enqueued
 *     asynchronously on `stream`; a device fault surfaces at the caller's
 *     next synchronisation.
 *   * A plan may be used from several threads / streams at once as long as
 *     each call has its own workspace.
 */
#ifndef RA_ATTN_H
#define RA_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RA_OK = 0,
  RA_ERR_INVALID_ARG = 1,   /* null pointer, bad enum, bad index */
  RA_ERR_SHAPE = 2,         /* non-positive or too large batch/heads/grid */
  RA_ERR_SEGMENTS = 3,      /* segments not even, not positive, or not summing to D */
  RA_ERR_DTYPE = 4,         /* unsupported input/output dtype */
  RA_ERR_ALIGNMENT = 5,     /* a device pointer is not 16-byte aligned */
  RA_ERR_WORKSPACE = 6,     /* workspace missing or smaller than required */
  RA_ERR_UNSUPPORTED = 7,   /* valid request this build does not implement */
  RA_ERR_OOM = 8,           /* device allocation of plan tables failed */
  RA_ERR_HIP = 9            /* a HIP runtime call or kernel launch failed */
} ra_status;

/* Rotation of Q and K after RoPE (RotateAttention review, Sec. 4.1 / Fig. 3
 * and Figs. 4-6): NONE; INTERLEAVED, R(pi/4) on each RoPE pair, merged into
 * the RoPE angles; HALF, H2 on (x_i, x_{i+L/2}) within each segment; FULL,
 * the dense comparator of Figs. 4-6 that rotates all D dimensions at once,
 * here the orthonormal Walsh-Hadamard matrix (binary32 butterflies h = 1, 2,
 * ..., D/2, then x f32(1/sqrt(D))) applied to the whole RoPE'd head row.
 * The bf16 path applies none of them. */
typedef enum { RA_ROT_NONE = 0, RA_ROT_INTERLEAVED = 1, RA_ROT_HALF = 2, RA_ROT_FULL = 3 } ra_rot;
typedef enum { RA_PREC_INT4 = 0, RA_PREC_BF16 = 1 } ra_prec;
typedef enum { RA_DT_F32 = 0, RA_DT_BF16 = 1 } ra_dtype;

/* Problem shape.  head_dim in {64, 128}; seg = (frame, height, width) even,
 * positive, summing to head_dim. */
typedef struct {
  int32_t batch, heads, head_dim;
  int32_t grid_f, grid_h, grid_w;
  int32_t seg[3];
} ra_shape;

/* Options.  rope_theta: RoPE base (10000 in the pages' models; > 0).
 * softmax_scale: 0 selects 1/sqrt(head_dim).  p_mode selects the INT4 map of
 * the attention probabilities p in [0, 1] (Sec. 4.2): 0 = range-optimized
 * (default; code = round(15 p) - 8, the full signed range [-8, 7]), 1 =
 * symmetric quantization, the baseline the pages improve on (code = round(7 p)
 * in [0, 7], half of the codes unused); other values return
 * RA_ERR_INVALID_ARG.  The bf16 path ignores it.
 * v_hadamard = 1 applies the V-side Hadamard of the pages (a standard
 * Hadamard transform fused into V; RotateAttention review, summary): each V
 * row is multiplied by H = H_D / sqrt(D) (Walsh-Hadamard, Sylvester order;
 * binary32 butterflies h = 1, 2, ..., D/2, then x f32(1/sqrt(D))) before its
 * per-channel INT4 quantization, and each output row by H again (H = H^-1),
 * so o is still attention(Q, K, V).  The V codes and scales reported by
 * ra_debug_prologue are then those of V H.  Default 0; values other than 0
 * and 1 return RA_ERR_INVALID_ARG; the bf16 path ignores it. */
typedef struct {
  int32_t rot;        /* ra_rot */
  int32_t prec;       /* ra_prec */
  int32_t in_dtype;   /* ra_dtype of q, k, v */
  int32_t out_dtype;  /* ra_dtype of o */
  double rope_theta;
  double softmax_scale;
  int32_t p_mode;
  int32_t v_hadamard; /* 0 or 1, see above */
} ra_opts;

typedef struct ra_plan_s* ra_plan;

/* Fill *opts with defaults: Half rotation, INT4, bf16 in, f32 out,
 * theta 10000, scale 1/sqrt(D), range-optimized P. */
ra_status ra_opts_default(ra_opts* opts);

/* Validate shape/opts, build the RoPE cos/sin tables on the host (binary64
 * angles, +pi/4 per pair for the merged Interleaved rotation, rounded to
 * binary32), the P map's thresholds (Sec. 4.2) and the byte table the INT4
 * kernels look the P codes up in, and, when a GPU is present, copy the
 * tables to the current device (one small allocation and
 * a synchronous copy; RA_ERR_OOM / RA_ERR_HIP if that fails, and then no
 * plan is returned).  *out receives a plan to be destroyed with
 * ra_plan_destroy. */
ra_status ra_plan_create(const ra_shape* shape, const ra_opts* opts, ra_plan* out);

/* Copy the plan's tables to the current device if they are not there yet
 * (allocates and synchronises; call it before using the plan on a device
 * other than the one current at ra_plan_create). */
ra_status ra_plan_upload(ra_plan plan);

/* Release the plan and its device table copies.  Null is accepted. */
ra_status ra_plan_destroy(ra_plan plan);

/* Workspace bytes one ra_attn_fwd call of this plan needs (the INT4 codes
 * of Q/K/V in the matrix-instruction operand format fp6 e2m3, 6 bits per
 * code, in 64-token tiles: 48 * D bytes per tile of each of Q, K and V; the
 * scales; or the bf16 copies for the bf16 path). */
ra_status ra_plan_workspace_size(ra_plan plan, size_t* bytes);

/* Same figure without a plan. */
ra_status ra_workspace_size(const ra_shape* shape, const ra_opts* opts, size_t* bytes);

/* o = attention(q, k, v) for the plan's shape and options; enqueue only (no
 * allocation, no host synchronisation).  Equivalent to ra_attn_prologue
 * followed by ra_attn_main on the same workspace.  RA_ERR_INVALID_ARG if the
 * plan's tables are not on the current device (see ra_plan_upload). */
ra_status ra_attn_fwd(ra_plan plan, const void* q, const void* k, const void* v, void* o,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of the device-resident workspace of ra_attn_fwd_noalloc (one copy
 * per GPU, held until the process ends). */
#define RA_NOALLOC_WORKSPACE_BYTES (64u << 20)

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): ra_attn_fwd with the
 * workspace taken from a fixed device-resident array of
 * RA_NOALLOC_WORKSPACE_BYTES per GPU instead of a caller buffer.  Same
 * kernels and results as ra_attn_fwd.  The caller still passes q, k, v and
 * o.  A plan whose workspace (ra_plan_workspace_size) exceeds
 * RA_NOALLOC_WORKSPACE_BYTES returns RA_ERR_WORKSPACE and enqueues nothing.
 * Allocates nothing; the first call on a device without a plan created
 * there looks the array's address up (no allocation).  Every call on one
 * GPU shares that GPU's array, which keeps the last call's contents: calls
 * that overlap on one GPU (other streams, other threads) race and must be
 * ordered by the caller.  Enqueue only. */
ra_status ra_attn_fwd_noalloc(ra_plan plan, const void* q, const void* k, const void* v, void* o,
                              hipStream_t stream);

/* Stage 1: RoPE + rotation + quantization (INT4) or RoPE + bf16 conversion
 * (bf16 path) of q, k, v into the workspace. */
ra_status ra_attn_prologue(ra_plan plan, const void* q, const void* k, const void* v,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Stage 2: the attention kernel on a workspace filled by stage 1. */
ra_status ra_attn_main(ra_plan plan, void* o, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* One-shot form: builds (and caches, under a mutex) a plan for these
 * arguments with theta 10000 and scale 1/sqrt(D), then runs ra_attn_fwd.
 * The first call with new arguments creates the plan (and so allocates and
 * synchronises once); later calls with the same arguments do not. */
ra_status ra_attn_fwd_simple(const void* q, const void* k, const void* v, void* o,
                             int32_t batch, int32_t heads, int32_t head_dim,
                             int32_t grid_f, int32_t grid_h, int32_t grid_w,
                             int32_t seg_f, int32_t seg_h, int32_t seg_w,
                             int32_t rot, int32_t prec, int32_t in_dtype, int32_t out_dtype,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Mixed-precision schedule (Sec. 5.1): full precision on the first
 * steps_head / last steps_tail sampling steps and on the first blocks_head /
 * last blocks_tail DiT blocks (either condition), INT4 elsewhere. */
typedef struct { int32_t steps_head, steps_tail, blocks_head, blocks_tail; } ra_schedule;
ra_prec ra_schedule_pick(const ra_schedule* sched, int32_t step, int32_t n_steps,
                         int32_t block, int32_t n_blocks);

const char* ra_status_str(ra_status status);
const char* ra_last_error_message(void);

/* The P map's thresholds (Sec. 4.2: u = round(P p), p = 2^d, rounded
 * half up; P = 15 for p_mode 0, 7 for p_mode 1): T[k], k = 0..P-1, the
 * smallest binary32 d with P 2^d >= k + 1/2, so that u = #{k : d >= T[k]}.
 * T (host) receives P floats.  p_mode outside {0, 1} or a null T returns
 * RA_ERR_INVALID_ARG.  Host only. */
ra_status ra_pmap_thresholds(int32_t p_mode, float* T);

/* The byte table the INT4 kernels look P codes up in (the one plans
 * upload), for p_mode 0 or 1: `bytes` must be at least
 * RA_PMAP_TABLE_BYTES.  Entry a (a = 0 .. 20111) is for the exponent cell
 * j = top - a, cells of width 2^-12 in x = -d (x rounded as rint(4096 x),
 * ties to even), and holds the fp8 e4m3 byte of u when every x of the cell
 * has the same u = #{k : x <= -T[k]}, or 0x80 | k when the cell holds
 * -T[k] and values above it; entries past top are 0.  Behind the entries,
 * at byte 20112, 16 records of 8 bytes: record k < P holds -T[k] / 8
 * (binary32) and the e4m3 bytes of k and k + 1; records k >= P are zero.
 * *top receives top.
 * Null arguments, a short buffer or p_mode outside {0, 1} return
 * RA_ERR_INVALID_ARG.  Host only. */
#define RA_PMAP_TABLE_BYTES 20240
ra_status ra_pmap_table(int32_t p_mode, uint8_t* out, size_t bytes, int32_t* top);

/* ---- parity / diagnostics exports (synchronous, test use) ---------------- */

/* Run stage 1 of an INT4 plan into `workspace`, wait for it, and copy the
 * quantized tensors to host buffers in plain layouts: codes [B, H, N, D] int8
 * (q, k, v), s_q and s_k [B, H, ceil(N/64)], s_v [B, H, D]. */
ra_status ra_debug_prologue(ra_plan plan, const void* q, const void* k, const void* v,
                            void* workspace, size_t workspace_bytes,
                            int8_t* q_codes, float* s_q, int8_t* k_codes, float* s_k,
                            int8_t* v_codes, float* s_v, hipStream_t stream);

/* On a workspace already filled by stage 1 of an INT4 plan, run the attention
 * step code for the 64 queries of Q block q_blk of head (b, h) up to key step
 * kv_blk and copy that step's exact integers to host buffers:
 * s_int [64, 64] (query, key) scores, p_codes [64, 64] P codes in [-8, 7]
 * (-8 for keys past N; [0, 7] and 0 for p_mode 1), pv_int [64, D] =
 * sum_j code * vhat, m_after [64] the running max (log2 units, binary32)
 * after the step.  Rows past N are unspecified. */
ra_status ra_debug_tile(ra_plan plan, void* workspace, size_t workspace_bytes,
                        int32_t b, int32_t h, int32_t q_blk, int32_t kv_blk,
                        int32_t* s_int, int8_t* p_codes, int32_t* pv_int, float* m_after,
                        hipStream_t stream);

/* Evaluate the attention kernels' P map of mode p_mode (see ra_opts) --
 * their table lookup, exact decision of the table cells that hold a
 * rounding boundary, and operand packing -- on n exponents d (device, f32,
 * d = log2 p <= 0) -> u (device, u8): u = round(15 2^d) = code + 8 for
 * p_mode 0, u = round(7 2^d) = code for p_mode 1.  p_mode outside {0, 1}
 * returns RA_ERR_INVALID_ARG.  The table is the one plans upload; its
 * first use per device and mode allocates and copies it synchronously
 * (kept until the process ends); later calls only enqueue. */
ra_status ra_debug_pmap(const float* d, uint8_t* u, int64_t n, int32_t p_mode, hipStream_t stream);

/* Stage 2 of an INT4 plan with f32 output (workspace filled by stage 1), run
 * by the parity variant of the attention kernel: the same kernel, launch
 * shape, LDS pipeline and step order, which also writes for every query row
 * r = (b * H + h) * N + n, into rows[4 r .. 4 r + 3] (device, uint32, 16-byte
 * aligned, B * H * N * 4 entries): the bits of the final running max (log2
 * units), the sum over all keys of u = code + zero-point, the sum of
 * u * (2654435761 (j + 1) mod 2^32) mod 2^32 over keys j, and the bits of
 * the row's final binary32 sum of u (rescaled, as the kernel keeps it).  o
 * receives the output as ra_attn_main would.  Enqueue only; for tests. */
ra_status ra_debug_row_digests(ra_plan plan, void* o, void* workspace, size_t workspace_bytes,
                               uint32_t* rows, hipStream_t stream);

/* Host copy of the plan's binary32 RoPE table of segment `seg` (0 frame,
 * 1 height, 2 width): cos and sin, each [positions, seg_len/2]. */
ra_status ra_debug_tables(ra_plan plan, int32_t seg, float* cos_out, float* sin_out);

/* Plain device-to-device copy kernel (bandwidth reference).  Enqueue only. */
ra_status ra_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);

/* Matrix-core throughput probe: a measurement helper beside the attention
 * path, used to state the sustained MFMA rate and the engine clock it is
 * reached at next to the published peaks.  kind: 0 INT8 (32x32x32 i8),
 * 1 fp8 x fp8, 2 fp6 x fp6, 3 fp6 A x fp8 B (32x32x64 f8f6f4), 4 bf16
 * (32x32x16).  Launches `blocks` workgroups of 4 waves; each wave issues
 * iters x 4 independent MFMAs of that kind.  clk (device, 4 x uint64_t)
 * receives, from wave 0 of workgroup 0, the shader cycle counter at its
 * start and end, then the 100 MHz real-time counter at its start and end.
 * sink (device, 1 float) keeps the results live and is not written for
 * these operands.  *ops_out (host) receives the operations of one launch
 * (2 per multiply-add).  Unknown kind, iters < 1 or blocks < 1 return
 * RA_ERR_INVALID_ARG.  Enqueue only. */
ra_status ra_bench_mfma_peak(int32_t kind, int32_t iters, int32_t blocks, float* sink, uint64_t* clk,
                             double* ops_out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RA_ATTN_H */
