/*
 * flux_attn.h - C ABI of the MI355X (gfx950) joint RoPE attention library.
 *
 * The operation.  One call computes, for every batch b and head h, the
 * non-causal softmax attention of the whole joint token sequence
 *
 *     O[b,i,h,:] = sum_j softmax_j( scale * <R(pos_i) Q[b,i,h,:], R(pos_j) K[b,j,h,:]> ) V[b,j,h,:]
 *
 * where R(p) is the multi-axis rotary position embedding of token position
 * p = (p0, p1, p2).  Sources:
 *   - "Welcome FLUX.3 Image Klein in Diffusers", Architecture section
 *     ("Two-Stage Processing"): text, noisy-image and reference tokens are
 *     concatenated and attend jointly in the joint blocks;
 *   - "FLUX.3 Image Klein Brings 2-Second AI Image Generation to Diffusers",
 *     Summary: five separate-stream blocks before 28 joint blocks (the
 *     segment-local entry point below is the separate-stream attention);
 *   - "Optimizing FLUX 3 Image Klein inference on NVIDIA Blackwell GPUs",
 *     "How it works": rotary position embeddings, and attention with query,
 *     key and value in FP8.
 * Conventions where the pages are silent: scale = 1/sqrt(head_dim); RoPE pairs
 * are adjacent elements (2j, 2j+1) inside each axis slice; head_dim is cut into
 * three slices of widths rope_axes_dim[0..2]; pair j of a slice of width d is
 * rotated by pos_axis * theta^(-2j/d); V is not rotated.  Precision: the
 * angles are formed in double; the kernels rotate in fp32 with cos and sin
 * rounded to fp16 (each within 2^-12), round the rotated Q (times scale *
 * log2 e) and K to bf16 (e4m3 for FP8 plans), accumulate in fp32 and round P
 * and the output to bf16.
 *
 * Layouts (all row-major, contiguous):
 *   q, k, v, out   [batch][tokens][num_heads][head_dim]
 *   pos_ids        [tokens][3] int32, shared by every batch entry
 *   qkv_scale      [3][batch][num_heads] float (FP8 only: q, k, v scales)
 *
 * Errors.  Every function returns a status code (flux_attn_status).  No C++
 * exception crosses this boundary.  forward() checks all arguments on the host
 * before any device work; on error nothing is launched and a thread-local
 * message is available from flux_attn_last_error().
 */
#ifndef FLUX_ATTN_H
#define FLUX_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FLUX_ATTN_ABI_VERSION 2

typedef enum {
  FLUX_ATTN_OK = 0,
  FLUX_ATTN_INVALID_ARGUMENT = 1, /* a pointer, size or shape is wrong */
  FLUX_ATTN_UNSUPPORTED = 2,      /* valid request that the library does not run */
  FLUX_ATTN_DEVICE_ERROR = 3,     /* a HIP runtime call failed */
  FLUX_ATTN_OUT_OF_MEMORY = 4     /* device allocation in create() failed */
} flux_attn_status;

typedef enum {
  FLUX_ATTN_BF16 = 0,     /* q, k, v are bfloat16 */
  FLUX_ATTN_FP8_E4M3 = 1  /* q, k, v are OCP e4m3 ("e4m3fn") codes + per-head scales */
} flux_attn_dtype;

typedef struct {
  int32_t batch;            /* >= 1 */
  int32_t num_heads;        /* >= 1 */
  int32_t head_dim;         /* 64 or 128 */
  int32_t max_tokens;       /* capacity: largest token count forward() will see;
                               one batch entry of q, k or v (max_tokens x num_heads
                               x head_dim elements) must stay under 4 GiB
                               (FLUX_ATTN_UNSUPPORTED otherwise): the kernels
                               address it through 32-bit buffer ranges */
  int32_t max_segments;     /* capacity of the segment list, >= 1 */
  int32_t rope_axes_dim[3]; /* even, multiples of 8, sum == head_dim */
  float rope_theta;         /* > 0, e.g. 10000 */
  float softmax_scale;      /* <= 0 selects 1/sqrt(head_dim) */
  int32_t dtype;            /* flux_attn_dtype */
} flux_attn_config;

typedef struct flux_attn_plan flux_attn_plan; /* opaque; owned by the library */

/* Fills *cfg with the defaults for (batch, num_heads, head_dim, max_tokens):
 * axes (D/4, 3D/8, 3D/8), theta 10000, scale 1/sqrt(D), bf16, 12 segments
 * (text + image + up to 10 references).  Host only; no device call. */
int flux_attn_default_config(flux_attn_config* cfg, int32_t batch, int32_t num_heads,
                             int32_t head_dim, int32_t max_tokens);

/* Checks a configuration without touching a device.  Host only. */
int flux_attn_validate_config(const flux_attn_config* cfg);

/* Checks the host-side arguments of a forward call (joint or segment-local:
 * both take the same arguments) against cfg without touching a device: segment
 * list (each >= 0, sum N with 1 <= N <= max_tokens, count <= max_segments),
 * non-null and 16-byte aligned tensors, out not overlapping q/k/v (by address
 * range), scales present iff FP8.  Host only. */
int flux_attn_validate_forward(const flux_attn_config* cfg, const void* q, const void* k,
                               const void* v, const float* qkv_scale,
                               const int32_t* segment_tokens, int32_t num_segments,
                               const int32_t* pos_ids, const void* out);

/* Creates a plan on the current HIP device: validates cfg and allocates the
 * plan's device workspace once (RoPE table of max_tokens x head_dim/2 x 8 bytes,
 * split-K/V partials; for bf16 plans also the tile-sparse tile means and
 * kept-tile lists, and the backward's row sums and rotated copies of q and k:
 * 2 x batch x max_tokens x num_heads x head_dim bf16).  *out receives the plan, or
 * NULL on error.  The environment variable FLUX_ATTN_SCHEDULE, read here,
 * overrides how the plan's dense bf16 launches split their work: "split" (whole
 * tiles plus K/V pieces of the last round) or "persistent" (one workgroup per
 * compute unit over equal slices); unset, the plan chooses by its cost model.
 * Results agree to rounding under every choice. */
int flux_attn_create(const flux_attn_config* cfg, flux_attn_plan** out);

/* Runs joint RoPE attention asynchronously on hip_stream (a hipStream_t; NULL
 * = the null stream): every token attends to all N tokens of the concatenated
 * sequence (the joint blocks).  q, k, v, out, pos_ids and qkv_scale are
 * device pointers owned by the caller and must stay valid until the stream
 * has passed this work; segment_tokens is a host array read before the call
 * returns.  N = sum(segment_tokens); the segment counts define N and are
 * validated, they do not change the arithmetic.  out is fully overwritten.
 * A plan runs one forward at a time (its workspace is shared between calls);
 * separate plans are independent.  Returns after launching. */
int flux_attn_forward(flux_attn_plan* plan, const void* q, const void* k, const void* v,
                      const float* qkv_scale, const int32_t* segment_tokens,
                      int32_t num_segments, const int32_t* pos_ids, void* out,
                      void* hip_stream);

/* Segment-local attention, same arguments and rules as flux_attn_forward: a
 * token of segment s attends only to the tokens of segment s, i.e. the formula
 * above with j restricted to the segment ("FLUX.3 Image Klein Brings 2-Second
 * AI Image Generation to Diffusers", Summary: the separate-stream blocks before
 * the joint ones).  The RoPE angles still come from the tokens' own position
 * ids, and empty segments are skipped. */
int flux_attn_forward_segment_local(flux_attn_plan* plan, const void* q, const void* k, const void* v,
                                    const float* qkv_scale, const int32_t* segment_tokens,
                                    int32_t num_segments, const int32_t* pos_ids, void* out,
                                    void* hip_stream);

/* Allocation-free joint forward, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  The same computation and arguments as flux_attn_forward,
 * without a plan: cfg (host) is validated as flux_attn_create does, and its
 * max_tokens only bounds N.  The RoPE table and the split partials live in a
 * static device array of FLUX_ATTN_NOALLOC_SCRATCH_BYTES (32 MiB) that every
 * device holds from the library's load until the process ends; the first call
 * on a device looks up its address there.  No call allocates host or device
 * memory.  Limit: the table, N x head_dim x 2 bytes, must fit in the array
 * (N <= 131,072 at head_dim 128, 262,144 at 64), FLUX_ATTN_UNSUPPORTED
 * otherwise; the rest of the array bounds how finely the last round of query
 * tiles is split, so results agree with flux_attn_forward to rounding, not
 * always bitwise.  Nothing is read from an earlier call.  All calls on one
 * device share its array: calls on one stream are ordered and safe, calls
 * that overlap on one device (several streams or threads) race and give wrong
 * results.  Not timed (no events). */
#define FLUX_ATTN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int flux_attn_forward_noalloc(const flux_attn_config* cfg, const void* q, const void* k, const void* v,
                              const float* qkv_scale, const int32_t* segment_tokens, int32_t num_segments,
                              const int32_t* pos_ids, void* out, void* hip_stream);

/* Training: forward with the per-row log-sum-exp, and the backward.  The
 * attention backward is the adjacent training workload (LoRA fine-tuning of
 * the base model, "FLUX.3 Image Klein Brings 2-Second AI Image Generation to
 * Diffusers", Summary); the pages give no formula, so these are the gradients
 * of the operation above.  Both need a bf16 plan (FLUX_ATTN_UNSUPPORTED
 * otherwise) and run joint attention over the whole sequence, asynchronously
 * on hip_stream, one call at a time per plan.
 *
 * flux_attn_forward_lse: forward() (joint) that also writes
 *   lse[b][h][i] = log sum_j exp(scale * <R(p_i) q_i, R(p_j) k_j>)
 * (natural log, fp32, device [batch][num_heads][N]).
 *
 * flux_attn_backward: given q, k, v, the forward's out and lse, and the
 * upstream gradient dout (all device, layouts as forward), writes dq, dk, dv
 * (device [batch][N][num_heads][head_dim] bf16, fully overwritten) with
 *   P = softmax rows of scale * S,  dV = P^T dO,  dS = P * (dO V^T - rowsum(dO * O)),
 *   dq = R^T (scale dS K~),  dk = R^T (scale dS^T Q~)
 * where Q~ = R q, K~ = R k and R^T rotates back by the negative angle.  The
 * gradients must not overlap any input or each other.  Timing pairs (see
 * below) bracket the backward kernels. */
int flux_attn_forward_lse(flux_attn_plan* plan, const void* q, const void* k, const void* v,
                          const int32_t* segment_tokens, int32_t num_segments, const int32_t* pos_ids, void* out,
                          float* lse, void* hip_stream);
int flux_attn_backward(flux_attn_plan* plan, const void* q, const void* k, const void* v, const void* out,
                       const void* dout, const float* lse, const int32_t* segment_tokens, int32_t num_segments,
                       const int32_t* pos_ids, void* dq, void* dk, void* dv, void* hip_stream);

/* Tile-sparse attention: skipping the work for less important token pairs by
 * a sparsity threshold tau ("Optimizing FLUX 3 Image Klein inference on NVIDIA
 * Blackwell GPUs", How it works; What you can do: tau).  The granularity and
 * importance measure are this library's reading of that passage:
 *   query tiles of 256 tokens x key tiles of 64 tokens of the joint sequence,
 *   QT = ceil(N / 256), KT = ceil(N / 64) (last tiles may be partial);
 *   mask: device uint8 [batch][num_heads][QT][KT], nonzero = the query tile
 *   attends to the key tile.
 * Both calls need a bf16 plan (FLUX_ATTN_UNSUPPORTED otherwise), take q, k, v,
 * segment_tokens and pos_ids as forward() does (joint sequence), run
 * asynchronously on hip_stream and share the plan's workspace (one call at a
 * time per plan). */

/* Writes the mask of the score-bound rule (scores s_ij = scale * log2(e) *
 * <R(p_i) q_i, R(p_j) k_j>, exp2 domain, from the same bf16 operands and
 * fp32 accumulation as the attention kernel): with L_i the largest score of
 * query i over the 4 key tiles aligned with its query tile (a lower bound of
 * its row maximum m_i), key tile t is kept for query tile Q when
 *     max over i in Q of ( max over j in t of s_ij  -  L_i )  >=  log2(tau),
 * 0 < tau <= 1.  Every skipped pair then has weight 2^(s_ij - m_i) < tau
 * relative to its row's largest, and the output moves from dense attention by
 * at most delta_i (max_j V[j,d] - min_j V[j,d]) per element, delta_i (the
 * dense softmax mass of row i's skipped keys) being below tau times the
 * number of skipped keys.  Its cost is one pass of Q K^T over all tiles.
 * N <= 131,072 (FLUX_ATTN_UNSUPPORTED beyond).  mask is written in full. */
int flux_attn_block_mask(flux_attn_plan* plan, const void* q, const void* k, const int32_t* segment_tokens,
                         int32_t num_segments, const int32_t* pos_ids, float tau, uint8_t* mask,
                         void* hip_stream);

/* Alternative rule without that guarantee, cheaper (tile means only): the
 * pooled score of a tile pair is scale * log2(e) * <mean over the query tile
 * of R(p_i) q_i, mean over the key tile of R(p_j) k_j> (fp32); a key tile is
 * kept when its pooled score is at least the query tile's largest plus
 * log2(tau), 0 < tau <= 1, so the largest is always kept.  mask is written in
 * full. */
int flux_attn_block_mask_pooled(flux_attn_plan* plan, const void* q, const void* k,
                                const int32_t* segment_tokens, int32_t num_segments, const int32_t* pos_ids,
                                float tau, uint8_t* mask, void* hip_stream);

/* Attention of each query over the keys of its query tile's kept key tiles:
 * the exact softmax over those keys (the others are left out); a query tile
 * that keeps no key tile gets 0.  mask may come from flux_attn_block_mask or
 * from the caller.  out is fully overwritten.  Timing pairs are recorded as
 * for forward(). */
int flux_attn_forward_sparse(flux_attn_plan* plan, const void* q, const void* k, const void* v,
                             const int32_t* segment_tokens, int32_t num_segments, const int32_t* pos_ids,
                             const uint8_t* mask, void* out, void* hip_stream);

/* Kernel timing.  flux_attn_timing_enable(plan, capacity) with capacity > 0
 * creates capacity triples of HIP events (capacity <= 4096) and a 16-byte
 * device counter; every following forward call records one triple (none once
 * all are used), on the stream its kernels run on: before the attention
 * kernel, after it, and after the exact merge of its split pieces (if any).
 * For segment-local calls the first two span the attention kernels of all
 * segments (the small merge kernels between them included).  The timed
 * attention kernels also add each workgroup's shader-clock cycles and
 * constant-rate wall-clock ticks to the counter.  capacity = 0 releases all.
 * flux_attn_timing_read() waits for the last recorded triple, writes the
 * durations in milliseconds of up to max_count recorded calls to host arrays:
 * attn_ms[i] (attention kernel) and, if total_ms is not NULL, total_ms[i]
 * (attention kernel plus merge); if clock_mhz is not NULL, the average shader
 * clock (MHz) the timed attention kernels' workgroups ran at (0 if none ran);
 * then starts over.  The caller must not read while another thread runs
 * forward calls on the plan. */
int flux_attn_timing_enable(flux_attn_plan* plan, int32_t capacity);
int flux_attn_timing_read(flux_attn_plan* plan, float* attn_ms, float* total_ms, double* clock_mhz,
                          int32_t max_count, int32_t* count);

/* Work split chosen by forward() for a launch (host only, no device call).
 * The kernel runs one 256-row query tile of one (batch, head) per workgroup,
 * one workgroup per compute unit.  Of `tiles` tiles, *whole_tiles run over all
 * kv_tiles 64-key tiles; the remaining *split_tiles are each cut into *split
 * key/value ranges whose fp32 partial softmax states are merged exactly, so
 * that the last round of workgroups fills num_cus units.  At most max_pieces
 * ranges are used.  *grid = *whole_tiles + *split_tiles * *split. */
int flux_attn_schedule(int32_t tiles, int32_t kv_tiles, int32_t num_cus, int32_t max_pieces,
                       int32_t head_dim, int32_t* whole_tiles, int32_t* split_tiles,
                       int32_t* split, int32_t* grid);

/* Copies the plan's configuration into *cfg. */
int flux_attn_get_config(const flux_attn_plan* plan, flux_attn_config* cfg);

/* Frees the plan and its workspace.  No work may be pending on it.
 * NULL is accepted and ignored. */
int flux_attn_destroy(flux_attn_plan* plan);

/* Static description of a status code. */
const char* flux_attn_status_string(int status);

/* Detail of the last error on the calling thread ("" if none). */
const char* flux_attn_last_error(void);

/* ABI version of the loaded library (FLUX_ATTN_ABI_VERSION). */
int flux_attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FLUX_ATTN_H */
