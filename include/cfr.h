/*
 * cfr.h — C ABI of the calibration-free MoE channel-selection reader for
 * AMD Instinct MI355X (gfx950).
 *
 * The reader replaces the routed-expert gated-MLP block of one MoE layer at
 * small-batch decode.  Per token it (1) rotates x by a block-128 randomized
 * Hadamard matrix and keeps, per block, the n_screen coordinates of largest
 * |Rx|; (2) estimates every candidate channel's gate/up activations from a
 * packed ternary sketch of the rotated rows, read only at those coordinates;
 * (3) scores channels in output units, s_j = w_j ||d_j|| |phi(g_hat_j) v_hat_j|,
 * and keeps exactly the top k across all routed experts; (4) computes kept
 * channels exactly from native BF16 rows and adds a rank-`rank` recovery term
 * U sum_{skipped} w_j b_j p_j.
 *
 * Sources (cited by page title and section):
 *   [zh §S] Chinese summary page of "Channel Selection for Mixture-of-Experts
 *           Decoding Needs No Calibration Data" (paper.rainbus.top), section S.
 *   [ko §S] Korean summary page of the same paper, "MoE 채널 선택은
 *           캘리브레이션 없이 top-k로 충분하다" (onedev.kr), section S.
 *
 * Conventions for every call:
 *   - Return 0 (CFR_OK) on success or a negative CFR_E* code; a thread-local
 *     message is then available from cfr_last_error().  No C++ exception
 *     crosses this boundary.
 *   - "host" pointers are ordinary CPU memory; "device" pointers are HIP
 *     device memory on the reader's device (for example a torch tensor's
 *     data_ptr()).  The caller owns every pointer it passes; the library
 *     owns the reader and all memory inside it.
 *   - Decode-time calls enqueue work on the caller's HIP stream (`stream`,
 *     a hipStream_t; NULL = the null stream), never synchronise the host
 *     and never allocate.  Calls that share a reader must be ordered on one
 *     stream: the reader's workspace is reused by every call.
 */
#ifndef CFR_H
#define CFR_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CFR_OK 0
#define CFR_EINVAL (-1)        /* bad argument (pointer, size, range)            */
#define CFR_ENOMEM (-2)        /* host or device allocation failed               */
#define CFR_EHIP (-3)          /* a HIP runtime call failed                      */
#define CFR_EUNSUPPORTED (-4)  /* shape outside what the kernels support         */
#define CFR_ESOLVER (-5)       /* the load-time eigensolver failed               */

typedef struct cfr_reader cfr_reader; /* opaque; owned by the library */

/* Layer shape and method constants, fixed at build time. */
typedef struct cfr_config {
  int32_t hidden;     /* H: model width, a multiple of 128, at most 4096              */
  int32_t n_experts;  /* E: experts in the layer                                        */
  int32_t inter;      /* I: channels per expert (expert intermediate size), 1..4096     */
  int32_t top;        /* routed experts per token, 1..16 and <= E                       */
  int32_t rank;       /* recovery rank, 0..64, a multiple of 8 (the pages use 32)       */
  int32_t n_screen;   /* coordinates screened per 128-block, 1..128 (the pages use 80) */
  int32_t max_batch;  /* largest batch a decode call may pass, 1..64                    */
  int32_t device;     /* HIP device ordinal the reader lives on                         */
  uint64_t rot_seed;  /* SplitMix64 seed of the rotation's sign vector                 */
  int32_t ranking;    /* how candidates are ranked ([zh §方法步骤详情] decode step (2)):
                       *   CFR_RANK_SCORE: output-unit score s_j = w_j ||d_j||
                       *     |phi(g_hat_j) v_hat_j| (the low budgets, 12.8% and
                       *     17.8%, with the partial screen);
                       *   CFR_RANK_EXPECTED_ERROR: the whole sketch is read
                       *     (n_screen must be 128) and candidates are ranked by
                       *     e_j = w_j ||d_j|| sqrt(p_j^2 + Var[a_j]), the root
                       *     of the expected squared output error of skipping j,
                       *     with Var[a_j] from the stored rho_b and the block
                       *     norms of x (budgets from 28.7% on).                  */
  int32_t exact_bits; /* format of the resident exact rows: 16 (or 0) for the native
                       * BF16 rows given to cfr_build_reader; 4 for a 4-bit
                       * checkpoint given to cfr_build_reader_q4 (the pages run the
                       * reader over a GPTQ 4-bit checkpoint, [zh §独立分析的弱点]
                       * item (2)); 4-bit readers rank by the output-unit score.  */
} cfr_config;

#define CFR_RANK_SCORE 0
#define CFR_RANK_EXPECTED_ERROR 1

/* Buffer sizes and layout constants implied by a config (see cfr_sizes_of()). */
typedef struct cfr_sizes {
  int32_t n_blocks;      /* H / 128                                                    */
  int32_t half_bytes;    /* Lp: bytes of one half (gate or up) of a sketch unit        */
  int32_t unit_bytes;    /* bytes of one sketch unit (one expert, block, coordinate)   */
  int32_t n_cand;        /* candidate channels per token = top * I                     */
  int64_t codes_bytes;   /* E * n_blocks * 128 * unit_bytes                            */
  int64_t scales_count;  /* E * n_blocks * 2 * I   (fp16 scales; rho has the same)     */
  int64_t norms_count;   /* E * I                  (fp32)                              */
  int64_t u_count;       /* H * rank               (fp16)                              */
  int64_t b_count;       /* E * I * rank           (fp16)                              */
  int64_t weights_bytes; /* E * I * 3 * H * 2      (native BF16 rows, resident)        */
} cfr_sizes;

/* Counted reads of one decode, in whole 32-byte sectors ([zh §前置知识 /
 * 显存带宽受限的解码]: every touched sector is charged). */
typedef struct cfr_read_stats {
  int64_t codes;   /* sketch codes of the screened coordinates                    */
  int64_t scales;  /* fp16 scales of the routed experts                            */
  int64_t norms;   /* ||d_j|| of the routed experts                                */
  int64_t rho;     /* fp16 rho_b of the routed experts (CFR_RANK_EXPECTED_ERROR)   */
  int64_t exact;   /* native gate row, up row and transposed down row, k channels */
  int64_t b;       /* recovery coefficients of the skipped channels                */
  int64_t u;       /* the recovery basis U                                         */
  int64_t total;   /* sum of the above                                             */
  int64_t dense;   /* all BF16 bytes of the routed experts (the dense block)       */
} cfr_read_stats;

/* Fill *out from *cfg.  Validates cfg.  Host only; no device work. */
int cfr_sizes_of(const cfr_config* cfg, cfr_sizes* out);

/* Counted reads per token for budget k ([zh §核心方法] read composition;
 * [zh §前置知识 / 显存带宽受限的解码]).  Host only. */
int cfr_read_bytes(const cfr_config* cfg, int32_t k, cfr_read_stats* out);

/*
 * Distinct reads of one batched decode call, in whole 32-byte sectors
 * ([zh §前置知识 / 显存带宽受限的解码]: every touched sector is charged, once):
 * the union over the batch's tokens of the sketch units of the screened
 * coordinates, the scale (and, for CFR_RANK_EXPECTED_ERROR, rho) blocks and
 * the norm rows of the routed experts, the exact rows of every channel some
 * token keeps, the b rows of every channel some token skips, and U once.
 * A sector several tokens read counts once.  `dense` is the BF16 bytes of
 * the distinct routed experts.  Inputs, host memory, as cfr_reader_decode_debug
 * returns them for the call:
 *   expert_ids int32 [batch][top]   sel uint8 [batch][H/128][n_screen]
 *   kept       int32 [batch][k]     (candidates slot * I + j; NULL if k = 0)
 * With batch = 1 and distinct ids and coordinates the result equals
 * cfr_read_bytes(cfg, k).  Host only.  CFR_EINVAL for a null pointer,
 * batch < 1, k outside 0..top*I, or an id, coordinate or candidate out of
 * range.
 */
int cfr_read_bytes_batch(const cfr_config* cfg, int32_t batch, int32_t k, const int32_t* expert_ids,
                         const uint8_t* sel, const int32_t* kept, cfr_read_stats* out);

/*
 * Bytes a batch-shared decode (cfr_reader_decode_shared) reads, counted as
 * cfr_read_bytes_batch does: the sketch units, scales and norms of the
 * batch's distinct routed experts at the coordinates any token screened,
 * the exact rows of the n_kept kept union candidates once, the b rows of
 * the other union candidates once, and U once.  ids int32 [batch][top] and
 * sel uint8 [batch][nblk][n_screen] (host memory, as for
 * cfr_read_bytes_batch); n_kept in 0 .. u * inter (u = distinct experts).
 */
int cfr_read_bytes_shared(const cfr_config* cfg, int32_t batch, const int32_t* expert_ids,
                          const uint8_t* sel, int32_t n_kept, cfr_read_stats* out);

/*
 * Load-time work for one layer ([zh §方法步骤详情] load steps (1)-(4);
 * [ko §어떻게 쓰나]):
 *   (1) rotate every gate/up row per 128-block and store TWN ternary codes,
 *       an FP16 scale and the block's mean squared quantisation error rho;
 *   (2) ||d_j|| of every down column;
 *   (3) the top-`rank` left singular vectors U of the stacked down columns
 *       of all experts (fp64 Gram + symmetric eigensolver on the device) and
 *       b_j = U^T d_j;
 *   (4) the down projection transposed, so a channel's gate row, up row and
 *       down column sit together.
 * Inputs (host, BF16 bit patterns, read only during the call):
 *   gate, up: [E][I][H]   down: [E][H][I]   router: [E][H] or NULL.
 * On success *out owns device memory for the native weights, the sketch,
 * norms, U, b, the router and a decode workspace sized for max_batch.
 * Errors: CFR_EINVAL (config/pointers, or a NaN or infinite weight),
 * CFR_EUNSUPPORTED, CFR_ENOMEM, CFR_EHIP, CFR_ESOLVER.  *out is left NULL on
 * failure.
 */
int cfr_build_reader(const cfr_config* cfg, const uint16_t* gate, const uint16_t* up,
                     const uint16_t* down, const uint16_t* router, cfr_reader** out);

/*
 * Builds a reader over a 4-bit checkpoint of the routed experts (the pages
 * run the reader over a GPTQ 4-bit checkpoint with the sketch unchanged,
 * [zh §独立分析的弱点] item (2)).  cfg->exact_bits must be 4.
 *   rows    uint8 [E][I][3][R] host, read only during the call: for each
 *           channel j of expert e its gate row g_j, up row v_j and down
 *           column d_j (over the H hidden units) as row records of
 *           R = roundup(H/2 + 3 H/128, 16) bytes: H/2 bytes of 4-bit codes
 *           (weight h in byte h/2, even h in the low nibble), then H/128
 *           fp16 group scales, then H/128 zero points (bytes, 0..15),
 *           then zero padding; weight h = scale_g (q_h - zero_g), g = h/128.
 *   router  bf16 [E][H] host or NULL, as for cfr_build_reader.
 * The sketch, the down norms and the recovery basis are built from the
 * dequantized weights (load steps (1)-(3)); the records themselves are the
 * resident exact rows, which the decode and the dense block dequantize as
 * they read them.  Errors: CFR_EINVAL for a zero point above 15 or a
 * non-finite scale, otherwise as cfr_build_reader.  The batch-shared decode
 * refuses 4-bit readers (CFR_EUNSUPPORTED).
 */
int cfr_build_reader_q4(const cfr_config* cfg, const uint8_t* rows, const uint16_t* router,
                        cfr_reader** out);

/*
 * Decode one batch ([zh §方法步骤详情] decode steps (1)-(4); [zh §核心方法];
 * [ko §어떻게 쓰나]).  All arrays are device memory:
 *   x          fp32  [batch][H]     token hidden states (not rotated)
 *   expert_ids int32 [batch][top]   routed experts, distinct per token, in [0,E)
 *   gate_w     fp32  [batch][top]   routing weight of each routed expert
 *   y          fp32  [batch][H]     output, written (not accumulated)
 * Each token keeps its own exact top-k over its top*I candidates
 * (0 <= k <= top*I; k = top*I keeps all and skips recovery; k = 0 returns the
 * recovery term alone).  Ties in any ranking go to the lower index.
 * Out-of-range expert ids are clamped into [0,E) and recorded in the
 * reader's status word (cfr_reader_status); ids are not otherwise checked.
 * Errors: CFR_EINVAL (null pointer, batch outside 1..max_batch, k outside
 * 0..top*I), CFR_EHIP (launch failure).
 */
int cfr_reader_decode(cfr_reader* r, const float* x, const int32_t* expert_ids,
                      const float* gate_w, int32_t batch, int32_t k, float* y, void* stream);

/*
 * cfr_reader_decode with the block's residual added in its last kernel:
 * y = resid + (the decode's output), in float32, the residual added to the
 * finished output (bit for bit what a separate add after cfr_reader_decode
 * gives).  resid fp32 [batch][H], device; it may be y itself (an in-place
 * residual stream x += block(RMSNorm(x))) but must not be x.  The pages'
 * reader replaces one MoE block of a transformer layer, whose output joins
 * the residual stream ([zh §前置知识 / Mixture-of-Experts (MoE)]).
 * Errors: those of cfr_reader_decode, and CFR_EINVAL if resid is NULL or x.
 */
int cfr_reader_decode_residual(cfr_reader* r, const float* x, const int32_t* expert_ids,
                               const float* gate_w, int32_t batch, int32_t k, const float* resid,
                               float* y, void* stream);

/*
 * cfr_reader_decode for callers that cannot allocate device memory during
 * the call (code under HIP graph capture, tight serving loops, harnesses
 * that forbid it): the same kernels and result, bit for bit, with the
 * decode's per-call buffers (screen sums, partial outputs) in a static
 * device array of the library, 8 MiB per device (kept until the process
 * ends), instead of the reader's workspace.  The call allocates nothing; the
 * first call on a device also clears the array with a fill kernel on
 * `stream`.  Every call on a device shares that device's array: calls that
 * overlap in time on one device (two streams, or two readers) race and
 * their outputs are unspecified; order them.  The array keeps the last
 * call's contents; the decode leaves its screen sums zero for the next call.
 * Errors: those of cfr_reader_decode, and CFR_EUNSUPPORTED when the call
 * would need more than the 8 MiB (for example batch 64 at 8192 candidates
 * per token); the message says how much it needs.
 */
int cfr_reader_decode_noalloc(cfr_reader* r, const float* x, const int32_t* expert_ids,
                              const float* gate_w, int32_t batch, int32_t k, float* y, void* stream);

/*
 * Same computation as cfr_reader_decode, also copying the intermediates to
 * the caller's device buffers (any may be NULL):
 *   xrot  fp32  [batch][H]              H_128 (sigma * x) per block, before the 1/sqrt(128)
 *   sel   uint8 [batch][H/128][n_screen] screened coordinates per block, ascending
 *   ghat, vhat, score  fp32 [batch][top*I]  candidate c = slot*I + j
 *   kept  int32 [batch][k]              kept candidates, ascending
 * For tests and measurement; not on the fast path.
 */
int cfr_reader_decode_debug(cfr_reader* r, const float* x, const int32_t* expert_ids,
                            const float* gate_w, int32_t batch, int32_t k, float* y,
                            float* xrot, uint8_t* sel, float* ghat, float* vhat,
                            float* score, int32_t* kept, void* stream);

/*
 * Batch-shared channel selection: one exact top-k for the whole batch
 * (the pages leave selecting channels jointly for the batch as the route to
 * larger-batch gains, [zh §未来方向] direction (1); [ko §전제와 한계]).
 * Candidates are the channels of the batch's distinct routed experts, union
 * candidate u * inter + j for the u-th distinct expert in ascending id
 * order; a candidate's batch score is the sum, over the (token, slot) pairs
 * routed to its expert (token-major, slot order), of the per-token score
 * w ||d_j|| |silu(g_hat_j) v_hat_j|; the k largest are kept (ties to the
 * lower union candidate).  Each kept channel's native rows are read once and
 * give the exact a_j of every token routed to its expert; each token
 * recovers its own skipped channels with its own p_j (rank-32 term).
 *   x, expert_ids, gate_w, y   as cfr_reader_decode; batch <= max_batch and
 *                              at most 8 (CFR_EUNSUPPORTED above)
 *   k        0 .. min(n_experts, batch * top) * inter; above the batch's
 *            union size u * inter every union candidate is kept
 *   bscore   fp32 [batch * top * inter] device or NULL: the batch scores of
 *            the union candidates (the first u * inter entries)
 *   kept     int32 [k] device or NULL: the kept union candidates, ascending
 *            (the first min(k, u * inter) entries)
 *   experts  int32 [1 + batch * top] device or NULL: u, then the union's
 *            experts ascending
 * Readers built for the expected-error ranking are refused
 * (CFR_EUNSUPPORTED).  Asynchronous on `stream`; allocates nothing.
 */
int cfr_reader_decode_shared(cfr_reader* r, const float* x, const int32_t* expert_ids,
                             const float* gate_w, int32_t batch, int32_t k, float* y,
                             float* bscore, int32_t* kept, int32_t* experts, void* stream);

/*
 * The experts a token activates and their weights, from the router weights
 * given at build time ([zh §前置知识 / Mixture-of-Experts (MoE)]; a channel's
 * routing weight is its expert's, [zh §核心方法]): logits = W_router u,
 * softmax over all n_experts, the `top` largest kept (ties to the lower
 * expert index) and their probabilities renormalised to sum to one.
 *   x          fp32  [batch][hidden]    device, read only
 *   x_norm     fp32  [batch][hidden]    device, written, or NULL
 *   expert_ids int32 [batch][top]       device, written: by weight, descending
 *   gate_w     fp32  [batch][top]       device, written
 * With x_norm NULL, u = x.  Otherwise u = x / sqrt(mean(x^2) + norm_eps), the
 * pre-norm of a transformer block with unit weights, written to x_norm for
 * the decode (the block reads u; the residual adds its output to x).
 * Outputs feed cfr_reader_decode directly.  Runs on `stream`; no host sync,
 * no allocation.  Route calls on one reader must not overlap in time (they
 * share its logit buffer and per-token arrival counters): serialise them on
 * one stream or clone the reader.  Float32 logits: experts whose logits
 * differ by a few float32 ulps from the top-th may be ordered differently
 * from a float64 computation.  A NaN logit ranks below every other value
 * (ties to the lower index), so every slot of expert_ids is written with
 * distinct experts; any non-finite logit sets bit 1 of the reader's status
 * word (cfr_reader_status) and leaves that token's weights unspecified.
 * CFR_EINVAL if the reader was built without router weights, batch is
 * outside 1..max_batch, norm_eps < 0 with x_norm given, or x_norm aliases x;
 * CFR_EUNSUPPORTED if the pick's 8 bytes of LDS per expert do not fit one
 * workgroup (n_experts above about 20 000).
 */
int cfr_reader_route(cfr_reader* r, const float* x, int32_t batch, float norm_eps, float* x_norm,
                     int32_t* expert_ids, float* gate_w, void* stream);

/*
 * The dense routed-expert gated MLP on the same resident BF16 weights
 * ([zh §前置知识 / 门控MLP与通道]): y = sum_s w_s D_e (phi(G_e x) * V_e x).
 * The baseline the reader is measured against.  Same argument rules as
 * cfr_reader_decode.
 */
int cfr_dense_decode(cfr_reader* r, const float* x, const int32_t* expert_ids,
                     const float* gate_w, int32_t batch, float* y, void* stream);

/* cfr_dense_decode with the residual added in its last kernel; the rules of
 * cfr_reader_decode_residual. */
int cfr_dense_decode_residual(cfr_reader* r, const float* x, const int32_t* expert_ids,
                              const float* gate_w, int32_t batch, const float* resid, float* y,
                              void* stream);

/* Stages of the decode path, in launch order; cfr_reader_decode_profile
 * reports one duration per stage. */
#define CFR_NUM_STAGES 3
/* 0 screen: rotate, partial screen, sketch screen sums (k_screen);
 * 1 select: scores, exact top-k, exact gather of the kept channels and the
 *   recovery projection of the skipped ones (k_select);
 * 2 reduce: sum of the partial outputs plus U z (k_reduce) */

/*
 * Measurement entry: the same computation as cfr_reader_decode with a HIP
 * event recorded on `stream` after every stage; waits for the stream and
 * writes each stage's duration in microseconds to stage_us (host,
 * CFR_NUM_STAGES floats; a stage that did not run reports 0).  Not for the
 * fast path: it synchronises the host.
 */
int cfr_reader_decode_profile(cfr_reader* r, const float* x, const int32_t* expert_ids,
                              const float* gate_w, int32_t batch, int32_t k, float* y,
                              float* stage_us, void* stream);

/*
 * Measurement entry: launches the kernel of one decode stage alone on
 * `stream` (stage 0, 1 or 2, as listed above), with the arguments
 * cfr_reader_decode would give it; no host synchronisation.  A stage reads
 * what the previous stage left in the reader's workspace, so y is the
 * decode's result only when stages 0, 1, 2 run in that order for the same
 * inputs; any other order reads stale but in-range workspace contents.  For
 * timing one kernel in isolation (for example many launches in a HIP graph).
 * Errors as cfr_reader_decode, plus CFR_EINVAL for a stage out of range.
 */
int cfr_reader_decode_stage(cfr_reader* r, int32_t stage, const float* x, const int32_t* expert_ids,
                            const float* gate_w, int32_t batch, int32_t k, float* y, void* stream);

/* Copy the built state to host buffers (any may be NULL); sizes from
 * cfr_sizes_of.  codes uint8, scales/rho/U/b fp16 bits, norms fp32,
 * sigma fp32 (+1/-1).  Synchronises the reader's device. */
int cfr_reader_export(const cfr_reader* r, uint8_t* codes, uint16_t* scales, uint16_t* rho,
                      float* norms, uint16_t* u, uint16_t* b, float* sigma);

/*
 * Host-only load steps (1) and (2): the sketch (codes, scales, rho) and the
 * down norms, exactly as cfr_build_reader computes them, into host buffers
 * sized by cfr_sizes_of (any output may be NULL).  No device is touched, so
 * the pack can be checked on a machine without a GPU.
 */
int cfr_pack_host(const cfr_config* cfg, const uint16_t* gate, const uint16_t* up,
                  const uint16_t* down, uint8_t* codes, uint16_t* scales, uint16_t* rho,
                  float* norms);

/* A second reader with the same configuration and a byte-identical copy of
 * every resident buffer at new device addresses (so benchmark loops can
 * cycle through layers the caches have not seen).  Fresh workspace. */
int cfr_reader_clone(const cfr_reader* src, cfr_reader** out);

/* Config the reader was built with. */
int cfr_reader_config(const cfr_reader* r, cfr_config* out);

/* Read (and clear) the reader's device status word: bit 0 = an expert id
 * was out of range and clamped; bit 1 = a router logit was not finite
 * (cfr_reader_route).  Synchronises the reader's device. */
int cfr_reader_status(cfr_reader* r, int32_t* flags);

/* Release the reader and all its device memory.  NULL-safe. */
void cfr_reader_free(cfr_reader* r);

/* Message of the calling thread's last error ("" if none). */
const char* cfr_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* CFR_H */
