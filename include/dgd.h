/*
 * dgd.h - C ABI of the MI355X (gfx950) denoising-step library (libdgd.so).
 *
 * The library performs the per-step update of uniform-state discrete
 * diffusion in the style of DiffusionGemma, as described by four pages:
 *   - the ComfyUI node page "DiffusionGemma Denoise (KV Cache)", Inputs table
 *     (knob names, units, defaults, the temperature schedule, block length);
 *   - the ComfyUI-DiffusionGemma pack README, sections "What it is" (lowest
 *     entropy positions freeze, the rest are re-noised) and "Terms and units";
 *   - the TensorSharp DiffusionGemma model doc, section "3. Sampler contract"
 *     (MaxDenoisingSteps, TMin/TMax, EntropyBound, StabilityThreshold,
 *     ConfidenceThreshold, Seed);
 *   - "The Annotated DiffusionGemma" walkthrough, section "Sampling" (apply
 *     temperature, compute entropy, keep a low-entropy prefix and renoise the
 *     rest, check for early stopping) and "Denoise, stage, commit, and
 *     generate".
 *
 * One step of one canvas (block b, step s, N steps per block, gstep = b*N+s):
 *   T_s   = t_max + (s/N)(t_min - t_max)                  (walkthrough, "Apply temperature")
 *   z     = H W_vocab^T, bf16 inputs, fp32 accumulation   (tied unembedding)
 *   x     = z / T_s
 *   H_p   = -sum_v p_v ln p_v, p = softmax(x)             (nats; "Compute entropy")
 *   a_p   = argmax_v x_v (first index on ties)
 *   tok_p = argmax_v (x_v + g_v), g = -ln(-ln u), u from Philox4x32-10
 *           word (v&3) of counter (v>>2, p_abs, gstep, 0), key = seed,
 *           u = ((w >> 9) + 1/2) 2^-23                       (Gumbel-max sample)
 *   converged = mean_p H_p < confidence AND argmax unchanged for
 *               stability_threshold steps (argmax before step 0 = all 0)
 *   final = converged OR s == N-1: every open position takes tok_p (or a_p
 *           when final_emit), all positions end committed, the canvas is done.
 *   otherwise: rank open positions by (H_p, p); rank r is accepted when the
 *           float64 sum of the entropies ranked before it is <= entropy_bound
 *           ("Keep a low-entropy prefix"); accepted positions take tok_p and
 *           become committed; the other ranked positions are re-noised to
 *           (w * V) >> 32 with w = Philox word 0 of (0, p_abs, gstep, 1).
 *   A block starts from tokens (w * V) >> 32, w = Philox word 0 of
 *   (0, p_abs, b, 2), with every position open.
 *
 * Memory.  Every device buffer is owned by the caller; the library allocates
 * no device memory.  Pointers marked "device" must be device memory of the
 * current HIP device; pointers marked "host" are read during the call only.
 * Layouts are row-major and densely packed.  bf16 values are IEEE bfloat16
 * bit patterns.
 *
 * Streams.  Work is enqueued on ctx->stream (a hipStream_t; NULL = the null
 * stream) and the call returns without synchronising, unless ctx->k1_ms asks
 * for kernel timing.  Outputs are valid once the stream has reached them.
 * Calls that share a workspace or state buffer must be ordered on one stream.
 *
 * Errors.  Every entry point returns DGD_OK (0) or a negative code and never
 * throws; dgd_last_error() describes the last failure of the calling thread.
 * Invalid arguments are refused, never adjusted.  Argument checks happen on
 * the host before any work is enqueued, so a refused call leaves every
 * buffer untouched.
 */
#ifndef DGD_H
#define DGD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DGD_OK            0
#define DGD_EINVAL       (-1)  /* null pointer, knob out of range, bad shape           */
#define DGD_EUNSUPPORTED (-2)  /* shape outside the limits below                        */
#define DGD_EWORKSPACE   (-3)  /* workspace smaller than dgd_workspace_bytes()          */
#define DGD_EHIP         (-4)  /* a HIP runtime call or kernel launch failed             */

#define DGD_MAX_CANVASES   64     /* B  <= 64                                           */
#define DGD_MAX_CANVAS_LEN 4096   /* L  <= 4096                                         */
#define DGD_MAX_GEN_LENGTH 8192   /* G  <= 8192 (node page, gen_length row range)        */
#define DGD_MAX_STEPS      1024   /* N  <= 1024 (node page, num_inference_steps range)   */
#define DGD_MAX_VOCAB      (1 << 24)
#define DGD_MAX_HIDDEN     65536

typedef uint16_t dgd_bf16;

/* Layouts of the vocabulary table W_vocab accepted by dgd_step / dgd_run. */
#define DGD_VOCAB_ROWS   0  /* [V][d] row-major: the tied embedding table as is          */
#define DGD_VOCAB_PACKED 1  /* the output of dgd_pack_vocab() (MFMA fragment order)      */
#define DGD_VOCAB_Q4     2  /* the output of dgd_pack_vocab_q4() (4-bit groups)           */

/* Largest self-conditioning top-K (dgd_ctx.sc_topk, dgd_sc_embed). */
#define DGD_SC_MAX_TOPK 32

/* Most labels one dgd_label_probs call reads. */
#define DGD_MAX_LABELS 512

/* Per-canvas status word of the state block (see the state layout). */
#define DGD_STATUS_OK        0
#define DGD_STATUS_NONFINITE 1  /* some position's logits were NaN or +inf (or all -inf):
                                   the canvas stopped at that step, untouched        */

/* Sampler knobs (node page "Inputs"; TensorSharp doc "3. Sampler contract").
 * Ranges are checked on every call:
 *   num_inference_steps  N in [1, 1024]
 *   t_min, t_max         finite, in [0, 1], and every T_s >= 1e-4 (so that
 *                        tempered fp32 logits stay finite)
 *   confidence           early-stop mean-entropy threshold in nats, [0, 1]
 *   stability_threshold  consecutive unchanged-argmax steps needed, [0, 1024]
 *   freeze               1: committed positions stay frozen (default);
 *                        0: every position is re-ranked each step
 *   final_emit           0: the last step writes samples (default);
 *                        1: it writes the argmax canvas                       */
typedef struct dgd_params {
  int32_t num_inference_steps;
  float   t_min;
  float   t_max;
  float   confidence;
  int32_t stability_threshold;
  int32_t freeze;
  int32_t final_emit;
} dgd_params;

/* Shapes, per-canvas knobs, scratch and optional outputs.
 *   B  canvases denoised together, [1, 64]
 *   L  canvas (block) length, [1, 4096]
 *   V  vocabulary size, [1, 2^24]
 *   d  hidden size, [8, 65536], a multiple of 8
 *   G  generated length per canvas, a multiple of L, G <= 8192
 *   entropy_bound  host float[B], nats, each in [0, 1]
 *   workspace      device, at least dgd_workspace_bytes(B, L, V, d) bytes,
 *                  256-byte aligned; contents need no initialisation
 *   state          device, dgd_state_bytes(B, L) bytes, layout below;
 *                  dgd_init_block() initialises it for a block
 *   stream         hipStream_t
 * Optional device outputs of dgd_step (NULL = not written), all for the step
 * just taken, row index r = c*L + p:
 *   entropy     float[B*L]   H_p in nats
 *   argmax      int32[B*L]   a_p
 *   token       int32[B*L]   tok_p (the Gumbel-max sample)
 *   gap         float[B*L]   top-two gap of the Gumbel-perturbed tempered logits, nats
 *   logits      float[B*L*V] z (fp32 accumulator, before temperature); validation only
 *   commit_step int16[B*G]   step index s at which the position was last committed
 *                            (untouched elsewhere; callers pre-fill, e.g. with -1)
 *   vocab_layout   DGD_VOCAB_ROWS (0) when W_vocab is the [V][d] table itself,
 *                  DGD_VOCAB_PACKED (1) when it is the output of dgd_pack_vocab()
 *                  for the same V and d (the faster path: every load of the
 *                  projection is a contiguous 1 KB MFMA fragment),
 *                  DGD_VOCAB_Q4 (2) when it is the output of dgd_pack_vocab_q4():
 *                  a 4-bit table the projection dequantizes as it streams it
 *                  (d a multiple of 32; no self-conditioning top-K)
 * Optional lm-head tail (walkthrough, "RMSNorm" and "Logit Softcapping";
 * TensorSharp doc, "2. Forward graph": output norm -> tied lm-head -> final
 * logit softcap).  Zero-initialised fields leave both off, and H is then
 * taken as already normalised.
 *   norm_weight  device bf16[d], 16-byte aligned, or NULL (no output norm).
 *                When set, each row x of H becomes
 *                  h = w * x * sqrt(d) / (||x||_2 + norm_eps)
 *                computed in fp64 and rounded once to bf16 (nearest, ties to
 *                even); the projection then uses h.
 *   norm_eps     added to the row's L2 norm (not to its mean square);
 *                finite, in [0, 1]
 *   norm_h       device bf16[B*L*d], 16-byte aligned, written with h each
 *                step; required when norm_weight is set, must not overlap H
 *   softcap      c: the logits become c * tanh(z / c) before the
 *                temperature; 0 = no cap, else in [0.01, 10000]
 * ctx->logits stays the projection z itself, before cap and temperature.
 * Optional self-conditioning outputs (walkthrough, "Complete DiffusionGemma
 * model" and "Denoise, stage, commit, and generate": the next forward takes
 * this step's tempered probabilities; TensorSharp doc: self-conditioning
 * top-K cutoff, default 32).  Needs vocab_layout = DGD_VOCAB_PACKED.
 *   sc_topk    K in [1, DGD_SC_MAX_TOPK], K <= V; 0 = off
 *   sc_prob    device float[B*L*K]: the K largest probabilities of
 *              softmax(z'/T_s) per position (z' the capped logits when the
 *              softcap is on), best first, ties by the lower id; exact
 *              probabilities, not renormalised over the K
 *   sc_id      device int32[B*L*K]: their vocabulary ids
 *   sc_status  device int32[B*L] or NULL: per position, how many parts of the
 *              vocabulary the selection recomputed exactly (0 almost always),
 *              or -1 if its recomputation budget ran out (the K ids are then
 *              the best found, not certified; ids of -1 mark empty slots),
 *              or -2 for a position with non-finite logits (ids -1, NaN
 *              probabilities; its canvas stops, see DGD_STATUS_NONFINITE)
 * Positions of canvases that are done are not written.
 * Optional host outputs (timing): when k1_ms is not NULL the call records HIP
 * events around every launch of the fused projection kernel, synchronises
 * before returning, and writes the summed kernel time in ms to *k1_ms and the
 * number of launches timed to *k1_launches (if not NULL); when tail_ms is also
 * set, *tail_ms receives the summed time from the end of each projection to
 * the end of its step's last kernel (merge, top-K, commit).                  */
typedef struct dgd_ctx {
  int32_t B, L, V, d, G;
  const float* entropy_bound;
  void*   workspace;
  size_t  workspace_bytes;
  void*   state;
  void*   stream;
  float*   entropy;
  int32_t* argmax;
  int32_t* token;
  float*   gap;
  float*   logits;
  int16_t* commit_step;
  double*  k1_ms;
  int32_t* k1_launches;
  int32_t  vocab_layout;   /* DGD_VOCAB_ROWS, DGD_VOCAB_PACKED or DGD_VOCAB_Q4 */
  const dgd_bf16* norm_weight;  /* output-norm weights or NULL */
  float    norm_eps;
  float    softcap;
  dgd_bf16* norm_h;             /* normalised H (scratch the caller owns) */
  int32_t  sc_topk;             /* self-conditioning top-K, 0 = off */
  float*   sc_prob;
  int32_t* sc_id;
  int32_t* sc_status;
  double*  tail_ms;             /* see the timing outputs above, or NULL */
} dgd_ctx;

/* State layout (device, int32/float words, in this order; the per-canvas
 * words carry the pack README's honesty readout, "What works today":
 * converged, committed fraction, steps used; plus a status and the step's
 * tie counts):
 *   int32 prev_argmax [B*L]  argmax canvas of the previous step of the block
 *   int32 stable_count[B]    consecutive steps with an unchanged argmax canvas
 *   int32 done        [B]    1 once the canvas has taken its final step (or stopped)
 *   int32 steps_used  [B]    steps taken in the current block
 *   int32 converged   [B]    1 if the block ended by the early-stop rule
 *   int32 n_committed [B]    committed positions of the current block
 *   float mean_entropy[B]    mean entropy of the last step, nats (NaN if stopped)
 *   int32 new_commits [B]    positions committed by the last step
 *   int32 status      [B]    DGD_STATUS_OK, or DGD_STATUS_NONFINITE: a position
 *                            of the last step had no finite distribution (NaN
 *                            or +inf logits, e.g. a non-finite row of H or an
 *                            fp32 overflow of the projection).  The canvas then
 *                            stopped: done = 1, converged = 0, canvas, committed
 *                            mask and prev_argmax untouched; that step's
 *                            entropy/gap outputs are NaN and argmax/token -1 at
 *                            the offending positions.  dgd_init_block clears it.
 *   Tie counts of the last step (positions where a decision rests on a float
 *   difference below the comparison bands of the step's arithmetic):
 *   int32 band_sample [B]    positions whose top-two Gumbel-perturbed logits
 *                            differ by < 1e-4 nats
 *   int32 band_commit [B]    ranked positions whose entropy lies within 1e-5
 *                            nats of the last accepted or the first rejected
 *                            entropy, or that are one of those two ranks with
 *                            the running sum before it within 1e-5 of the
 *                            bound (0 on a final step)
 *   int32 band_conv   [B]    1 if |mean_entropy - confidence| < 1e-5
 * The step reads and writes it; callers may read it after a stream sync, and
 * may overwrite it to resume from a saved state.                            */
size_t dgd_state_bytes(int32_t B, int32_t L);

/* Bytes of scratch the step needs (per-slice softmax/entropy/Gumbel partials
 * and per-position results); 0 if the shape is unsupported. */
size_t dgd_workspace_bytes(int32_t B, int32_t L, int32_t V, int32_t d);

/* Start block `block` of every canvas (walkthrough, "Lazy Sampling": the
 * first step samples from all-equal logits, i.e. a uniform canvas; node page,
 * gen_length row: a longer generation runs more blocks): uniform initial
 * tokens (Philox word 0 of counter (0, p_abs, block, 2)) over positions
 * [block*L, (block+1)*L), committed = 0 there, and a fresh state for the
 * block.  Earlier and later positions are untouched.
 *   canvas     device int32[B*G], committed device uint8[B*G]
 *   seed       host uint64[B] (Philox key: low word, high word)            */
int dgd_init_block(int32_t* canvas, uint8_t* committed, int32_t block,
                   const dgd_params* params, const uint64_t* seed, const dgd_ctx* ctx);

/* One denoising step (walkthrough, "Sampling": apply temperature, compute
 * entropy, keep a low-entropy prefix and renoise the rest, check for early
 * stopping; taken eagerly, the forward's hidden states H first) for block
 * `block`, step `step` in [0, N), of every canvas that is not done.  H: device bf16[B*L*d], the final hidden states of the B
 * canvases for this step (row r = c*L + p).  W_vocab: device, the tied
 * embedding table in the layout ctx->vocab_layout names (bf16[V*d] row-major,
 * or dgd_packed_vocab_bytes(V, d) bytes from dgd_pack_vocab).  H and W_vocab
 * must be 16-byte aligned.  canvas/committed: device int32/uint8[B*G], updated
 * in place.  seed: host uint64[B].  The [B*L x V] logits never reach HBM
 * unless ctx->logits asks for them. */
int dgd_step(const dgd_bf16* H, const dgd_bf16* W_vocab, int32_t* canvas, uint8_t* committed,
             int32_t block, int32_t step, const dgd_params* params, const uint64_t* seed,
             const dgd_ctx* ctx);

/* dgd_step for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same step, with
 * the same kernels and results, whose scratch is a 32 MiB device array of the
 * library (one per GPU, held until the process ends) instead of
 * ctx->workspace, which is ignored (may be NULL).  The call allocates
 * nothing: no hipMalloc or hipFree, no events (ctx->k1_ms must be NULL).  The
 * first call on a device looks the array's address up on that device.
 * Shapes whose scratch exceeds the array are refused with DGD_EUNSUPPORTED:
 * the step needs 32 B per (position, vocabulary group) record (groups =
 * min(ceil(V/256), 256)), 24 B per position, and with a top-K 128 B more per
 * record; e.g. 256 positions at V = 262144 need 2.1 MB (10.5 MB with a
 * top-K), 2048 positions 16.8 MB (without).  Nothing is carried in the array
 * from one call to the next, but every call on a GPU uses that GPU's one
 * array: calls that overlap on one GPU (other streams, other threads) race
 * and must not be issued.  Everything else (state, outputs, errors) is as
 * for dgd_step. */
int dgd_step_noalloc(const dgd_bf16* H, const dgd_bf16* W_vocab, int32_t* canvas,
                     uint8_t* committed, int32_t block, int32_t step, const dgd_params* params,
                     const uint64_t* seed, const dgd_ctx* ctx);

/* Whole generation (walkthrough, "Denoise, stage, commit, and generate";
 * node page, gen_length row): for every block b in [0, G/L): dgd_init_block,
 * then up to N steps (steps after a canvas is done leave it untouched;
 * nothing synchronises with the host).  H_steps: device bf16[(G/L)*N*B*L*d], laid
 * out [block][step][canvas][position][hidden].  Per-step outputs of ctx, if
 * set, hold the last step taken. */
int dgd_run(const dgd_bf16* H_steps, const dgd_bf16* W_vocab, int32_t* canvas,
            uint8_t* committed, const dgd_params* params, const uint64_t* seed,
            const dgd_ctx* ctx);

/* Part of a generation, as dgd_run takes it: the n_steps global steps
 * g = first_step .. first_step + n_steps - 1 in order, where g = b*N + s is
 * step s of block b; at every s == 0 the block is first started as by
 * dgd_init_block.  dgd_run is dgd_run_steps(0, (G/L)*N).  A caller resumes a
 * generation from a saved state by running its remaining steps.
 * first_step >= 0, n_steps >= 0, first_step + n_steps <= (G/L)*N; H_steps
 * as for dgd_run (the whole [G/L][N][B][L][d] array). */
int dgd_run_steps(const dgd_bf16* H_steps, const dgd_bf16* W_vocab, int32_t* canvas,
                  uint8_t* committed, int32_t first_step, int32_t n_steps,
                  const dgd_params* params, const uint64_t* seed, const dgd_ctx* ctx);

/* The self-conditioning input of the next forward from a step's top-K
 * (walkthrough, "Complete DiffusionGemma model": the decoder adds
 * (P @ W_embed) * sqrt(hidden), with P cast to the model dtype):
 *   out[r][k] = bf16( scale * sum_{j<K} bf16(sc_prob[r][j]) * E[sc_id[r][j]][k] )
 * summed in fp32 in j order; bf16() rounds to nearest, ties to even.  Ids
 * outside [0, V) are skipped.
 *   sc_prob, sc_id  device float/int32[rows*K] (as dgd_step writes them)
 *   W_vocab         device, the table in vocab_layout (rows or packed), 16-B aligned
 *   scale           finite; the walkthrough's embed scale is sqrt(d)
 *   out             device bf16[rows*d], 16-byte aligned, written
 * Enqueued on `stream`; 0 or a negative DGD_E* code. */
int dgd_sc_embed(const float* sc_prob, const int32_t* sc_id, int32_t rows, int32_t K,
                 const dgd_bf16* W_vocab, int32_t vocab_layout, int32_t V, int32_t d, float scale,
                 dgd_bf16* out, void* stream);

/* Sparse label read for typed decisions (TensorSharp doc, "1. Origin and
 * intent": label probabilities read from a canvas in one denoising step
 * through a sparse output projection):
 *   logits[r][l] = z = H[r] . E[labels[l]]  (fp32 sum), then c tanh(z / c)
 *                  when softcap c > 0
 *   probs[r][l]  = softmax over l of logits[r][l] / temperature
 * Only the label rows of the table are read; the probabilities are
 * normalised over the labels, not over the vocabulary.
 *   H          device bf16[rows*d], 16-byte aligned (rows that already went
 *              through the model's output norm, e.g. dgd_ctx.norm_h)
 *   W_vocab    device, the table in vocab_layout (rows or packed), 16-B aligned
 *   labels     HOST int32[n_labels], each in [0, V), 1 <= n_labels <= DGD_MAX_LABELS
 *              (repeats allowed)
 *   temperature  finite, >= 1e-4;  softcap  0 or in [0.01, 10000]
 *   logits     device float[rows*n_labels] or NULL; probs device float[rows*n_labels]
 * Enqueued on `stream`; 0 or a negative DGD_E* code. */
int dgd_label_probs(const dgd_bf16* H, int32_t rows, const dgd_bf16* W_vocab, int32_t vocab_layout,
                    int32_t V, int32_t d, const int32_t* labels, int32_t n_labels, float temperature,
                    float softcap, float* logits, float* probs, void* stream);

/* A 4-bit table (the pages' quantized checkpoints: INT4 W4A16 and GGUF
 * 4-bit files, ComfyUI pack "What works today" and "Downloads"): each row is
 * cut into groups of 32 hidden elements sharing a bf16 scale s and minimum m;
 * element k keeps a 4-bit code q and stands for
 *   w = bf16( fp32(s) * q + fp32(m) )   (one fp32 rounding, then nearest-even)
 * The step with ctx->vocab_layout = DGD_VOCAB_Q4 is the step on that table.
 * dgd_q4_vocab_bytes: size of the streaming form, ceil(V/64)*64 rows x
 * ceil(d/64) chunks x 40 bytes per 64 elements; 0 if V or d is outside the
 * limits or d is not a multiple of 32.
 * dgd_pack_vocab_q4 rewrites the natural form into it, once per table:
 *   codes   device uint8[V*d/2]: element 2i of a row in the low nibble of byte
 *           i, element 2i+1 in the high nibble; 16-byte aligned
 *   scales, mins  device bf16[V*(d/32)], group g of row v at v*(d/32) + g
 *   W_q4    device, dgd_q4_vocab_bytes(V, d) bytes, 16-byte aligned, written;
 *           must not overlap the inputs
 * Enqueued on `stream`; 0 or a negative DGD_E* code. */
size_t dgd_q4_vocab_bytes(int32_t V, int32_t d);
int dgd_pack_vocab_q4(const uint8_t* codes, const dgd_bf16* scales, const dgd_bf16* mins, void* W_q4,
                      int32_t V, int32_t d, void* stream);

/* Size in bytes of the packed vocabulary table for (V, d):
 * ceil(V/64)*64 * ceil(d/64)*64 * 2; 0 if V or d is outside the limits. */
size_t dgd_packed_vocab_bytes(int32_t V, int32_t d);

/* Rewrite the tied embedding table once into the order in which the fused
 * projection streams it (a permutation of W_vocab's elements, zero-padded to
 * whole 64-row groups and 64-element hidden chunks).  The table's values are
 * the ones the pages' unembedding uses (walkthrough, "Setup + Load Model":
 * tied [V x d] embedding); only the byte order changes.
 *   W_vocab   device bf16[V*d] row-major, read only
 *   W_packed  device, dgd_packed_vocab_bytes(V, d) bytes, written; must not
 *             overlap W_vocab
 * Both 16-byte aligned.  Enqueued on `stream` (hipStream_t).  Pack once per
 * table; a packed table serves every later step with ctx->vocab_layout =
 * DGD_VOCAB_PACKED. */
int dgd_pack_vocab(const dgd_bf16* W_vocab, dgd_bf16* W_packed, int32_t V, int32_t d, void* stream);

/* Validation helper: for n 32-bit Philox words (device uint32[n]) write the
 * Gumbel noise the fused step adds to its logits, in base-2 units:
 * out[i] = -log2(-log2(u_i)) with u_i = ((w_i >> 9) + 1/2) 2^-23, so that the
 * natural-unit noise is out[i]*ln 2 - ln(ln 2).  Device float[n] output. */
int dgd_debug_gumbel(const uint32_t* words, float* out, int64_t n, void* stream);

/* Validation helper: Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel
 * Random Numbers: As Easy as 1, 2, 3", SC'11) as the kernels compute it.
 *   ctr  device uint32[n*4]: call i's counter (c0, c1, c2, c3), 16-byte aligned
 *   key  device uint32[n*2]: call i's key (k0, k1), 8-byte aligned; or NULL to
 *        use uniform_key (k0 = low word, k1 = high word) for every call, the
 *        form the fused step runs with its key in scalar registers
 *   out  device uint32[n*4]: the four output words, 16-byte aligned */
int dgd_debug_philox(const uint32_t* ctr, const uint32_t* key, uint64_t uniform_key, uint32_t* out,
                     int64_t n, void* stream);

/* Measurement helpers (not part of the step): what this GPU sustains on the
 * two resources the projection uses, for reports against measured ceilings
 * beside the published peaks.  The caller times them (e.g. with events).
 * dgd_ceiling_hbm_read: reads `bytes` (a multiple of 16) of device memory at
 *   `buf` once, 16-byte non-temporal loads from 4096 workgroups, folding
 *   them into sink (device uint32[1024], XOR-accumulated: clear it first).
 * dgd_ceiling_mfma_bf16: `workgroups` workgroups of 4 waves (one per SIMD),
 *   each wave `rounds` x 64 independent v_mfma_f32_32x32x16_bf16 (32768 flop
 *   each) on operands read once from `ops` (device, `bytes` >= 256); writes
 *   device float[workgroups*256] to sink. */
int dgd_ceiling_hbm_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);
int dgd_ceiling_mfma_bf16(const void* ops, size_t bytes, int64_t rounds, int32_t workgroups, float* sink,
                          void* stream);

/* Measurement helper (not part of the step): phase times of the packed
 * projection, for a profile of where its time goes.  Only a library built
 * with DGD_PHASE_TIMING defined records them (build.py writes that build as
 * libdgd_phase.so beside libdgd.so); its packed projection then stores, for
 * workgroups 0..1023 and each of their 4 waves, 16 slots of 64 bits:
 *   slot 0        100 MHz wall clock at kernel start; slot 1 shader clock there
 *   slot 2+3t     wall clock at the start of tile t (t = 0..3, the first four
 *                 vocabulary tiles of the workgroup)
 *   slot 3+3t     wall clock at the end of tile t's K loop (all MFMAs issued)
 *   slot 4+3t     wall clock at the end of tile t's epilogue
 *   slot 14       wall clock at kernel end; slot 15 shader clock there
 * at entry (workgroup*4 + wave)*16 + slot.  Each launch overwrites the last;
 * slots of tiles a workgroup does not run keep older values.
 *   dst  host uint64[n], n <= 1024*4*16; copied synchronously, so the caller
 *        synchronises its stream first.
 * Returns DGD_EUNSUPPORTED (nothing copied) in a library built without it. */
int dgd_phase_times(uint64_t* dst, size_t n);

/* Description of the last failure on the calling thread ("" if none). */
const char* dgd_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DGD_H */
