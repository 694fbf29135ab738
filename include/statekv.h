/*
 * statekv.h - C ABI of the StateKV streaming-prefill frame step on AMD MI355X
 * (gfx950).
 *
 * The operation is the per-layer, per-frame step of the paper note "Linear
 * Scaling Video VLMs for Long Video Understanding" (papernotes.org, ECCV 2026),
 * section 方法详解:
 *   - 整体框架 / 关键设计 1: each layer keeps a compressed state C (capacity B)
 *     and a detailed state D holding every processed token; the queries of
 *     frame n attend only over [Kbar_{n-1}; K_n] and the result goes to the
 *     next layer;
 *   - 关键设计 2: the candidate pool is the old state plus the frame's T tokens;
 *     each candidate is scored by the average attention the frame's queries
 *     pay to it; the B best form the next state;
 *   - 关键设计 3: RoPE angles use the virtual stream position L_n = nT and one
 *     global scaling factor alpha fixed before the stream starts.
 *
 * Readings taken where the text is silent (equations are missing from it):
 *   - attention is softmax(sigma * Q K^T) V, causal inside the frame, with the
 *     whole compressed state visible;
 *   - a candidate's score is its attention weight averaged over all T queries
 *     and all Hq query heads of the layer (masked pairs count as zero), kept
 *     as fp32; one index set per layer is shared by all KV heads;
 *   - Top-B orders by (score descending, position ascending): ties keep the
 *     older token.  The state keeps its slots: kept frame tokens take the
 *     slots of evicted ones, so the state is a set in slot order (not sorted
 *     by position);
 *   - alpha > 1 applies the YaRN frequency ramp (original window
 *     rope_orig_ctx) and the logit scale sigma = (0.1 ln alpha + 1)^2/sqrt(d);
 *   - K and D store keys after RoPE (positions never change); V has no RoPE.
 *
 * Conventions (all entry points):
 *   - Return 0 on success or a negative STATEKV_E* code.  Arguments are
 *     checked before anything is enqueued, so a failed call leaves the state
 *     unchanged.  Errors reported by the HIP runtime return STATEKV_EDEVICE.
 *   - Device pointers are HIP device memory on the state's device.  Tensors
 *     are dense, row-major, in the element type of the configuration
 *     (bf16 as raw 16-bit words, or fp32).
 *   - A state belongs to one HIP stream (statekv_set_stream); its work is
 *     asynchronous on that stream.  Calls on one state are not thread-safe.
 */
#ifndef STATEKV_H
#define STATEKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define STATEKV_OK          0
#define STATEKV_EINVAL     -1  /* a null pointer, bad size or unsupported shape */
#define STATEKV_EORDER     -2  /* n is not the next frame of the stream, or a frame
                                  after the text phase has begun */
#define STATEKV_ECAPACITY  -3  /* the detailed cache is full (max_frames or max_text reached) */
#define STATEKV_ENOMEM     -4  /* device allocation failed */
#define STATEKV_EDEVICE    -5  /* the HIP runtime reported an error */
#define STATEKV_ENONFINITE -6  /* an input frame held NaN or Inf */
#define STATEKV_ESCRATCH   -7  /* statekv_prefill_frame_static: the frame step needs more
                                  working memory than STATEKV_STATIC_SCRATCH_BYTES */

#define STATEKV_DTYPE_BF16  1
#define STATEKV_DTYPE_F32   2

/* Shape and RoPE parameters of one layer; n_layers > 1 makes the state a
 * stack of L such layers, each with its own compressed state and detailed
 * cache, that advance frame by frame together (the layers of one stream
 * position in a frame x layer wavefront, or independent streams of one
 * shape).  Every frame-step kernel then covers all L layers in one launch. */
typedef struct statekv_layer_cfg {
  int32_t n_q_heads;        /* Hq >= 1 */
  int32_t n_kv_heads;       /* Hkv >= 1, Hq % Hkv == 0; query head h uses KV head h / (Hq/Hkv) */
  int32_t head_dim;         /* d: 64 or 128 */
  int32_t tokens_per_frame; /* T >= 1 */
  int32_t max_frames;       /* frames the detailed cache holds (N_max >= 1) */
  int32_t dtype;            /* STATEKV_DTYPE_BF16 or STATEKV_DTYPE_F32 */
  double  rope_base;        /* RoPE base (> 1) */
  int32_t rope_orig_ctx;    /* original context of the YaRN ramp (>= 1) */
  int32_t max_text;         /* text tokens the detailed cache holds after the
                               frames (>= 0; 0 disables statekv_decode) */
  int32_t n_layers;         /* L: independent layers held by one state and
                               stepped together (0 or 1: a single layer) */
} statekv_layer_cfg;

typedef struct statekv_state statekv_state;

/* A non-owning window on device memory held by the state. */
typedef struct statekv_view {
  const void*    k;            /* keys after RoPE */
  const void*    v;            /* values */
  const int32_t* pos;          /* [count] absolute stream positions in slot order
                                  (compressed view); NULL for the detailed view */
  int64_t        count;        /* tokens in the view */
  int64_t        head_stride;  /* elements between consecutive KV heads */
  int64_t        token_stride; /* elements between consecutive tokens */
  int32_t        n_kv_heads;
  int32_t        head_dim;
  int32_t        dtype;
  int32_t        frames_done;  /* frames processed so far */
  int32_t        n_layers;     /* L */
  int64_t        layer_stride; /* elements of k / v between consecutive layers */
  int64_t        pos_layer_stride; /* elements of pos between consecutive layers */
} statekv_view;

/* Scores and selection of the most recent frame that computed them. */
typedef struct statekv_scores_view {
  const float*   scores;    /* [pool] fp32 mean attention of each candidate */
  const int32_t* pool_pos;  /* [pool] positions of the candidates (state slots, then frame) */
  const int32_t* keep_flag; /* [pool] 1 if the candidate stayed in the state, else 0 */
  int32_t        pool;      /* candidates: min(B, n*T) + T */
  int32_t        kept;      /* min(B, pool) */
  int32_t        frame;     /* frame index, or -1 if no frame has computed scores */
  int32_t        n_layers;  /* L */
  int64_t        layer_stride; /* elements of scores / pool_pos / keep_flag between layers */
} statekv_scores_view;

/*
 * Create the per-layer state (per layer of a stack of cfg->n_layers):
 * compressed state of capacity B (empty), the detailed cache for
 * cfg->max_frames * T + cfg->max_text tokens, and all scratch buffers, on
 * the current HIP device.  1 <= n_layers <= 256.  Everything is allocated here;
 * later calls do not allocate.  alpha >= 1 is the global RoPE scaling factor (关键设计 3), fixed
 * for the life of the state.  Requires B >= 1 and B + T <= 32768, except
 * when B >= max_frames * T: such a state never evicts (full causal attention
 * over the stream, the quadratic baseline) and may hold any number of tokens.
 * On success *out receives the state; the caller releases it with
 * statekv_destroy.  Errors: EINVAL, ENOMEM, EDEVICE.
 */
int statekv_create(const statekv_layer_cfg* cfg, int32_t budget_B, float alpha,
                   statekv_state** out);

/* Launch subsequent work on hip_stream (a hipStream_t on the state's device;
 * NULL = default stream).  The new stream is ordered after all work already
 * queued for the state on the old one (an event recorded on the old stream,
 * waited on by the new one; the event is created with the state, so this call
 * allocates nothing), so frames may move between streams without a host
 * synchronisation.  Inputs written on another stream must be ordered before a
 * call by the caller.  Errors: EINVAL (null state), EDEVICE; on error the state
 * keeps its old stream. */
int statekv_set_stream(statekv_state* s, void* hip_stream);

/*
 * One StateKV step of frame n (0-based; page frame n+1) for this layer (for
 * every layer of a stack: each layer is stepped exactly as a state of its own).
 *   Q [L][T][Hq][d], K [L][T][Hkv][d], V [L][T][Hkv][d]: projected, pre-RoPE
 *     inputs (device, caller-owned, read only; L = 1: [T][H][d]);
 *   O [L][T][Hq][d]: attention output (device, caller-owned, written).
 * Rotates Q and K at positions nT..nT+T-1, attends over [compressed state;
 * frame], appends the rotated K and V to the detailed cache, scores the pool
 * and keeps min(B, pool) candidates as the next compressed state.
 * n must equal the number of frames already processed (EORDER otherwise);
 * ECAPACITY once max_frames frames are done; EINVAL for a frame that would
 * score a pool of more than 32768 candidates (possible only with
 * STATEKV_FLAG_ALWAYS_SCORE on a state that never evicts).  Asynchronous: O and the views
 * are valid after the stream reaches this point.  A NaN or Inf in Q, K or V is
 * detected on the device and reported by the next view call (ENONFINITE).
 */
int statekv_prefill_frame(statekv_state* s, const void* Q, const void* K,
                          const void* V, int32_t n, void* O);

/* Bytes of the static device scratch behind statekv_prefill_frame_static (per device). */
#define STATEKV_STATIC_SCRATCH_BYTES (32u << 20)

/*
 * The frame step of statekv_prefill_frame, for callers that cannot allocate
 * device memory at the time of the call (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): same arguments, same
 * results (bit-identical), but the step's working buffers (rotated queries,
 * the key-split partial outputs and their statistics) live in one static
 * device array of STATEKV_STATIC_SCRATCH_BYTES per device instead of the
 * state's own.  Calls nothing that allocates.  The array's address on the
 * state's device is resolved when a state is first created there (or, failing
 * that, on the first call).  Every call on one device shares that array and
 * leaves its contents behind (nothing in it needs to start cleared): calls that
 * overlap on one device, on different streams or states, race and must not be
 * issued.  Errors: those of statekv_prefill_frame, and ESCRATCH (nothing
 * enqueued, state unchanged) when the state's shapes need more working memory
 * than the array holds: (rotated queries + split partials + statistics) of all
 * L layers; e.g. the single-layer Hq=14/Hkv=2/d=64/T=256/B=4096 step uses about
 * 9 MB.
 */
int statekv_prefill_frame_static(statekv_state* s, const void* Q, const void* K,
                                 const void* V, int32_t n, void* O);

/*
 * Compressed state C after the last frame: k, v are [Hkv][count][d] with
 * head_stride (elements between KV heads: the row capacity times d) and
 * token_stride = d; pos[count] gives each slot's
 * stream position (slot order; sort by position for a sequence view).
 * Layer l of a stack starts at k + l*layer_stride (v likewise) and
 * pos + l*pos_layer_stride; every layer holds count tokens.
 * Synchronises the state's stream.  Valid until the next prefill_frame or
 * destroy.  Returns ENONFINITE if an input frame held NaN or Inf.
 */
int statekv_compressed_view(const statekv_state* s, statekv_view* out);

/*
 * Detailed state D: k, v are [count][Hkv][d] (token_stride = Hkv*d,
 * head_stride = d), row p holding the token at stream position p:
 * count = frames_done*T + the text tokens decoded so far; layer l of a stack
 * starts at k + l*layer_stride.  Synchronises the
 * state's stream.  Valid until destroy.  Returns ENONFINITE as above.
 */
int statekv_detailed_view(const statekv_state* s, statekv_view* out);

/*
 * Scores, pool positions and kept indices of the last frame that computed
 * them (frames whose pool does not exceed B skip scoring unless
 * STATEKV_FLAG_ALWAYS_SCORE is set); layer l's arrays start layer_stride*l
 * elements further.  Synchronises the stream; valid until the
 * next prefill_frame or destroy.
 */
int statekv_scores(const statekv_state* s, statekv_scores_view* out);

/*
 * Text phase (整体框架 and 关键设计 1: once the frames are done, generation
 * uses the whole detailed cache D as its context; 关键设计 3: the same fixed
 * alpha, positions continuing the virtual length).  Appends t text tokens
 * (prompt chunk or generated tokens) at stream positions P0..P0+t-1, with
 * P0 = frames_done*T + text tokens already decoded, and attends them causally
 * over every row of D:
 *   Q [L][t][Hq][d], K [L][t][Hkv][d], V [L][t][Hkv][d]: projected, pre-RoPE
 *     inputs (device, caller-owned, read only; L = 1: [t][H][d]);
 *   O [L][t][Hq][d]: attention output (device, caller-owned, written).
 * Query i sees D rows 0..P0+i (all frame tokens, earlier text, itself).  The
 * compressed state is neither read nor changed.  1 <= t <= T (EINVAL
 * otherwise); ECAPACITY when the text would exceed cfg->max_text.  After the
 * first decode, statekv_prefill_frame returns EORDER.  Asynchronous like
 * prefill_frame; non-finite inputs are reported by the next view.
 */
int statekv_decode(statekv_state* s, const void* Q, const void* K, const void* V,
                   int32_t t, void* O);

#define STATEKV_FLAG_ALWAYS_SCORE  1u  /* score the pool even while it fits in B */
#define STATEKV_FLAG_KERNEL_TIMING 2u  /* time each kernel with HIP events */
/* Keep the B most recent tokens (a sliding window over the stream, the
 * compute-matched ReKV baseline of 实验关键数据) instead of the B best-scoring
 * candidates.  The score pass is skipped unless STATEKV_FLAG_ALWAYS_SCORE is
 * also set (then the scores are computed and reported, but not used). */
#define STATEKV_FLAG_RECENT_WINDOW 4u

/* Set option flags (STATEKV_FLAG_*).  Takes effect from the next frame. */
int statekv_set_flags(statekv_state* s, uint32_t flags);

/* Kernels of one step, in launch order, as indexed by statekv_kernel_times.
 * A frame step is three launches: the frame launch, pass 1, and the score +
 * merge launch.  The Top-B decision of a frame (and the moves of kept rows
 * into evicted slots) is made in the next frame's frame launch, beside that
 * frame's RoPE, or in a launch of its own when a view asks for the state. */
#define STATEKV_K_ROPE     0  /* frame launch: the previous frame's Top-B decision
                                 and moves; virtual-position RoPE + append to D */
#define STATEKV_K_ATTN     1  /* fused attention, pass 1 (split over keys) */
#define STATEKV_K_SCORE    2  /* merge of the key splits into O; recompute pass:
                                 per-key column sums */
#define STATEKV_K_SELECT   3  /* a pending Top-B decision made for a view */
#define STATEKV_K_DEC_ROPE  4 /* text phase: RoPE of the text tokens + append to D */
#define STATEKV_K_DEC_ATTN  5 /* text phase: attention over D, split over keys */
#define STATEKV_K_DEC_MERGE 6 /* text phase: merge of the key splits into O */
#define STATEKV_K_COUNT    7

/*
 * With STATEKV_FLAG_KERNEL_TIMING set, per-kernel device time is summed over
 * frames: each timed kernel is dispatched with a start and a stop HIP event
 * that the dispatch itself records (hipExtLaunchKernel), so the time is the
 * kernel's execution, without the gaps between launches.  Copies up to n_kernels sums in
 * milliseconds into ms[] and launch counts into launches[] (either may be
 * NULL), synchronising the stream; reset != 0 clears the sums afterwards.
 */
int statekv_kernel_times(statekv_state* s, float* ms, int32_t* launches,
                         int32_t n_kernels, int32_t reset);

/* Release every device buffer of the state.  Accepts NULL. */
void statekv_destroy(statekv_state* s);

/* Static description of an error code. */
const char* statekv_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* STATEKV_H */
