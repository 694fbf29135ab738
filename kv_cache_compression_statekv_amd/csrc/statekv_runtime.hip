// Host runtime and C ABI of the StateKV frame step (see include/statekv.h).
//
// State layout in HBM (one layer; a stack of L layers holds L copies of every
// per-layer array back to back, layer-major, so that its KV heads number
// layer*Hkv + head in the head-major arrays):
//   kpool, vpool      [Hkv][cap][d], cap = B + 2T.  Rows [0, count) hold the
//                     compressed state (one slot per token, in slot order).
//                     While the state fills, frame n is written right after
//                     it (rows [count, count+T)); once frames evict, they
//                     alternate between rows [B, B+T) and [B+T, B+2T).  After
//                     the Top-B decision the kept frame rows at or beyond B
//                     move into the evicted slots below B (at most T rows per
//                     KV head); the next frame's RoPE kernel performs these
//                     moves, as its own rows lie in the other region.  A view
//                     of the state performs pending moves first.
//   ppos              [cap] absolute stream positions of those rows.
//   dk, dv            [max_frames*T + max_text][Hkv][d]: the detailed cache D
//                     (row = stream position: the frames, then the text).
//   qrot              [Hkv][G*T][d]: the frame's rotated queries, rows grouped
//                     by KV head (row = token*G + head-in-group).
//   opart/mpart/lpart split-over-keys partials of attention pass 1 (merged
//                     into O by the select kernel's merge work-groups; the
//                     score pass forms its row statistics from mpart/lpart).
//   rope_tab          [max_frames*T + max_text][d/2] fp32 (cos, sin) of the
//                     scaled angles.
//   dec_opart/mpart/lpart  split-over-keys partials of the text-phase attention.
//   colsum            [2][cap] per-key column sums, 64-bit fixed point, two
//                     buffers used by alternate scored frames: the select
//                     launch reads one and its merge work-groups clear the other.
//   scores, keep_flag              scores of the last scored pool, rebuilt on
//                                  request by statekv_scores.
//   move_dst, move_src, move_count the moves of the last selection.
//   evicted_pos                    [B] positions the last moves overwrote, by slot.
//   score_pos                      positions of the last scored pool, rebuilt
//                                  on request by statekv_scores.
// Everything is allocated in statekv_create; a frame step only launches.
#include "statekv.h"
#include "statekv_internal.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>

using namespace statekv;

// Working memory of statekv_prefill_frame_static: the per-step buffers of a
// frame step (rotated queries, pass-1 partials and split statistics) for
// callers that cannot allocate.  Every device the library runs on holds its own
// copy until the process ends; its address on a device is resolved once, with
// that device current (hipGetSymbolAddress), and only that address is handed
// to kernels.  Calls that overlap on one device share it and race.
static __device__ __align__(256) unsigned char scratch[STATEKV_STATIC_SCRATCH_BYTES];

// Per-step working buffers of a frame step: written and read within one
// step, so nothing in them needs clearing between steps.
struct StepScratch {
  void* qrot;      // [L*Hkv][G*T][d] rotated queries
  void* opart;     // pass-1 partial outputs, whole groups of 32 rows
  int8_t* epart;   // exponents of the fp16 partials
  float* mpart;    // split maxima
  double* lpart;   // split row sums
};

struct statekv_state {
  statekv_layer_cfg cfg;
  int32_t B;
  float alpha;
  Dt dt;
  int esize, Hq, Hkv, D, T, G, R, cap;
  int L;                 // layers of the stack
  int HkvAll;            // L * Hkv: KV heads over all layers
  int64_t det_ls;        // elements of dk / dv per layer
  int device;
  hipStream_t stream;
  hipEvent_t stream_ev;  // orders a newly set stream after the work queued on the old one

  // launch geometry
  int attn_tiles, attn_splits_max;
  int stat_ss;           // split stride of the pass-1 partials (kMaxSplits with a text phase)
  bool never_evicts;
  int score_rsplits_max;
  int score_slots;       // score work-groups resident on the device at once (0: unknown)
  int score_slots8;      // the same for the 8-wave score kernel (bf16)
  int dec_target_wgs;

  void* kpool;
  void* vpool;
  int32_t* ppos;
  void* dk;
  void* dv;
  // The state's own per-step buffers, two sets used by alternate frames: a
  // frame's pass 1 then never writes the lines the previous frame's merge and
  // score pass have just read on other XCDs (measured 2 us faster at B = 4096).
  StepScratch work[2];
  float2* rope_tab;
  unsigned long long* colsum;
  float* scores;
  int32_t* score_pos;
  int32_t* keep_flag;
  int32_t* move_dst;
  int32_t* move_src;
  int32_t* move_count;
  int32_t* evicted_pos;
  double* inv_freq;
  int32_t* nonfinite;
  float* dec_opart;
  float* dec_mpart;
  double* dec_lpart;

  float c_hi, c_lo;  // softmax scale times log2(e), as a float pair

  int count;         // tokens in the compressed state
  int frames_done;
  int text_done;     // text tokens appended to D by statekv_decode

  // Rows of the last frame, and its Top-B decision (with the moves it
  // implies) when not yet made: it runs in the next frame's first launch, or
  // in a launch of its own before a view of the state.
  int frame_base;
  mutable bool sel_pending;
  int sel_P, sel_k0, sel_foff, sel_mode, sel_recent, sel_colsum;

  // scores of the last frame that computed them
  int score_frame, score_pool, score_k0, score_foff;
  int colsum_next;       // column-sum buffer of the next scored frame (0 or 1)
  int colsum_last;       // buffer of the last scored frame
  bool score_evicted;

  uint32_t flags;
  // Kernel timing: a ring of (start, stop) event pairs per kernel, drained
  // lazily so that recording never waits for the device.
  static constexpr int kRing = 64;
  hipEvent_t ev[kRing][STATEKV_K_COUNT][2];
  bool ev_pending[kRing][STATEKV_K_COUNT];
  int ev_slot;
  bool ev_ok;
  float ktime_ms[STATEKV_K_COUNT];
  int32_t klaunch[STATEKV_K_COUNT];
};

namespace {

int check(hipError_t e) { return e == hipSuccess ? STATEKV_OK : STATEKV_EDEVICE; }

template <class P>
int alloc(P** p, size_t bytes) {
  *p = nullptr;
  if (bytes == 0) bytes = 16;
  hipError_t e = hipMalloc((void**)p, bytes);
  if (e != hipSuccess) {
    *p = nullptr;
    return e == hipErrorOutOfMemory ? STATEKV_ENOMEM : STATEKV_EDEVICE;
  }
  return STATEKV_OK;
}

void release(statekv_state* s) {
  for (StepScratch& w : s->work) {
    void* wb[] = {w.qrot, w.opart, w.epart, w.mpart, w.lpart};
    for (void* b : wb)
      if (b) (void)hipFree(b);
  }
  void* bufs[] = {s->kpool, s->vpool, s->ppos, s->dk, s->dv, s->rope_tab, s->colsum, s->scores,
                  s->score_pos, s->keep_flag,
                  s->move_dst, s->move_src, s->move_count, s->evicted_pos, s->inv_freq,
                  s->nonfinite, s->dec_opart, s->dec_mpart, s->dec_lpart};
  for (void* b : bufs)
    if (b) (void)hipFree(b);
  for (auto& ring : s->ev)
    for (auto& e : ring) {
      if (e[0]) (void)hipEventDestroy(e[0]);
      if (e[1]) (void)hipEventDestroy(e[1]);
    }
  if (s->stream_ev) (void)hipEventDestroy(s->stream_ev);
}

// Add a finished (start, stop) pair of ring slot r, kernel k to the sums.
void drain_slot(statekv_state* s, int r, int k) {
  if (!s->ev_pending[r][k]) return;
  s->ev_pending[r][k] = false;
  if (hipEventSynchronize(s->ev[r][k][1]) != hipSuccess) return;
  float ms = 0.f;
  if (hipEventElapsedTime(&ms, s->ev[r][k][0], s->ev[r][k][1]) == hipSuccess) {
    s->ktime_ms[k] += ms;
    s->klaunch[k] += 1;
  }
}

// Frequencies of the rotation pairs: theta_k = base^(-2k/d), and under a
// fixed scaling factor alpha > 1 the YaRN ramp over r_k = L_orig theta_k / 2pi:
// gamma = clamp((r - 1) / 31, 0, 1), theta'_k = (1 - gamma) theta_k / alpha + gamma theta_k.
void scaled_inv_freq(int d, double base, double alpha, int orig_ctx, double* out) {
  for (int k = 0; k < d / 2; ++k) {
    const double kk = (double)k;
    const double th = pow(base, -2.0 * kk / (double)d);
    if (alpha == 1.0) {
      out[k] = th;
      continue;
    }
    const double r = (double)orig_ctx * th / (2.0 * M_PI);
    const double gamma = std::min(std::max((r - 1.0) / (32.0 - 1.0), 0.0), 1.0);
    out[k] = (1.0 - gamma) * th / alpha + gamma * th;
  }
}

int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Byte sizes of the per-step buffers (StepScratch order) for the state's
// shapes and its split stride stat_ss.
void step_scratch_sizes(const statekv_state* s, size_t (&bytes)[5]) {
  const size_t E = s->esize, D = s->D, S = s->stat_ss;
  const size_t rows_all = (size_t)s->HkvAll * s->R;
  const size_t stat_rows = (rows_all + 31) / 32 * 32;   // whole groups of 32 rows
  bytes[0] = rows_all * D * E;
  bytes[1] = (S * rows_all + 31) / 32 * 32 * D * E;
  bytes[2] = S * rows_all * sizeof(int8_t);
  bytes[3] = stat_rows * S * sizeof(float);
  bytes[4] = stat_rows * S * sizeof(double);
}

// Lays the per-step buffers out from base (256-byte aligned pieces); returns
// the bytes they span.
size_t carve_step_scratch(const statekv_state* s, char* base, StepScratch* w) {
  size_t bytes[5];
  step_scratch_sizes(s, bytes);
  size_t off[5], at = 0;
  for (int i = 0; i < 5; ++i) {
    off[i] = at;
    at += (bytes[i] + 255) / 256 * 256;
  }
  if (w) {
    w->qrot = base + off[0];
    w->opart = base + off[1];
    w->epart = reinterpret_cast<int8_t*>(base + off[2]);
    w->mpart = reinterpret_cast<float*>(base + off[3]);
    w->lpart = reinterpret_cast<double*>(base + off[4]);
  }
  return at;
}

// Device address of the static scratch array, per device.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Resolves the address of `scratch` on `device`, which must be current;
// once per device.
int resolve_static_scratch(int device) {
  if (device < 0 || device >= kMaxDevices) return STATEKV_EDEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device]) return STATEKV_OK;
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return STATEKV_EDEVICE;
  g_scratch_ptr[device] = p;
  return STATEKV_OK;
}

// Pass 1 runs best with one work-group (8 waves) per compute unit: about 256
// work-groups; the score pass with about 8 waves per compute unit.
constexpr int kAttnTargetWGs = 256;
constexpr int kAttnHeadMajorMin = 4;   // KV heads from which a single layer's pass 1 runs head-major
constexpr int kScoreTargetWaves = 256 * 8;

// Key splits of pass 1 for a pool of P keys: enough work-groups to fill the
// chip, at least 4 blocks of 64 keys per split.
void attn_geometry(const statekv_state* s, int P, int* splits, int* kps) {
  const int base = s->attn_tiles * s->HkvAll;
  const int bn = attn_block_keys(s->dt, s->D);
  int sp = std::max(1, std::min(ceil_div(kAttnTargetWGs, base), ceil_div(P, 4 * bn)));
  sp = std::min(sp, s->attn_splits_max);
  int k = ceil_div(ceil_div(P, sp), bn) * bn;
  *splits = ceil_div(P, k);
  *kps = k;
}

// Row splits of the score pass.  Every work-group holds its key block and
// walks its rows; with the resident work-group count known, the split
// minimises (dispatch rounds) x (rows per work-group + a fixed cost of about
// kScoreWGRows rows), so that a last, nearly empty round of work-groups is
// avoided.  Otherwise: about 8 waves per CU.  That model is the 4-wave
// kernel's.  When the 8-wave kernel (bf16: twice the keys per work-group,
// half the Q traffic) fits the whole pool in one round of resident
// work-groups, it runs instead, with the most rows per work-group that one
// round allows (a single layer at B = 4096; long pools and stacks take
// several rounds and keep 4 waves, which measured faster there).
constexpr int kScoreWGRows = 48;

void score_geometry(const statekv_state* s, int P, int* key_blocks, int* rsplits, int* rps, int* waves) {
  const int w0 = 4;
  const int kb = ceil_div(P, score_keys_per_wg(s->dt, w0));
  const int base = kb * s->HkvAll;
  const int rs_lo = ceil_div(s->R, kScoreMaxRows);   // rows per work-group fit the LDS statistics
  int rs;
  if (s->score_slots > 0) {
    const int rs_hi = std::max(rs_lo, std::min(s->score_rsplits_max, ceil_div(s->R, 32)));
    long best = -1;
    rs = rs_lo;
    for (int x = rs_lo; x <= rs_hi; ++x) {
      const int r = ceil_div(ceil_div(s->R, x), 32) * 32;
      const long wgs = (long)base * ceil_div(s->R, r);
      const long cost = (wgs + s->score_slots - 1) / s->score_slots * (long)(r + kScoreWGRows);
      if (best < 0 || cost < best) {
        best = cost;
        rs = x;
      }
    }
  } else {
    const int target = kScoreTargetWaves / w0;
    rs = std::max(1, std::min(ceil_div(target, base), ceil_div(s->R, 128)));
    rs = std::min(rs, s->score_rsplits_max);
    rs = std::max(rs, rs_lo);
  }
  int r = ceil_div(ceil_div(s->R, rs), 32) * 32;
  int w = w0, kbw = kb;
  if (s->dt == Dt::BF16 && s->score_slots8 > 0) {
    const int kb8 = ceil_div(P, score_keys_per_wg(s->dt, 8));
    const int rs8 = std::min(s->score_slots8 / (kb8 * s->HkvAll), std::min(s->score_rsplits_max, ceil_div(s->R, 32)));
    if (rs8 >= rs_lo) {
      w = 8;
      kbw = kb8;
      r = ceil_div(ceil_div(s->R, rs8), 32) * 32;
    }
  }
  *key_blocks = kbw;
  *rsplits = ceil_div(s->R, r);
  *rps = r;
  *waves = w;
}

// Text phase: t tokens over P keys.  Row tiles of 32 rows per KV head; key
// splits of whole blocks, about one work-group per CU (measured best for
// long contexts).
constexpr int kDecodeTargetWGs = 256;

void decode_geometry(const statekv_state* s, int64_t P, int* splits, int* kps) {
  const int bk = decode_block_keys(s->dt);
  const int64_t blocks = (P + bk - 1) / bk;
  int sp = (int)std::max<int64_t>(1, std::min<int64_t>(ceil_div(s->dec_target_wgs, s->HkvAll), blocks));
  sp = std::min(sp, kDecodeMaxSplits);
  const int64_t k = ((P + sp - 1) / sp + bk - 1) / bk * bk;
  *splits = (int)((P + k - 1) / k);
  *kps = (int)k;
}

// Text chunks with more than 32 query rows per KV head: pass 1 over D, row
// tiles of the pass-1 kernel.  The split partials are sized for a frame's
// rows and stat_ss splits; a chunk of t tokens has fewer rows, so it may use
// proportionally more splits (up to kMaxMergeSplits): short prompts over a
// long cache then still fill the chip.
int chunk_split_cap(const statekv_state* s, int t) {
  const int64_t rows_all = (int64_t)s->HkvAll * s->R;
  const int64_t rows = (int64_t)s->HkvAll * s->G * t;
  const int64_t by_partials = (int64_t)s->stat_ss * rows_all / rows;
  const int64_t by_stats = (int64_t)s->stat_ss * ((rows_all + 31) / 32) / ((rows + 31) / 32);
  return (int)std::max<int64_t>(1, std::min<int64_t>(kMaxMergeSplits, std::min(by_partials, by_stats)));
}

// At least kChunkSplitBlocks blocks per split: shorter splits cost more in
// per-work-group overhead and merge traffic than they gain (measured on a
// 16k-key cache).
constexpr int kChunkSplitBlocks = 12;

void chunk_geometry(const statekv_state* s, int t, int64_t P, int* tiles, int* splits, int* kps) {
  const int tl = ceil_div(s->G * t, attn_rows_per_wg(s->dt, s->D));
  const int bn = attn_block_keys(s->dt, s->D);
  const int64_t min_keys = (int64_t)kChunkSplitBlocks * bn;
  int sp = (int)std::max<int64_t>(1, std::min<int64_t>(ceil_div(kAttnTargetWGs, tl * s->HkvAll),
                                                       (P + min_keys - 1) / min_keys));
  sp = std::min(sp, chunk_split_cap(s, t));
  const int64_t k = ((P + sp - 1) / sp + bn - 1) / bn * bn;
  *tiles = tl;
  *splits = (int)((P + k - 1) / k);
  *kps = (int)k;
}

struct KernelTimer {
  statekv_state* s;
  int k;
  bool on;
  LaunchTiming lt;   // events the timed dispatch records itself
  KernelTimer(statekv_state* st, int kernel)
      : s(st), k(kernel), on((st->flags & STATEKV_FLAG_KERNEL_TIMING) && st->ev_ok) {
    if (!on) return;
    drain_slot(s, s->ev_slot, k);  // the pair recorded kRing frames ago
    lt.start = s->ev[s->ev_slot][k][0];
    lt.stop = s->ev[s->ev_slot][k][1];
  }
  void done() {
    if (on) s->ev_pending[s->ev_slot][k] = true;
  }
};

// The pending selection of the last frame (layer 0's arrays; the kernel
// offsets the other layers).
// Selection arguments for a pool of P candidates (state rows [0, k0), frame
// rows from k0 + foff) in the given mode, scores from column-sum buffer
// colsum_buf.
SelArgs sel_args_for(const statekv_state* s, int P, int k0, int foff, int mode, int recent, int colsum_buf) {
  SelArgs a{};
  a.colsum = s->colsum + (size_t)colsum_buf * s->L * s->cap;
  a.pool_pos = s->ppos;
  a.evicted_pos = s->evicted_pos;
  a.move_dst = s->move_dst;
  a.move_src = s->move_src;
  a.move_count = s->move_count;
  a.kpool = s->kpool;
  a.vpool = s->vpool;
  a.P = P;
  a.B = s->B;
  a.mode = mode;
  a.recent = recent;
  a.k0 = k0;
  a.foff = foff;
  a.score_scale = 1.0 / ((double)(1ull << kScoreFracBits) * (double)s->Hq * (double)s->T);
  a.Hkv = s->Hkv;
  a.cap = s->cap;
  a.row_bytes = s->D * s->esize;
  a.list_stride = s->T;
  return a;
}

// The pending decision of the last frame.
SelArgs sel_args(const statekv_state* s) {
  return sel_args_for(s, s->sel_P, s->sel_k0, s->sel_foff, s->sel_mode, s->sel_recent, s->sel_colsum);
}

// Makes the last frame's pending Top-B decision and its moves (one launch of
// the selection work-groups alone).
int resolve_pending_selection(const statekv_state* s) {
  if (!s->sel_pending) return STATEKV_OK;
  RopeArgs a{};
  a.nsel = 1;
  a.sel = sel_args(s);
  a.cap = s->cap;
  KernelTimer tm(const_cast<statekv_state*>(s), STATEKV_K_SELECT);
  const int rc = check(launch_frame(s->dt, s->D, a, s->L, s->stream, tm.lt));
  tm.done();
  if (!rc) s->sel_pending = false;
  return rc;
}

int read_nonfinite(const statekv_state* s) {
  int32_t h = 0;
  if (hipMemcpy(&h, s->nonfinite, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess)
    return STATEKV_EDEVICE;
  return h ? STATEKV_ENONFINITE : STATEKV_OK;
}

int sync_state(const statekv_state* s) {
  if (hipSetDevice(s->device) != hipSuccess || hipStreamSynchronize(s->stream) != hipSuccess)
    return STATEKV_EDEVICE;
  return STATEKV_OK;
}

}  // namespace

extern "C" {

const char* statekv_strerror(int code) {
  switch (code) {
    case STATEKV_OK: return "ok";
    case STATEKV_EINVAL: return "invalid argument";
    case STATEKV_EORDER: return "frame index is not the next frame of the stream";
    case STATEKV_ECAPACITY: return "detailed cache is full";
    case STATEKV_ENOMEM: return "device memory allocation failed";
    case STATEKV_EDEVICE: return "HIP runtime error";
    case STATEKV_ENONFINITE: return "an input frame held NaN or Inf";
    case STATEKV_ESCRATCH: return "the frame step needs more working memory than the static scratch holds";
    default: return "unknown error";
  }
}

int statekv_create(const statekv_layer_cfg* cfg, int32_t budget_B, float alpha,
                   statekv_state** out) {
  if (!cfg || !out) return STATEKV_EINVAL;
  *out = nullptr;
  const statekv_layer_cfg c = *cfg;
  if (c.n_q_heads < 1 || c.n_kv_heads < 1 || c.n_q_heads % c.n_kv_heads != 0) return STATEKV_EINVAL;
  if (c.head_dim != 64 && c.head_dim != 128) return STATEKV_EINVAL;
  // Rows of the detailed cache are Hkv*d elements apart; the kernels form
  // in-block row offsets as 24-bit products.
  if ((int64_t)c.n_kv_heads * c.head_dim >= (1 << 24)) return STATEKV_EINVAL;
  if (c.tokens_per_frame < 1 || c.max_frames < 1) return STATEKV_EINVAL;
  if (c.dtype != STATEKV_DTYPE_BF16 && c.dtype != STATEKV_DTYPE_F32) return STATEKV_EINVAL;
  if (!(c.rope_base > 1.0) || !isfinite(c.rope_base) || c.rope_orig_ctx < 1) return STATEKV_EINVAL;
  if (!(alpha >= 1.0f) || !isfinite(alpha)) return STATEKV_EINVAL;
  if (c.max_text < 0) return STATEKV_EINVAL;
  const int layers = c.n_layers == 0 ? 1 : c.n_layers;
  if (layers < 1 || layers > kMaxLayers) return STATEKV_EINVAL;
  const int64_t positions = (int64_t)c.max_frames * c.tokens_per_frame;   // frame tokens
  const int64_t all_positions = positions + c.max_text;                   // rows of D
  if (all_positions > INT32_MAX) return STATEKV_EINVAL;
  // The selection runs in one work-group over at most kMaxPool candidates; a
  // budget that holds every token of the stream never selects (full
  // attention) and has no such limit.
  const bool never_evicts = budget_B >= positions;
  if (budget_B < 1 || (!never_evicts && (int64_t)budget_B + c.tokens_per_frame > kMaxPool))
    return STATEKV_EINVAL;
  const int64_t rows = (int64_t)c.n_q_heads * c.tokens_per_frame;
  if (rows > kMaxRowsTimesHeads) return STATEKV_EINVAL;

  statekv_state* s = (statekv_state*)calloc(1, sizeof(statekv_state));
  if (!s) return STATEKV_ENOMEM;
  s->cfg = c;
  s->B = budget_B;
  s->alpha = alpha;
  s->dt = c.dtype == STATEKV_DTYPE_BF16 ? Dt::BF16 : Dt::F32;
  s->esize = c.dtype == STATEKV_DTYPE_BF16 ? 2 : 4;
  s->Hq = c.n_q_heads;
  s->Hkv = c.n_kv_heads;
  s->D = c.head_dim;
  s->T = c.tokens_per_frame;
  s->G = s->Hq / s->Hkv;
  s->R = s->G * s->T;
  s->L = layers;
  s->HkvAll = layers * s->Hkv;
  // Rows: the state, then two frame regions (frames alternate once they
  // evict); a stream that never evicts needs one row per token.
  s->never_evicts = budget_B >= (int64_t)c.max_frames * c.tokens_per_frame;
  s->cap = s->never_evicts ? c.max_frames * c.tokens_per_frame : budget_B + 2 * s->T;
  s->stream = nullptr;
  s->score_frame = -1;
  s->dec_target_wgs = kDecodeTargetWGs;

  int rc = check(hipGetDevice(&s->device));
  if (rc) {
    free(s);
    return rc;
  }

  s->attn_tiles = ceil_div(s->R, attn_rows_per_wg(s->dt, s->D));
  s->attn_splits_max = std::min(std::min(kMaxSplits, ceil_div(kAttnTargetWGs, s->attn_tiles * s->HkvAll)),
                                std::max(1, ceil_div(s->cap, 4 * attn_block_keys(s->dt, s->D))));
  s->score_rsplits_max = std::max(ceil_div(s->R, kScoreMaxRows), ceil_div(s->R, 32));
  {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, s->device) != hipSuccess) cus = 0;
    s->score_slots = cus * score_wgs_per_cu(s->dt, s->D);
    s->score_slots8 = s->dt == Dt::BF16 ? cus * score8_wgs_per_cu(s->D) : 0;
    if (const char* e = getenv("STATEKV_SCORE_SLOTS")) s->score_slots = atoi(e);
  }
  // Tuning overrides (launch geometry only; the result does not depend on them).
  if (const char* e = getenv("STATEKV_ATTN_SPLITS")) {
    const int v = atoi(e);
    if (v >= 1) s->attn_splits_max = std::min(v, s->attn_splits_max);
  }
  if (const char* e = getenv("STATEKV_DECODE_WGS")) {
    const int v = atoi(e);
    if (v >= 1) s->dec_target_wgs = v;
  }
  if (const char* e = getenv("STATEKV_SCORE_RSPLITS")) {
    const int v = atoi(e);
    if (v >= 1)
      s->score_rsplits_max = std::max(ceil_div(s->R, kScoreMaxRows), std::min(v, s->score_rsplits_max));
  }

  const size_t E = s->esize, D = s->D, Ls = s->L;
  const size_t pool_bytes = Ls * s->Hkv * s->cap * D * E;
  s->det_ls = all_positions * s->Hkv * (int64_t)D;
  const size_t det_bytes = Ls * (size_t)s->det_ls * E;
  // Text-phase partials of the single-tile kernel: splits times rows, for
  // the largest chunk it takes (G*t <= 32).
  size_t dec_rows = 0;
  if (c.max_text > 0 && s->G <= 32) {
    int sp, kp;
    decode_geometry(s, all_positions, &sp, &kp);
    if (sp > 1) dec_rows = (size_t)sp * s->HkvAll * 32;
  }
  // Text chunks of more than 32 query rows per KV head run through pass 1
  // over D and may use up to kMaxSplits key splits.
  s->stat_ss = c.max_text > 0 ? kMaxSplits : s->attn_splits_max;
  size_t wbytes[5];
  step_scratch_sizes(s, wbytes);
  rc = alloc(&s->kpool, pool_bytes);
  if (!rc) rc = alloc(&s->vpool, pool_bytes);
  if (!rc) rc = alloc(&s->ppos, Ls * s->cap * sizeof(int32_t));
  if (!rc) rc = alloc(&s->dk, det_bytes);
  if (!rc) rc = alloc(&s->dv, det_bytes);
  for (StepScratch& w : s->work) {
    if (!rc) rc = alloc(&w.qrot, wbytes[0]);
    if (!rc) rc = alloc(&w.opart, wbytes[1]);
    if (!rc) rc = alloc(&w.epart, wbytes[2]);
    if (!rc) rc = alloc(&w.mpart, wbytes[3]);
    if (!rc) rc = alloc(&w.lpart, wbytes[4]);
  }
  if (!rc) rc = alloc(&s->rope_tab, (size_t)all_positions * (D / 2) * sizeof(float2));
  if (!rc) rc = alloc(&s->colsum, 2 * Ls * s->cap * sizeof(unsigned long long));
  if (!rc) rc = alloc(&s->scores, Ls * s->cap * sizeof(float));
  if (!rc) rc = alloc(&s->score_pos, Ls * s->cap * sizeof(int32_t));
  if (!rc) rc = alloc(&s->keep_flag, Ls * s->cap * sizeof(int32_t));
  if (!rc) rc = alloc(&s->move_dst, Ls * s->T * sizeof(int32_t));
  if (!rc) rc = alloc(&s->move_src, Ls * s->T * sizeof(int32_t));
  if (!rc) rc = alloc(&s->move_count, Ls * sizeof(int32_t));
  if (!rc) rc = alloc(&s->evicted_pos, Ls * s->B * sizeof(int32_t));
  if (!rc) rc = alloc(&s->inv_freq, D / 2 * sizeof(double));
  if (!rc) rc = alloc(&s->nonfinite, sizeof(int32_t));
  if (!rc) rc = alloc(&s->dec_opart, dec_rows * D * sizeof(float));
  if (!rc) rc = alloc(&s->dec_mpart, dec_rows * sizeof(float));
  if (!rc) rc = alloc(&s->dec_lpart, dec_rows * sizeof(double));
  if (!rc) {
    double table[64];
    scaled_inv_freq(s->D, c.rope_base, (double)alpha, c.rope_orig_ctx, table);
    rc = check(hipMemcpy(s->inv_freq, table, D / 2 * sizeof(double), hipMemcpyHostToDevice));
  }
  if (!rc) {
    RopeTableArgs ta{};
    ta.inv_freq = s->inv_freq;
    ta.table = s->rope_tab;
    ta.npos = (int32_t)all_positions;
    ta.half = s->D / 2;
    rc = check(launch_rope_table(ta, nullptr));
  }
  if (!rc) rc = check(hipMemset(s->nonfinite, 0, sizeof(int32_t)));
  if (!rc) rc = check(hipMemset(s->colsum, 0, 2 * Ls * s->cap * sizeof(unsigned long long)));
  if (!rc) rc = check(hipMemset(s->ppos, 0, Ls * s->cap * sizeof(int32_t)));
  if (!rc) rc = check(hipMemset(s->move_count, 0, Ls * sizeof(int32_t)));
  if (!rc) rc = check(hipDeviceSynchronize());
  if (!rc) rc = check(hipEventCreateWithFlags(&s->stream_ev, hipEventDisableTiming));
  // The static scratch of statekv_prefill_frame_static on this device (a
  // failure here is reported by that entry point, which retries).
  if (!rc) (void)resolve_static_scratch(s->device);
  if (!rc) {
    s->ev_ok = true;
    for (auto& ring : s->ev)
      for (auto& e : ring)
        if (s->ev_ok && (hipEventCreate(&e[0]) != hipSuccess || hipEventCreate(&e[1]) != hipSuccess))
          s->ev_ok = false;
  }
  if (rc) {
    release(s);
    free(s);
    return rc;
  }
  // Softmax scale: sigma = mscale^2 / sqrt(d), mscale = 0.1 ln(alpha) + 1 (1 when
  // alpha = 1), applied as 2^(sigma log2(e) x) with the constant split in two
  // floats so that the score pass carries it to fp64 accuracy.
  const double mscale = alpha <= 1.0f ? 1.0 : 0.1 * log((double)alpha) + 1.0;
  const double cexp = mscale * mscale / sqrt((double)s->D) * M_LOG2E;
  s->c_hi = (float)cexp;
  s->c_lo = (float)(cexp - (double)s->c_hi);
  *out = s;
  return STATEKV_OK;
}

int statekv_set_stream(statekv_state* s, void* hip_stream) {
  if (!s) return STATEKV_EINVAL;
  const hipStream_t next = (hipStream_t)hip_stream;
  if (next == s->stream) return STATEKV_OK;
  // Work already queued on the old stream (earlier frames, pending moves)
  // completes before anything later queued on the new one starts.
  int rc = check(hipSetDevice(s->device));
  if (!rc) rc = check(hipEventRecord(s->stream_ev, s->stream));
  if (!rc) rc = check(hipStreamWaitEvent(next, s->stream_ev, 0));
  if (rc) return rc;
  s->stream = next;
  return STATEKV_OK;
}

int statekv_set_flags(statekv_state* s, uint32_t flags) {
  if (!s) return STATEKV_EINVAL;
  if (flags & ~(STATEKV_FLAG_ALWAYS_SCORE | STATEKV_FLAG_KERNEL_TIMING | STATEKV_FLAG_RECENT_WINDOW))
    return STATEKV_EINVAL;
  s->flags = flags;
  return STATEKV_OK;
}

}  // extern "C"

namespace {

// Argument checks of a frame step; 0 if the frame may run.
int check_frame(const statekv_state* s, const void* Q, const void* K, const void* V, int32_t n,
                const void* O) {
  if (!s || !Q || !K || !V || !O) return STATEKV_EINVAL;
  if (n != s->frames_done || s->text_done > 0) return STATEKV_EORDER;
  if (n >= s->cfg.max_frames) return STATEKV_ECAPACITY;
  const int P = s->count + s->T;
  const bool scored = (P > s->B && !(s->flags & STATEKV_FLAG_RECENT_WINDOW)) ||
                      (s->flags & STATEKV_FLAG_ALWAYS_SCORE);
  return STATEKV_OK;
}

// The frame step (arguments already checked, device current) with its
// per-step buffers in w.
// The split merge of a frame step into O.
MergeArgs merge_args(const statekv_state* s, const StepScratch& w, void* O, int splits) {
  MergeArgs m{};
  m.opart = w.opart;
  m.epart = w.epart;
  m.mpart = w.mpart;
  m.lpart = w.lpart;
  m.out = O;
  m.Hkv = s->HkvAll;
  m.R = s->R;
  m.G = s->G;
  m.Hq = s->Hq;
  m.S = splits;
  m.ss = s->stat_ss;
  m.lh = s->Hkv;
  m.out_ls = (int64_t)s->T * s->Hq * s->D;
  return m;
}

int frame_step(statekv_state* s, const void* Q, const void* K, const void* V, int32_t n, void* O,
               const StepScratch& w) {
  int rc = STATEKV_OK;
  const int k0 = s->count;   // the state after the last frame's (possibly pending) selection
  const int P = k0 + s->T;
  const hipStream_t st = s->stream;
  const bool evict = P > s->B;
  const bool recent = (s->flags & STATEKV_FLAG_RECENT_WINDOW) != 0;
  const bool scored = (evict && !recent) || (s->flags & STATEKV_FLAG_ALWAYS_SCORE);
  // Rows of this frame: right after the state, or, while the last frame's
  // evictions are pending (its kept rows at or beyond B are about to move),
  // the frame region its rows do not occupy.
  const bool prev_moves = s->sel_pending && s->sel_mode == kSelEvict;
  const int F = prev_moves ? (s->frame_base == (int)s->B + s->T ? (int)s->B : (int)s->B + s->T) : k0;
  const int foff = F - k0;
  const size_t cs_n = (size_t)s->L * s->cap;

  // 1. The last frame's Top-B decision and moves, beside this frame's RoPE and
  //    appends (disjoint rows), which also clear this frame's column sums.
  {
    KernelTimer tm(s, STATEKV_K_ROPE);
    RopeArgs a{};
    a.q = Q;
    a.k = K;
    a.v = V;
    a.table = s->rope_tab;
    a.qrot = w.qrot;
    a.kpool = s->kpool;
    a.vpool = s->vpool;
    a.pool_pos = s->ppos;
    a.dk = s->dk;
    a.dv = s->dv;
    a.nonfinite = s->nonfinite;
    a.pos0 = n * s->T;
    a.T = s->T;
    a.Hq = s->Hq;
    a.Hkv = s->Hkv;
    a.G = s->G;
    a.cap = s->cap;
    a.frame_base = F;
    a.rope_pairs = rope_pairs_for(s->T, s->Hq, s->Hkv, s->D, s->esize, s->L);
    a.rope_blocks = rope_blocks(s->T, s->Hq, s->Hkv, s->D, s->esize, a.rope_pairs);
    a.det_ls = s->det_ls;
    if (scored) {
      a.clear = s->colsum + (size_t)s->colsum_next * cs_n;
      a.clear_n = P;
    }
    if (s->sel_pending) {
      a.nsel = 1;
      a.sel = sel_args(s);
    }
    rc = check(launch_frame(s->dt, s->D, a, s->L, st, tm.lt));
    tm.done();
    if (rc) return rc;
    s->sel_pending = false;
  }
  // 2. Attention pass 1, split over keys.
  int splits, kps;
  attn_geometry(s, P, &splits, &kps);
  {
    KernelTimer tm(s, STATEKV_K_ATTN);
    AttnArgs a{};
    a.qrot = w.qrot;
    a.kpool = s->kpool;
    a.vpool = s->vpool;
    a.opart = w.opart;
    a.epart = w.epart;
    a.mpart = w.mpart;
    a.lpart = w.lpart;
    a.c_hi = s->c_hi;
    a.R = s->R;
    a.G = s->G;
    a.cap = s->cap;
    a.P = P;
    a.k0 = k0;
    a.foff = foff;
    a.kps = kps;
    a.ss = s->stat_ss;
    a.Hkv = s->HkvAll;
    a.lh = s->Hkv;
    // Head-major work-group order for a single layer with many KV heads:
    // measured faster at 8 heads (qwen3vl_2b-like and stress shapes), slower
    // at 2 (ivl3_1b-like); on 28-layer stacks it left pass 1 unchanged and
    // made the next frame launch slower.
    a.head_major = s->L == 1 && s->HkvAll >= kAttnHeadMajorMin ? 1 : 0;
    a.kv_hs = (int64_t)s->cap * s->D;
    a.kv_rs = s->D;
    a.kv_ls = (int64_t)s->Hkv * s->cap * s->D;
    rc = check(launch_attn(s->dt, s->D, a, s->attn_tiles, splits, st, tm.lt));
    tm.done();
    if (rc) return rc;
  }
  // 3. The merge of the key splits into O and, for a scored frame, the score
  //    pass.  Under the recency policy an evicting frame's decision needs
  //    positions only: it is made here, beside the merge, instead of waiting
  //    for the next frame.
  const bool decide_now = evict && recent && !scored;
  if (decide_now) {
    KernelTimer tm(s, STATEKV_K_SCORE);
    SelectMergeArgs a{};
    a.mg = merge_args(s, w, O, splits);
    a.sel = sel_args_for(s, P, k0, foff, kSelEvict, 1, 0);
    a.layers = s->L;
    rc = check(launch_select_merge(s->dt, s->D, a, merge_wgs((int64_t)s->HkvAll * s->R), st, tm.lt));
    tm.done();
    if (rc) return rc;
  } else {
    KernelTimer tm(s, STATEKV_K_SCORE);
    ScoreMergeArgs a{};
    a.mg = merge_args(s, w, O, splits);
    a.merge_wgs = merge_wgs((int64_t)s->HkvAll * s->R);
    int waves = s->dt == Dt::BF16 ? 8 : 4;
    if (scored) {
      int key_blocks, rsplits, rps;
      score_geometry(s, P, &key_blocks, &rsplits, &rps, &waves);
      ScoreArgs& c = a.sc;
      c.qrot = w.qrot;
      c.kpool = s->kpool;
      c.mpart = w.mpart;
      c.lpart = w.lpart;
      c.S = splits;
      c.ss = s->stat_ss;
      c.colsum = s->colsum + (size_t)s->colsum_next * cs_n;
      c.c_hi = s->c_hi;
      c.c_lo = s->c_lo;
      c.R = s->R;
      c.G = s->G;
      c.cap = s->cap;
      c.P = P;
      c.k0 = k0;
      c.foff = foff;
      c.rps = rps;
      c.Hkv = s->HkvAll;
      c.lh = s->Hkv;
      a.key_blocks = key_blocks;
      a.rsplits = rsplits;
      // The merge rides on the score work-groups whose key block starts
      // before k0, each taking an equal slice of its row range's (row, 4
      // dims) tasks, when a slice fits in one task per thread.
      const int bnk = score_keys_per_wg(s->dt, waves);
      const int mkb = std::min(key_blocks, ceil_div(k0, bnk));
      if (mkb > 0 && score_merge_fusable(s->dt, s->D, waves)) {
        const int mtpw = ceil_div(ceil_div(rps * (s->D / 4), mkb), 32) * 32;
        if (mtpw <= 64 * waves) {
          a.fused = 1;
          a.mkb = mkb;
          a.mtpw = mtpw;
          a.merge_wgs = 0;
        }
      }
    }
    rc = check(launch_score_merge(s->dt, s->D, a, waves, st, tm.lt));
    tm.done();
    if (rc) return rc;
  }
  // Otherwise the Top-B decision of this frame waits for the next frame's
  // first launch (or a view of the state).
  if ((evict || scored) && !decide_now) {
    s->sel_pending = true;
    s->sel_P = P;
    s->sel_k0 = k0;
    s->sel_foff = foff;
    s->sel_mode = evict ? kSelEvict : kSelScores;
    s->sel_recent = recent ? 1 : 0;
    s->sel_colsum = scored ? s->colsum_next : 0;
  }
  s->frame_base = F;
  if (scored) {
    s->colsum_last = s->colsum_next;
    s->colsum_next ^= 1;
    s->score_frame = n;
    s->score_pool = P;
    s->score_k0 = k0;
    s->score_foff = foff;
    s->score_evicted = evict;
  } else if (evict) {
    s->score_frame = -1;   // the pool changes: earlier scores no longer describe it
  }
  s->count = evict ? (int)s->B : P;
  s->frames_done = n + 1;
  s->ev_slot = (s->ev_slot + 1) % statekv_state::kRing;
  return STATEKV_OK;
}

}  // namespace

extern "C" {

int statekv_prefill_frame(statekv_state* s, const void* Q, const void* K, const void* V,
                          int32_t n, void* O) {
  int rc = check_frame(s, Q, K, V, n, O);
  if (!rc) rc = check(hipSetDevice(s->device));
  if (rc) return rc;
  return frame_step(s, Q, K, V, n, O, s->work[n & 1]);
}

int statekv_prefill_frame_static(statekv_state* s, const void* Q, const void* K, const void* V,
                                 int32_t n, void* O) {
  int rc = check_frame(s, Q, K, V, n, O);
  if (rc) return rc;
  if (carve_step_scratch(s, nullptr, nullptr) > (size_t)STATEKV_STATIC_SCRATCH_BYTES)
    return STATEKV_ESCRATCH;
  rc = check(hipSetDevice(s->device));
  if (!rc) rc = resolve_static_scratch(s->device);
  if (rc) return rc;
  StepScratch w;
  carve_step_scratch(s, static_cast<char*>(g_scratch_ptr[s->device]), &w);
  return frame_step(s, Q, K, V, n, O, w);
}

int statekv_decode(statekv_state* s, const void* Q, const void* K, const void* V, int32_t t,
                   void* O) {
  if (!s || !Q || !K || !V || !O) return STATEKV_EINVAL;
  if (t < 1 || t > s->T) return STATEKV_EINVAL;
  if ((int64_t)s->text_done + t > s->cfg.max_text) return STATEKV_ECAPACITY;
  int rc = check(hipSetDevice(s->device));
  if (rc) return rc;
  const hipStream_t st = s->stream;
  const int P0 = s->frames_done * s->T + s->text_done;   // keys before the text chunk
  const int P = P0 + t;
  const int R = s->G * t;
  if (R <= 32) {
    // Few query rows: one kernel streams D (rotating the text tokens and
    // appending them to D itself), then the merge of its key splits.
    int splits, kps;
    decode_geometry(s, P, &splits, &kps);
    {
      KernelTimer tm(s, STATEKV_K_DEC_ATTN);
      DecodeArgs a{};
      a.q = Q;
      a.k = K;
      a.v = V;
      a.table = s->rope_tab;
      a.nonfinite = s->nonfinite;
      a.dk = s->dk;
      a.dv = s->dv;
      a.opart = s->dec_opart;
      a.mpart = s->dec_mpart;
      a.lpart = s->dec_lpart;
      a.out = O;
      a.c_hi = s->c_hi;
      a.R = R;
      a.G = s->G;
      a.Hq = s->Hq;
      a.Hkv = s->Hkv;
      a.P = P;
      a.k0 = P0;
      a.kps = kps;
      a.S = splits;
      a.L = s->L;
      a.det_ls = s->det_ls;
      rc = check(launch_decode(s->dt, s->D, a, st, tm.lt));
      tm.done();
      if (rc) return rc;
    }
    if (splits > 1) {
      KernelTimer tm(s, STATEKV_K_DEC_MERGE);
      DecodeMergeArgs a{};
      a.opart = s->dec_opart;
      a.mpart = s->dec_mpart;
      a.lpart = s->dec_lpart;
      a.out = O;
      a.R = R;
      a.G = s->G;
      a.Hq = s->Hq;
      a.Hkv = s->Hkv;
      a.S = splits;
      a.L = s->L;
      rc = check(launch_decode_merge(s->dt, s->D, a, st, tm.lt));
      tm.done();
      if (rc) return rc;
    }
  } else {
    // A longer chunk (a prompt): the frame step's kernels over D.  RoPE and
    // append, attention pass 1 with D's strides, the merge of the splits.
    {
      KernelTimer tm(s, STATEKV_K_DEC_ROPE);
      RopeArgs a{};
      a.q = Q;
      a.k = K;
      a.v = V;
      a.table = s->rope_tab;
      a.qrot = s->work[0].qrot;
      a.dk = s->dk;
      a.dv = s->dv;
      a.nonfinite = s->nonfinite;
      a.pos0 = P0;
      a.T = t;
      a.Hq = s->Hq;
      a.Hkv = s->Hkv;
      a.G = s->G;
      a.cap = s->cap;
      a.rope_pairs = rope_pairs_for(t, s->Hq, s->Hkv, s->D, s->esize, s->L);
      a.rope_blocks = rope_blocks(t, s->Hq, s->Hkv, s->D, s->esize, a.rope_pairs);
      a.det_ls = s->det_ls;
      rc = check(launch_frame(s->dt, s->D, a, s->L, st, tm.lt));
      tm.done();
      if (rc) return rc;
    }
    int tiles, splits, kps;
    chunk_geometry(s, t, P, &tiles, &splits, &kps);
    {
      KernelTimer tm(s, STATEKV_K_DEC_ATTN);
      AttnArgs a{};
      a.qrot = s->work[0].qrot;
      a.kpool = s->dk;
      a.vpool = s->dv;
      a.opart = s->work[0].opart;
      a.epart = s->work[0].epart;
      a.mpart = s->work[0].mpart;
      a.lpart = s->work[0].lpart;
      a.c_hi = s->c_hi;
      a.R = R;
      a.G = s->G;
      a.cap = s->cap;
      a.P = P;
      a.k0 = P0;
      a.foff = 0;
      a.kps = kps;
      a.ss = splits;   // the chunk's statistics stride (chunk_split_cap sized it)
      a.Hkv = s->HkvAll;
      a.lh = s->Hkv;
      a.kv_hs = s->D;
      a.kv_rs = (int64_t)s->Hkv * s->D;
      a.kv_ls = s->det_ls;
      rc = check(launch_attn(s->dt, s->D, a, tiles, splits, st, tm.lt));
      tm.done();
      if (rc) return rc;
    }
    {
      KernelTimer tm(s, STATEKV_K_DEC_MERGE);
      ScoreMergeArgs a{};
      MergeArgs& m = a.mg;
      m.opart = s->work[0].opart;
      m.epart = s->work[0].epart;
      m.mpart = s->work[0].mpart;
      m.lpart = s->work[0].lpart;
      m.out = O;
      m.Hkv = s->HkvAll;
      m.R = R;
      m.G = s->G;
      m.Hq = s->Hq;
      m.S = splits;
      m.ss = splits;
      m.lh = s->Hkv;
      m.out_ls = (int64_t)t * s->Hq * s->D;
      a.merge_wgs = merge_wgs((int64_t)s->HkvAll * R);
      rc = check(launch_score_merge(s->dt, s->D, a, s->dt == Dt::BF16 ? 8 : 4, st, tm.lt));
      tm.done();
      if (rc) return rc;
    }
  }
  s->text_done += t;
  s->ev_slot = (s->ev_slot + 1) % statekv_state::kRing;
  return STATEKV_OK;
}

int statekv_compressed_view(const statekv_state* s, statekv_view* out) {
  if (!s || !out) return STATEKV_EINVAL;
  int rc = check(hipSetDevice(s->device));
  if (!rc) rc = resolve_pending_selection(s);
  if (!rc) rc = sync_state(s);
  if (!rc) rc = read_nonfinite(s);
  if (rc) return rc;
  memset(out, 0, sizeof(*out));
  out->k = s->kpool;
  out->v = s->vpool;
  out->pos = s->ppos;
  out->count = s->count;
  out->head_stride = (int64_t)s->cap * s->D;
  out->token_stride = s->D;
  out->n_kv_heads = s->Hkv;
  out->head_dim = s->D;
  out->dtype = s->cfg.dtype;
  out->frames_done = s->frames_done;
  out->n_layers = s->L;
  out->layer_stride = (int64_t)s->Hkv * s->cap * s->D;
  out->pos_layer_stride = s->cap;
  return STATEKV_OK;
}

int statekv_detailed_view(const statekv_state* s, statekv_view* out) {
  if (!s || !out) return STATEKV_EINVAL;
  int rc = sync_state(s);
  if (!rc) rc = read_nonfinite(s);
  if (rc) return rc;
  memset(out, 0, sizeof(*out));
  out->k = s->dk;
  out->v = s->dv;
  out->pos = nullptr;
  out->count = (int64_t)s->frames_done * s->T + s->text_done;
  out->head_stride = s->D;
  out->token_stride = (int64_t)s->Hkv * s->D;
  out->n_kv_heads = s->Hkv;
  out->head_dim = s->D;
  out->dtype = s->cfg.dtype;
  out->frames_done = s->frames_done;
  out->n_layers = s->L;
  out->layer_stride = s->det_ls;
  out->pos_layer_stride = 0;
  return STATEKV_OK;
}

int statekv_scores(const statekv_state* s, statekv_scores_view* out) {
  if (!s || !out) return STATEKV_EINVAL;
  int rc = check(hipSetDevice(s->device));
  if (!rc) rc = sync_state(s);
  if (rc) return rc;
  memset(out, 0, sizeof(*out));
  out->frame = s->score_frame;
  if (s->score_frame < 0) return STATEKV_OK;
  // Scores from the frame's column sums, keep flags from its move list, and
  // positions at scoring time: those of the pool rows, except in the slots
  // that the selection's moves have filled since.
  rc = resolve_pending_selection(s);
  if (!rc) {
    ScoreViewArgs a{};
    a.colsum = s->colsum + (size_t)s->colsum_last * s->L * s->cap;
    a.pool_pos = s->ppos;
    a.evicted_pos = s->evicted_pos;
    a.move_dst = s->move_dst;
    a.move_src = s->move_src;
    a.move_count = s->move_count;
    a.scores = s->scores;
    a.keep_flag = s->keep_flag;
    a.score_pos = s->score_pos;
    a.score_scale = 1.0 / ((double)(1ull << kScoreFracBits) * (double)s->Hq * (double)s->T);
    a.P = s->score_pool;
    a.B = s->B;
    a.k0 = s->score_k0;
    a.foff = s->score_foff;
    a.moved = s->score_evicted ? 1 : 0;
    a.cap = s->cap;
    a.list_stride = s->T;
    rc = check(launch_score_view(a, s->L, s->stream));
  }
  if (!rc) rc = check(hipStreamSynchronize(s->stream));
  if (rc) return rc;
  out->scores = s->scores;
  out->pool_pos = s->score_pos;
  out->keep_flag = s->keep_flag;
  out->pool = s->score_pool;
  out->kept = std::min(s->score_pool, (int)s->B);
  out->n_layers = s->L;
  out->layer_stride = s->cap;
  return STATEKV_OK;
}

int statekv_kernel_times(statekv_state* s, float* ms, int32_t* launches, int32_t n_kernels,
                         int32_t reset) {
  if (!s || n_kernels < 0) return STATEKV_EINVAL;
  const int rc = sync_state(s);
  if (rc) return rc;
  for (int r = 0; r < statekv_state::kRing; ++r)
    for (int k = 0; k < STATEKV_K_COUNT; ++k) drain_slot(s, r, k);
  const int n = std::min<int>(n_kernels, STATEKV_K_COUNT);
  for (int k = 0; k < n; ++k) {
    if (ms) ms[k] = s->ktime_ms[k];
    if (launches) launches[k] = s->klaunch[k];
  }
  if (reset) {
    memset(s->ktime_ms, 0, sizeof(s->ktime_ms));
    memset(s->klaunch, 0, sizeof(s->klaunch));
  }
  return STATEKV_OK;
}

void statekv_destroy(statekv_state* s) {
  if (!s) return;
  (void)hipSetDevice(s->device);
  (void)hipStreamSynchronize(s->stream);
  release(s);
  free(s);
}

}  // extern "C"
