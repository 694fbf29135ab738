// Internal declarations shared by the StateKV runtime and its HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace statekv {

enum class Dt : int { BF16 = 1, F32 = 2 };

constexpr int kAttnThreads = 256;
constexpr int kAttnBN = 64;          // keys per LDS block in attention pass 1
constexpr int kMaxSplits = 24;       // key splits of a frame's pass 1 (merges unroll over them)
constexpr int kMaxMergeSplits = 512; // key splits of a text chunk's pass 1 (merged in a loop)
constexpr int kScoreMaxRows = 512;   // rows of one score work-group (row statistics in LDS)
constexpr int kSelectThreads = 1024;  // frame launch: selection and RoPE work-groups
constexpr int kMaxPool = 32768;      // B + T limit of the single-work-group select
constexpr int kSelectBins = 4096;
constexpr int kSelCand = kSelectThreads;  // boundary candidates resolved by rank counting (one per thread)
constexpr int kDecodeMaxSplits = 1024;  // key splits of the text-phase attention
// Column sums are accumulated as unsigned 64-bit fixed point with this many
// fractional bits: integer addition is associative, so the sum does not depend
// on the order in which work-groups add their partials.  A sum is at most
// Hq*T (every weight 1), which stays below 2^63 for Hq*T <= 2^22.
constexpr int kScoreFracBits = 40;
constexpr int64_t kMaxRowsTimesHeads = 1 << 22;
constexpr int kMaxLayers = 256;      // layers of one state (a stack stepped together)

// Cos / sin table of the scaled RoPE angles, built once per state.
struct RopeTableArgs {
  const double* inv_freq;  // [d/2] scaled frequencies
  float2* table;           // [npos][d/2] (cos, sin) rounded to fp32
  int32_t npos, half;
};

// Top-B decision of a scored (or evicting) frame and the moves it implies:
// the evicted slots below B receive, in ascending order, the kept rows at or
// beyond B (K and V of every KV head, and their positions; the position a slot
// held is saved in evicted_pos[slot]).  One work-group per layer makes the
// decision and performs its moves, in the next frame's first launch (beside
// that frame's RoPE work-groups, which write the other frame region) or in a
// launch of its own before a view of the state.  Pointers address layer 0 of a
// stack; layer l's arrays follow at fixed strides: cap (colsum, pool_pos), B
// (evicted_pos), list_stride (move lists), 1 (move_count), Hkv*cap rows (pools).
struct SelArgs {
  const unsigned long long* colsum;  // [cap] fixed-point column sums of the frame
  int32_t* pool_pos;           // [cap] positions of the pool rows (by row)
  int32_t* evicted_pos;        // [B] out
  int32_t* move_dst;           // [T] out: evicted state slots (< B), ascending
  int32_t* move_src;           // [T] out: rows of the kept frame tokens at or beyond B, ascending
  int32_t* move_count;         // [1] out
  void* kpool;
  void* vpool;
  int32_t P, B, mode;          // mode: kSelScores or kSelEvict
  int32_t recent;              // 1: keep the B most recent candidates (positions), not the best scores
  int32_t k0, foff;            // pool index -> row
  double score_scale;          // 2^-kScoreFracBits / (Hq * T)
  int32_t Hkv, cap, row_bytes, list_stride;   // Hkv: KV heads per layer
};
constexpr int kSelScores = 1;  // scores only, everything kept
constexpr int kSelEvict = 2;   // scores (or positions) and Top-B

// Arguments of the frame launch: the RoPE + append work for T tokens at
// stream positions pos0..pos0+T-1 (a frame, or a chunk of text tokens), and
// in front of it (nsel = 1) the previous frame's selection work-group.  The
// RoPE work-groups also clear the column sums this frame's score pass will
// accumulate.  Text tokens go to D only (kpool, vpool and pool_pos null).
// Layer l of a stack (grid y) finds its inputs and qrot T*H*d elements per
// layer further, its pool Hkv*cap*d, pool_pos cap and D det_ls.
struct RopeArgs {
  const void* q;          // [T][Hq][d]
  const void* k;          // [T][Hkv][d]
  const void* v;          // [T][Hkv][d]
  const float2* table;    // [positions][d/2]
  void* qrot;             // [Hkv][G*T][d], row r = token*G + head-in-group
  void* kpool;            // [Hkv][cap][d]: state rows; this frame's rows at frame_base
  void* vpool;            // [Hkv][cap][d]
  int32_t* pool_pos;      // [cap] position of every row
  void* dk;               // [positions][Hkv][d]
  void* dv;               // [positions][Hkv][d]
  int32_t* nonfinite;     // set to 1 when an input element is NaN or Inf
  int32_t pos0, T, Hq, Hkv, G, cap, frame_base, rope_blocks;
  int32_t rope_pairs;     // rotation pairs per RoPE task (rope_pairs_for)
  int64_t det_ls;         // elements between layers of dk / dv
  unsigned long long* clear;  // [L][cap] column sums cleared (null: none)
  int32_t clear_n;            // elements per layer
  int32_t nsel;           // selection work-groups per layer in front of the RoPE ones (0 or 1)
  SelArgs sel;
};

// Pool index j (state slots, then the frame's tokens) -> row of the pool
// arrays: the frame's tokens sit at frame_base = k0 + foff.
__host__ __device__ inline int pool_row(int j, int k0, int foff) { return j < k0 ? j : j + foff; }

// Attention pass 1: one work-group per (row tile, KV head, key split).
// Per split and row it leaves (m_s, l_s, O_s) with m_s an integer (log2 units)
// so that merging splits scales by exact powers of two.  The KV heads of a
// stack's layers are numbered layer-major (head = layer*lh + head in layer):
// qrot and the partials are head-major over all of them; keys and values of
// head (l, h) start at l*kv_ls + h*kv_hs.
struct AttnArgs {
  const void* qrot;       // [Hkv][R][d]
  const void* kpool;      // [Hkv][cap][d]
  const void* vpool;      // [Hkv][cap][d]
  void* opart;            // [S][Hkv][R][d] unnormalised partial outputs, lane-order groups
                          // of 32 rows: fp16 scaled by 2^-e_s for bf16 streams, else fp32
  int8_t* epart;          // [S][Hkv][R] e_s of the fp16 partials
  float* mpart;           // reference maxima (integers, -inf if empty) and partial row
  double* lpart;          // sums of 2^(x*c - m_s), per (row, split): split-major inside
                          // groups of 32 rows
  float c_hi;             // sigma * log2(e) rounded to fp32
  int32_t R, G, cap, P, k0, foff, kps, Hkv;   // Hkv: KV heads of all layers
  int32_t ss;             // split stride of the statistics (maximum splits)
  int32_t lh;             // KV heads per layer
  int32_t head_major;     // work-group order: 1 = (row tile, split, KV head), 0 = (row tile, KV head, split)
  // Element strides of the key / value rows: between KV heads and between
  // rows.  The pool is [Hkv][cap][d] (cap*d, d); the detailed cache, read by
  // text chunks, is [positions][Hkv][d] (d, Hkv*d).
  int64_t kv_hs, kv_rs;
  int64_t kv_ls;          // elements between layers of the key / value arrays
};

// Score pass: one work-group per (key block, KV head, row split); KV heads
// of all layers of a stack, layer-major as in pass 1.
struct ScoreArgs {
  const void* qrot;
  const void* kpool;
  const float* mpart;
  const double* lpart;
  unsigned long long* colsum;  // [L][cap] column sums, fixed point (2^-kScoreFracBits units)
  float c_hi, c_lo;            // sigma * log2(e) = c_hi + c_lo
  int32_t R, G, cap, P, k0, foff, rps, Hkv, S, ss;
  int32_t lh;                  // KV heads per layer
};

// Text-phase attention over the detailed cache D (token-major rows) for at
// most 32 query rows per KV head: one work-group per (KV head, key split),
// over the KV heads of all L layers of a stack (grid x = L*Hkv, layer-major).
// Pointers address layer 0: layer l's inputs and output follow t*H*d
// elements per layer further, its D rows det_ls further; the partials are
// head-major over all L*Hkv heads.
// Its NW waves take the 32-key sub-tiles of every block of 32*NW keys and are
// merged in LDS at the end.  With one split the work-group writes O;
// otherwise it leaves (m_s, l_s, O_s) for the merge kernel.
struct DecodeArgs {
  // The text tokens' projected inputs: the kernel rotates queries and keys
  // itself (R = G*t <= 32 rows per KV head, one row tile) and appends the
  // rotated keys and the values to D.
  const void* q;          // [t][Hq][d]
  const void* k;          // [t][Hkv][d]
  const void* v;          // [t][Hkv][d]
  const float2* table;    // [positions][d/2]
  int32_t* nonfinite;
  const void* dk;         // [positions][Hkv][d]
  const void* dv;         // [positions][Hkv][d]
  float* opart;           // [S][Hkv][R][d] unnormalised partial outputs (S > 1)
  float* mpart;           // [S][Hkv][R] reference maxima (integers, log2 units)
  double* lpart;          // [S][Hkv][R] row sums of 2^(x*c - m_s)
  void* out;              // [t][Hq][d] (S == 1)
  float c_hi;             // sigma * log2(e) rounded to fp32
  int32_t R, G, Hq, Hkv, P, k0, kps, S;  // P = k0 + t keys; k0 keys precede the text
  int32_t L;              // layers
  int64_t det_ls;         // elements between layers of dk / dv
};

struct DecodeMergeArgs {
  const float* opart;
  const float* mpart;
  const double* lpart;
  void* out;              // [L][t][Hq][d]
  int32_t R, G, Hq, Hkv, S, L;   // Hkv per layer
};

// Merge of the key splits of pass 1 into O, one work-group per group of 32
// flat rows (flat row = g*R + r over the KV heads of all layers).
struct MergeArgs {
  const void* opart;
  const int8_t* epart;
  const float* mpart;
  const double* lpart;
  void* out;                   // [L][T][Hq][d]
  int32_t Hkv, R, G, Hq, S, ss;   // Hkv: KV heads of all layers (layer-major)
  int32_t lh;                  // KV heads per layer
  int64_t out_ls;              // elements of out between layers
};

// The launch after pass 1: merge work-groups first (merge_wgs, a multiple of
// the XCD count), then the score pass's (key block, KV head, row split)
// work-groups.  Either part may be empty.
// With fused = 1 there are no merge work-groups: the score work-groups whose
// key block starts before k0 (the first mkb of each (KV head, row split))
// also merge the split partials of their row range, mtpw (row, 4 dims) tasks
// each, rows fastest; such a block's row statistics cover its whole range.
// The launch after pass 1 under the recency policy: the frame's own eviction
// decision (positions only) and moves, one work-group per layer, beside the
// split merge (merge groups numbered across the stack's layers).
struct SelectMergeArgs {
  SelArgs sel;
  MergeArgs mg;
  int32_t layers;
};

struct ScoreMergeArgs {
  ScoreArgs sc;
  MergeArgs mg;
  int32_t merge_wgs, key_blocks, rsplits;
  int32_t fused, mkb, mtpw;
};

// Start / stop events that the dispatch itself records (kernel timing): the
// elapsed time between them is the kernel's execution, without the launch
// gaps that separately recorded events would include.  Null: not timed.
struct LaunchTiming {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// Rows handled by one pass-1 work-group / keys by one score work-group.
int attn_rows_per_wg(Dt dt, int d);
// Keys per LDS block of pass 1 (key splits are whole blocks).
int attn_block_keys(Dt dt, int d);
int score_keys_per_wg(Dt dt, int waves);
// Score work-groups resident per CU (occupancy of the instantiation in use).
int score_wgs_per_cu(Dt dt, int d);
int score8_wgs_per_cu(int d);
// Rotation pairs per RoPE task for a launch over `layers` layers of T
// tokens: 4, or 16 bytes of each half of a head (8 for bf16) when the launch
// is large enough to be bound by memory bandwidth rather than latency.
int rope_pairs_for(int T, int Hq, int Hkv, int d, int esize, int layers);
// Work-groups of the RoPE part of the frame launch for T tokens.
int rope_blocks(int T, int Hq, int Hkv, int d, int esize, int pairs);

hipError_t launch_rope_table(const RopeTableArgs& a, hipStream_t s);
// The frame launch (RoPE + append, the previous frame's selection); with
// a.rope_blocks = 0 only the selection.
hipError_t launch_frame(Dt dt, int d, const RopeArgs& a, int layers, hipStream_t s,
                        const LaunchTiming& tm = {});
hipError_t launch_attn(Dt dt, int d, const AttnArgs& a, int row_tiles, int splits, hipStream_t s,
                       const LaunchTiming& tm = {});
// Recency policy: the frame's decision and moves beside the split merge.
hipError_t launch_select_merge(Dt dt, int d, const SelectMergeArgs& a, int merge_groups, hipStream_t s,
                               const LaunchTiming& tm = {});
// Score pass (with `waves` waves per work-group) and merge in one launch.  The
// merge rides on the score work-groups (fused) only where score_merge_fusable:
// bf16 with 8 waves, the single-layer grids resident all at once, where
// separate merge work-groups would push score work-groups into a second round
// (the 4-wave kernel has no registers to spare for the merge at d = 128).
hipError_t launch_score_merge(Dt dt, int d, const ScoreMergeArgs& a, int waves, hipStream_t s,
                              const LaunchTiming& tm = {});
// Work-groups of the merge for `rows` flat rows (a multiple of the XCD count).
int merge_wgs(int64_t rows);
inline bool score_merge_fusable(Dt dt, int, int waves) { return dt == Dt::BF16 && waves == 8; }
// Keys per block of the text-phase attention kernel.
int decode_block_keys(Dt dt);
hipError_t launch_decode(Dt dt, int d, const DecodeArgs& a, hipStream_t s, const LaunchTiming& tm = {});
hipError_t launch_decode_merge(Dt dt, int d, const DecodeMergeArgs& a, hipStream_t s,
                               const LaunchTiming& tm = {});
// Positions of a scored pool of P candidates: the position of its row, or
// for an evicted slot below B that a move has since filled, the saved one.
// The scores view of the last scored pool of P candidates, rebuilt on
// request: scores from the column sums, keep flags from the move lists of
// the selection (a slot below B stays unless it is a move destination; a row
// at or beyond B stays only if it is a move source) and positions (the row's,
// or for a slot below B that a move has since filled, the saved one).  Layer
// l's arrays follow cap (colsum, scores, keep_flag, score_pos, pool_pos), B
// (evicted_pos), list_stride (move lists) and 1 (move_count) elements further.
struct ScoreViewArgs {
  const unsigned long long* colsum;
  const int32_t* pool_pos;
  const int32_t* evicted_pos;
  const int32_t* move_dst;
  const int32_t* move_src;
  const int32_t* move_count;
  float* scores;
  int32_t* keep_flag;
  int32_t* score_pos;
  double score_scale;          // 2^-kScoreFracBits / (Hq * T)
  int32_t P, B, k0, foff, moved, cap, list_stride;
};
hipError_t launch_score_view(const ScoreViewArgs& a, int layers, hipStream_t s);

}  // namespace statekv
