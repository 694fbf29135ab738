// Internal declarations shared by the StateKV runtime and its HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace statekv {

enum class Dt : int { BF16 = 1, F32 = 2 };

// Per-frame arguments of the RoPE + append kernel.
struct RopeArgs {
  const void* q;          // [T][Hq][d]
  const void* k;          // [T][Hkv][d]
  const void* v;          // [T][Hkv][d]
  const double* inv_freq; // [d/2] scaled RoPE frequencies
  void* qrot;             // [Hkv][G*T][d], row r = token*G + head-in-group
  void* kpool;            // [Hkv][cap][d]: state rows, then this frame's rows
  void* vpool;            // [Hkv][cap][d]
  int32_t* pool_pos;      // [cap]
  void* dk;               // [max_frames*T][Hkv][d]
  void* dv;               // [max_frames*T][Hkv][d]
  int32_t* nonfinite;     // set to 1 when an input element is NaN or Inf
  int32_t n, T, Hq, Hkv, G, cap, k0;
};

// Attention pass 1: one work-group per (row tile, KV head, key split).
struct AttnArgs {
  const void* qrot;       // [Hkv][R][d]
  const void* kpool;      // [Hkv][cap][d]
  const void* vpool;      // [Hkv][cap][d]
  float* opart;           // [S][Hkv][R][d] unnormalised partial outputs
  float* mpart;           // [S][Hkv][R] partial row maxima (scaled, log2 units)
  double* lpart;          // [S][Hkv][R] partial row sums of exp2
  float c_hi, c_lo;       // sigma * log2(e) split into two floats
  int32_t R, G, cap, P, k0, kps, Hkv;
};

struct CombineArgs {
  const float* opart;
  const float* mpart;
  const double* lpart;
  void* out;              // [T][Hq][d]
  float* row_m;           // [Hkv][R] final row maxima
  float* row_rinv;        // [Hkv][R] 1 / row sums
  int32_t R, G, Hq, Hkv, S;
};

// Score pass: one work-group per (key block, KV head, row split).
struct ScoreArgs {
  const void* qrot;
  const void* kpool;
  const float* row_m;
  const float* row_rinv;
  double* colpart;        // [RS][Hkv][cap] per-key column sums
  float c_hi, c_lo;
  int32_t R, G, cap, P, k0, rps, Hkv;
};

struct SelectArgs {
  const double* colpart;  // [nparts][cap]
  float* scores;          // [P]
  int32_t* keep;          // [B]
  int32_t nparts, cap, P, B;
  double denom;           // Hq * T
};

struct GatherArgs {
  const void* kcur;
  const void* vcur;
  const int32_t* pcur;
  void* knext;
  void* vnext;
  int32_t* pnext;
  const int32_t* keep;
  int32_t Hkv, cap, B, row_bytes;
};

constexpr int kAttnThreads = 256;
constexpr int kAttnBN = 64;          // keys per block in pass 1
constexpr int kSelectThreads = 1024;
constexpr int kMaxPool = 32768;      // B + T limit of the single-work-group select
constexpr int kSelectBins = 4096;

// Rows handled by one pass-1 work-group / keys by one score work-group.
int attn_rows_per_wg(Dt dt);
int score_keys_per_wg(Dt dt);

hipError_t launch_rope(Dt dt, int d, const RopeArgs& a, hipStream_t s);
hipError_t launch_attn(Dt dt, int d, const AttnArgs& a, int row_tiles, int splits, hipStream_t s);
hipError_t launch_combine(Dt dt, int d, const CombineArgs& a, hipStream_t s);
hipError_t launch_score(Dt dt, int d, const ScoreArgs& a, int key_blocks, int rsplits, hipStream_t s);
hipError_t launch_select(const SelectArgs& a, hipStream_t s);
hipError_t launch_gather(const GatherArgs& a, hipStream_t s);

}  // namespace statekv
