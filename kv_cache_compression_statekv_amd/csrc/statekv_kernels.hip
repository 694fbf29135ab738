// HIP kernels of the StateKV frame step for AMD CDNA4 (gfx950, wave64).
//
// Paper note "Linear Scaling Video VLMs for Long Video Understanding"
// (papernotes.org, ECCV 2026), section 方法详解:
//   rope_wg             关键设计 3: RoPE at the virtual position nT + i with the
//   (in frame_kernel)   fixed scaled frequencies; 整体框架 / flowchart node E:
//                       the frame's K, V are appended to the detailed cache D.
//   attn_fwd_kernel     关键设计 1: the frame's queries attend over
//                       [Kbar_{n-1}; K_n] (bf16 MFMA, online softmax, split
//                       over keys).
//   score_merge_kernel  关键设计 1: merge of pass 1's key splits into the
//                       output; 关键设计 2: score of candidate j = attention
//                       weight paid to j averaged over the frame's queries and
//                       query heads, recomputed with the final row max / sum.
//   frame_kernel        关键设计 3 + flowchart node E: the RoPE work-groups
//                       (rope_wg); 关键设计 2: in front of them, the previous
//                       frame's TopK({s_j}, B), ties kept toward the older
//                       token, and C_n built from the kept candidates (kept
//                       frame rows move into the evicted slots).
//   decode_attn_kernel  整体框架 / 关键设计 1, 3: after the frames, text
//   decode_merge_kernel tokens attend over the whole detailed cache D at the
//                       continuing virtual positions (split over keys, then
//                       merged).  Longer text chunks reuse the frame launch's
//                       RoPE work-groups, attn_fwd_kernel (with D's strides)
//                       and the merge.
//
// Matrix-core tiles use v_mfma_f32_32x32x16_bf16 (bf16 storage) or
// v_mfma_f32_32x32x2_f32 (fp32 storage).  Accumulator layout of a 32x32 tile:
// lane l, register i holds row 8*(i/4) + 4*(l/32) + i%4 and column l%32.
// Operand layout: lane l supplies row (A) / column (B) l%32 and the reduction
// slice [KL*(l/32), KL*(l/32) + KL) of the instruction's KS-deep reduction.
#include "statekv_internal.h"

#include <hip/hip_ext.h>

#include <math.h>
#include <stdlib.h>

#include <algorithm>
#include <type_traits>

namespace statekv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

struct BF16 { typedef uint16_t T; };
struct F32 { typedef float T; };

template <class E> struct Mma;

template <> struct Mma<BF16> {
  static constexpr int KS = 16;  // reduction depth of one instruction
  static constexpr int KL = 8;   // reduction elements supplied per lane
  typedef bf16x8_t Frag;
  static __device__ __forceinline__ f32x16_t mma(Frag a, Frag b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ Frag ld(const uint16_t* p) {
    return *reinterpret_cast<const bf16x8_t*>(p);
  }
  static __device__ __forceinline__ Frag zero() {
    u32x4_t z = {0u, 0u, 0u, 0u};
    return __builtin_bit_cast(bf16x8_t, z);
  }
  static __device__ __forceinline__ Frag from(const uint16_t* y) {
    u32x4_t v;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = (uint32_t)y[2 * j] | ((uint32_t)y[2 * j + 1] << 16);
    return __builtin_bit_cast(bf16x8_t, v);
  }
};

template <> struct Mma<F32> {
  static constexpr int KS = 2;
  static constexpr int KL = 1;
  typedef float Frag;
  static __device__ __forceinline__ f32x16_t mma(Frag a, Frag b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ Frag ld(const float* p) { return *p; }
  static __device__ __forceinline__ Frag zero() { return 0.0f; }
  static __device__ __forceinline__ Frag from(const float* y) { return y[0]; }
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// Nearest-even bf16 of a double, rounded once: first to fp32 by round-to-odd
// (truncate toward zero, then set the last bit if anything was discarded),
// then to bf16 by nearest-even.  fp32 keeps 16 more bits than bf16, so the
// two steps equal a single correct rounding.
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
  float f = (float)x;
  if (fabs((double)f) > fabs(x)) f = __uint_as_float(__float_as_uint(f) - 1u);
  uint32_t b = __float_as_uint(f);
  if ((double)f != x) b |= 1u;
  if ((b & 0x7f800000u) == 0x7f800000u) {
    return (b & 0x007fffffu) ? (uint16_t)((b >> 16) | 0x40u) : (uint16_t)(b >> 16);
  }
  b += 0x7fffu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7f800000u) == 0x7f800000u) {
    return (b & 0x007fffffu) ? (uint16_t)((b >> 16) | 0x40u) : (uint16_t)(b >> 16);
  }
  b += 0x7fffu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

template <class E> struct Store;
template <> struct Store<BF16> {
  static __device__ __forceinline__ float load(const uint16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ uint16_t from_f64(double x) { return f64_to_bf16(x); }
  static __device__ __forceinline__ uint16_t from_f32(float x) { return f32_to_bf16(x); }
};
template <> struct Store<F32> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ float from_f64(double x) { return (float)x; }
  static __device__ __forceinline__ float from_f32(float x) { return x; }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Lane l combined with lane l ^ 32: v_permlane32_swap exchanges the wave's
// two halves in one VALU instruction (no LDS round trip).  Of its two
// results, one holds lane l's own value and the other its partner's, in
// either order; max and sum are symmetric, so both lanes of a pair get the
// same bits.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ double halves_sum(double x) {
  const uint64_t b = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)b, hi = (uint32_t)(b >> 32);
  const auto rl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
  const auto rh = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
  const double a = __builtin_bit_cast(double, (uint64_t)rl[0] | ((uint64_t)rh[0] << 32));
  const double c = __builtin_bit_cast(double, (uint64_t)rl[1] | ((uint64_t)rh[1] << 32));
  return a + c;
}

// ---------------------------------------------------------------------------
// RoPE at virtual positions + append to the detailed cache.
// Every (token, head, 8 rotation pairs) has its own thread: x1 = x[k..k+8),
// x2 = x[k+d/2..k+d/2+8) are rotated by the table's fp32 cos / sin of
// position nT + i in fp64, with one fused multiply-add per output (the other
// product is exact in fp64), and rounded once to storage.  Rotated queries go
// to the grouped query buffer; rotated keys and the values go to the pool's
// frame rows and to D.
// ---------------------------------------------------------------------------
template <class E> struct Vec8;
template <> struct Vec8<BF16> {
  static __device__ __forceinline__ void load(const uint16_t* p, float* x) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = __uint_as_float(v[j] << 16);
      x[2 * j + 1] = __uint_as_float(v[j] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void store(uint16_t* p, const uint16_t* y) {
    u32x4_t v;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = (uint32_t)y[2 * j] | ((uint32_t)y[2 * j + 1] << 16);
    *reinterpret_cast<u32x4_t*>(p) = v;
  }
};
template <> struct Vec8<F32> {
  static __device__ __forceinline__ void load(const float* p, float* x) {
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p);
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(p + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = a[j];
      x[4 + j] = b[j];
    }
  }
  static __device__ __forceinline__ void store(float* p, const float* y) {
    *reinterpret_cast<f32x4_t*>(p) = f32x4_t{y[0], y[1], y[2], y[3]};
    *reinterpret_cast<f32x4_t*>(p + 4) = f32x4_t{y[4], y[5], y[6], y[7]};
  }
};

// One rotation pair: (u, v) by the fp32 (c, s) of its angle, in fp64 with one
// fused multiply-add per output (the other product is exact in fp64), rounded
// once to storage.
template <class E>
__device__ __forceinline__ void rope_pair(float u, float v, float2 cs, typename E::T& y1, typename E::T& y2) {
  const double du = u, dv = v, c = cs.x, sn = cs.y;
  y1 = Store<E>::from_f64(fma(du, c, -(dv * sn)));
  y2 = Store<E>::from_f64(fma(dv, c, du * sn));
}

// cos / sin of (p * theta_k) for every stream position p and frequency k,
// evaluated in fp64 and rounded to fp32; built once when the state is created.
__global__ __launch_bounds__(256) void rope_table_kernel(RopeTableArgs a) {
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (size_t)a.npos * a.half) return;
  const int p = (int)(t / a.half), k = (int)(t - (size_t)p * a.half);
  double sn, cs;
  sincos((double)p * a.inv_freq[k], &sn, &cs);
  a.table[t] = float2{(float)cs, (float)sn};
}

// Partial outputs of pass 1.  bf16 streams store each row of O_s as fp16
// scaled by a power of two 2^-e_s (e_s per row, so that the row's largest
// magnitude is below 1): relative rounding 2^-11, half the bytes of fp32.  The
// merge folds 2^e_s into its exact power-of-two weight.  fp32 streams store
// fp32 with e_s = 0.
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
template <class E> struct PartialOut;
template <> struct PartialOut<BF16> {
  typedef f16x4_t V;
  static __device__ __forceinline__ V pack(float a, float b, float c, float d, float sc) {
    return V{(_Float16)(a * sc), (_Float16)(b * sc), (_Float16)(c * sc), (_Float16)(d * sc)};
  }
  static __device__ __forceinline__ f32x4_t unpack(V v) {
    return f32x4_t{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
  }
};
template <> struct PartialOut<F32> {
  typedef f32x4_t V;
  static __device__ __forceinline__ V pack(float a, float b, float c, float d, float) { return V{a, b, c, d}; }
  static __device__ __forceinline__ f32x4_t unpack(V v) { return v; }
};

// Partial outputs of pass 1 are stored in groups of 32 flat rows (flat row =
// (split*Hkv + g)*R + r): inside a group, quad q of the dims of flat row ri is
// f32x4 number q*32 + ri%32, so that a wave's store instruction writes 1 KB
// contiguous.  Returns the f32x4 index of the group of flat row ri.  The
// buffer holds whole groups.
__host__ __device__ inline size_t opart_group(size_t ri, int D) { return (ri >> 5) * (size_t)(D / 4) * 32; }

// Split statistics of pass 1 are stored split-major inside groups of 32 rows
// (row = g*R + r): a wave's store is 32 consecutive values, and the
// statistics of one row are 32 elements apart.
// ss = splits per group (the maximum number of splits).
__host__ __device__ inline size_t stat_index(size_t row, int split, int ss) {
  return ((row >> 5) * ss + split) * 32 + (row & 31);
}
__device__ __forceinline__ void load_split_stats(const float* mpart, const double* lpart, size_t row, int S,
                                                 int ss, float (&ms)[kMaxSplits], double (&ls)[kMaxSplits]) {
  const float* mrow = mpart + stat_index(row, 0, ss);
  const double* lrow = lpart + stat_index(row, 0, ss);
#pragma unroll
  for (int sp = 0; sp < kMaxSplits; ++sp) {
    ms[sp] = sp < S ? mrow[sp * 32] : -INFINITY;
    ls[sp] = sp < S ? lrow[sp * 32] : 0.0;
  }
}

// m = max_s m_s, l = sum_s 2^(m_s - m) l_s: exact powers of two, fp64 sum in
// split order; splits that saw no key of the row (m_s = -inf) are skipped.
__device__ __forceinline__ void merge_split_stats(const float (&ms)[kMaxSplits], const double (&ls)[kMaxSplits],
                                                  float& m, double& l) {
  m = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < kMaxSplits; ++sp) m = fmaxf(m, ms[sp]);
  l = 0.0;
#pragma unroll
  for (int sp = 0; sp < kMaxSplits; ++sp)
    if (ms[sp] != -INFINITY) l += ldexp(ls[sp], (int)(ms[sp] - m));
}

// Work-groups are dispatched round-robin over the 8 XCDs, each with its own
// L2.  Renumbering the linear work-group id this way makes consecutive
// logical indices run on the same XCD, so work-groups that read the same data
// share one L2.  A permutation of [0, n): results do not depend on it.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_remap(int id, int n) {
  const int xcd = id % kXcds, local = id / kXcds;
  const int q = n / kXcds, r = n % kXcds;   // XCDs below r receive q + 1 work-groups
  return xcd * q + min(xcd, r) + local;
}

// Four rotation pairs of one (token, head): x1 = x[k..k+4), x2 = x[k+d/2..).
template <class E> struct Vec4;
template <> struct Vec4<BF16> {
  static __device__ __forceinline__ void load(const uint16_t* p, float* x) {
    const u32x2_t v = *reinterpret_cast<const u32x2_t*>(p);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      x[2 * j] = __uint_as_float(v[j] << 16);
      x[2 * j + 1] = __uint_as_float(v[j] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void store(uint16_t* p, const uint16_t* y) {
    *reinterpret_cast<u32x2_t*>(p) = u32x2_t{(uint32_t)y[0] | ((uint32_t)y[1] << 16),
                                             (uint32_t)y[2] | ((uint32_t)y[3] << 16)};
  }
};
template <> struct Vec4<F32> {
  static __device__ __forceinline__ void load(const float* p, float* x) {
    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = v[j];
  }
  static __device__ __forceinline__ void store(float* p, const float* y) {
    *reinterpret_cast<f32x4_t*>(p) = f32x4_t{y[0], y[1], y[2], y[3]};
  }
};

// Threads of the RoPE launch: one task each, (token, head, 4 rotation pairs)
// for the query and key heads, then (token, KV head, 16 bytes) for the
// values.  Short per-thread work keeps the launch's latency chain (load,
// fp64 rotation, store) short; the value loads are issued by their own
// threads, beside the rotations.
__host__ __device__ inline int64_t rope_qk_tasks(int T, int Hq, int Hkv, int d, int pairs) {
  return (int64_t)T * (Hq + Hkv) * (d / 2 / pairs);
}
__host__ __device__ inline int64_t rope_v_tasks(int T, int Hkv, int d, int esize) {
  return (int64_t)T * Hkv * (d * esize / 16);
}

// The RoPE + append work of RoPE work-group `wg` (kSelectThreads tasks) of
// layer `layer`, RP rotation pairs per task; it also clears its share of the
// layer's column sums.
template <class E, int D, int RP>
__device__ void rope_wg_t(const RopeArgs& a0, size_t layer, int wg) {
  typedef typename E::T T;
  constexpr int HALF = D / 2;
  constexpr int CH = HALF / RP;                  // tasks per head
  constexpr int VEC = 16 / (int)sizeof(T);
  constexpr int VCH = D / VEC;                   // value chunks per head
  const int tid = threadIdx.x;
  if (a0.clear) {
    unsigned long long* c = a0.clear + layer * a0.cap;
    for (int i = wg * kSelectThreads + tid; i < a0.clear_n; i += a0.rope_blocks * kSelectThreads) c[i] = 0ull;
  }
  RopeArgs a = a0;
  {
    const size_t q_ls = (size_t)a.T * a.Hq * D, kv_ls = (size_t)a.T * a.Hkv * D;
    const size_t pool_ls = (size_t)a.Hkv * a.cap * D;
    a.q = (const T*)a.q + layer * q_ls;
    a.k = (const T*)a.k + layer * kv_ls;
    a.v = (const T*)a.v + layer * kv_ls;
    a.qrot = (T*)a.qrot + layer * q_ls;
    if (a.kpool) {
      a.kpool = (T*)a.kpool + layer * pool_ls;
      a.vpool = (T*)a.vpool + layer * pool_ls;
      a.pool_pos += layer * a.cap;
    }
    a.dk = (T*)a.dk + layer * a.det_ls;
    a.dv = (T*)a.dv + layer * a.det_ls;
  }
  const int nh = a.Hq + a.Hkv;
  const int64_t nqk = rope_qk_tasks(a.T, a.Hq, a.Hkv, D, RP);
  const int64_t nv = rope_v_tasks(a.T, a.Hkv, D, (int)sizeof(T));
  const int64_t t = (int64_t)wg * kSelectThreads + tid;
  bool finite = true;
  if (t < nqk) {
    const int c = (int)(t % CH);
    const int64_t rest = t / CH;
    const int hd = (int)(rest % nh);
    const int tok = (int)(rest / nh);
    const int k = c * RP;
    const int pos = a.pos0 + tok;
    const T* src;
    T* dst0;
    T* dst1 = nullptr;
    if (hd < a.Hq) {
      const int g = hd / a.G, hl = hd - g * a.G;
      src = (const T*)a.q + ((size_t)tok * a.Hq + hd) * D;
      dst0 = (T*)a.qrot + ((size_t)g * a.G * a.T + (size_t)tok * a.G + hl) * D;
    } else {
      const int g = hd - a.Hq;
      src = (const T*)a.k + ((size_t)tok * a.Hkv + g) * D;
      dst0 = (T*)a.dk + ((size_t)pos * a.Hkv + g) * D;
      if (a.kpool) dst1 = (T*)a.kpool + ((size_t)g * a.cap + a.frame_base + tok) * D;
      if (a.pool_pos && g == 0 && c == 0) a.pool_pos[a.frame_base + tok] = pos;
    }
    typedef typename std::conditional<RP == 8, Vec8<E>, Vec4<E>>::type VP;
    float x1[RP], x2[RP];
    VP::load(src + k, x1);
    VP::load(src + k + HALF, x2);
    const f32x4_t* tb = reinterpret_cast<const f32x4_t*>(a.table + (size_t)pos * HALF + k);
    f32x4_t cs4[RP / 2];   // (cos, sin) of pairs k + 2 i and k + 2 i + 1
#pragma unroll
    for (int i = 0; i < RP / 2; ++i) cs4[i] = tb[i];
    T y1[RP], y2[RP];
#pragma unroll
    for (int j = 0; j < RP; ++j) {
      finite &= isfinite(x1[j]) && isfinite(x2[j]);
      rope_pair<E>(x1[j], x2[j], float2{cs4[j >> 1][2 * (j & 1)], cs4[j >> 1][2 * (j & 1) + 1]}, y1[j], y2[j]);
    }
    VP::store(dst0 + k, y1);
    VP::store(dst0 + k + HALF, y2);
    if (dst1) {
      VP::store(dst1 + k, y1);
      VP::store(dst1 + k + HALF, y2);
    }
  } else if (t < nqk + nv) {
    // Values: copied unrotated to the pool and to D, 16 bytes per task.
    const int64_t tv = t - nqk;
    const int c = (int)(tv % VCH);
    const int64_t rest = tv / VCH;
    const int g = (int)(rest % a.Hkv);
    const int tok = (int)(rest / a.Hkv);
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>((const T*)a.v + ((size_t)tok * a.Hkv + g) * D + c * VEC);
    if constexpr (sizeof(T) == 2) {
      float x[8];
      Vec8<BF16>::load(reinterpret_cast<const uint16_t*>(&v), x);
#pragma unroll
      for (int j = 0; j < 8; ++j) finite &= isfinite(x[j]);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) finite &= isfinite(__uint_as_float(v[j]));
    }
    if (a.vpool)
      *reinterpret_cast<u32x4_t*>((T*)a.vpool + ((size_t)g * a.cap + a.frame_base + tok) * D + c * VEC) = v;
    *reinterpret_cast<u32x4_t*>((T*)a.dv + ((size_t)(a.pos0 + tok) * a.Hkv + g) * D + c * VEC) = v;
  }
  if (!finite) atomicOr(a.nonfinite, 1);
}

template <class E, int D>
__device__ void rope_wg(const RopeArgs& a, size_t layer, int wg) {
  if (sizeof(typename E::T) == 2 && a.rope_pairs == 8) rope_wg_t<E, D, 8>(a, layer, wg);
  else rope_wg_t<E, D, 4>(a, layer, wg);
}

// ---------------------------------------------------------------------------
// Attention pass 1.  Work-group = NW waves; each wave owns QT tiles of 32 query
// rows of one KV group (rows r = token*G + head-in-group) and the work-group
// walks its key split in blocks of 64 keys, double-buffered in LDS: the next
// block's global loads are in flight while the current block is computed.
//
// S^T = K Q^T puts one query per lane column, so row max / row sum reduce
// inside the lane plus one exchange with lane l^32.  O^T = V^T P^T reuses the
// S^T accumulators directly as the B operand: for bf16 the eight keys a lane
// supplies to one instruction are keys {16m + 8(t/4) + 4(l/32) + t%4}.  V
// stays row-major in LDS and gfx950's transposing LDS read (ds_read_b64_tr_b16)
// gathers those keys of the lane's dimension, two reads per operand; fp32
// streams write V^T to LDS instead.
//
// Visibility: key j is visible to a query of token i iff j < k0 + i + 1 (all
// state keys, the frame's keys causally) and j lies in this split.  Blocks
// that every row of the work-group sees in full take the unmasked path.
// Exponent: p = 2^(x*c_hi - m) with c_hi = sigma*log2(e) rounded to fp32; the
// row sum l only needs the weights near the maximum, whose exponent error
// c_lo*x is common to them, so it stays within about 1e-7 of the exact sum.
// ---------------------------------------------------------------------------
// Raw buffer resource over [base, base + 2^32): loads address base + a
// 32-bit byte offset, with the base in scalar registers.  Word 3 selects a
// 32-bit data format, which untyped loads need to return data.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, -1, 0x00020000);
}

// VROW (bf16 only): V kept row-major in LDS ([BN][VSTR], rows padded by 64
// bytes so that the transposing reads of four rows by 32 lanes hit distinct
// banks) and read as V^T by ds_read_b64_tr_b16; otherwise V^T is written to
// LDS ([D][VSTR]) from registers.
template <class E, int D, int NT, int BN_ = kAttnBN, bool VROW = false>
struct AttnStage {
  typedef typename E::T T;
  static constexpr int BN = BN_;
  static constexpr int EPV = 16 / (int)sizeof(T);
  static constexpr int KSTR = D + EPV;
  static_assert(!VROW || sizeof(T) == 2, "row-major V needs 16-bit elements");
  static constexpr int VSTR = VROW ? D + 32 : BN + EPV;
  static constexpr int VSIZE = VROW ? BN * VSTR : D * VSTR;   // elements of one V buffer
  static constexpr bool VROW_ = VROW;
  static constexpr int KCH = BN * (D / EPV) / NT;          // 16-byte K chunks / thread
  // bf16 V^T: tasks of KG consecutive keys x 8 dims
  static constexpr int KG = (BN / 4) * (D / 8) >= NT ? 4 : 2;
  static constexpr int VTASKS = (BN / KG) * (D / 8);
  static constexpr int VT_PER = (VTASKS + NT - 1) / NT;
  static constexpr int VCH = VROW ? KCH : (sizeof(T) == 2 ? KG * VT_PER : KCH);
  static_assert(KCH >= 1 && (BN * (D / EPV)) % NT == 0, "K staging shape");

  u32x4_t kr[KCH];
  u32x4_t vr[VCH];

  // Key j of the block is row pool_row(j, k0, foff) of kbase / vbase; rows
  // are rs elements apart (rs < 2^24).  Loads are buffer loads: the block's
  // base is a scalar resource (kbase / vbase advanced by the block's first
  // row) and each lane adds a byte offset.  Row kb + r of the block sits at
  // (kb + r) * rs, plus foff * rs from key k0 on.  When the whole block lies
  // on one side of k0 (nearly every block) the lane offsets r * rs do not
  // change from block to block: they are formed once (off_uniform) and no
  // vector instruction is spent on addresses in the loop.  Keys at or beyond
  // kend (the last block of a range) read the row of key kend - 1 instead:
  // the softmax masks them, so these finite rows only fill the tile, and no
  // load needs a branch.
  struct Offsets {
    uint32_t k[KCH];
    uint32_t v[VCH];
  };
  template <class RowOff>
  __device__ __forceinline__ static void offsets(Offsets& o, RowOff row_off, int tid) {
    constexpr int CPR = D / EPV;
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      const int t = tid + j * NT;
      const int rr = t / CPR, cc = t - rr * CPR;
      o.k[j] = row_off(rr) + (uint32_t)(cc * 16);
    }
    if constexpr (VROW) {
#pragma unroll
      for (int j = 0; j < VCH; ++j) {
        const int t = tid + j * NT;
        const int rr = t / CPR, cc = t - rr * CPR;
        o.v[j] = row_off(rr) + (uint32_t)(cc * 16);
      }
    } else if constexpr (sizeof(T) == 2) {
      constexpr int NKQ = BN / KG;
#pragma unroll
      for (int u = 0; u < VT_PER; ++u) {
        const int t = min(tid + u * NT, VTASKS - 1);
        const int kq = t % NKQ, dc = t / NKQ;
#pragma unroll
        for (int j = 0; j < KG; ++j) o.v[u * KG + j] = row_off(kq * KG + j) + (uint32_t)(dc * 16);
      }
    } else {
#pragma unroll
      for (int j = 0; j < VCH; ++j) {
        const int t = tid + j * NT;
        const int rr = t % BN, cc = t / BN;
        o.v[j] = row_off(rr) + (uint32_t)(cc * 16);
      }
    }
  }
  __device__ __forceinline__ static void off_uniform(Offsets& o, size_t rs, int tid) {
    const uint32_t rb = (uint32_t)rs * (uint32_t)sizeof(T);
    offsets(o, [&](int rr) -> uint32_t { return (uint32_t)rr * rb; }, tid);
  }

  __device__ __forceinline__ void load(const T* kbase, const T* vbase, int kb, int kend, int k0,
                                       int foff, size_t rs, Offsets& ou, int tid) {
    const int64_t blk = (int64_t)kb * (int64_t)rs;
    const int64_t fo = (int64_t)foff * (int64_t)rs;
    // Whole block on one side of k0 (nearly every block): one uniform base
    // and the loop-invariant offsets.  Otherwise rows are clamped and the
    // frame's rows shifted by foff one by one, in the same registers, which
    // get their loop-invariant values back once the loads are issued.
    if (kb + BN <= kend && (kb + BN <= k0 || kb >= k0)) {
      const int64_t ub = blk + (kb >= k0 ? fo : 0);
      load_rows(kbase + ub, vbase + ub, ou);
    } else {
      const uint32_t rb = (uint32_t)rs * (uint32_t)sizeof(T);
      const uint32_t fob = (uint32_t)fo * (uint32_t)sizeof(T);
      const int rlast = kend - 1 - kb;   // last valid row of the block (>= 0)
      offsets(ou, [&](int rr) -> uint32_t {
        const int rc = min(rr, rlast);
        return (uint32_t)rc * rb + (kb + rc >= k0 ? fob : 0u);
      }, tid);
      load_rows(kbase + blk, vbase + blk, ou);
      off_uniform(ou, rs, tid);
    }
  }

  // The same block through 64-bit global addresses, for the text-phase
  // kernel: its K and V come from D, a stream read once, and its registers
  // are at their limit, so loop-invariant offsets would cost it more than the
  // address arithmetic they save (measured 25 % slower per token at 131k keys).
  __device__ __forceinline__ void load_global(const T* kbase, const T* vbase, int kb, int kend, size_t rs,
                                              int tid) {
    const int64_t blk = (int64_t)kb * (int64_t)rs;
    const uint32_t rs32 = (uint32_t)rs;
    const int rlast = kend - 1 - kb;   // last valid row of the block (>= 0)
    if (kb + BN <= kend) {
      load_rows_global(kbase + blk, vbase + blk,
                       [&](int rr) -> int64_t { return (int64_t)__umul24((uint32_t)rr, rs32); }, tid);
    } else {
      load_rows_global(kbase + blk, vbase + blk, [&](int rr) -> int64_t {
        return (int64_t)__umul24((uint32_t)min(rr, rlast), rs32);
      }, tid);
    }
  }

  // Row r of the block is at kb_ + row_off(r) (keys) and vb_ + row_off(r).
  template <class RowOff>
  __device__ __forceinline__ void load_rows_global(const T* kb_, const T* vb_, RowOff row_off, int tid) {
    constexpr int CPR = D / EPV;
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      const int t = tid + j * NT;
      const int rr = t / CPR, cc = t - rr * CPR;
      kr[j] = *reinterpret_cast<const u32x4_t*>(kb_ + row_off(rr) + cc * EPV);
    }
    if constexpr (sizeof(T) == 2) {
      constexpr int NKQ = BN / KG;
#pragma unroll
      for (int u = 0; u < VT_PER; ++u) {
        const int t = tid + u * NT;
        const int kq = t % NKQ, dc = t / NKQ;
#pragma unroll
        for (int j = 0; j < KG; ++j) {
          vr[u * KG + j] = u32x4_t{0u, 0u, 0u, 0u};
          if (VTASKS % NT == 0 || t < VTASKS)
            vr[u * KG + j] = *reinterpret_cast<const u32x4_t*>(vb_ + row_off(kq * KG + j) + dc * 8);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < VCH; ++j) {
        const int t = tid + j * NT;
        const int rr = t % BN, cc = t / BN;
        vr[j] = *reinterpret_cast<const u32x4_t*>(vb_ + row_off(rr) + cc * 4);
      }
    }
  }

  // Every thread loads (threads beyond the V^T tasks repeat the last task's
  // rows and do not store them): no branch around the loads.
  __device__ __forceinline__ void load_rows(const T* kb_, const T* vb_, const Offsets& o) {
    const __amdgpu_buffer_rsrc_t kr_ = buffer_rsrc(kb_);
    const __amdgpu_buffer_rsrc_t vr_ = buffer_rsrc(vb_);
#pragma unroll
    for (int j = 0; j < KCH; ++j) kr[j] = __builtin_amdgcn_raw_buffer_load_b128(kr_, o.k[j], 0, 0);
#pragma unroll
    for (int j = 0; j < VCH; ++j) vr[j] = __builtin_amdgcn_raw_buffer_load_b128(vr_, o.v[j], 0, 0);
  }

  __device__ __forceinline__ void store(T* Ks, T* Vt, int tid) const {
    constexpr int CPR = D / EPV;
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      const int t = tid + j * NT;
      const int rr = t / CPR, cc = t - rr * CPR;
      *reinterpret_cast<u32x4_t*>(&Ks[rr * KSTR + cc * EPV]) = kr[j];
    }
    if constexpr (VROW) {
#pragma unroll
      for (int j = 0; j < VCH; ++j) {
        const int t = tid + j * NT;
        const int rr = t / CPR, cc = t - rr * CPR;
        *reinterpret_cast<u32x4_t*>(&Vt[rr * VSTR + cc * EPV]) = vr[j];
      }
    } else if constexpr (sizeof(T) == 2) {
      constexpr int NKQ = BN / KG;
#pragma unroll
      for (int u = 0; u < VT_PER; ++u) {
        const int t = tid + u * NT;
        if (t >= VTASKS) continue;
        const int kq = t % NKQ, dc = t / NKQ;
        const int kk = kq * KG;
        const int slot = (kk & ~12) | ((kk & 4) << 1) | ((kk & 8) >> 1);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          uint32_t w[KG];
#pragma unroll
          for (int j = 0; j < KG; ++j) w[j] = vr[u * KG + j][e >> 1];
          if constexpr (KG == 4) {
            uint32_t lo, hi;
            if (e & 1) {
              lo = (w[0] >> 16) | (w[1] & 0xffff0000u);
              hi = (w[2] >> 16) | (w[3] & 0xffff0000u);
            } else {
              lo = (w[0] & 0xffffu) | (w[1] << 16);
              hi = (w[2] & 0xffffu) | (w[3] << 16);
            }
            *reinterpret_cast<u32x2_t*>(&Vt[(dc * 8 + e) * VSTR + slot]) = u32x2_t{lo, hi};
          } else {
            const uint32_t lo = (e & 1) ? ((w[0] >> 16) | (w[1] & 0xffff0000u))
                                        : ((w[0] & 0xffffu) | (w[1] << 16));
            *reinterpret_cast<uint32_t*>(&Vt[(dc * 8 + e) * VSTR + slot]) = lo;
          }
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < VCH; ++j) {
        const int t = tid + j * NT;
        const int rr = t % BN, cc = t / BN;
#pragma unroll
        for (int e = 0; e < 4; ++e) Vt[(cc * 4 + e) * VSTR + rr] = __uint_as_float(vr[j][e]);
      }
    }
  }
};

// Online softmax over one 32-key sub-tile (S^T accumulators: 16 keys per lane
// for the lane's query, the other 16 in lane l^32).  Overwrites the scores
// with p = 2^(x*c_hi - m) and returns in alpha the factor that rescales the
// earlier output.  The reference m is an integer (log2 units) that moves only
// when the row maximum exceeds it by more than kLazyRescale, to ceil(max): the
// weights stay below 2^kLazyRescale, rescaling is rare and every rescale or
// merge factor 2^(m_old - m_new) is an exact power of two.
constexpr float kLazyRescale = 8.f;

// First half: masking, the sub-tile's row maximum and the reference update
// (alpha, and l rescaled).  Second half (softmax_exp): the weights and their
// row sum.  online_softmax is the two in sequence.
template <int QT, bool MASK>
__device__ __forceinline__ void softmax_max(f32x16_t (&sacc)[QT], float (&m_run)[QT],
                                            double (&l_run)[QT], float (&alpha)[QT],
                                            const int (&lim)[QT], int kb, int hh, float c_hi) {
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if constexpr (MASK) {
        const int key = kb + 8 * (i >> 2) + 4 * hh + (i & 3);
        sacc[qt][i] = key < lim[qt] ? sacc[qt][i] : -INFINITY;
      }
      mx = fmaxf(mx, sacc[qt][i]);
    }
    mx = halves_max(mx) * c_hi;
    alpha[qt] = 1.f;
    if (__ballot(mx > m_run[qt] + kLazyRescale)) {   // rare after the first sub-tile
      if (mx > m_run[qt] + kLazyRescale) {
        const float m_new = ceilf(mx);
        if (m_run[qt] == -INFINITY) {
          alpha[qt] = 0.f;
          l_run[qt] = 0.0;
        } else {
          const int dm = (int)(m_run[qt] - m_new);
          alpha[qt] = ldexpf(1.f, dm);
          l_run[qt] = ldexp(l_run[qt], dm);
        }
        m_run[qt] = m_new;
      }
    }
  }
}

template <int QT>
__device__ __forceinline__ void softmax_exp(f32x16_t (&sacc)[QT], const float (&m_run)[QT],
                                            double (&l_run)[QT], float c_hi) {
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float m_use = m_run[qt] == -INFINITY ? 0.f : m_run[qt];
    // Row sum in a fixed order: four interleaved partial sums, then pairwise.
    float r4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = fast_exp2(fmaf(sacc[qt][i], c_hi, -m_use));
      sacc[qt][i] = p;
      r4[i & 3] += p;
    }
    l_run[qt] += (double)((r4[0] + r4[1]) + (r4[2] + r4[3]));
  }
}

template <int QT, bool MASK>
__device__ __forceinline__ void online_softmax(f32x16_t (&sacc)[QT], float (&m_run)[QT],
                                               double (&l_run)[QT], float (&alpha)[QT],
                                               const int (&lim)[QT], int kb, int hh,
                                               float c_hi) {
  softmax_max<QT, MASK>(sacc, m_run, l_run, alpha, lim, kb, hh, c_hi);
  softmax_exp<QT>(sacc, m_run, l_run, c_hi);
}

// Scheduling groups of a straight-line region: R0 LDS reads (the first
// matrix operands), V0 VALU instructions while they are in flight, then N
// times (one MFMA, RI further LDS reads, V VALU instructions), so that each
// matrix instruction runs beside the wave's vector work and later operands
// are read meanwhile.
template <int R0, int V0, int N, int RI, int V>
__device__ __forceinline__ void interleave_mfma_valu() {
  __builtin_amdgcn_sched_group_barrier(0x100, R0, 0);   // LDS reads
  __builtin_amdgcn_sched_group_barrier(0x002, V0, 0);   // VALU
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    if (RI > 0) __builtin_amdgcn_sched_group_barrier(0x100, RI, 0);   // LDS reads
    __builtin_amdgcn_sched_group_barrier(0x002, V, 0);   // VALU
  }
}

// WPE: waves per SIMD the registers are sized for.  With d = 64 two 8-wave
// work-groups fit on a CU when registers are capped at 128 per lane (WPE =
// 4): worth it when the grid has more work-groups than CUs; otherwise the
// uncapped build (WPE = 1) runs faster.
template <class E, int D, int QT, int NW, int NPF = 1, int BN_ = kAttnBN, int WPE = 1>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(WPE)))
void attn_fwd_kernel(AttnArgs a) {
  typedef typename E::T T;
  typedef Mma<E> M;
  constexpr int NT = 64 * NW;
  constexpr int BN = BN_;
  typedef AttnStage<E, D, NT, BN, sizeof(T) == 2> Stage;
  constexpr int NSUB = BN / 32;   // 32-key sub-tiles per block
  constexpr int KSTR = Stage::KSTR;
  constexpr int VSTR = Stage::VSTR;
  constexpr int NKS = D / M::KS;
  constexpr int NDT = D / 32;
  constexpr int BM = NW * 32 * QT;
  __shared__ __attribute__((aligned(16))) T Ks[2][BN * KSTR];
  __shared__ __attribute__((aligned(16))) T Vt[2][Stage::VSIZE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hh = lane >> 5;
  // MFMA operand V^T for dims [32 dt, 32 dt + 32) and the 16 keys from key0
  // of an LDS block: this lane's row 32 dt + col and its 8 keys, in the order
  // the P operand holds them (key key0 + 8 (t / 4) + 4 hh + t % 4 for t < 8).
  // Row-major V (bf16): two transposing reads; lane s of each 16-lane group
  // reads 4 dims of key key0 + 8 c + 4 hh + s / 4 and the read hands lane i of
  // the group element i % 4 of lane 4 e + i / 4, i.e. key e of its own dim.
  const int vlane = Stage::VROW_ ? (4 * hh + (lane & 15) / 4) * VSTR + 16 * ((lane >> 4) & 1) + 4 * (lane & 3)
                                 : col * VSTR + hh * 8;
  auto v_operand = [&](const T* vt_, int key0, int dt) {
    if constexpr (Stage::VROW_) {
      typedef short s16x4_t __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
      const T* p = vt_ + key0 * VSTR + dt * 32 + vlane;
      const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p));
      const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p + 8 * VSTR));
      const u32x4_t w = {__builtin_bit_cast(u32x2_t, lo)[0], __builtin_bit_cast(u32x2_t, lo)[1],
                         __builtin_bit_cast(u32x2_t, hi)[0], __builtin_bit_cast(u32x2_t, hi)[1]};
      return __builtin_bit_cast(bf16x8_t, w);
    } else {
      return *reinterpret_cast<const bf16x8_t*>(&vt_[dt * 32 * VSTR + key0 + vlane]);
    }
  };
  // Logical (row tile, KV head, split), or (row tile, split, KV head) with
  // head_major; the row tiles of one (head, split) share its K/V blocks and
  // run on one XCD.  Head-major order gives each XCD the query rows of few
  // heads (many KV heads: each XCD would otherwise read every head's queries).
  // Heaviest row tiles first (later tokens see more keys).
  const int wl = xcd_remap(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z),
                           gridDim.x * gridDim.y * gridDim.z);
  const int tile = wl % gridDim.x, wrest = wl / gridDim.x;
  const int g = a.head_major ? (int)(wrest / gridDim.z) : (int)(wrest % gridDim.y);
  const int split = a.head_major ? (int)(wrest % gridDim.z) : (int)(wrest / gridDim.y);
  const int row_wg = (gridDim.x - 1 - tile) * BM;
  const int row_last = min(a.R, row_wg + BM) - 1;
  const int tok_min = row_wg / a.G;
  const int need_end = a.k0 + row_last / a.G + 1;  // keys beyond are masked for every row
  const int kbeg = split * a.kps;
  const int kend = min(min(kbeg + a.kps, need_end), a.P);
  // Blocks ending at or before this key are visible to every row of the work-group.
  const int full_end = min(kend, a.k0 + tok_min + 1);

  const T* qbase = (const T*)a.qrot + (size_t)g * a.R * D;
  const int layer = g / a.lh, gl = g - layer * a.lh;
  const size_t kvo = (size_t)layer * a.kv_ls + (size_t)gl * a.kv_hs;
  const T* kbase = (const T*)a.kpool + kvo;
  const T* vbase = (const T*)a.vpool + kvo;
  const size_t rs = (size_t)a.kv_rs;

  typename M::Frag qf[QT][NKS];
  int qrow[QT], lim[QT];
  // bf16: buffer loads through a resource that ends at row R (rows past it
  // read as zero), so no load sits behind a branch and the compiler's wait
  // counts stay exact.
  const __amdgpu_buffer_rsrc_t qres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T*>(qbase), (short)0, a.R * D * (int)sizeof(T), 0x00020000);
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int r = row_wg + (wave * QT + qt) * 32 + col;
    qrow[qt] = r;
    lim[qt] = min(kend, a.k0 + (r < a.R ? r / a.G : -1) + 1);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if constexpr (sizeof(T) == 2) {
        const uint32_t off = (uint32_t)((r * D + ks * M::KS + hh * M::KL) * (int)sizeof(T));
        qf[qt][ks] = __builtin_bit_cast(typename M::Frag, __builtin_amdgcn_raw_buffer_load_b128(qres, off, 0, 0));
      } else {
        qf[qt][ks] = r < a.R ? M::ld(qbase + (size_t)r * D + ks * M::KS + hh * M::KL) : M::zero();
      }
    }
  }

  f32x16_t o[QT][NDT];
  float m_run[QT];
  double l_run[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[qt][dt] = f32x16_t{};
    m_run[qt] = -INFINITY;
    l_run[qt] = 0.0;
  }

  // NPF register stages: block b's loads are issued NPF blocks ahead of its
  // compute and it is stored to LDS after block b-1's compute, so a load has
  // NPF blocks of compute to arrive in, and short splits (a few blocks per
  // work-group) have all their loads in flight at once.  Blocks pass through
  // two LDS buffers.  Loads past the last block repeat it (every stage is
  // loaded on every path, so the compiler's wait counts are exact); they are
  // never stored.
  Stage st[NPF];
  typename Stage::Offsets so;
  Stage::off_uniform(so, rs, tid);
  const int nblk = kend > kbeg ? (kend - kbeg + BN - 1) / BN : 0;
  const int kb_last = kbeg + max(nblk - 1, 0) * BN;
  // A work-group without keys (nblk = 0) loads the pool's first rows instead
  // (valid rows, never used).
  const int kend_ld = nblk > 0 ? kend : a.P;
#pragma unroll
  for (int i = 0; i < NPF; ++i)
    st[i].load(kbase, vbase, nblk > 0 ? min(kbeg + i * BN, kb_last) : 0, kend_ld, a.k0, a.foff, rs, so, tid);
  st[0].store(Ks[0], Vt[0], tid);
  // The query fragments and block 0 have arrived here on every path (at most
  // the later stages' loads are outstanding); saying so keeps the compiler
  // from waiting for the loop's own prefetch loads before the first matrix
  // instruction of a block.
  constexpr int kStageLoads = Stage::KCH + Stage::VCH;   // buffer loads per stage and thread
  static_assert(kStageLoads * (NPF - 1) < 16, "wait count fits the low vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (kStageLoads * (NPF - 1)));
  __syncthreads();

  auto compute = [&](int kb, int buf) {
    const T* ks_ = Ks[buf];
    const T* vt_ = Vt[buf];

    if constexpr (sizeof(T) == 2) {
      // NSUB sub-tiles of 32 keys, software-pipelined inside the wave:
      //   QK(0); max(0);
      //   for s: rescale(s-1); [PV(s-1), QK(s+1)] beside [exp(s), pack(s)]; max(s+1)
      //   rescale(NSUB-1); PV(NSUB-1)
      // so the matrix pipe works while the VALU computes the weights.  Per
      // row the arithmetic and its order are those of online_softmax: max(s)
      // fixes the reference of sub-tile s and rescales l; O is rescaled for
      // it after PV(s-1) and right before PV(s).  The rescale (a rare,
      // wave-uniform branch) stays ahead of each interleaved region: inside
      // one, it split the region in two, and the exponentials of sub-tile 0
      // were placed after all four QK(1) instructions instead of beside them.
      auto qk = [&](int sub, f32x16_t (&acc)[QT]) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) acc[qt] = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const typename M::Frag af = M::ld(&ks_[(sub * 32 + col) * KSTR + ks * M::KS + hh * M::KL]);
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) acc[qt] = M::mma(af, qf[qt][ks], acc[qt]);
        }
      };
      auto pack = [&](const f32x16_t (&acc)[QT], bf16x8_t (&pf)[2][QT]) {
#pragma unroll
        for (int mm = 0; mm < 2; ++mm)
#pragma unroll
          for (int qt = 0; qt < QT; ++qt)
#pragma unroll
            for (int t = 0; t < 8; ++t) pf[mm][qt][t] = (__bf16)acc[qt][8 * mm + t];
      };
      auto pv = [&](int sub, const bf16x8_t (&pf)[2][QT]) {
#pragma unroll
        for (int mm = 0; mm < 2; ++mm)
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            const bf16x8_t af = v_operand(vt_, sub * 32 + mm * 16, dt);
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) o[qt][dt] = M::mma(af, pf[mm][qt], o[qt][dt]);
          }
      };
      auto rescale = [&](const float (&alpha)[QT]) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          if (__ballot(alpha[qt] != 1.f)) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) o[qt][dt] *= alpha[qt];
          }
      };
      auto smax = [&](int sub, f32x16_t (&acc)[QT], float (&alpha)[QT]) {
        const int ksub = kb + 32 * sub;
        if (ksub + 32 > full_end)
          softmax_max<QT, true>(acc, m_run, l_run, alpha, lim, ksub, hh, a.c_hi);
        else
          softmax_max<QT, false>(acc, m_run, l_run, alpha, lim, ksub, hh, a.c_hi);
      };
      f32x16_t sb[2][QT];          // S of sub-tiles s and s+1
      bf16x8_t pb[2][2][QT];       // P of sub-tiles s-1 and s
      float alpha[2][QT];          // O's rescale for sub-tiles s and s+1
      qk(0, sb[0]);
      smax(0, sb[0], alpha[0]);
#pragma unroll
      for (int sub = 0; sub < NSUB; ++sub) {
        const int c = sub & 1;
        if (sub >= 1) rescale(alpha[c ^ 1]);              // O for sub-tile s-1's reference
        if (sub >= 1) pv(sub - 1, pb[c ^ 1]);
        if (sub + 1 < NSUB) qk(sub + 1, sb[c ^ 1]);
        softmax_exp<QT>(sb[c], m_run, l_run, a.c_hi);
        pack(sb[c], pb[c]);
        if (sub >= 1 && sub + 1 < NSUB)
          interleave_mfma_valu<4, 12, (NKS + 2 * NDT) * QT, 1, 3>();
        else if (sub + 1 < NSUB)
          interleave_mfma_valu<NKS, 12, NKS * QT, 0, 6>();
        else
          interleave_mfma_valu<2 * NDT, 12, 2 * NDT * QT, 0, 6>();
        if (sub + 1 < NSUB) smax(sub + 1, sb[c ^ 1], alpha[c ^ 1]);
      }
      rescale(alpha[(NSUB - 1) & 1]);
      pv(NSUB - 1, pb[(NSUB - 1) & 1]);
      return;
    }

    f32x16_t sacc[2][QT];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) sacc[sub][qt] = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const typename M::Frag af = M::ld(&ks_[(sub * 32 + col) * KSTR + ks * M::KS + hh * M::KL]);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) sacc[sub][qt] = M::mma(af, qf[qt][ks], sacc[sub][qt]);
      }
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int ksub = kb + sub * 32;
      float alpha[QT];
      if (ksub + 32 > full_end)
        online_softmax<QT, true>(sacc[sub], m_run, l_run, alpha, lim, ksub, hh, a.c_hi);
      else
        online_softmax<QT, false>(sacc[sub], m_run, l_run, alpha, lim, ksub, hh, a.c_hi);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
        if (__ballot(alpha[qt] != 1.f)) {
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) o[qt][dt] *= alpha[qt];
        }

      if constexpr (sizeof(T) == 2) {
        // Each 16-key slice of P is packed to bf16 right before its MFMAs.
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          bf16x8_t pf[QT];
#pragma unroll
          for (int qt = 0; qt < QT; ++qt)
#pragma unroll
            for (int t = 0; t < 8; ++t) pf[qt][t] = (__bf16)sacc[sub][qt][8 * mm + t];
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            const bf16x8_t af = v_operand(vt_, sub * 32 + mm * 16, dt);
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) o[qt][dt] = M::mma(af, pf[qt], o[qt][dt]);
          }
        }
      } else {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            const int kin = sub * 32 + 8 * (t >> 2) + 4 * hh + (t & 3);
            const float af = vt_[(dt * 32 + col) * VSTR + kin];
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) o[qt][dt] = M::mma(af, sacc[sub][qt][t], o[qt][dt]);
          }
      }
    }

  };

  // Splits of at most SLN blocks (a single layer's short splits) run as
  // straight-line code, so that each block waits only for its own loads (a
  // loop makes the compiler wait for the prologue's stages before entering
  // it, and copy them into the loop's registers).
  constexpr int SLN = NPF > 4 ? NPF : 4;
  if (nblk <= SLN) {
#pragma unroll
    for (int b = 0; b < SLN; ++b) {
      const int buf = b & 1;
      // Stage b % NPF held block b (stored after the previous block).
      if (b + NPF < SLN) st[b % NPF].load(kbase, vbase, min(kbeg + (b + NPF) * BN, kb_last), kend_ld, a.k0, a.foff, rs, so, tid);
      if (b < nblk) compute(kbeg + b * BN, buf);
      if (b + 1 < nblk) {   // every load above is issued on every path, so the waits stay exact
        st[(b + 1) % NPF].store(Ks[buf ^ 1], Vt[buf ^ 1], tid);
        __syncthreads();
      }
    }
  } else {
    for (int b0 = 0; b0 < nblk; b0 += NPF) {
#pragma unroll
      for (int i = 0; i < NPF; ++i) {
        const int b = b0 + i;
        if (b < nblk) {
          const int kb = kbeg + b * BN;
          const int buf = b & 1;
          // Stage i held block b (stored after the previous block); it takes
          // block b + NPF.  Block b+1 (loaded NPF blocks ago) goes to the
          // other buffer after this block's compute: that buffer was last
          // read before the previous barrier, and the barrier below
          // publishes it.
          st[i].load(kbase, vbase, min(kb + NPF * BN, kb_last), kend, a.k0, a.foff, rs, so, tid);
          compute(kb, buf);
          if (b + 1 < nblk) st[(i + 1) % NPF].store(Ks[buf ^ 1], Vt[buf ^ 1], tid);
          __syncthreads();
        }
      }
    }
  }

  // Partial results of this key split.
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const double lt = halves_sum(l_run[qt]);
    const int r = qrow[qt];
    if (r < a.R) {
      const size_t ri = ((size_t)split * a.Hkv + g) * a.R + r;
      if (hh == 0) {
        const size_t si = stat_index((size_t)g * a.R + r, split, a.ss);
        a.mpart[si] = m_run[qt];
        a.lpart[si] = lt;
      }
      if (m_run[qt] != -INFINITY) {
        int e = 0;
        if constexpr (sizeof(T) == 2) {
          float amax = 0.f;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(o[qt][dt][i]));
          amax = halves_max(amax);
          (void)frexpf(amax, &e);   // amax < 2^e
          if (hh == 0) a.epart[ri] = (int8_t)max(-127, min(127, e));
        }
        const float sc = ldexpf(1.f, -e);
        // Lane-order layout: one store instruction writes 512 B (fp16) or
        // 1 KB (fp32) contiguous.
        typedef typename PartialOut<E>::V PV;
        PV* op = reinterpret_cast<PV*>(a.opart) + opart_group(ri, D) + (ri & 31);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            op[(dt * 8 + 2 * j + hh) * 32] = PartialOut<E>::pack(o[qt][dt][4 * j], o[qt][dt][4 * j + 1],
                                                                o[qt][dt][4 * j + 2], o[qt][dt][4 * j + 3], sc);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Text-phase attention over the detailed cache D for t text tokens with
// G*t <= 32 query rows per KV head (single-token decode and short chunks).
// Few queries make this a stream over D's rows: HBM-bound.  A work-group owns
// one KV head and a contiguous key split; each block of BN = 32*NW keys is
// loaded with 16-byte coalesced reads (D rows are Hkv*d elements apart),
// staged in LDS as K and V^T (as in pass 1), and wave w computes the block's
// w-th 32-key sub-tile: S^T = K Q^T, online softmax, O^T += V^T P^T.  The next
// block's loads are in flight during the compute.
// The text tokens themselves are not yet in D: the work-group rotates its
// query rows from the projected input (the RoPE kernel's arithmetic), stages
// the text keys of its split in a separate LDS tile (rotated K, V) that is
// attended after the block loop, and appends those rows to D for later calls.
// At the end the waves' (m, l, O) are merged with exact power-of-two factors.
// Visibility: key j is seen by the query of text token i iff j < k0 + i + 1.
// ---------------------------------------------------------------------------
template <class E, int D, int NW, int NPF = 1>
__global__ __launch_bounds__(64 * NW, NPF > 1 ? 1 : 2) void decode_attn_kernel(DecodeArgs a0) {
  typedef typename E::T T;
  typedef Mma<E> M;
  constexpr int NT = 64 * NW;
  constexpr int BN = 32 * NW;
  typedef AttnStage<E, D, NT, BN> Stage;
  constexpr int KSTR = Stage::KSTR;
  constexpr int VSTR = Stage::VSTR;
  constexpr int NKS = D / M::KS;
  constexpr int NDT = D / 32;
  constexpr int KBYTES = BN * KSTR * (int)sizeof(T);
  constexpr int VBYTES = D * VSTR * (int)sizeof(T);
  constexpr int OSTR = D + 4;                       // fp32 row stride of the wave merge
  constexpr int RBYTES = NW * 32 * OSTR * 4;
  constexpr int LBYTES = KBYTES + VBYTES > RBYTES ? KBYTES + VBYTES : RBYTES;
  constexpr int VSTR_T = 32 + 16 / (int)sizeof(T);  // V^T row stride of the text tile
  __shared__ __attribute__((aligned(16))) char lds[LBYTES];
  __shared__ __attribute__((aligned(16))) T Kt[32 * KSTR];
  __shared__ __attribute__((aligned(16))) T Vtt[D * VSTR_T];
  __shared__ float wm[NW][32];
  __shared__ double wsum[NW][32];
  T* Ks = reinterpret_cast<T*>(lds);
  T* Vt = reinterpret_cast<T*>(lds + KBYTES);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hh = lane >> 5;
  const int gf = blockIdx.x, split = blockIdx.y;   // KV head over all layers
  const int layer = gf / a0.Hkv, g = gf - layer * a0.Hkv;
  DecodeArgs a = a0;   // layer's slice of inputs, D and output
  {
    const size_t t_ = (size_t)(a.R / a.G);
    a.q = (const T*)a.q + layer * t_ * a.Hq * D;
    a.out = (T*)a.out + layer * t_ * a.Hq * D;
    a.k = (const T*)a.k + layer * t_ * a.Hkv * D;
    a.v = (const T*)a.v + layer * t_ * a.Hkv * D;
    a.dk = (const T*)a.dk + (size_t)layer * a.det_ls;
    a.dv = (const T*)a.dv + (size_t)layer * a.det_ls;
  }
  const int row0 = 0;
  const int row_last = a.R - 1;
  const int kbeg = split * a.kps;
  const int kend = min(min(kbeg + a.kps, a.k0 + row_last / a.G + 1), a.P);
  const int full_end = min(kend, a.k0 + row0 / a.G + 1);   // visible to every row of the tile
  const size_t rs = (size_t)a.Hkv * D;
  const T* kbase = (const T*)a.dk + (size_t)g * D;
  const T* vbase = (const T*)a.dv + (size_t)g * D;

  const int r = row0 + col;
  // The block loop streams D's keys below k0; the split's text keys
  // [tbeg, kend) (at most 32) are staged from the projected inputs into their
  // own LDS tile up front (K rotated here), attended last, and appended to D
  // for later calls.
  const int dend = min(kend, a.k0);                         // keys read from D
  const int tbeg = max(kbeg, a.k0);
  const int ntext = max(0, kend - tbeg);
  int lim[1] = {min(kend, a.k0 + (r < a.R ? r / a.G : -1) + 1)};
  int lim_d[1] = {min(lim[0], dend)};
  // NPF register stages: block b's loads are issued NPF blocks ahead of its
  // compute (more bytes in flight per CU for the HBM stream).
  Stage st[NPF];
  const int nblk = dend > kbeg ? (dend - kbeg + BN - 1) / BN : 0;
  bool finite = true;
#pragma unroll
  for (int i = 0; i < NPF; ++i)
    if (i < nblk) st[i].load_global(kbase, vbase, kbeg + i * BN, dend, rs, tid);

  typename M::Frag qf[NKS];
  {
    constexpr int HALF = D / 2;
    constexpr int QSTR = D + 16 / (int)sizeof(T);
    const T zero = Store<E>::from_f32(0.f);
    // Query rows, rotated at positions k0 + token (the RoPE kernel's
    // arithmetic), through LDS that the first block has not yet claimed.
    T* Qs = reinterpret_cast<T*>(lds);
    for (int task = tid; task < 32 * HALF; task += NT) {
      const int rr = task / HALF, i = task - rr * HALF;
      const int row = row0 + rr;
      T y1 = zero, y2 = zero;
      if (row < a.R) {
        const int tok = row / a.G;
        const int h = g * a.G + (row - tok * a.G);
        const T* qs = (const T*)a.q + ((size_t)tok * a.Hq + h) * D;
        const float u = Store<E>::load(qs + i), v = Store<E>::load(qs + i + HALF);
        finite &= isfinite(u) && isfinite(v);
        rope_pair<E>(u, v, a.table[(size_t)(a.k0 + tok) * HALF + i], y1, y2);
      }
      Qs[rr * QSTR + i] = y1;
      Qs[rr * QSTR + i + HALF] = y2;
    }
    // Text tile: 32 key rows of K and the matching V^T columns (zeros beyond
    // the text keys), with the block layout of the stage.
    for (int task = tid; task < 32 * HALF; task += NT) {
      const int kk = task / HALF, i = task - kk * HALF;
      T y1 = zero, y2 = zero;
      if (kk < ntext) {
        const int key = tbeg + kk;
        const T* row = (const T*)a.k + ((size_t)(key - a.k0) * a.Hkv + g) * D;
        const float u = Store<E>::load(row + i), v = Store<E>::load(row + i + HALF);
        finite &= isfinite(u) && isfinite(v);
        rope_pair<E>(u, v, a.table[(size_t)key * HALF + i], y1, y2);
        T* drow = (T*)a.dk + ((size_t)key * a.Hkv + g) * D;   // append to D
        drow[i] = y1;
        drow[i + HALF] = y2;
      }
      Kt[kk * KSTR + i] = y1;
      Kt[kk * KSTR + i + HALF] = y2;
    }
    for (int task = tid; task < 32 * D; task += NT) {
      const int e = task / 32, kk = task - e * 32;
      T x = zero;
      if (kk < ntext) {
        const int key = tbeg + kk;
        x = ((const T*)a.v)[((size_t)(key - a.k0) * a.Hkv + g) * D + e];
        finite &= isfinite(Store<E>::load(&x));
        ((T*)a.dv)[((size_t)key * a.Hkv + g) * D + e] = x;     // append to D
      }
      const int slot = sizeof(T) == 2 ? (kk & ~12) | ((kk & 4) << 1) | ((kk & 8) >> 1) : kk;
      Vtt[e * VSTR_T + slot] = x;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = M::ld(&Qs[col * QSTR + ks * M::KS + hh * M::KL]);
    __syncthreads();   // the first block's store reuses the query rows' LDS
  }

  f32x16_t o[1][NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[0][dt] = f32x16_t{};
  float m_run[1] = {-INFINITY};
  double l_run[1] = {0.0};

  // One 32-key sub-tile: keys kb + 0..31 are rows koff.. of Kb and columns
  // koff.. of Vb.  S^T = K Q^T, online softmax, O^T += V^T P^T.
  auto subtile = [&](int kb, const T* Kb, const T* Vb, int vstr, int koff, const int (&lm)[1], int fend) {
    f32x16_t sacc[1] = {f32x16_t{}};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const typename M::Frag af = M::ld(&Kb[(koff + col) * KSTR + ks * M::KS + hh * M::KL]);
      sacc[0] = M::mma(af, qf[ks], sacc[0]);
    }
    float alpha[1];
    if (kb + 32 > fend)
      online_softmax<1, true>(sacc, m_run, l_run, alpha, lm, kb, hh, a.c_hi);
    else
      online_softmax<1, false>(sacc, m_run, l_run, alpha, lm, kb, hh, a.c_hi);
    if (__ballot(alpha[0] != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[0][dt] *= alpha[0];
    }
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        bf16x8_t pf;
#pragma unroll
        for (int t = 0; t < 8; ++t) pf[t] = (__bf16)sacc[0][8 * mm + t];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(
              &Vb[(dt * 32 + col) * vstr + koff + mm * 16 + hh * 8]);
          o[0][dt] = M::mma(af, pf, o[0][dt]);
        }
      }
    } else {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const int kin = koff + 8 * (t >> 2) + 4 * hh + (t & 3);
          o[0][dt] = M::mma(Vb[(dt * 32 + col) * vstr + kin], sacc[0][t], o[0][dt]);
        }
    }
  };

  const int full_end_d = min(full_end, dend);
  for (int b0 = 0; b0 < nblk; b0 += NPF) {
#pragma unroll
    for (int i = 0; i < NPF; ++i) {
      const int b = b0 + i;
      if (b < nblk) {
        const int kb = kbeg + b * BN;
        if (b > 0) __syncthreads();   // every wave is done with the previous block
        st[i].store(Ks, Vt, tid);
        __syncthreads();
        if (b + NPF < nblk) st[i].load_global(kbase, vbase, kb + NPF * BN, dend, rs, tid);
        if (kb + wave * 32 < dend) subtile(kb + wave * 32, Ks, Vt, VSTR, wave * 32, lim_d, full_end_d);
      }
    }
  }
  if (ntext > 0 && wave == 0) subtile(tbeg, Kt, Vtt, VSTR_T, 0, lim, full_end);

  if (!finite) atomicOr(a.nonfinite, 1);
  // Merge of the waves: m = max_w m_w; each wave's l and O scale by the exact
  // factor 2^(m_w - m); the sums run in wave order.
  const double lt = halves_sum(l_run[0]);
  __syncthreads();                  // the last block's LDS reads are done
  if (hh == 0) {
    wm[wave][col] = m_run[0];
    wsum[wave][col] = lt;
  }
  __syncthreads();
  float m = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) m = fmaxf(m, wm[w][col]);
  const float fw = m_run[0] == -INFINITY ? 0.f : ldexpf(1.f, (int)(m_run[0] - m));
  float* red = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<f32x4_t*>(&red[(wave * 32 + col) * OSTR + dt * 32 + 8 * j + 4 * hh]) =
          f32x4_t{o[0][dt][4 * j], o[0][dt][4 * j + 1], o[0][dt][4 * j + 2], o[0][dt][4 * j + 3]} * fw;
  __syncthreads();
  // Thread task: (row, 4 dims); rows of the tile in order.
  constexpr int CPR = D / 4;
  for (int e = tid; e < 32 * CPR; e += NT) {
    const int rr = e / CPR, c = e - rr * CPR;
    const int row = row0 + rr;
    if (row >= a.R) continue;
    float mr = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mr = fmaxf(mr, wm[w][rr]);
    double l = 0.0;
#pragma unroll
    for (int w = 0; w < NW; ++w)
      if (wm[w][rr] != -INFINITY) l += ldexp(wsum[w][rr], (int)(wm[w][rr] - mr));
    f32x4_t acc = *reinterpret_cast<const f32x4_t*>(&red[rr * OSTR + 4 * c]);
#pragma unroll
    for (int w = 1; w < NW; ++w) acc += *reinterpret_cast<const f32x4_t*>(&red[(w * 32 + rr) * OSTR + 4 * c]);
    if (a.S == 1) {
      const float inv = (float)(1.0 / l);
      const int tok = row / a.G;
      const int h = g * a.G + (row - tok * a.G);
      T* out = (T*)a.out + ((size_t)tok * a.Hq + h) * D + c * 4;
      if constexpr (sizeof(T) == 2) {
        const u32x2_t v = {(uint32_t)f32_to_bf16(acc[0] * inv) | ((uint32_t)f32_to_bf16(acc[1] * inv) << 16),
                           (uint32_t)f32_to_bf16(acc[2] * inv) | ((uint32_t)f32_to_bf16(acc[3] * inv) << 16)};
        *reinterpret_cast<u32x2_t*>(out) = v;
      } else {
        *reinterpret_cast<f32x4_t*>(out) = acc * inv;
      }
    } else {
      const size_t ri = ((size_t)split * a.L * a.Hkv + gf) * a.R + row;
      *reinterpret_cast<f32x4_t*>(a.opart + ri * D + c * 4) = acc;
      if (c == 0) {
        a.mpart[ri] = mr;
        a.lpart[ri] = l;
      }
    }
  }
}

// Merge of the text-phase key splits: one work-group per (KV head, row), one
// thread per split for the statistics.  m = max_s m_s; the weights
// 2^(m_s - m) are exact; l and O are summed in a fixed order (a fixed
// butterfly inside each wave, then waves in order; per thread over its
// splits, then thread groups in order), so the result does not depend on
// scheduling.  Splits that saw no key hold zeros and weigh 0.
constexpr int kDecodeMergeThreads = 1024;
static_assert(kDecodeMaxSplits <= kDecodeMergeThreads, "one split per merge thread");

template <class E, int D>
__global__ __launch_bounds__(kDecodeMergeThreads) void decode_merge_kernel(DecodeMergeArgs a) {
  typedef typename E::T T;
  constexpr int NT = kDecodeMergeThreads;
  constexpr int NWV = NT / 64;
  constexpr int CPR = D / 4;
  constexpr int SG = NT / CPR;                       // split groups of the accumulation
  __shared__ float wts[kDecodeMaxSplits];
  __shared__ float wmax[NWV];
  __shared__ double wl[NWV];
  __shared__ __attribute__((aligned(16))) f32x4_t redo[SG][CPR];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const size_t nrows = (size_t)a.L * a.Hkv * a.R;
  const size_t row = blockIdx.x;                     // = (layer*Hkv + g)*R + r
  const int c = tid % CPR, sg = tid / CPR;
  // Every load is issued before the first reduction: the statistics of this
  // thread's split and the first PF partial outputs of its split group.
  constexpr int PF = 8;
  f32x4_t os[PF];
#pragma unroll
  for (int j = 0; j < PF; ++j) {
    const int s = sg + j * SG;
    os[j] = s < a.S ? *reinterpret_cast<const f32x4_t*>(a.opart + (s * nrows + row) * D + c * 4)
                    : f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const float ms = tid < a.S ? a.mpart[tid * nrows + row] : -INFINITY;
  const double ls = tid < a.S ? a.lpart[tid * nrows + row] : 0.0;
  float mx = ms;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if (lane == 0) wmax[wave] = mx;
  __syncthreads();
  float m = wmax[0];
#pragma unroll
  for (int w = 1; w < NWV; ++w) m = fmaxf(m, wmax[w]);
  const float wt = ms != -INFINITY ? ldexpf(1.f, (int)(ms - m)) : 0.f;
  if (tid < a.S) wts[tid] = wt;
  double lw = wt != 0.f ? (double)wt * ls : 0.0;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) lw += __shfl_xor(lw, o);
  if (lane == 0) wl[wave] = lw;
  __syncthreads();
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < PF; ++j) {
    const int s = sg + j * SG;
    const float w = s < a.S ? wts[s] : 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = fmaf(w, os[j][e], acc[e]);
  }
#pragma unroll 1
  for (int s = sg + PF * SG; s < a.S; s += SG) {
    const float w = wts[s];
    const f32x4_t os = *reinterpret_cast<const f32x4_t*>(a.opart + (s * nrows + row) * D + c * 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = fmaf(w, os[e], acc[e]);
  }
  redo[sg][c] = acc;
  __syncthreads();
  if (tid >= CPR) return;
  acc = redo[0][c];
  for (int j = 1; j < SG; ++j) acc += redo[j][c];
  double l = wl[0];
#pragma unroll
  for (int w = 1; w < NWV; ++w) l += wl[w];
  const float inv = (float)(1.0 / l);
  const int gf = (int)(row / a.R), r = (int)(row - (size_t)gf * a.R);
  const int layer = gf / a.Hkv, g = gf - layer * a.Hkv;
  const int tok = r / a.G;
  const int h = g * a.G + (r - tok * a.G);
  T* out = (T*)a.out + (size_t)layer * (a.R / a.G) * a.Hq * D + ((size_t)tok * a.Hq + h) * D + c * 4;
  if constexpr (sizeof(T) == 2) {
    const u32x2_t v = {(uint32_t)f32_to_bf16(acc[0] * inv) | ((uint32_t)f32_to_bf16(acc[1] * inv) << 16),
                       (uint32_t)f32_to_bf16(acc[2] * inv) | ((uint32_t)f32_to_bf16(acc[3] * inv) << 16)};
    *reinterpret_cast<u32x2_t*>(out) = v;
  } else {
    *reinterpret_cast<f32x4_t*>(out) = acc * inv;
  }
}

// ---------------------------------------------------------------------------
// Score pass.  Work-group = NW waves; each wave keeps KT tiles of 32 keys in
// registers (the B operand of S = Q K^T) and all waves stream the same
// 32-row Q tiles through double-buffered LDS (the next tile is loaded while
// the current one is computed).  The row statistics of the work-group's rows
// (reference max m and row sum l) are formed once, up front, from the
// key-split partials of pass 1.  With queries as rows, a lane holds 16 rows of one key
// column, so the column sum of P = 2^(x*c - m) / l is accumulated
// in the lane: fp32 over the tile's 16 rows, then fp64 across tiles; the two
// lane halves are added at the end and the work-group's sum is added to the
// key's fixed-point total.  Every sum has a fixed order (or is an integer
// sum), so the scores are deterministic.
// ---------------------------------------------------------------------------
constexpr int16_t kNoWeight = -32768;
// Exponent of a merge weight 2^(ms - m) <= 1 (an integer); exponents below the
// fp32 range give weight 0 either way.
__device__ __forceinline__ int16_t weight_exp(float e) { return (int16_t)max(-1000, (int)e); }

// LDS bytes of one score work-group: two Q tiles, row statistics.
template <class E, int D>
constexpr int score_lds_bytes() {
  return 2 * 32 * (D + 16 / (int)sizeof(typename E::T)) * (int)sizeof(typename E::T) + 3 * kScoreMaxRows * 4;
}

// Score work-group `wid` of `nwg` (logical (key block, KV head, row split),
// key_blocks x a.Hkv x row splits), LDS at smem (score_lds_bytes).
// FM: this instantiation can merge split partials in its score work-groups
// (ScoreMergeArgs::fused); the merge's registers fit beside the score pass's
// only in some shapes.
template <class E, int D, int KT, int NW, int NPF, bool FM>
__device__ void score_wg(const ScoreArgs& a, int wid, int nwg, int key_blocks, const ScoreMergeArgs& fm,
                         char* smem) {
  typedef typename E::T T;
  typedef Mma<E> M;
  constexpr int RT = 32;
  constexpr int EPV = 16 / (int)sizeof(T);
  constexpr int QSTR = D + EPV;
  constexpr int NKS = D / M::KS;
  constexpr int NT = 64 * NW;
  constexpr int BNK = NW * 32 * KT;
  constexpr int CPR = D / EPV;                       // 16-byte chunks per Q row
  constexpr int QCH = (RT * CPR + NT - 1) / NT;
  T* const Qs0 = reinterpret_cast<T*>(smem);         // [2][RT * QSTR]
  float* const sm = reinterpret_cast<float*>(smem + 2 * RT * QSTR * sizeof(T));
  float* const sr = sm + kScoreMaxRows;
  int* const slim = reinterpret_cast<int*>(sr + kScoreMaxRows);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hh = lane >> 5;
  // Logical work-group order (consecutive ids run on one XCD and share its
  // L2).  The 8-wave kernel (grids resident all at once): (key block, KV
  // head, row split), the key blocks of one (head, row split) sharing its Q
  // rows.  The 4-wave kernel (grids of several rounds, long pools): (row
  // split, key block, KV head), consecutive ids sharing a key block's K and a
  // head's key blocks sharing its Q tiles; with the key blocks fastest a
  // head's K (4.3 MB at the stress shape) streamed through the L2 once per
  // row split, and the launch fetched 157 MB instead of 55.
  const int wl = xcd_remap(wid, nwg);
  int kblock, g, rsplit;
  if constexpr (NW == 4) {
    rsplit = wl % fm.rsplits;
    const int wrest = wl / fm.rsplits;
    kblock = wrest % key_blocks;
    g = wrest / key_blocks;
  } else {
    kblock = wl % key_blocks;
    const int wrest = wl / key_blocks;
    g = wrest % a.Hkv;
    rsplit = wrest / a.Hkv;
  }
  const int key_wg = kblock * BNK;
  const int key_w = key_wg + wave * 32 * KT;

  const T* qbase = (const T*)a.qrot + (size_t)g * a.R * D;
  const T* kbase = (const T*)a.kpool + (size_t)g * a.cap * D;

  typename M::Frag kf[KT][NKS];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    const int key = key_w + kt * 32 + col;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      kf[kt][ks] = key < a.P ? M::ld(kbase + (size_t)pool_row(key, a.k0, a.foff) * D + ks * M::KS + hh * M::KL)
                             : M::zero();
  }
  double cs[KT];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) cs[kt] = 0.0;

  const int r0 = rsplit * a.rps;
  const int r1 = min(a.R, r0 + a.rps);
  // Rows whose token precedes every frame key of this work-group see none of them.
  int rstart = r0;
  if (key_wg >= a.k0) rstart = max(r0, (key_wg - a.k0) * a.G);
  const int nrow = r1 - rstart;
  const int ntile = nrow > 0 ? (nrow + RT - 1) / RT : 0;

  // NPF register stages of Q tiles: tile it's loads are issued NPF tiles
  // ahead of its compute; tiles pass through two LDS buffers.  The first
  // NPF tiles' loads are issued before the row statistics are merged, so the
  // two latencies overlap.
  u32x4_t qr[NPF][QCH];
  // Tile loads are buffer loads from the tile's first row: rows at or beyond
  // r1 lie past the resource's extent and read as zero, and threads without a
  // chunk (t >= RT * CPR) use an offset past any extent, so no load needs a
  // branch and the lane offsets are formed once.
  uint32_t qoff[QCH];
#pragma unroll
  for (int j = 0; j < QCH; ++j) {
    const int t = tid + j * NT;
    const int rr = t / CPR, cc = t - rr * CPR;
    qoff[j] = t < RT * CPR ? (uint32_t)(rr * D * (int)sizeof(T) + cc * 16) : 0x80000000u;
  }
  auto load_tile = [&](u32x4_t (&q)[QCH], int rt) {
    const __amdgpu_buffer_rsrc_t rsq = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T*>(qbase + (size_t)rt * D), (short)0, max(r1 - rt, 0) * D * (int)sizeof(T), 0x00020000);
#pragma unroll
    for (int j = 0; j < QCH; ++j) q[j] = __builtin_amdgcn_raw_buffer_load_b128(rsq, qoff[j], 0, 0);
  };
  auto store_tile = [&](const u32x4_t (&q)[QCH], int buf) {
#pragma unroll
    for (int j = 0; j < QCH; ++j) {
      const int t = tid + j * NT;
      const int rr = t / CPR, cc = t - rr * CPR;
      if (t < RT * CPR) *reinterpret_cast<u32x4_t*>(&Qs0[buf * RT * QSTR + rr * QSTR + cc * EPV]) = q[j];
    }
  };

  // Tiles past the last one read as zero (no rows in their extent), so every
  // stage is loaded unconditionally and the compiler knows which loads each
  // wait is for.
#pragma unroll
  for (int i = 0; i < NPF; ++i) load_tile(qr[i], rstart + i * RT);

  // Fused merge: task tid of this work-group's slice, (row, 4 dims) of the
  // rows [r0, r1) (rows fastest).  Its loads are in flight while the row
  // statistics are merged; the merge itself uses those statistics (this key
  // block starts before k0, so rstart = r0 and they cover every row).
  typedef typename PartialOut<E>::V PV;
  constexpr int MCPR = D / 4;
  PV mo[kMaxSplits];
  int8_t me[kMaxSplits];
  float mm[kMaxSplits];
  int m_row = -1, m_c = 0;
  if (FM && fm.fused && kblock < fm.mkb && tid < fm.mtpw) {
    const int nrow_m = r1 - r0;
    const int t = kblock * fm.mtpw + tid;
    if (t < nrow_m * MCPR) {
      m_row = r0 + t % nrow_m;
      m_c = t / nrow_m;
    }
  }
  if (FM && m_row >= 0) {
    const MergeArgs& mg = fm.mg;
    const size_t nrows = (size_t)mg.Hkv * mg.R;
    const size_t base = (size_t)g * mg.R + m_row;
#pragma unroll
    for (int sp = 0; sp < kMaxSplits; ++sp) {
      mm[sp] = -INFINITY;
      if (sp < mg.S) {
        const size_t ri = sp * nrows + base;
        mo[sp] = reinterpret_cast<const PV*>(mg.opart)[opart_group(ri, D) + (size_t)m_c * 32 + (ri & 31)];
        me[sp] = sizeof(T) == 2 ? mg.epart[ri] : (int8_t)0;
        mm[sp] = mg.mpart[stat_index(base, sp, mg.ss)];
      }
    }
  }
  // Row statistics of the work-group's rows (padded to whole tiles), from the
  // key-split partials of pass 1: m = max_s m_s, l = sum_s 2^(m_s - m) l_s
  // (exact powers of two, fp64 sum).  Padding rows get 1/l = 0.
  for (int i = tid; i < ntile * RT; i += NT) {
    const int r = rstart + i;
    float m = 0.f, rinv = 0.f;
    int lim = 0;
    if (r < r1) {
      float ms[kMaxSplits];
      double ls[kMaxSplits];
      load_split_stats(a.mpart, a.lpart, (size_t)g * a.R + r, a.S, a.ss, ms, ls);
      double l;
      merge_split_stats(ms, ls, m, l);
      rinv = (float)(1.0 / l);
      lim = a.k0 + r / a.G + 1;   // keys below this are visible to row r
    }
    sm[i] = m;
    sr[i] = rinv;
    slim[i] = lim;
  }

  if (ntile > 0) store_tile(qr[0], 0);
  // Every load issued so far has arrived on every path (the statistics were
  // issued after the first tiles, and the merge needs its partials next);
  // saying so keeps the compiler from waiting for the loop's own prefetch
  // loads before the first matrix instruction of a tile.
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();
  if (FM && m_row >= 0) {
    // m and 1/l of the row, as the split merge forms them; the same weights,
    // arithmetic and order as merge_group, so O does not depend on which
    // work-groups merge it.
    const MergeArgs& mg = fm.mg;
    const float m = sm[m_row - rstart];
    const float inv = sr[m_row - rstart];
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sp = 0; sp < kMaxSplits; ++sp) {
      if (sp < mg.S && mm[sp] != -INFINITY) {
        const float w = ldexpf(1.f, weight_exp(mm[sp] - m));
        if (w != 0.f) {
          const f32x4_t o4 = PartialOut<E>::unpack(mo[sp]);
          const float wo = sizeof(T) == 2 ? ldexpf(w, (int)me[sp]) : w;
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] = fmaf(wo, o4[e], acc[e]);
        }
      }
    }
    const int layer = g / mg.lh;
    const int tok = m_row / mg.G;
    const int h = (g - layer * mg.lh) * mg.G + (m_row - tok * mg.G);
    T* out = (T*)mg.out + (size_t)layer * mg.out_ls + ((size_t)tok * mg.Hq + h) * D + m_c * 4;
    if constexpr (sizeof(T) == 2) {
      const u32x2_t v = {(uint32_t)f32_to_bf16(acc[0] * inv) | ((uint32_t)f32_to_bf16(acc[1] * inv) << 16),
                         (uint32_t)f32_to_bf16(acc[2] * inv) | ((uint32_t)f32_to_bf16(acc[3] * inv) << 16)};
      *reinterpret_cast<u32x2_t*>(out) = v;
    } else {
      *reinterpret_cast<f32x4_t*>(out) = acc * inv;
    }
  }
  for (int it0 = 0; it0 < ntile; it0 += NPF)
#pragma unroll
  for (int ip = 0; ip < NPF; ++ip) {
    const int it = it0 + ip;
    if (it >= ntile) break;
    const int buf = it & 1;
    const int ro = it * RT;   // tile offset inside the statistics arrays
    load_tile(qr[ip], rstart + (it + NPF) * RT);
    // S = Q K^T for the KT key tiles: Q fragments read once per k-slice and
    // fed to KT independent accumulation chains.
    f32x16_t acc[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) acc[kt] = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const typename M::Frag af = M::ld(&Qs0[buf * RT * QSTR + col * QSTR + ks * M::KS + hh * M::KL]);
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) acc[kt] = M::mma(af, kf[kt][ks], acc[kt]);
    }
    // Statistics of the lane's 16 rows of this tile.
    f32x4_t mv[4], rv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      mv[j] = *reinterpret_cast<const f32x4_t*>(&sm[ro + 8 * j + 4 * hh]);
      rv[j] = *reinterpret_cast<const f32x4_t*>(&sr[ro + 8 * j + 4 * hh]);
    }
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      const int key_t0 = key_w + kt * 32;
      const int key = key_t0 + col;
      // The lane's 16 weights of this key summed as a tree (four partial sums
      // over the row groups, then pairwise): fewer roundings in series than a
      // running sum.
      float part[4];
      if (key_t0 + 31 >= a.k0) {  // tile holds frame keys: causal visibility per row
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int4 lv = *reinterpret_cast<const int4*>(&slim[ro + 8 * j + 4 * hh]);
          const int lvv[4] = {lv.x, lv.y, lv.z, lv.w};
          float pq[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float x = acc[kt][4 * j + q];
            const float p = fast_exp2(fmaf(x, a.c_lo, fmaf(x, a.c_hi, -mv[j][q]))) * rv[j][q];
            pq[q] = key < lvv[q] ? p : 0.f;
          }
          part[j] = (pq[0] + pq[1]) + (pq[2] + pq[3]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float pq[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float x = acc[kt][4 * j + q];
            pq[q] = fast_exp2(fmaf(x, a.c_lo, fmaf(x, a.c_hi, -mv[j][q]))) * rv[j][q];
          }
          part[j] = (pq[0] + pq[1]) + (pq[2] + pq[3]);
        }
      }
      cs[kt] += (double)((part[0] + part[1]) + (part[2] + part[3]));
    }
    if (it + 1 < ntile) store_tile(qr[(ip + 1) % NPF], buf ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    const double tot = halves_sum(cs[kt]);
    const int key = key_w + kt * 32 + col;
    if (hh == 0 && key < a.P && tot > 0.0) {
      const unsigned long long fx =
          (unsigned long long)(tot * (double)(1ull << kScoreFracBits) + 0.5);
      atomicAdd(&a.colsum[(size_t)(g / a.lh) * a.cap + key], fx);
    }
  }
}

// ---------------------------------------------------------------------------
// Top-B selection (work-group 0 of frame_kernel, 1024 threads).  With the
// recency window the selection value is the position instead of the score, so
// the same steps evict the oldest tokens.
// Scores s_j = (fixed-point column sum) / (Hq*T), rounded to fp32.  The pool
// keeps its B best under (score descending, position ascending), i.e. it
// evicts the E = P - B smallest 64-bit keys
//     key_j = (bits of s_j) << 32 | ~pos_j
// (non-negative fp32 values order like their bit patterns; among equal scores
// the newer token has the smaller key).  The keys are distinct, so the evicted
// set is unique.  The score bits live in LDS.  The E-th smallest key is
// bracketed by refining a range of score bits with histograms of up to 4096
// power-of-two-wide buckets until the boundary bucket holds at most kSelCand
// candidates (usually after one round).  If the boundary is a single score
// shared by more candidates (exact ties), the same refinement runs over ~pos
// of the tied rows.  The candidates are then ranked by their keys; positions
// are read only for candidates whose score bits tie.  The state keeps its
// slots: evicted slots below B receive, in ascending order, the kept rows at
// or beyond B (the frame's tail), so at most T rows move per KV head; the move
// list is built with one block-wide scan.
// ---------------------------------------------------------------------------

// Inclusive prefix sum over the 64 lanes of a wave (row shifts within rows of
// 16 lanes, then the row broadcasts of lanes 15 and 31).
__device__ __forceinline__ int wave_incl_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Minimum / maximum of the wave, valid in lane 63 (same lane pattern).
__device__ __forceinline__ uint32_t wave_min_last(uint32_t x) {
  const int id = -1;
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x111, 0xf, 0xf, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x112, 0xf, 0xf, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x114, 0xf, 0xf, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x118, 0xf, 0xf, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x142, 0xa, 0xf, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x143, 0xc, 0xf, false));
  return x;
}
__device__ __forceinline__ uint32_t wave_max_last(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false));
  return x;
}

// Exclusive prefix sum over the work-group; *total receives the sum.  One
// barrier; sh[] must not be written again before the caller's next barrier.
__device__ int block_excl_scan(int v, int* sh, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int inc = wave_incl_sum(v);
  if (lane == 63) sh[wave] = inc;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSelectThreads / 64; ++w) {
    const int x = sh[w];
    before += w < wave ? x : 0;
    tot += x;
  }
  *total = tot;
  return before + inc - v;
}

// Moves kept in LDS (the histogram's space) when the list holds at most this many.
constexpr int kSelListMax = kSelectBins / 2;

struct SelectShared {
  int hist[kSelectBins];
  uint32_t cand_v[kSelCand];
  uint32_t cand_np[kSelCand];
  int cand_idx[kSelCand];
  int scan[kSelectThreads / 64];
  uint32_t red_lo[kSelectThreads / 64], red_hi[kSelectThreads / 64];
  int bucket, below, cnt, ncand, any_tie;
};

// One refinement of the boundary: histogram of the values get(idx) in
// [lo, hi] (get returns false for rows outside the set), then the bucket
// holding the need-th smallest becomes the new [lo, hi].  Returns that
// bucket's count.  The histogram is all zero on entry and on return: each
// thread clears the bins it scanned, and the next round's counts come after
// its first barrier.  sh.bucket/below/cnt are written by the one thread whose
// bins hold the need-th value; the next round writes them only after its
// first barrier, when every thread has read them.
constexpr int kBinsPerThread = kSelectBins / kSelectThreads;
static_assert(kBinsPerThread * kSelectThreads == kSelectBins, "histogram scan shape");
template <class Get>
__device__ int refine_boundary(SelectShared& sh, int P, uint32_t& lo, uint32_t& hi, int& need, Get get) {
  const int tid = threadIdx.x;
  const uint32_t span = hi - lo;
  const int bits = span ? 32 - __clz((int)span) : 0;
  const int shift = bits > 12 ? bits - 12 : 0;
  const int nb = (int)(span >> shift) + 1;
  for (int idx = tid; idx < P; idx += kSelectThreads) {
    uint32_t v;
    if (get(idx, v) && v >= lo && v <= hi) atomicAdd(&sh.hist[(int)((v - lo) >> shift)], 1);
  }
  __syncthreads();
  int cb[kBinsPerThread];
  int sb = 0;
#pragma unroll
  for (int u = 0; u < kBinsPerThread; ++u) {
    const int q = tid * kBinsPerThread + u;
    cb[u] = q < nb ? sh.hist[q] : 0;
    sb += cb[u];
  }
  int total;
  int run = block_excl_scan(sb, sh.scan, &total);
#pragma unroll
  for (int u = 0; u < kBinsPerThread; ++u) {
    const int q = tid * kBinsPerThread + u;
    if (q < nb && run < need && need <= run + cb[u]) {
      sh.bucket = q;
      sh.below = run;
      sh.cnt = cb[u];
    }
    run += cb[u];
    sh.hist[q] = 0;
  }
  __syncthreads();
  need -= sh.below;
  const uint32_t blo = lo + ((uint32_t)sh.bucket << shift);
  const uint32_t width_m1 = (uint32_t)((1ull << shift) - 1ull);
  hi = (hi - blo > width_m1) ? blo + width_m1 : hi;
  lo = blo;
  return sh.cnt;
}

// val: [P] words of dynamic LDS, the score bits of the pool rows (bit 31 set
// once a row is evicted).
__device__ void select_top_b(const SelArgs& a, SelectShared& sh, uint32_t* val) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Row j*kSelectThreads + tid of the pool belongs to thread tid, so that every
  // global access of a wave is contiguous.  No global store precedes a
  // barrier (a barrier waits for the wave's outstanding stores): the outputs
  // are written after the last one.
  const int C = (a.P + kSelectThreads - 1) / kSelectThreads;
  constexpr int kChunk = 8;
  // Zero state of the refinement and the candidate count; the barrier after
  // the loads publishes it.
#pragma unroll
  for (int u = 0; u < kBinsPerThread; ++u) sh.hist[tid * kBinsPerThread + u] = 0;
  if (tid == 0) {
    sh.ncand = 0;
    sh.any_tie = 0;
  }
  uint32_t flo = ~0u, fhi = 0u;
  for (int j0 = 0; j0 < C; j0 += kChunk) {
    unsigned long long fx[kChunk];
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      const int idx = (j0 + j) * kSelectThreads + tid;
      fx[j] = 0ull;
      if (idx < a.P)
        fx[j] = a.recent ? (unsigned long long)a.pool_pos[pool_row(idx, a.k0, a.foff)] : a.colsum[idx];
    }
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      const int idx = (j0 + j) * kSelectThreads + tid;
      if (idx < a.P) {
        // Selection value: the score's bits, or for the recency window the
        // position (older tokens have smaller values and are evicted first).
        const uint32_t fb = a.recent ? (uint32_t)fx[j]
                                     : __float_as_uint((float)((double)fx[j] * a.score_scale));
        val[idx] = fb;
        flo = min(flo, fb);
        fhi = max(fhi, fb);
      }
    }
  }

  if (a.mode == kSelEvict) {
    // Range of the score bits.
    flo = wave_min_last(flo);
    fhi = wave_max_last(fhi);
    if (lane == 63) {
      sh.red_lo[wave] = flo;
      sh.red_hi[wave] = fhi;
    }
    __syncthreads();
    uint32_t lo = ~0u, hi = 0u;
#pragma unroll
    for (int w = 0; w < kSelectThreads / 64; ++w) {
      lo = min(lo, sh.red_lo[w]);
      hi = max(hi, sh.red_hi[w]);
    }

    int need = a.P - a.B;  // keys still to evict inside the boundary range
    int cnt;
    do {
      cnt = refine_boundary(sh, a.P, lo, hi, need, [&](int idx, uint32_t& v) {
        v = val[idx];
        return true;
      });
    } while (cnt > kSelCand && lo != hi);

    // Exact ties beyond kSelCand at one score: refine over ~pos of the tied rows.
    uint32_t plo = 0u, phi = ~0u;
    const bool tie_stage = cnt > kSelCand;
    if (tie_stage) {
      const uint32_t tied = lo;
      do {
        cnt = refine_boundary(sh, a.P, plo, phi, need, [&](int idx, uint32_t& v) {
          if (val[idx] != tied) return false;
          v = ~(uint32_t)a.pool_pos[pool_row(idx, a.k0, a.foff)];
          return true;
        });
      } while (cnt > kSelCand && plo != phi);
    }

    // Rows below the boundary are evicted (bit 31 of their entry); the
    // candidates are collected.
    for (int idx = tid; idx < a.P; idx += kSelectThreads) {
      const uint32_t v = val[idx];
      bool ev = v < lo;
      bool cand = v >= lo && v <= hi;
      if (cand && tie_stage) {
        const uint32_t np = ~(uint32_t)a.pool_pos[pool_row(idx, a.k0, a.foff)];
        ev = np < plo;
        cand = np >= plo && np <= phi;
      }
      if (cand) {
        const int slot = atomicAdd(&sh.ncand, 1);
        if (slot < kSelCand) {   // always true when positions are unique
          sh.cand_v[slot] = v;
          sh.cand_idx[slot] = idx;
        }
      }
      if (ev) val[idx] = v | 0x80000000u;
    }
    __syncthreads();
    // Rank of each candidate among the candidates: by score bits, and by ~pos
    // among equal score bits (read only when such ties exist).
    const int nc = min(sh.ncand, kSelCand);
    int rank = 0, eq = 0;
    uint32_t mine = 0u;
    if (tid < nc) {
      mine = sh.cand_v[tid];
      for (int c = 0; c < nc; ++c) {
        const uint32_t o = sh.cand_v[c];
        rank += o < mine ? 1 : 0;
        eq += o == mine ? 1 : 0;
      }
      if (eq == 1 && rank < need) val[sh.cand_idx[tid]] |= 0x80000000u;
      if (eq > 1) sh.any_tie = 1;
    }
    __syncthreads();
    if (sh.any_tie) {
      uint32_t np = 0u;
      if (tid < nc && eq > 1) {
        np = ~(uint32_t)a.pool_pos[pool_row(sh.cand_idx[tid], a.k0, a.foff)];
        sh.cand_np[tid] = np;
      }
      __syncthreads();
      if (tid < nc && eq > 1) {
        for (int c = 0; c < nc; ++c)
          rank += (sh.cand_v[c] == mine && sh.cand_np[c] < np) ? 1 : 0;
        if (rank < need) val[sh.cand_idx[tid]] |= 0x80000000u;
      }
      __syncthreads();
    }
  }

  // Without the eviction steps nothing is evicted and nothing moves.
  if (a.mode != kSelEvict) {
    if (tid == 0) *a.move_count = 0;
    return;
  }
  // Move list from the flags: every thread takes a contiguous range of C rows
  // (at most 32: P <= kMaxPool) so that holes (evicted slots below B) and
  // movers (kept rows at or beyond B) come out ascending.  Its holes and
  // movers are kept as bit masks, so the list writes below visit only them.
  static_assert(kMaxPool <= 32 * kSelectThreads, "a thread's rows fit a 32-bit mask");
  const int i0 = tid * C;
  const int i1 = min(a.P, i0 + C);
  uint32_t hmask = 0u, mmask = 0u;
  for (int j0 = 0; j0 < C; j0 += kChunk) {
#pragma unroll
    for (int j = j0; j < j0 + kChunk; ++j) {
      const int idx = i0 + j;
      if (j < C && idx < i1) {
        const uint32_t ev = val[idx] >> 31;
        hmask |= (idx < a.B && ev) ? (1u << j) : 0u;
        mmask |= (idx >= a.B && !ev) ? (1u << j) : 0u;
      }
    }
  }
  const int holes = __popc(hmask), movers = __popc(mmask);
  int total;
  const int base = block_excl_scan(holes | (movers << 16), sh.scan, &total);

  // Outputs: the move list only.  Scores, keep flags and positions of the
  // scored pool are rebuilt on request from the column sums and the move
  // list.  With unique positions exactly P - B rows are evicted, so at most
  // min(T, B) moves exist; the writes are still bounded by the lists'
  // capacity, so inconsistent inputs cannot write past them.  When the list
  // fits in LDS (the histogram's space, free by now) it goes there, and every
  // global store waits until after the barrier below (which would otherwise
  // wait for them).
  const bool lds_list = a.list_stride <= kSelListMax;
  int* l_dst = sh.hist;
  int* l_src = sh.hist + kSelListMax;
  {
    int bh = base & 0xffff, bm = base >> 16;
    for (; hmask != 0u && bh < a.list_stride; ++bh) {
      const int idx = i0 + __builtin_ctz(hmask);
      hmask &= hmask - 1u;
      if (lds_list) l_dst[bh] = idx;
      else a.move_dst[bh] = idx;
    }
    for (; mmask != 0u && bm < a.list_stride; ++bm) {
      const int row = pool_row(i0 + __builtin_ctz(mmask), a.k0, a.foff);
      mmask &= mmask - 1u;
      if (lds_list) l_src[bm] = row;
      else a.move_src[bm] = row;
    }
  }
  const int moves = min(min(total & 0xffff, total >> 16), a.list_stride);
  if (moves == 0) {
    if (tid == 0) *a.move_count = 0;
    return;
  }
  __syncthreads();
  // The moves: K and V of every KV head (16 bytes per task), and the
  // positions.  A round issues all its loads before its stores: one memory
  // round trip per round (one round for a frame of up to 1024 moves of
  // 4 * 1024 chunks).
  const int cpr = a.row_bytes / 16;
  const int per_move = a.Hkv * cpr;
  const int tasks = moves * per_move;
  constexpr int kMoveRound = 4;
  for (int t0 = 0, mp0 = 0; t0 < tasks || mp0 < moves; t0 += kMoveRound * kSelectThreads, mp0 += kSelectThreads) {
    u32x4_t kv[kMoveRound], vv[kMoveRound];
    size_t dof[kMoveRound];
#pragma unroll
    for (int m = 0; m < kMoveRound; ++m) {
      const int t = t0 + tid + m * kSelectThreads;
      dof[m] = ~(size_t)0;
      if (t < tasks) {
        const int mi = t / per_move;
        const int rem = t - mi * per_move;
        const int g = rem / cpr, c = rem - g * cpr;
        const int dst = min(max(lds_list ? l_dst[mi] : a.move_dst[mi], 0), a.B - 1);
        const int src = min(max(lds_list ? l_src[mi] : a.move_src[mi], a.B), a.cap - 1);
        const size_t so = ((size_t)g * a.cap + src) * a.row_bytes + (size_t)c * 16;
        dof[m] = ((size_t)g * a.cap + dst) * a.row_bytes + (size_t)c * 16;
        kv[m] = *reinterpret_cast<const u32x4_t*>((const char*)a.kpool + so);
        vv[m] = *reinterpret_cast<const u32x4_t*>((const char*)a.vpool + so);
      }
    }
    // One position move per thread and round.
    const int mp = mp0 + tid;
    int pdst = -1, psrc = 0, pd = 0, ps = 0;
    if (mp < moves) {
      pdst = min(max(lds_list ? l_dst[mp] : a.move_dst[mp], 0), a.B - 1);
      psrc = min(max(lds_list ? l_src[mp] : a.move_src[mp], a.B), a.cap - 1);
      pd = a.pool_pos[pdst];
      ps = a.pool_pos[psrc];
    }
#pragma unroll
    for (int m = 0; m < kMoveRound; ++m) {
      if (dof[m] == ~(size_t)0) continue;
      *reinterpret_cast<u32x4_t*>((char*)a.kpool + dof[m]) = kv[m];
      *reinterpret_cast<u32x4_t*>((char*)a.vpool + dof[m]) = vv[m];
    }
    if (pdst >= 0) {
      a.evicted_pos[pdst] = pd;
      a.pool_pos[pdst] = ps;
      if (lds_list) {
        a.move_dst[mp] = pdst;
        a.move_src[mp] = psrc;
      }
    }
  }
  if (tid == 0) *a.move_count = moves;
}

// Merge of the key splits of pass 1:
//   m = max_s m_s,  l = sum_s 2^(m_s - m) l_s,  O = sum_s 2^(m_s - m) O_s / l,
// for one group of 32 flat rows (flat row = g*R + r), written to O [T][Hq][d].
// A task is (row, 4 dims) with rows fastest, matching the lane-order layout of
// the partials; a work-group of NT threads takes TPT tasks per thread.  One
// thread per row merges the row's split statistics into LDS (weights
// 2^(m_s - m), exact powers of two, and 1/l), which the row's other tasks
// read.  Partials of splits that saw no key of a row were never written, so
// they are selected out, not multiplied.  Up to kMaxSplits splits (a frame)
// the statistics sit in registers; more (a text chunk over a long cache, up to
// kMaxMergeSplits) are merged in two loops over the splits with the same
// arithmetic in the same order.  LDS: merge_lds_bytes(S).
// LDS bytes of a merge work-group for S splits.
__host__ __device__ inline int merge_lds_bytes(int S) {
  return 32 * 4 + 32 * (S <= kMaxSplits ? kMaxSplits : S) * 2;
}

template <class E, int D, int NT>
__device__ void merge_group(const MergeArgs& a, int grp, float* lds) {
  typedef typename E::T T;
  constexpr int CPR = D / 4;
  constexpr int TASKS = 32 * CPR;
  constexpr int TPT = (TASKS + NT - 1) / NT;      // tasks per thread
  // Partial loads in flight per task (a frame's 17 splits at B = 4096 arrive
  // in two rounds with one task per thread).
  constexpr int MCH = sizeof(T) == 2 ? (TPT == 1 ? 9 : (TPT == 2 ? 5 : 3)) : (TPT == 1 ? 4 : 2);
  const int wstr = a.S <= kMaxSplits ? kMaxSplits : a.S;   // weights per row
  // Weights are exact powers of two, kept as their exponents (kNoWeight: the
  // split saw no key of the row).
  float* rinv = lds;                                        // [32]
  int16_t* wexp = reinterpret_cast<int16_t*>(lds + 32);     // [32][wstr]
  typedef typename PartialOut<E>::V PV;
  const int tid = threadIdx.x;
  const size_t nrows = (size_t)a.Hkv * a.R;
  const size_t row0 = (size_t)grp * 32;
  PV os[TPT][MCH];
  int8_t ep[TPT][MCH];
  auto load_chunk = [&](int s0) {
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int task = tid + u * NT;
      const int rr = task & 31, c = task >> 5;
      const size_t base = row0 + rr;
#pragma unroll
      for (int j = 0; j < MCH; ++j) {
        const int sp = s0 + j;
        if (task < TASKS && sp < a.S && base < nrows) {
          const size_t ri = sp * nrows + base;
          os[u][j] = reinterpret_cast<const PV*>(a.opart)[opart_group(ri, D) + (size_t)c * 32 + (ri & 31)];
          ep[u][j] = sizeof(T) == 2 ? a.epart[ri] : (int8_t)0;
        }
      }
    }
  };
  load_chunk(0);
  if (tid < 32) {
    const size_t base = row0 + tid;
    if (a.S > kMaxSplits) {
      float inv = 0.f;
      if (base < nrows) {
        float m = -INFINITY;
        for (int sp = 0; sp < a.S; ++sp) m = fmaxf(m, a.mpart[stat_index(base, sp, a.ss)]);
        double l = 0.0;
        for (int sp = 0; sp < a.S; ++sp) {
          const float ms = a.mpart[stat_index(base, sp, a.ss)];
          int16_t we = kNoWeight;
          if (ms != -INFINITY) {
            we = weight_exp(ms - m);
            l += ldexp(a.lpart[stat_index(base, sp, a.ss)], (int)(ms - m));
          }
          wexp[tid * wstr + sp] = we;
        }
        inv = (float)(1.0 / l);
      } else {
        for (int sp = 0; sp < a.S; ++sp) wexp[tid * wstr + sp] = kNoWeight;
      }
      rinv[tid] = inv;
    } else {
      int16_t w[kMaxSplits];
      float inv = 0.f;
#pragma unroll
      for (int sp = 0; sp < kMaxSplits; ++sp) w[sp] = kNoWeight;
      if (base < nrows) {
        float ms[kMaxSplits];
        double ls[kMaxSplits];
        load_split_stats(a.mpart, a.lpart, base, a.S, a.ss, ms, ls);
        float m;
        double l;
        merge_split_stats(ms, ls, m, l);
#pragma unroll
        for (int sp = 0; sp < kMaxSplits; ++sp) w[sp] = ms[sp] != -INFINITY ? weight_exp(ms[sp] - m) : kNoWeight;
        inv = (float)(1.0 / l);
      }
#pragma unroll
      for (int sp = 0; sp < kMaxSplits; ++sp) wexp[tid * kMaxSplits + sp] = w[sp];
      rinv[tid] = inv;
    }
  }
  __syncthreads();
  f32x4_t acc[TPT];
#pragma unroll
  for (int u = 0; u < TPT; ++u) acc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < a.S; s0 += MCH) {
    if (s0 > 0) load_chunk(s0);
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int rr = (tid + u * NT) & 31;
#pragma unroll
      for (int j = 0; j < MCH; ++j) {
        const int sp = s0 + j;
        // Splits that saw no key of the row have weight 0 and unwritten partials.
        const int we = sp < a.S ? wexp[rr * wstr + sp] : kNoWeight;
        const float w = we == kNoWeight ? 0.f : ldexpf(1.f, we);
        if (w != 0.f) {
          const f32x4_t o4 = PartialOut<E>::unpack(os[u][j]);
          const float wo = sizeof(T) == 2 ? ldexpf(w, (int)ep[u][j]) : w;
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[u][e] = fmaf(wo, o4[e], acc[u][e]);
        }
      }
    }
  }
#pragma unroll
  for (int u = 0; u < TPT; ++u) {
    const int task = tid + u * NT;
    const int rr = task & 31, c = task >> 5;
    const size_t base = row0 + rr;
    if (task >= TASKS || base >= nrows) continue;
    const float inv = rinv[rr];
    const int g = (int)(base / a.R), r = (int)(base - (size_t)g * a.R);
    const int layer = g / a.lh;
    const int tok = r / a.G;
    const int h = (g - layer * a.lh) * a.G + (r - tok * a.G);
    T* out = (T*)a.out + (size_t)layer * a.out_ls + ((size_t)tok * a.Hq + h) * D + c * 4;
    if constexpr (sizeof(T) == 2) {
      const u32x2_t v = {(uint32_t)f32_to_bf16(acc[u][0] * inv) | ((uint32_t)f32_to_bf16(acc[u][1] * inv) << 16),
                         (uint32_t)f32_to_bf16(acc[u][2] * inv) | ((uint32_t)f32_to_bf16(acc[u][3] * inv) << 16)};
      *reinterpret_cast<u32x2_t*>(out) = v;
    } else {
      *reinterpret_cast<f32x4_t*>(out) = acc[u] * inv;
    }
  }
}

// The frame launch: per layer (grid y), work-group 0 makes the previous
// frame's Top-B decision and its moves when nsel = 1; the others rotate and
// append this frame's tokens.  Dynamic LDS: the selection's P score words.
// The selection of layer `layer` of a stack (its slices of every array).
__device__ void select_layer(SelArgs b, size_t layer, SelectShared& sh, uint32_t* val) {
  const size_t pool_bytes = (size_t)b.Hkv * b.cap * b.row_bytes;
  b.colsum += layer * b.cap;
  b.pool_pos += layer * b.cap;
  b.evicted_pos += layer * b.B;
  b.move_dst += layer * b.list_stride;
  b.move_src += layer * b.list_stride;
  b.move_count += layer;
  b.kpool = (char*)b.kpool + layer * pool_bytes;
  b.vpool = (char*)b.vpool + layer * pool_bytes;
  select_top_b(b, sh, val);
}

template <class E, int D>
__global__ __launch_bounds__(kSelectThreads) void frame_kernel(RopeArgs a) {
  const size_t layer = blockIdx.y;
  if ((int)blockIdx.x < a.nsel) {
    __shared__ SelectShared sh;
    extern __shared__ __attribute__((aligned(16))) uint32_t sel_val[];
    select_layer(a.sel, layer, sh, sel_val);
    return;
  }
  rope_wg<E, D>(a, layer, (int)blockIdx.x - a.nsel);
}

// Recency policy, the launch after pass 1: work-group l < layers evicts the
// oldest rows of layer l's pool and makes its moves (the merge reads only the
// split partials, never the pool), the others merge the key splits into O.
// Dynamic LDS: the selection's P score words, or the merge's weights.
template <class E, int D>
__global__ __launch_bounds__(kSelectThreads) void select_merge_kernel(SelectMergeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t dyn[];
  if ((int)blockIdx.x < a.layers) {
    __shared__ SelectShared sh;
    select_layer(a.sel, blockIdx.x, sh, dyn);
    return;
  }
  merge_group<E, D, kSelectThreads>(a.mg, (int)blockIdx.x - a.layers, reinterpret_cast<float*>(dyn));
}

// The launch after pass 1: merge work-groups first, then the score pass.
template <class E, int D, int KT, int NW, int NPF = 1, bool FM = false>
__global__ __launch_bounds__(64 * NW, 1) void score_merge_kernel(ScoreMergeArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int wg = blockIdx.x;
  if (wg < a.merge_wgs) {
    merge_group<E, D, 64 * NW>(a.mg, wg, reinterpret_cast<float*>(smem));
    return;
  }
  score_wg<E, D, KT, NW, NPF, FM>(a.sc, wg - a.merge_wgs, (int)gridDim.x - a.merge_wgs, a.key_blocks, a, smem);
}

// The scores view of the last scored pool (one thread per candidate, layer
// blockIdx.y): the fp32 score of the column sum (the value the selection
// ranked), the keep flag from the move list, and the candidate's position.
__global__ __launch_bounds__(256) void score_view_kernel(ScoreViewArgs a) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= a.P) return;
  const size_t l = blockIdx.y, lc = l * a.cap;
  const int row = pool_row(j, a.k0, a.foff);
  const int32_t* mdst = a.move_dst + l * a.list_stride;
  const int32_t* msrc = a.move_src + l * a.list_stride;
  const int cnt = min(a.move_count[l], a.list_stride);
  int keep;
  if (j < a.B) {
    keep = 1;
    for (int i = 0; i < cnt; ++i) keep &= mdst[i] != j;
  } else {
    keep = 0;
    for (int i = 0; i < cnt; ++i) keep |= msrc[i] == row;
  }
  a.scores[lc + j] = (float)((double)a.colsum[lc + j] * a.score_scale);
  a.keep_flag[lc + j] = keep;
  a.score_pos[lc + j] = (a.moved && j < a.B && !keep) ? a.evicted_pos[l * a.B + j] : a.pool_pos[lc + row];
}

}  // namespace

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
static constexpr int kKtBf16 = 2;  // key tiles per wave in the score pass
static constexpr int kKtF32 = 1;

// Register stages of pass 1's block prefetch (a block's loads are issued
// NPF blocks ahead of its compute): 4 for d = 64, so that the 4-block splits
// of a single layer at B = 4096 load every block in the prologue (pass 1
// 11.4 -> 10.6 us at ivl3_1b); 2 for d = 128, the most its registers allow
// without spills.
static constexpr int attn_prefetch(int d) { return d == 128 ? 2 : 4; }

// Compute units of the current device (0 if unknown).
static int device_cus() {
  static int cus = -1;
  if (cus < 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      n = 0;
    cus = n;
  }
  return cus;
}

// Keys per pass-1 block (128-key blocks measured slower: fewer resident
// stages per LDS byte).
int attn_block_keys(Dt, int) { return kAttnBN; }

// Pass-1 shape: bf16 uses 8 waves of one 32-query tile each (two waves per
// SIMD, so one wave's matrix work overlaps the other's softmax); fp32 (tiny
// shapes) uses 4 waves.
int attn_rows_per_wg(Dt dt, int) { return dt != Dt::BF16 ? 4 * 32 : 8 * 32; }
// Score pass shape: 4 waves (256 keys per work-group), or for bf16 8 waves
// (512 keys), which halves the Q traffic: faster when the whole grid is
// resident at once (a single layer at B = 4096: 9.9 -> 9.4 us), slower on the
// long-pool shapes and stacks, whose grids take several rounds (stress shape
// 69 -> 78 us).  The runtime picks per frame.
// Register stages of the score pass's Q-tile prefetch (4-wave kernel): 4 for
// d = 128 (5-7 % faster on the long-pool shapes), 2 for d = 64, where it
// leaves room for three waves per SIMD (16 % faster on the 28-layer ivl3_1b
// stack).
static constexpr int score_prefetch(int d) { return d == 64 ? 2 : 4; }

// Work-groups of the (4-wave) score kernel that fit on one CU at once (0 if unknown).
int score_wgs_per_cu(Dt dt, int d) {
  int n = 0;
  hipError_t e = hipSuccess;
  if (dt == Dt::BF16) {
    e = d == 64 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(
                      &n, score_merge_kernel<BF16, 64, kKtBf16, 4, score_prefetch(64)>, 256,
                      score_lds_bytes<BF16, 64>())
                : hipOccupancyMaxActiveBlocksPerMultiprocessor(
                      &n, score_merge_kernel<BF16, 128, kKtBf16, 4, score_prefetch(128)>, 256,
                      score_lds_bytes<BF16, 128>());
  }
  return e == hipSuccess ? n : 0;
}
// Work-groups of the 8-wave score kernel (bf16) that fit on one CU at once.
int score8_wgs_per_cu(int d) {
  int n = 0;
  const hipError_t e = d == 64
      ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, score_merge_kernel<BF16, 64, kKtBf16, 8>, 512,
                                                     score_lds_bytes<BF16, 64>())
      : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, score_merge_kernel<BF16, 128, kKtBf16, 8>, 512,
                                                     score_lds_bytes<BF16, 128>());
  return e == hipSuccess ? n : 0;
}
int score_keys_per_wg(Dt dt, int waves) { return waves * 32 * (dt == Dt::BF16 ? kKtBf16 : kKtF32); }

int merge_wgs(int64_t rows) {
  const int64_t groups = (rows + 31) / 32;
  return (int)((groups + kXcds - 1) / kXcds * kXcds);
}

hipError_t launch_rope_table(const RopeTableArgs& a, hipStream_t s) {
  const size_t total = (size_t)a.npos * a.half;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

// Four pairs per task keep each thread's load, rotation and store chain short
// (latency-bound launches: a single layer of a few hundred tokens); with more
// than 2^20 such tasks in the launch (large frames, stacks) 16-byte accesses
// move the bytes faster (28-layer qwen3vl_2b stack: 161 -> 135 us).
int rope_pairs_for(int T, int Hq, int Hkv, int d, int esize, int layers) {
  if (esize != 2) return 4;
  return (int64_t)layers * rope_qk_tasks(T, Hq, Hkv, d, 4) > (int64_t(1) << 20) ? 8 : 4;
}

// Work-groups of the RoPE part of a launch for T tokens (after the selection
// work-group).
int rope_blocks(int T, int Hq, int Hkv, int d, int esize, int pairs) {
  return (int)((rope_qk_tasks(T, Hq, Hkv, d, pairs) + rope_v_tasks(T, Hkv, d, esize) + kSelectThreads - 1) /
               kSelectThreads);
}

template <class E, int D>
static hipError_t launch_frame_t(const RopeArgs& a, int layers, hipStream_t s, const LaunchTiming& tm) {
  const dim3 grid(a.nsel + a.rope_blocks, layers);
  const size_t lds = a.nsel ? (size_t)a.sel.P * sizeof(uint32_t) : 0;
  // The selection's LDS may exceed the default dynamic limit (a failure here
  // surfaces as a launch error below).
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&frame_kernel<E, D>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     kMaxPool * (int)sizeof(uint32_t));
  (void)attr;
  hipExtLaunchKernelGGL((frame_kernel<E, D>), grid, dim3(kSelectThreads), lds, s, tm.start, tm.stop, 0, a);
  return hipGetLastError();
}

template <class E, int D>
static hipError_t launch_select_merge_t(const SelectMergeArgs& a, int merge_groups, hipStream_t s,
                                        const LaunchTiming& tm) {
  const size_t lds = std::max((size_t)a.sel.P * sizeof(uint32_t), (size_t)merge_lds_bytes(a.mg.S));
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&select_merge_kernel<E, D>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     kMaxPool * (int)sizeof(uint32_t));
  (void)attr;
  hipExtLaunchKernelGGL((select_merge_kernel<E, D>), dim3(a.layers + merge_groups), dim3(kSelectThreads), lds, s,
                        tm.start, tm.stop, 0, a);
  return hipGetLastError();
}

hipError_t launch_select_merge(Dt dt, int d, const SelectMergeArgs& a, int merge_groups, hipStream_t s,
                               const LaunchTiming& tm) {
  if (dt == Dt::BF16)
    return d == 64 ? launch_select_merge_t<BF16, 64>(a, merge_groups, s, tm)
                   : launch_select_merge_t<BF16, 128>(a, merge_groups, s, tm);
  return d == 64 ? launch_select_merge_t<F32, 64>(a, merge_groups, s, tm)
                 : launch_select_merge_t<F32, 128>(a, merge_groups, s, tm);
}

hipError_t launch_frame(Dt dt, int d, const RopeArgs& a, int layers, hipStream_t s, const LaunchTiming& tm) {
  if (a.nsel + a.rope_blocks == 0) return hipSuccess;
  if (dt == Dt::BF16) return d == 64 ? launch_frame_t<BF16, 64>(a, layers, s, tm) : launch_frame_t<BF16, 128>(a, layers, s, tm);
  return d == 64 ? launch_frame_t<F32, 64>(a, layers, s, tm) : launch_frame_t<F32, 128>(a, layers, s, tm);
}

hipError_t launch_attn(Dt dt, int d, const AttnArgs& a, int row_tiles, int splits, hipStream_t s,
                       const LaunchTiming& tm) {
  const dim3 grid(row_tiles, a.Hkv, splits);
  if (dt == Dt::BF16) {
    if (d == 64 && (long)row_tiles * a.Hkv * splits > device_cus())
      hipExtLaunchKernelGGL((attn_fwd_kernel<BF16, 64, 1, 8, 1, kAttnBN, 4>), grid, dim3(512), 0, s, tm.start, tm.stop, 0, a);
    else if (d == 64)
      hipExtLaunchKernelGGL((attn_fwd_kernel<BF16, 64, 1, 8, attn_prefetch(64)>), grid, dim3(512), 0, s, tm.start, tm.stop, 0, a);
    else
      hipExtLaunchKernelGGL((attn_fwd_kernel<BF16, 128, 1, 8, attn_prefetch(128)>), grid, dim3(512), 0, s, tm.start, tm.stop, 0, a);
  } else {
    if (d == 64) hipExtLaunchKernelGGL((attn_fwd_kernel<F32, 64, 1, 4>), grid, dim3(256), 0, s, tm.start, tm.stop, 0, a);
    else hipExtLaunchKernelGGL((attn_fwd_kernel<F32, 128, 1, 4>), grid, dim3(256), 0, s, tm.start, tm.stop, 0, a);
  }
  return hipGetLastError();
}

template <class E, int D, int KT, int NW, int NPF, bool FM = false>
static hipError_t launch_sm_t(const ScoreMergeArgs& a, hipStream_t s, const LaunchTiming& tm) {
  const int score_wgs = a.key_blocks * a.sc.Hkv * a.rsplits;
  const int grid = a.merge_wgs + score_wgs;
  if (grid == 0) return hipSuccess;
  size_t lds = a.merge_wgs ? (size_t)merge_lds_bytes(a.mg.S) : 0;
  if (score_wgs) lds = std::max(lds, (size_t)score_lds_bytes<E, D>());
  hipExtLaunchKernelGGL((score_merge_kernel<E, D, KT, NW, NPF, FM>), dim3(grid), dim3(64 * NW), lds, s, tm.start,
                        tm.stop, 0, a);
  return hipGetLastError();
}

hipError_t launch_score_merge(Dt dt, int d, const ScoreMergeArgs& a, int waves, hipStream_t s,
                              const LaunchTiming& tm) {
  if (dt == Dt::BF16) {
    if (waves == 8 && a.fused)
      return d == 64 ? launch_sm_t<BF16, 64, kKtBf16, 8, 1, true>(a, s, tm)
                     : launch_sm_t<BF16, 128, kKtBf16, 8, 1, true>(a, s, tm);
    if (waves == 8)
      return d == 64 ? launch_sm_t<BF16, 64, kKtBf16, 8, 1>(a, s, tm) : launch_sm_t<BF16, 128, kKtBf16, 8, 1>(a, s, tm);
    return d == 64 ? launch_sm_t<BF16, 64, kKtBf16, 4, score_prefetch(64)>(a, s, tm)
                   : launch_sm_t<BF16, 128, kKtBf16, 4, score_prefetch(128)>(a, s, tm);
  }
  return d == 64 ? launch_sm_t<F32, 64, kKtF32, 4, 1>(a, s, tm) : launch_sm_t<F32, 128, kKtF32, 4, 1>(a, s, tm);
}

// Waves of the text-phase attention kernel: 4 (bf16) or 2 (fp32, whose
// staged block would otherwise not leave room for two work-groups per CU).
constexpr int kDecodeWavesBf16 = 4;
constexpr int kDecodeWavesF32 = 2;
int decode_block_keys(Dt dt) { return 32 * (dt == Dt::BF16 ? kDecodeWavesBf16 : kDecodeWavesF32); }

// Register stages of the text-phase kernel's block prefetch: 2 for d = 128
// (about 6 % more bandwidth on the long caches), 1 for d = 64.
static constexpr int decode_prefetch(int d) { return d == 128 ? 2 : 1; }

hipError_t launch_decode(Dt dt, int d, const DecodeArgs& a, hipStream_t s, const LaunchTiming& tm) {
  const dim3 grid(a.L * a.Hkv, a.S);
  if (dt == Dt::BF16) {
    const dim3 block(64 * kDecodeWavesBf16);
    if (d == 64) hipExtLaunchKernelGGL((decode_attn_kernel<BF16, 64, kDecodeWavesBf16, decode_prefetch(64)>), grid, block, 0, s, tm.start, tm.stop, 0, a);
    else hipExtLaunchKernelGGL((decode_attn_kernel<BF16, 128, kDecodeWavesBf16, decode_prefetch(128)>), grid, block, 0, s, tm.start, tm.stop, 0, a);
  } else {
    const dim3 block(64 * kDecodeWavesF32);
    if (d == 64) hipExtLaunchKernelGGL((decode_attn_kernel<F32, 64, kDecodeWavesF32>), grid, block, 0, s, tm.start, tm.stop, 0, a);
    else hipExtLaunchKernelGGL((decode_attn_kernel<F32, 128, kDecodeWavesF32>), grid, block, 0, s, tm.start, tm.stop, 0, a);
  }
  return hipGetLastError();
}

hipError_t launch_decode_merge(Dt dt, int d, const DecodeMergeArgs& a, hipStream_t s,
                               const LaunchTiming& tm) {
  const dim3 grid((unsigned)((size_t)a.L * a.Hkv * a.R)), block(kDecodeMergeThreads);
  if (dt == Dt::BF16) {
    if (d == 64) hipExtLaunchKernelGGL((decode_merge_kernel<BF16, 64>), grid, block, 0, s, tm.start, tm.stop, 0, a);
    else hipExtLaunchKernelGGL((decode_merge_kernel<BF16, 128>), grid, block, 0, s, tm.start, tm.stop, 0, a);
  } else {
    if (d == 64) hipExtLaunchKernelGGL((decode_merge_kernel<F32, 64>), grid, block, 0, s, tm.start, tm.stop, 0, a);
    else hipExtLaunchKernelGGL((decode_merge_kernel<F32, 128>), grid, block, 0, s, tm.start, tm.stop, 0, a);
  }
  return hipGetLastError();
}

hipError_t launch_score_view(const ScoreViewArgs& a, int layers, hipStream_t s) {
  hipLaunchKernelGGL(score_view_kernel, dim3((unsigned)((a.P + 255) / 256), layers), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace statekv
