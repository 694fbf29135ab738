// HIP kernels of the StateKV frame step for AMD CDNA4 (gfx950, wave64).
//
// Paper note "Linear Scaling Video VLMs for Long Video Understanding"
// (papernotes.org, ECCV 2026), section 方法详解:
//   rope_append_kernel  关键设计 3: RoPE at the virtual position nT + i with the
//                       fixed scaled frequencies; 整体框架 / flowchart node E:
//                       the frame's K, V are appended to the detailed cache D.
//   attn_fwd_kernel     关键设计 1: the frame's queries attend over
//   combine_kernel      [Kbar_{n-1}; K_n] (bf16 MFMA, online softmax, split
//                       over keys, then merged).
//   attn_score_kernel   关键设计 2: score of candidate j = attention weight paid
//                       to j averaged over the frame's queries and query heads;
//                       recomputed with the final row max / sum of pass 1.
//   topb_select_kernel  关键设计 2: TopK({s_j}, B), ties kept toward the older
//                       token, emitted in ascending position.
//   gather_kernel       关键设计 2: build C_n from the kept candidates.
//
// Matrix-core tiles use v_mfma_f32_32x32x16_bf16 (bf16 storage) or
// v_mfma_f32_32x32x2_f32 (fp32 storage).  Accumulator layout of a 32x32 tile:
// lane l, register i holds row 8*(i/4) + 4*(l/32) + i%4 and column l%32.
// Operand layout: lane l supplies row (A) / column (B) l%32 and the reduction
// slice [KL*(l/32), KL*(l/32) + KL) of the instruction's KS-deep reduction.
#include "statekv_internal.h"

#include <math.h>

namespace statekv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
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

// ---------------------------------------------------------------------------
// RoPE at virtual positions + append to the detailed cache.
// One thread per (token, group of 4 rotation pairs), looping over all heads so
// that each cos/sin is evaluated once.  Rotation of the pair (x1, x2) =
// (x[k], x[k + d/2]) is computed in fp64 with one fused multiply-add per
// output (the other product is exact in fp64) and rounded once to storage.
// ---------------------------------------------------------------------------
template <class E, int D>
__global__ __launch_bounds__(256) void rope_append_kernel(RopeArgs a) {
  typedef typename E::T T;
  constexpr int HALF = D / 2;
  constexpr int PPT = 4;
  constexpr int TPT = HALF / PPT;
  const int gt = blockIdx.x * blockDim.x + threadIdx.x;
  const int tok = gt / TPT;
  if (tok >= a.T) return;
  const int k = (gt - tok * TPT) * PPT;
  const int pos = a.n * a.T + tok;

  double c[PPT], s[PPT];
#pragma unroll
  for (int j = 0; j < PPT; ++j) {
    double sn, cs;
    sincos((double)pos * a.inv_freq[k + j], &sn, &cs);
    c[j] = (double)(float)cs;
    s[j] = (double)(float)sn;
  }
  bool finite = true;

  auto rotate = [&](const T* src, T* dst0, T* dst1) {
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const float x1f = Store<E>::load(src + k + j);
      const float x2f = Store<E>::load(src + k + j + HALF);
      finite &= isfinite(x1f) && isfinite(x2f);
      const double x1 = x1f, x2 = x2f;
      const T y1 = Store<E>::from_f64(fma(x1, c[j], -(x2 * s[j])));
      const T y2 = Store<E>::from_f64(fma(x2, c[j], x1 * s[j]));
      dst0[k + j] = y1;
      dst0[k + j + HALF] = y2;
      if (dst1) {
        dst1[k + j] = y1;
        dst1[k + j + HALF] = y2;
      }
    }
  };

  const size_t rows_per_group = (size_t)a.G * a.T;
  for (int h = 0; h < a.Hq; ++h) {
    const int g = h / a.G;
    const int hl = h - g * a.G;
    const T* src = (const T*)a.q + ((size_t)tok * a.Hq + h) * D;
    T* dst = (T*)a.qrot + ((size_t)g * rows_per_group + (size_t)tok * a.G + hl) * D;
    rotate(src, dst, nullptr);
  }
  for (int g = 0; g < a.Hkv; ++g) {
    const T* src = (const T*)a.k + ((size_t)tok * a.Hkv + g) * D;
    T* pool = (T*)a.kpool + ((size_t)g * a.cap + a.k0 + tok) * D;
    T* det = (T*)a.dk + ((size_t)pos * a.Hkv + g) * D;
    rotate(src, pool, det);
    const T* vs = (const T*)a.v + ((size_t)tok * a.Hkv + g) * D;
    T* vpool = (T*)a.vpool + ((size_t)g * a.cap + a.k0 + tok) * D;
    T* vdet = (T*)a.dv + ((size_t)pos * a.Hkv + g) * D;
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const T v1 = vs[k + j], v2 = vs[k + j + HALF];
      finite &= isfinite(Store<E>::load(&v1)) && isfinite(Store<E>::load(&v2));
      vpool[k + j] = v1;
      vpool[k + j + HALF] = v2;
      vdet[k + j] = v1;
      vdet[k + j + HALF] = v2;
    }
  }
  if (k == 0) a.pool_pos[a.k0 + tok] = pos;
  if (!finite) atomicOr(a.nonfinite, 1);
}

// ---------------------------------------------------------------------------
// Attention pass 1.  Work-group = 4 waves; each wave owns QT tiles of 32 query
// rows of one KV group (rows r = token*G + head-in-group) and the work-group
// walks its key split in blocks of 64 keys staged in LDS.
//
// S^T = K Q^T puts one query per lane column, so row max / row sum reduce
// inside the lane plus one exchange with lane l^32.  O^T = V^T P^T reuses the
// S^T accumulators directly as the B operand: for bf16 the eight keys a lane
// supplies to one instruction are keys {16m + 8(t/4) + 4(l/32) + t%4}, so V^T
// is written to LDS with bits 2 and 3 of the key index swapped inside each
// group of 16, which makes those eight keys contiguous (one 16-byte read).
// ---------------------------------------------------------------------------
template <class E, int D, int QT>
__global__ __launch_bounds__(256, 1) void attn_fwd_kernel(AttnArgs a) {
  typedef typename E::T T;
  typedef Mma<E> M;
  constexpr int BN = kAttnBN;
  constexpr int EPV = 16 / (int)sizeof(T);  // elements per 16-byte vector
  constexpr int KSTR = D + EPV;              // LDS pitch of K rows
  constexpr int VSTR = BN + EPV;             // LDS pitch of V^T rows
  constexpr int NKS = D / M::KS;
  constexpr int NDT = D / 32;
  constexpr int BM = 4 * 32 * QT;
  __shared__ __attribute__((aligned(16))) T Ks[BN * KSTR];
  __shared__ __attribute__((aligned(16))) T Vt[D * VSTR];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hh = lane >> 5;
  const int g = blockIdx.y, split = blockIdx.z;
  const int row_wg = blockIdx.x * BM;
  const int row_last = min(a.R, row_wg + BM) - 1;
  const int tok_min = row_wg / a.G;
  const int need_end = a.k0 + row_last / a.G + 1;  // keys beyond are masked for every row
  const int kbeg = split * a.kps;
  const int kend = min(min(kbeg + a.kps, need_end), a.P);

  const T* qbase = (const T*)a.qrot + (size_t)g * a.R * D;
  const T* kbase = (const T*)a.kpool + (size_t)g * a.cap * D;
  const T* vbase = (const T*)a.vpool + (size_t)g * a.cap * D;

  typename M::Frag qf[QT][NKS];
  int qrow[QT], qtok[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int r = row_wg + (wave * QT + qt) * 32 + col;
    qrow[qt] = r;
    qtok[qt] = r < a.R ? r / a.G : -1;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      qf[qt][ks] = r < a.R ? M::ld(qbase + (size_t)r * D + ks * M::KS + hh * M::KL) : M::zero();
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

  for (int kb = kbeg; kb < kend; kb += BN) {
    __syncthreads();
    // Stage K rows [kb, kb + BN) (zero past the split end).
    {
      constexpr int CPR = D / EPV;
      for (int t = tid; t < BN * CPR; t += kAttnThreads) {
        const int rr = t / CPR, cc = t - rr * CPR;
        const int key = kb + rr;
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (key < kend) v = *reinterpret_cast<const u32x4_t*>(kbase + (size_t)key * D + cc * EPV);
        *reinterpret_cast<u32x4_t*>(&Ks[rr * KSTR + cc * EPV]) = v;
      }
    }
    // Stage V^T.
    if constexpr (sizeof(T) == 2) {
      constexpr int NKQ = BN / 4;  // key quads
      for (int t = tid; t < NKQ * (D / 8); t += kAttnThreads) {
        const int kq = t % NKQ, dc = t / NKQ;
        const int key0 = kb + kq * 4;
        u32x4_t r4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          r4[j] = u32x4_t{0u, 0u, 0u, 0u};
          if (key0 + j < kend)
            r4[j] = *reinterpret_cast<const u32x4_t*>(vbase + (size_t)(key0 + j) * D + dc * 8);
        }
        const int kk = kq * 4;
        const int slot = (kk & ~12) | ((kk & 4) << 1) | ((kk & 8) >> 1);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t w0 = r4[0][e >> 1], w1 = r4[1][e >> 1];
          const uint32_t w2 = r4[2][e >> 1], w3 = r4[3][e >> 1];
          uint32_t lo, hi;
          if (e & 1) {
            lo = (w0 >> 16) | (w1 & 0xffff0000u);
            hi = (w2 >> 16) | (w3 & 0xffff0000u);
          } else {
            lo = (w0 & 0xffffu) | (w1 << 16);
            hi = (w2 & 0xffffu) | (w3 << 16);
          }
          *reinterpret_cast<u32x2_t*>(&Vt[(dc * 8 + e) * VSTR + slot]) = u32x2_t{lo, hi};
        }
      }
    } else {
      for (int t = tid; t < BN * (D / 4); t += kAttnThreads) {
        const int rr = t % BN, cc = t / BN;
        const int key = kb + rr;
        f32x4_t v = {0.f, 0.f, 0.f, 0.f};
        if (key < kend) v = *reinterpret_cast<const f32x4_t*>(vbase + (size_t)key * D + cc * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) Vt[(cc * 4 + e) * VSTR + rr] = v[e];
      }
    }
    __syncthreads();

    // S^T tiles: 2 sub-tiles of 32 keys x QT tiles of 32 queries.
    f32x16_t sacc[2][QT];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) sacc[sub][qt] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const typename M::Frag af = M::ld(&Ks[(sub * 32 + col) * KSTR + ks * M::KS + hh * M::KL]);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) sacc[sub][qt] = M::mma(af, qf[qt][ks], sacc[sub][qt]);
      }
    }

    // Online softmax, one query per lane column.
    const bool need_mask = (kb + BN > a.k0 + tok_min) || (kb + BN > kend);
    float pv[QT][2][16];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float mx = -INFINITY;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float x = sacc[sub][qt][i];
          bool vis = true;
          if (need_mask) {
            const int key = kb + sub * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
            vis = key < kend && (key < a.k0 || key - a.k0 <= qtok[qt]);
          }
          mx = vis ? fmaxf(mx, x) : mx;
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      float m_new = m_run[qt];
      if (mx != -INFINITY) m_new = fmaxf(m_new, mx * a.c_hi);
      float rs = 0.f;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float x = sacc[sub][qt][i];
          float p = 0.f;
          if (m_new != -INFINITY) p = fast_exp2(fmaf(x, a.c_lo, fmaf(x, a.c_hi, -m_new)));
          if (need_mask) {
            const int key = kb + sub * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
            const bool vis = key < kend && (key < a.k0 || key - a.k0 <= qtok[qt]);
            p = vis ? p : 0.f;
          }
          pv[qt][sub][i] = p;
          rs += p;
        }
      }
      float alpha = 1.f;
      if (m_new != m_run[qt]) {
        const double al = exp2((double)m_run[qt] - (double)m_new);
        l_run[qt] *= al;
        alpha = (float)al;
      }
      l_run[qt] += (double)rs;
      m_run[qt] = m_new;
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[qt][dt] *= alpha;
      }
    }

    // O^T += V^T P^T.
    if constexpr (sizeof(T) == 2) {
      bf16x8_t pf[QT][2][2];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int mm = 0; mm < 2; ++mm)
#pragma unroll
            for (int t = 0; t < 8; ++t) pf[qt][sub][mm][t] = (__bf16)pv[qt][sub][8 * mm + t];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int mm = 0; mm < 2; ++mm) {
            const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(
                &Vt[(dt * 32 + col) * VSTR + sub * 32 + mm * 16 + hh * 8]);
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) o[qt][dt] = M::mma(af, pf[qt][sub][mm], o[qt][dt]);
          }
    } else {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            const int kin = sub * 32 + 8 * (t >> 2) + 4 * hh + (t & 3);
            const float af = Vt[(dt * 32 + col) * VSTR + kin];
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) o[qt][dt] = M::mma(af, pv[qt][sub][t], o[qt][dt]);
          }
    }
  }

  // Partial results of this key split.
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const double lt = l_run[qt] + __shfl_xor(l_run[qt], 32);
    const int r = qrow[qt];
    if (r < a.R) {
      const size_t ri = ((size_t)split * a.Hkv + g) * a.R + r;
      if (hh == 0) {
        a.mpart[ri] = m_run[qt];
        a.lpart[ri] = lt;
      }
      if (m_run[qt] != -INFINITY) {
        float* op = a.opart + ri * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            f32x4_t v = {o[qt][dt][4 * j], o[qt][dt][4 * j + 1], o[qt][dt][4 * j + 2],
                         o[qt][dt][4 * j + 3]};
            *reinterpret_cast<f32x4_t*>(op + dt * 32 + 8 * j + 4 * hh) = v;
          }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Merge of the key splits: O = sum_s 2^(m_s - m) O_s / l, l = sum_s 2^(m_s - m) l_s.
// Writes O in [T][Hq][d] and the row statistics used by the score pass.
// ---------------------------------------------------------------------------
template <class E, int D>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  typedef typename E::T T;
  constexpr int CPR = D / 4;
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t total = (size_t)a.Hkv * a.R * CPR;
  if (t >= total) return;
  const int c = (int)(t % CPR);
  const size_t gr = t / CPR;
  const int r = (int)(gr % a.R);
  const int g = (int)(gr / a.R);
  const size_t stride = (size_t)a.Hkv * a.R;
  const size_t base = (size_t)g * a.R + r;
  float m = -INFINITY;
  for (int s = 0; s < a.S; ++s) m = fmaxf(m, a.mpart[s * stride + base]);
  double l = 0.0;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < a.S; ++s) {
    const float ms = a.mpart[s * stride + base];
    if (ms == -INFINITY) continue;
    const double w = exp2((double)ms - (double)m);
    l += a.lpart[s * stride + base] * w;
    const f32x4_t os = *reinterpret_cast<const f32x4_t*>(a.opart + (s * stride + base) * D + c * 4);
    acc += (float)w * os;
  }
  const float inv = (float)(1.0 / l);
  const int tok = r / a.G;
  const int h = g * a.G + (r - tok * a.G);
  T* out = (T*)a.out + ((size_t)tok * a.Hq + h) * D + c * 4;
#pragma unroll
  for (int e = 0; e < 4; ++e) out[e] = Store<E>::from_f32(acc[e] * inv);
  if (c == 0) {
    a.row_m[base] = m;
    a.row_rinv[base] = inv;
  }
}

// ---------------------------------------------------------------------------
// Score pass.  Work-group = 4 waves; each wave keeps KT tiles of 32 keys in
// registers (the B operand of S = Q K^T) and all waves stream the same
// 32-row Q tiles through LDS.  With queries as rows, a lane holds 16 rows of
// one key column, so the column sum of P = 2^(s*c - m) / l is accumulated in
// the lane: fp32 over the tile's 16 rows, then fp64 across tiles; the two lane
// halves are added at the end.  The order of every sum is fixed, so the
// result is deterministic.
// ---------------------------------------------------------------------------
template <class E, int D, int KT>
__global__ __launch_bounds__(256, 1) void attn_score_kernel(ScoreArgs a) {
  typedef typename E::T T;
  typedef Mma<E> M;
  constexpr int RT = 32;
  constexpr int EPV = 16 / (int)sizeof(T);
  constexpr int QSTR = D + EPV;
  constexpr int NKS = D / M::KS;
  constexpr int BNK = 4 * 32 * KT;
  __shared__ __attribute__((aligned(16))) T Qs[RT * QSTR];
  __shared__ __attribute__((aligned(16))) float sm[RT];
  __shared__ __attribute__((aligned(16))) float sr[RT];
  __shared__ int stok[RT];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hh = lane >> 5;
  const int g = blockIdx.y, rsplit = blockIdx.z;
  const int key_wg = blockIdx.x * BNK;
  const int key_w = key_wg + wave * 32 * KT;

  const T* qbase = (const T*)a.qrot + (size_t)g * a.R * D;
  const T* kbase = (const T*)a.kpool + (size_t)g * a.cap * D;
  const float* mbase = a.row_m + (size_t)g * a.R;
  const float* rbase = a.row_rinv + (size_t)g * a.R;

  typename M::Frag kf[KT][NKS];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    const int key = key_w + kt * 32 + col;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      kf[kt][ks] = key < a.P ? M::ld(kbase + (size_t)key * D + ks * M::KS + hh * M::KL) : M::zero();
  }
  double cs[KT];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) cs[kt] = 0.0;

  const int r0 = rsplit * a.rps;
  const int r1 = min(a.R, r0 + a.rps);
  // Rows whose token precedes every frame key of this work-group see none of them.
  int rstart = r0;
  if (key_wg >= a.k0) rstart = max(r0, (key_wg - a.k0) * a.G);

  for (int rt = rstart; rt < r1; rt += RT) {
    __syncthreads();
    {
      constexpr int CPR = D / EPV;
      for (int t = tid; t < RT * CPR; t += kAttnThreads) {
        const int rr = t / CPR, cc = t - rr * CPR;
        const int r = rt + rr;
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (r < r1) v = *reinterpret_cast<const u32x4_t*>(qbase + (size_t)r * D + cc * EPV);
        *reinterpret_cast<u32x4_t*>(&Qs[rr * QSTR + cc * EPV]) = v;
      }
      if (tid < RT) {
        const int r = rt + tid;
        const bool ok = r < r1;
        sm[tid] = ok ? mbase[r] : 0.f;
        sr[tid] = ok ? rbase[r] : 0.f;
        stok[tid] = ok ? r / a.G : -1;
      }
    }
    __syncthreads();
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      const int key_t0 = key_w + kt * 32;
      if (key_t0 >= a.P) break;
      f32x16_t acc = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const typename M::Frag af = M::ld(&Qs[col * QSTR + ks * M::KS + hh * M::KL]);
        acc = M::mma(af, kf[kt][ks], acc);
      }
      const bool causal = key_t0 + 31 >= a.k0;
      const int ktok = key_t0 + col - a.k0;
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4_t mv = *reinterpret_cast<const f32x4_t*>(&sm[8 * j + 4 * hh]);
        const f32x4_t rv = *reinterpret_cast<const f32x4_t*>(&sr[8 * j + 4 * hh]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float x = acc[4 * j + q];
          float p = fast_exp2(fmaf(x, a.c_lo, fmaf(x, a.c_hi, -mv[q]))) * rv[q];
          if (causal && ktok > stok[8 * j + 4 * hh + q]) p = 0.f;
          sum += p;
        }
      }
      cs[kt] += (double)sum;
    }
  }
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    const double tot = cs[kt] + __shfl_xor(cs[kt], 32);
    const int key = key_w + kt * 32 + col;
    if (hh == 0 && key < a.P) a.colpart[((size_t)rsplit * a.Hkv + g) * a.cap + key] = tot;
  }
}

// ---------------------------------------------------------------------------
// Top-B selection in one work-group of 1024 threads.
// Scores s_j = (sum of the column partials in fixed order) / (Hq*T), rounded
// to fp32.  Non-negative fp32 values order like their bit patterns, so the
// B-th largest bit pattern tau is found by refining a value range [lo, hi]:
// histogram the candidates in [lo, hi] into up to 4096 equal-width buckets,
// pick the bucket holding the B-th largest, repeat until lo == hi.  Then keep
// every score > tau and, among scores == tau, the lowest pool indices (the
// older tokens).  The keep list is written in ascending pool index.
// ---------------------------------------------------------------------------
__device__ int block_excl_scan(int v, int* sh, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  if (wave == 0) {
    const int w = lane < kSelectThreads / 64 ? sh[lane] : 0;
    int xs = w;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(xs, o);
      if (lane >= o) xs += y;
    }
    if (lane < kSelectThreads / 64) sh[lane] = xs - w;
    if (lane == kSelectThreads / 64 - 1) sh[kSelectThreads / 64] = xs;
  }
  __syncthreads();
  const int res = sh[wave] + x - v;
  *total = sh[kSelectThreads / 64];
  __syncthreads();
  return res;
}

constexpr int kSelMaxPerThread = kMaxPool / kSelectThreads;  // 32

__global__ __launch_bounds__(1024, 1) void topb_select_kernel(SelectArgs a) {
  __shared__ uint32_t sbits[kMaxPool];
  __shared__ int hist[kSelectBins];
  __shared__ int scan_sh[kSelectThreads / 64 + 1];
  __shared__ uint32_t red_lo[kSelectThreads / 64], red_hi[kSelectThreads / 64];
  __shared__ int s_bucket, s_above;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int j = tid; j < a.P; j += kSelectThreads) {
    double s = 0.0;
    for (int q = 0; q < a.nparts; ++q) s += a.colpart[(size_t)q * a.cap + j];
    const float f = (float)(s / a.denom);
    a.scores[j] = f;
    sbits[j] = __float_as_uint(f);
  }
  __syncthreads();

  if (a.P <= a.B) {
    for (int j = tid; j < a.P; j += kSelectThreads) a.keep[j] = j;
    return;
  }

  const int C = (a.P + kSelectThreads - 1) / kSelectThreads;
  const int i0 = tid * C;
  const int cnt = max(0, min(C, a.P - i0));
  uint32_t b[kSelMaxPerThread];
  uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
  for (int j = 0; j < kSelMaxPerThread; ++j) {
    b[j] = 0u;
    if (j < cnt) {
      b[j] = sbits[i0 + j];
      lo = min(lo, b[j]);
      hi = max(hi, b[j]);
    }
  }
  // block min / max
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    lo = min(lo, (uint32_t)__shfl_xor((int)lo, o));
    hi = max(hi, (uint32_t)__shfl_xor((int)hi, o));
  }
  if (lane == 0) {
    red_lo[wave] = lo;
    red_hi[wave] = hi;
  }
  __syncthreads();
  lo = 0xffffffffu;
  hi = 0u;
  for (int w = 0; w < kSelectThreads / 64; ++w) {
    lo = min(lo, red_lo[w]);
    hi = max(hi, red_hi[w]);
  }

  int need = a.B;
  while (lo < hi) {
    const uint64_t range = (uint64_t)hi - lo + 1u;
    const int nb = (int)(range < (uint64_t)kSelectBins ? range : (uint64_t)kSelectBins);
    for (int x = tid; x < nb; x += kSelectThreads) hist[x] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kSelMaxPerThread; ++j) {
      if (j < cnt && b[j] >= lo && b[j] <= hi) {
        const int bk = (int)(((uint64_t)(b[j] - lo) * (uint64_t)nb) / range);
        atomicAdd(&hist[bk], 1);
      }
    }
    __syncthreads();
    // Walk buckets from the top: position q holds bucket nb-1-q.
    int c4[4];
    int s4 = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = tid * 4 + u;
      c4[u] = q < nb ? hist[nb - 1 - q] : 0;
      s4 += c4[u];
    }
    if (tid == 0) {
      s_bucket = 0;
      s_above = 0;
    }
    int total;
    int run = block_excl_scan(s4, scan_sh, &total);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = tid * 4 + u;
      if (q < nb && run < need && need <= run + c4[u]) {
        s_bucket = nb - 1 - q;
        s_above = run;
      }
      run += c4[u];
    }
    __syncthreads();
    const uint64_t x = (uint64_t)s_bucket;
    need -= s_above;
    const uint64_t off_lo = (x * range + nb - 1) / nb;
    const uint64_t off_hi = ((x + 1) * range + nb - 1) / nb - 1;
    hi = lo + (uint32_t)off_hi;
    lo = lo + (uint32_t)off_lo;
    __syncthreads();
  }
  const uint32_t tau = lo;

  int my_eq = 0;
#pragma unroll
  for (int j = 0; j < kSelMaxPerThread; ++j) my_eq += (j < cnt && b[j] == tau) ? 1 : 0;
  int eq_total;
  int eqr = block_excl_scan(my_eq, scan_sh, &eq_total);
  uint32_t keepmask = 0u;
  int my_keep = 0;
#pragma unroll
  for (int j = 0; j < kSelMaxPerThread; ++j) {
    if (j < cnt) {
      bool k = b[j] > tau;
      if (b[j] == tau) {
        k = eqr < need;
        ++eqr;
      }
      if (k) {
        keepmask |= 1u << j;
        ++my_keep;
      }
    }
  }
  int kept_total;
  int out = block_excl_scan(my_keep, scan_sh, &kept_total);
#pragma unroll
  for (int j = 0; j < kSelMaxPerThread; ++j)
    if ((keepmask >> j) & 1u) a.keep[out++] = i0 + j;
}

// ---------------------------------------------------------------------------
// Gather of the kept rows (K, V of every KV head, and positions) into the
// other state buffer, 16 bytes per thread, consecutive threads on
// consecutive bytes of a row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
  const int cpr = a.row_bytes / 16;
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t total = (size_t)a.Hkv * a.B * cpr;
  if (t >= total) return;
  const int c = (int)(t % cpr);
  const size_t gr = t / cpr;
  const int r = (int)(gr % a.B);
  const int g = (int)(gr / a.B);
  // keep[] holds pool indices; clamping only guards the copy against a
  // malformed list, it never changes a valid one.
  const int src = min(max(a.keep[r], 0), a.cap - 1);
  const size_t so = ((size_t)g * a.cap + src) * a.row_bytes + (size_t)c * 16;
  const size_t dof = ((size_t)g * a.cap + r) * a.row_bytes + (size_t)c * 16;
  *reinterpret_cast<u32x4_t*>((char*)a.knext + dof) =
      *reinterpret_cast<const u32x4_t*>((const char*)a.kcur + so);
  *reinterpret_cast<u32x4_t*>((char*)a.vnext + dof) =
      *reinterpret_cast<const u32x4_t*>((const char*)a.vcur + so);
  if (g == 0 && c == 0) a.pnext[r] = a.pcur[src];
}

}  // namespace

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
static constexpr int kQtBf16 = 2;  // query tiles per wave in pass 1 (bf16)
static constexpr int kQtF32 = 1;
static constexpr int kKtBf16 = 2;  // key tiles per wave in the score pass
static constexpr int kKtF32 = 1;

int attn_rows_per_wg(Dt dt) { return 4 * 32 * (dt == Dt::BF16 ? kQtBf16 : kQtF32); }
int score_keys_per_wg(Dt dt) { return 4 * 32 * (dt == Dt::BF16 ? kKtBf16 : kKtF32); }

hipError_t launch_rope(Dt dt, int d, const RopeArgs& a, hipStream_t s) {
  const int tpt = d / 8;
  const int blocks = (a.T * tpt + 255) / 256;
  if (dt == Dt::BF16) {
    if (d == 64) hipLaunchKernelGGL((rope_append_kernel<BF16, 64>), dim3(blocks), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((rope_append_kernel<BF16, 128>), dim3(blocks), dim3(256), 0, s, a);
  } else {
    if (d == 64) hipLaunchKernelGGL((rope_append_kernel<F32, 64>), dim3(blocks), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((rope_append_kernel<F32, 128>), dim3(blocks), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_attn(Dt dt, int d, const AttnArgs& a, int row_tiles, int splits, hipStream_t s) {
  const dim3 grid(row_tiles, a.Hkv, splits), block(kAttnThreads);
  if (dt == Dt::BF16) {
    if (d == 64) hipLaunchKernelGGL((attn_fwd_kernel<BF16, 64, kQtBf16>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((attn_fwd_kernel<BF16, 128, kQtBf16>), grid, block, 0, s, a);
  } else {
    if (d == 64) hipLaunchKernelGGL((attn_fwd_kernel<F32, 64, kQtF32>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((attn_fwd_kernel<F32, 128, kQtF32>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_combine(Dt dt, int d, const CombineArgs& a, hipStream_t s) {
  const size_t total = (size_t)a.Hkv * a.R * (d / 4);
  const dim3 grid((unsigned)((total + 255) / 256)), block(256);
  if (dt == Dt::BF16) {
    if (d == 64) hipLaunchKernelGGL((combine_kernel<BF16, 64>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((combine_kernel<BF16, 128>), grid, block, 0, s, a);
  } else {
    if (d == 64) hipLaunchKernelGGL((combine_kernel<F32, 64>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((combine_kernel<F32, 128>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_score(Dt dt, int d, const ScoreArgs& a, int key_blocks, int rsplits, hipStream_t s) {
  const dim3 grid(key_blocks, a.Hkv, rsplits), block(kAttnThreads);
  if (dt == Dt::BF16) {
    if (d == 64) hipLaunchKernelGGL((attn_score_kernel<BF16, 64, kKtBf16>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((attn_score_kernel<BF16, 128, kKtBf16>), grid, block, 0, s, a);
  } else {
    if (d == 64) hipLaunchKernelGGL((attn_score_kernel<F32, 64, kKtF32>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((attn_score_kernel<F32, 128, kKtF32>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(topb_select_kernel, dim3(1), dim3(kSelectThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs& a, hipStream_t s) {
  const size_t total = (size_t)a.Hkv * a.B * (a.row_bytes / 16);
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace statekv
