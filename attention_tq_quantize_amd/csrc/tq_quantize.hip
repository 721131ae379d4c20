// Quantize kernels for gfx950 (CDNA4, wave64) and their launcher.
//
// What is computed follows [NIK] = S. Nikolenko, "Eternal mathematics of
// TurboQuant" (blog.sergeynikolenko.ru): "Step 0: normalization", "Step 1:
// random rotation", "Step 2: optimal scalar quantization (Lloyd-Max)", "QJL:
// a one-bit method", "TurboQuant proper"; and [NAH] = "What exactly TurboQuant
// showed" (nahornyi.ai): prod keys need a dedicated attention kernel.
//
// Matrix-core building block: v_mfma_f32_16x16x32_bf16. For C = A*B + C with
// A 16x32, B 32x16 and lane l = r + 16*g (r in 0..15, g in 0..3):
//   A: lane l holds A[r][8g .. 8g+7];  B: lane l holds B[8g .. 8g+7][r];
//   C: lane l holds C[4g .. 4g+3][r].
// fp32 accuracy for the rotations comes from splitting each matrix (and fp32
// inputs) into bf16 hi + lo parts (16 significant bits) and accumulating in
// fp32; bf16 inputs are exact as they are.
//
// The rotation's rows are permuted so that lane group g owns output
// coordinates [g D/4, (g+1) D/4) of its vector: 16-row output block q gives
// the lane coordinates g D/4 + 4q + i, i = 0..3. The kernel walks the blocks
// from the last to the first and shifts each plane bit into a 32-bit word, so
// the vector-layout words are complete in registers with no lane exchange.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <type_traits>

#include "tq_device.h"

namespace tq {
namespace {

// ===========================================================================
// Quantize: [NIK] Step 0 (norm, unit vector), Step 1 (y = Pi u), Step 2
// (nearest centroid, b-bit index); prod adds the residual, |r| and sign(S r).
// A wave handles 16 T vectors per step as T 16-vector MFMA tiles; workgroups
// are persistent over the steps of one group and keep the group's rotation
// fragments in LDS (d <= 128).
// ===========================================================================
constexpr int kQWaves = 8;
constexpr int kQThreads = 64 * kQWaves;

struct QuantParams {
  const void* x;
  int64_t x_row_bytes;    // bytes from one input vector to the next
  int64_t n_per_group;
  int n_groups;
  int64_t group_base;     // first group of this launch (vectors index from it)
  uint8_t* codes;
  uint8_t* signs;
  float* norms;
  float* rnorms;
  float* rot_dbg;
  float* proj_dbg;
  float thr[15];
  float cen[16];
  unsigned thr_key[8];  // magnitude-search keys of the upper thresholds (P >= 3)
  const uint16_t* pi_frag[kMaxGroupsPerLaunch];
  const uint16_t* sp_frag[kMaxGroupsPerLaunch];
};

// One part of an outlier-channel split ([NIK] "Experiments", KV cache) over up
// to kQSplitGroups groups, for d = 128 heads: the part's d_p x d_p rotation is
// laid into a 128 x 128 matrix M with M[o][c] = Pi_p[o][j] where channel c is
// coordinate j of the part (o < d_p), zero elsewhere; likewise S' = S Pi^T on
// the first d_p rotated coordinates. Lane groups g < d_p / 32 then hold the
// part's rotated coordinates and write its records.
//
// Fused two-part split (both parts of a 128-channel head whose dimensions are
// multiples of 32 and add up to 128, same variant): one pass over the row. The
// two rotations form one block-diagonal 128 x 128 matrix (part 0 on output
// coordinates [0, d_0), part 1 on [d_0, 128)), so each lane group's 32 output
// coordinates belong to one part; the part with fewer planes runs the same
// P-plane search on its thresholds with +inf above them (its top planes come out
// 0 and are not stored).
constexpr int kQSplitGroups = 16;
constexpr uint8_t kNoChannel = 0xFF;
struct QuantSplitParams {
  int dp;                                // d_p (fused: d_0), a multiple of 32 up to 128
  unsigned chan_mask[kQSplitGroups][4];  // bit b of word w: channel 32 w + b is in the part (fused: part 0)
  uint8_t inv[kQSplitGroups][128];       // channel -> (part << 7) | its coordinate in the part; kNoChannel: none
  const float* pi[kQSplitGroups];        // Pi_p, fp32 [d_p][d_p]
  const float* sp[kQSplitGroups];        // prod: S' = S_p Pi_p^T, fp32 [d_p][d_p]
  // fused only: part 1's dimension and tables, both parts' plane counts, their
  // thresholds and centroids laid on the P-plane search, part 1's records
  int dp1, planes0, planes1;
  unsigned chan_mask1[kQSplitGroups][4];
  const float* pi1[kQSplitGroups];
  const float* sp1[kQSplitGroups];
  float thr_e[2][15], cen_e[2][16];
  uint8_t* codes1;
  uint8_t* signs1;
  float* norms1;
  float* rnorms1;
  float* rot1;
  float* proj1;
};
struct QuantNoSplit {};

// 16-vector tiles per wave step (the block layout needs two: a block is 32 vectors)
__host__ __device__ constexpr int q_tiles(int D, bool prod, bool xf32, bool blk) {
  return (D == 256 && (prod || xf32) && !blk) ? 1 : 2;
}
// waves per SIMD: 4 where the registers allow (bf16 mse up to d = 128, not the
// fused two-part split, which keeps both parts' norms), else 2
__host__ __device__ constexpr int q_waves_per_simd(int D, bool prod, bool xf32, bool fused = false) {
  return (D <= 128 && !prod && !xf32 && !fused) ? 4 : 2;
}
__host__ __device__ constexpr bool q_prefetch(int D, bool xf32) { return !(D == 256 && xf32); }

// Raw input of one 16-vector tile for lane (r, g): vector r, coordinates
// [g D/4, (g+1) D/4) as 16-byte loads (bf16: D/32 loads, fp32: D/16 loads).
template <int D, bool XF32>
struct XTile {
  static constexpr int NR = XF32 ? D / 16 : D / 32;
  u32x4 raw[NR];
};

// Loads of one tile: base = the tile's first row (wave-uniform), rel = this
// lane's row relative to it, clamped by the caller to an existing row (rows
// past the end are read again and never stored).
template <int D, bool XF32>
__device__ __forceinline__ void load_tile(const uint8_t* base, unsigned rel, int64_t row_bytes, int g,
                                          XTile<D, XF32>& t) {
  constexpr int ROW = D * (XF32 ? 4 : 2);
  const u32x4* src = (const u32x4*)(base + (int64_t)rel * row_bytes + g * (ROW / 4));
#pragma unroll
  for (int i = 0; i < XTile<D, XF32>::NR; ++i) t.raw[i] = src[i];
}

// This lane's part of |x|^2 for bf16 input, exactly in fp64 (the fallback of
// tile_operands for tiny or huge vectors).
template <int D>
__device__ __forceinline__ double sumsq_bf16_exact(const XTile<D, false>& t) {
  double acc = 0.0;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    const u32x4 v = t.raw[ks];
    const unsigned w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = bf16_val(w[e] & 0xFFFFu), b = bf16_val(w[e] >> 16);
      acc = fma((double)a, (double)a, acc);
      acc = fma((double)b, (double)b, acc);
    }
  }
  return acc;
}

// Channels outside a split part read as zero: lane group g's bit b of cm is
// channel 32 g + b (d = 128; bf16 words hold two channels, fp32 words one).
template <int D, bool XF32>
__device__ __forceinline__ void mask_tile(XTile<D, XF32>& t, unsigned cm) {
  auto bit = [&](int pos) -> unsigned { return (unsigned)(((int)(cm << (31 - pos))) >> 31); };
#pragma unroll
  for (int i = 0; i < XTile<D, XF32>::NR; ++i) {
    unsigned w[4] = {t.raw[i].x, t.raw[i].y, t.raw[i].z, t.raw[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (XF32)
        w[j] &= bit(4 * i + j);
      else
        w[j] &= (bit(8 * i + 2 * j) & 0xFFFFu) | (bit(8 * i + 2 * j + 1) << 16);
    }
    t.raw[i] = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// This lane's part of |x|^2 over the channels of cm (split parts): as
// tile_operands (v_dot2 pairs for bf16, fp64 fma for fp32) on the masked words,
// and the exact fp64 sum for bf16 (the fallback for tiny or huge vectors).
template <int D, bool XF32>
__device__ __forceinline__ double sumsq_masked(const XTile<D, XF32>& t, unsigned cm, bool exact) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  auto bit = [&](int pos) -> unsigned { return (unsigned)(((int)(cm << (31 - pos))) >> 31); };
  double acc = 0.0;
#pragma unroll
  for (int i = 0; i < XTile<D, XF32>::NR; ++i) {
    unsigned w[4] = {t.raw[i].x, t.raw[i].y, t.raw[i].z, t.raw[i].w};
    if constexpr (XF32) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float f = __uint_as_float(w[j] & bit(4 * i + j));
        acc = fma((double)f, (double)f, acc);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] &= (bit(8 * i + 2 * j) & 0xFFFFu) | (bit(8 * i + 2 * j + 1) << 16);
      if (exact) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float a = bf16_val(w[j] & 0xFFFFu), b = bf16_val(w[j] >> 16);
          acc = fma((double)a, (double)a, acc);
          acc = fma((double)b, (double)b, acc);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const bf2 h0 = __builtin_bit_cast(bf2, w[2 * e]), h1 = __builtin_bit_cast(bf2, w[2 * e + 1]);
          acc += (double)__builtin_amdgcn_fdot2_f32_bf16(h1, h1, __builtin_amdgcn_fdot2_f32_bf16(h0, h0, 0.0f, false),
                                                         false);
        }
      }
    }
  }
  return acc;
}

// |x|^2 of bf16 input from the fast part sums is used when it lies in
// [2^-90, 2^100]: there no square is subnormal or infinite in fp32 enough to
// matter (the ones below 2^-126 add at most 2^-119 in all), and the result
// keeps the bound of tile_operands.
constexpr double kSumsqFastLo = 0x1p-90, kSumsqFastHi = 0x1p100;

// MFMA operands of a tile (K index 8g + e of k-step ks <-> coordinate
// g D/4 + 8 ks + e) and this lane's part of |x|^2. fp32 input: fp64 fma per
// coordinate. bf16 input: the two squares of a dword are exact in fp32 and
// v_dot2 adds them to its accumulator with one rounding; a chain of two covers
// four coordinates and the partials are added in fp64, so the relative error
// is at most about 2^-23 (the norm's about 2^-24, within one fp32 ulp).
template <int D, bool XF32>
__device__ __forceinline__ double tile_operands(const XTile<D, XF32>& t, u32x4* xh, u32x4* xl) {
  constexpr int NK = D / 32;
  double acc = 0.0;
#pragma unroll
  for (int ks = 0; ks < NK; ++ks) {
    if constexpr (!XF32) {
      typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
      const u32x4 v = t.raw[ks];
      xh[ks] = v;
      const unsigned w[4] = {v.x, v.y, v.z, v.w};
      float q[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const bf2 h0 = __builtin_bit_cast(bf2, w[2 * e]), h1 = __builtin_bit_cast(bf2, w[2 * e + 1]);
        q[e] = __builtin_amdgcn_fdot2_f32_bf16(h1, h1, __builtin_amdgcn_fdot2_f32_bf16(h0, h0, 0.0f, false), false);
      }
      acc += (double)q[0];
      acc += (double)q[1];
    } else {
      const u32x4 u0 = t.raw[2 * ks], u1 = t.raw[2 * ks + 1];
      const float f[8] = {__uint_as_float(u0.x), __uint_as_float(u0.y), __uint_as_float(u0.z), __uint_as_float(u0.w),
                          __uint_as_float(u1.x), __uint_as_float(u1.y), __uint_as_float(u1.z), __uint_as_float(u1.w)};
      unsigned h[8], l[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        h[e] = bf16_part(f[e], false);
        l[e] = bf16_part(f[e], true);
        acc = fma((double)f[e], (double)f[e], acc);
      }
      xh[ks] = u32x4{pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7])};
      xl[ks] = u32x4{pack2(l[0], l[1]), pack2(l[2], l[3]), pack2(l[4], l[5]), pack2(l[6], l[7])};
    }
  }
  return acc;
}

// v in a VGPR the compiler cannot see through: keeps "c ? t[a] : t[b]" a register
// select instead of a load from a computed kernel-argument address
__device__ __forceinline__ float opaque_vgpr(float v) {
  asm volatile("" : "+v"(v));
  return v;
}

// ---- nearest-centroid search on wave masks ----
// The compare results stay in SGPR lane masks and feed the threshold selects
// and the bit shift-in directly: per plane one v_cmp, one v_addc (w = 2w + bit)
// and the selects of the binary search. Plain ALU instructions only. Their
// inputs must come from ordinary VALU code, never straight from an MFMA result:
// the compiler does not add the MFMA-to-VALU wait states for asm operands.
typedef unsigned long long lanemask;
__device__ __forceinline__ lanemask cmp_gt(float a, float b) {  // lanes with a > b
  lanemask m;
  asm("v_cmp_gt_f32_e64 %0, %1, %2" : "=s"(m) : "v"(a), "v"(b));
  return m;
}
__device__ __forceinline__ float sel(lanemask m, float a, float b) {  // lane-wise m ? b : a
  float r;
  asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "s"(m));
  return r;
}
__device__ __forceinline__ unsigned shift_in(unsigned w, lanemask m) {  // 2 w + (lane bit of m)
  unsigned r;
  lanemask c;
  asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(r), "=s"(c) : "v"(w), "s"(m));
  return r;
}

// Plane masks of the nearest-centroid indices of N values y: binary search
// over the fp32 thresholds (t_i = largest fp32 not above the midpoint of
// centroids i and i+1, so y > t_i <=> strictly nearer centroid i+1; ties go
// low). The N searches advance level by level so independent compares fill
// each other's SGPR write-to-read gaps.
template <int P>
struct PlaneMasks {
  lanemask m[P > 0 ? P : 1];
};
template <int P, int N>
__device__ __forceinline__ void nearest_planes(const float* y, const float* T, PlaneMasks<P>* r) {
  if constexpr (P >= 1) {
    constexpr int top = (1 << (P - 1)) - 1;  // threshold index of the top plane
#pragma unroll
    for (int i = 0; i < N; ++i) r[i].m[P - 1] = cmp_gt(y[i], T[top]);
  }
  if constexpr (P == 2) {
#pragma unroll
    for (int i = 0; i < N; ++i) r[i].m[0] = cmp_gt(y[i], sel(r[i].m[1], T[0], T[2]));
  } else if constexpr (P == 3) {
    float a[N], b[N];
#pragma unroll
    for (int i = 0; i < N; ++i) r[i].m[1] = cmp_gt(y[i], sel(r[i].m[2], T[1], T[5]));
#pragma unroll
    for (int i = 0; i < N; ++i) {
      a[i] = sel(r[i].m[2], T[0], T[4]);
      b[i] = sel(r[i].m[2], T[2], T[6]);
    }
#pragma unroll
    for (int i = 0; i < N; ++i) r[i].m[0] = cmp_gt(y[i], sel(r[i].m[1], a[i], b[i]));
  } else if constexpr (P == 4) {
#pragma unroll
    for (int i = 0; i < N; ++i) r[i].m[2] = cmp_gt(y[i], sel(r[i].m[3], T[3], T[11]));
    float a[N], b[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
      a[i] = sel(r[i].m[3], T[1], T[9]);
      b[i] = sel(r[i].m[3], T[5], T[13]);
    }
#pragma unroll
    for (int i = 0; i < N; ++i) r[i].m[1] = cmp_gt(y[i], sel(r[i].m[2], a[i], b[i]));
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const float c0 = sel(r[i].m[3], T[0], T[8]), c1 = sel(r[i].m[3], T[2], T[10]);
      const float c2 = sel(r[i].m[3], T[4], T[12]), c3 = sel(r[i].m[3], T[6], T[14]);
      a[i] = sel(r[i].m[1], c0, c1);
      b[i] = sel(r[i].m[1], c2, c3);
    }
#pragma unroll
    for (int i = 0; i < N; ++i) r[i].m[0] = cmp_gt(y[i], sel(r[i].m[2], a[i], b[i]));
  }
}
// Nearest centroid of a symmetric codebook (C[K-1-i] = -C[i], so the middle
// threshold is 0) from the magnitude, for P >= 3. With neg = [y <= 0] and
// key = 2 bits(|y|) + neg (bits(y) + bits(y) + carry: the add drops the sign
// bit), one unsigned compare key > TK[j] against
//   TK[j] = 2 bits(t_u) + (1 if the midpoint behind t_u is not a float32)
// for the upper thresholds t_u (u = K/2 + j) decides both sides: y > 0 is past
// the midpoint when |y| > t_u; y <= 0 is below its mirror when |y| >= the
// midpoint (the tie goes to the lower index, which on the negative side is the
// one farther from zero), i.e. |y| > t_u unless the midpoint is a float32 and
// equals t_u. J = the number of upper midpoints passed is found by a binary
// search over TK; then idx = neg ? K/2 - 1 - J : K/2 + J, so the top plane is
// !neg and the lower planes are J's bits flipped when neg (mask XORs on the
// scalar unit). Per value one float compare, the key add, P - 1 integer
// compares and 2^(P-2) - 1 selects, against P compares and 2^(P-1) - 1 selects
// of the plain search.
__device__ __forceinline__ lanemask cmp_le0(float a) {  // lanes with a <= 0
  lanemask m;
  asm("v_cmp_ge_f32_e64 %0, 0, %1" : "=s"(m) : "v"(a));
  return m;
}
__device__ __forceinline__ lanemask cmp_gt_u(unsigned a, unsigned b) {  // lanes with a > b (unsigned)
  lanemask m;
  asm("v_cmp_gt_u32_e64 %0, %1, %2" : "=s"(m) : "v"(a), "v"(b));
  return m;
}
__device__ __forceinline__ unsigned sel_u(lanemask m, unsigned a, unsigned b) {  // lane-wise m ? b : a
  unsigned r;
  asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "s"(m));
  return r;
}
template <int P, int N>
__device__ __forceinline__ void nearest_planes_sym(const float* y, const unsigned* TK, PlaneMasks<P>* r) {
  static_assert(P == 3 || P == 4, "magnitude search: 3 or 4 planes");
  lanemask neg[N];
  unsigned key[N];
#pragma unroll
  for (int i = 0; i < N; ++i) neg[i] = cmp_le0(y[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) key[i] = shift_in(__float_as_uint(y[i]), neg[i]);
  if constexpr (P == 3) {
#pragma unroll
    for (int i = 0; i < N; ++i) r[i].m[1] = cmp_gt_u(key[i], TK[1]);
#pragma unroll
    for (int i = 0; i < N; ++i) r[i].m[0] = cmp_gt_u(key[i], sel_u(r[i].m[1], TK[0], TK[2]));
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) r[i].m[2] = cmp_gt_u(key[i], TK[3]);
#pragma unroll
    for (int i = 0; i < N; ++i) r[i].m[1] = cmp_gt_u(key[i], sel_u(r[i].m[2], TK[1], TK[5]));
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const unsigned a = sel_u(r[i].m[2], TK[0], TK[4]), b = sel_u(r[i].m[2], TK[2], TK[6]);
      r[i].m[0] = cmp_gt_u(key[i], sel_u(r[i].m[1], a, b));
    }
  }
#pragma unroll
  for (int i = 0; i < N; ++i) {
#pragma unroll
    for (int p = 0; p < P - 1; ++p) r[i].m[p] ^= neg[i];
    r[i].m[P - 1] = ~neg[i];
  }
}

// centroid C[idx] of the index whose plane masks are r
template <int P>
__device__ __forceinline__ float plane_centroid(const PlaneMasks<P>& r, const float* C) {
  if constexpr (P == 0) {
    return 0.0f;
  } else if constexpr (P == 1) {
    return sel(r.m[0], C[0], C[1]);
  } else if constexpr (P == 2) {
    return sel(r.m[1], sel(r.m[0], C[0], C[1]), sel(r.m[0], C[2], C[3]));
  } else if constexpr (P == 3) {
    const float lo = sel(r.m[1], sel(r.m[0], C[0], C[1]), sel(r.m[0], C[2], C[3]));
    const float hi = sel(r.m[1], sel(r.m[0], C[4], C[5]), sel(r.m[0], C[6], C[7]));
    return sel(r.m[2], lo, hi);
  } else {
    static_assert(P <= 3, "prod keeps at most 3 planes");
    return 0.0f;
  }
}

// OR of a value over the four lanes of a quad (DPP quad permutations)
__device__ __forceinline__ unsigned quad_or(unsigned w) {
  w |= (unsigned)__builtin_amdgcn_mov_dpp((int)w, 0xB1, 0xF, 0xF, true);  // lanes ^ 1
  w |= (unsigned)__builtin_amdgcn_mov_dpp((int)w, 0x4E, 0xF, 0xF, true);  // lanes ^ 2
  return w;
}

// SPLIT: 0 whole vectors, 1 one part of a channel split, 2 the fused two-part split
// The work of one workgroup: by is its row of the grid (the group, and at
// d = 256 mse the half of the rotation's output rows), blockIdx.x / gridDim.x
// its place among the persistent workgroups of that row.
template <int D, int P, bool PROD, bool XF32, bool BLK, bool DBG, int SPLIT = 0>
__device__ __forceinline__ void quantize_body(const QuantParams& prm,
                                              const std::conditional_t<SPLIT != 0, QuantSplitParams, QuantNoSplit>& sx,
                                              const int by) {
  static_assert(!SPLIT || D == 128, "split parts: d = 128 heads");
  constexpr bool FUSED = SPLIT == 2;
  constexpr int NQ = D / 16, NK = D / 32, Q4 = D / 4;
  constexpr int T = q_tiles(D, PROD, XF32, BLK);
  // split mse at four waves per SIMD has no registers for the next step's tiles
  // d = 256 prod (bf16 input): the 16-row fragment blocks of Pi and S' stream
  // through a double-buffered LDS slot shared by the workgroup's waves, one
  // block per barrier, in the order the rotation (blocks 15..0 of Pi) and the
  // projection (blocks 15..0 of S') use them
  constexpr bool STREAM = D == 256 && PROD && !XF32 && SPLIT == 0;
  constexpr bool PREF = q_prefetch(D, XF32) && !(SPLIT == 1 && !PROD && !XF32) && !STREAM;
  constexpr int WPL = Q4 >= 32 ? Q4 / 32 : 1;  // 32-bit words per plane per lane (vector layout)
  constexpr int PP = P > 0 ? P : 1;
  // d = 256 mse: two workgroup sets, each for half of the output rows (16-row
  // blocks [QH h, QH h + QH) and 32-bit words h of the vector layout), whose
  // fragments (128 KB) fit in LDS; every vector is read by both
  constexpr bool HALF = D == 256 && !PROD && SPLIT == 0;
  constexpr int QH = HALF ? NQ / 2 : NQ;  // 16-row blocks per workgroup
  constexpr bool LDS_FRAG = D <= 128 || HALF;
  constexpr int FRAG_VECS = 2 * QH * NK * 64;  // u32x4 of this workgroup's fragments per matrix (hi + lo)
  extern __shared__ u32x4 smem_frag[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int grp = HALF ? (by >> 1) : by;
  const int hq = HALF ? (by & 1) : 0;  // this workgroup's half of the output rows
  const int q0 = hq * QH;
  // record width (d_p of a split part), whether this lane group holds record
  // coordinates, and its channel mask. Fused split: this lane's part (by lane
  // group for vectors, by coordinate group r16 / 4 for blocks), its plane count,
  // its lane group within the part and its record arrays.
  int RD = D;
  bool gv = true;
  unsigned cm = ~0u, cm0 = 0u, cm1 = 0u;
  int part = 0, RP = P, gl = g, G0 = 4;
  uint8_t* r_codes = prm.codes;
  uint8_t* r_signs = prm.signs;
  float* r_rot = prm.rot_dbg;
  float* r_proj = prm.proj_dbg;
  if constexpr (SPLIT) {
    RD = sx.dp;
    gv = g < sx.dp / Q4;
    cm = sx.chan_mask[grp][g];
  }
  if constexpr (FUSED) {
    G0 = sx.dp / Q4;
    cm0 = sx.chan_mask[grp][g];
    cm1 = sx.chan_mask1[grp][g];
    cm = cm0 | cm1;
    gv = true;
    part = (BLK ? (r16 >> 2) : g) >= G0 ? 1 : 0;
    RD = part ? sx.dp1 : sx.dp;
    RP = part ? sx.planes1 : sx.planes0;
    gl = g - (part ? G0 : 0);
    r_codes = part ? sx.codes1 : prm.codes;
    r_signs = part ? sx.signs1 : prm.signs;
    r_rot = part ? sx.rot1 : prm.rot_dbg;
    r_proj = part ? sx.proj1 : prm.proj_dbg;
  }
  const int64_t n = prm.n_per_group;
  const int64_t gbase = (prm.group_base + grp) * n;
  const int64_t steps = (n + 16 * T - 1) / (16 * T);
  constexpr int NTHR = P > 0 ? (1 << P) - 1 : 1;
  constexpr int NCEN = 1 << (P > 0 ? P : 0);
  float thr[NTHR], cen[NCEN];
  // the magnitude search (whole vectors, 3 or 4 planes)
  constexpr bool SYM = SPLIT == 0 && P >= 3;
  constexpr int NTK = SYM ? (1 << (P - 1)) - 1 : 1;
  unsigned tkey[NTK];
#pragma unroll
  for (int i = 0; i < NTK; ++i) tkey[i] = SYM ? __float_as_uint(opaque_vgpr(__uint_as_float(prm.thr_key[i]))) : 0u;
#pragma unroll
  for (int i = 0; i < NTHR; ++i) {
    if constexpr (FUSED)
      thr[i] = opaque_vgpr(part ? sx.thr_e[1][i] : sx.thr_e[0][i]);
    else
      thr[i] = opaque_vgpr(prm.thr[i]);
  }
#pragma unroll
  for (int i = 0; i < NCEN; ++i) {
    if constexpr (FUSED)
      cen[i] = PROD ? opaque_vgpr(part ? sx.cen_e[1][i] : sx.cen_e[0][i]) : 0.0f;
    else
      cen[i] = PROD ? opaque_vgpr(prm.cen[i]) : 0.0f;
  }
  const int64_t stride = (int64_t)gridDim.x * kQWaves;
  int64_t step = (int64_t)blockIdx.x * kQWaves + wave;

  XTile<D, XF32> cur[T], nxt[T];
  const int64_t xrow = prm.x_row_bytes;
  auto load_step = [&](int64_t s, XTile<D, XF32>(&dst)[T]) {
    const int64_t vb = s * 16 * T;  // first vector of step s
    const uint8_t* base = (const uint8_t*)prm.x + (gbase + vb) * xrow;
    const int64_t left = n - 1 - vb;  // last existing row, relative
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int rel = 16 * t + r16;
      load_tile<D, XF32>(base, (unsigned)(rel < left ? rel : left), xrow, g, dst[t]);
    }
  };
  // streamed kernels run every step of the workgroup in every wave (the barriers
  // need all of them): a wave past the end works on a clamped step and stores nothing
  if constexpr (STREAM) {
    load_step(step < steps ? step : steps - 1, cur);
  } else {
    if (step < steps) load_step(step, cur);  // in flight while the fragments are staged
  }

  const u32x4* fpi;
  const u32x4* fsp;
  if constexpr (SPLIT) {
    // fragments of the part's matrices laid over the head's channels, built here
    // from the fp32 tables (hi = bf16(v), lo = bf16(v - hi), as on the host)
    // (fused: block-diagonal, part 0 on output rows [0, d_0), part 1 below)
    constexpr int HALF = FRAG_VECS / 2;
    const int dp0 = sx.dp;
    const uint8_t* inv = sx.inv[grp];
    for (int w = 0; w < (PROD ? 2 : 1); ++w) {
      for (int i = threadIdx.x; i < HALF; i += kQThreads) {
        const int l = i & 63, ks = (i >> 6) % NK, q = (i >> 6) / NK;
        const int m = l & 15;
        const int row = Q4 * (m >> 2) + 4 * q + (m & 3);
        const int col = Q4 * (l >> 4) + 8 * ks;
        const int prow = (FUSED && row >= dp0) ? 1 : 0;  // the part of this output row
        const int r = row - (prow ? dp0 : 0), dpr = prow ? sx.dp1 : dp0;
        const float* M = w ? (prow ? sx.sp1[grp] : sx.sp[grp]) : (prow ? sx.pi1[grp] : sx.pi[grp]);
        unsigned h[8], lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          // Pi_p: input channel col + e is coordinate inv of its part; S': the
          // residual's coordinate is col + e itself (minus d_0 in part 1)
          int j;
          if (w) {
            const int c = col + e, pc = (FUSED && c >= dp0) ? 1 : 0;
            j = pc == prow ? c - (pc ? dp0 : 0) : -1;
          } else {
            const unsigned iv = inv[col + e];
            j = (iv != kNoChannel && (int)(iv >> 7) == prow) ? (int)(iv & 0x7Fu) : -1;
          }
          const float v = (r < dpr && j >= 0 && j < dpr) ? M[r * dpr + j] : 0.0f;
          h[e] = bf16_part(v, false);
          lo[e] = bf16_part(v, true);
        }
        smem_frag[w * FRAG_VECS + i] = u32x4{pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7])};
        smem_frag[w * FRAG_VECS + HALF + i] =
            u32x4{pack2(lo[0], lo[1]), pack2(lo[2], lo[3]), pack2(lo[4], lo[5]), pack2(lo[6], lo[7])};
      }
    }
    __syncthreads();
    fpi = smem_frag;
    fsp = smem_frag + FRAG_VECS;
  } else if constexpr (LDS_FRAG) {
    const u32x4* src = (const u32x4*)prm.pi_frag[grp];
    if constexpr (HALF) {
      // blocks [q0, q0 + QH) of the hi and of the lo fragments ([hilo][q][ks][lane] in memory)
      for (int i = threadIdx.x; i < FRAG_VECS; i += kQThreads) {
        const int hl = i / (QH * NK * 64), rest = i % (QH * NK * 64);
        smem_frag[i] = src[(hl * NQ + q0) * NK * 64 + rest];
      }
    } else {
      for (int i = threadIdx.x; i < FRAG_VECS; i += kQThreads) smem_frag[i] = src[i];
    }
    if constexpr (PROD) {
      const u32x4* s2 = (const u32x4*)prm.sp_frag[grp];
      for (int i = threadIdx.x; i < FRAG_VECS; i += kQThreads) smem_frag[FRAG_VECS + i] = s2[i];
    }
    __syncthreads();
    fpi = smem_frag;
    fsp = smem_frag + FRAG_VECS;
  } else {
    fpi = (const u32x4*)prm.pi_frag[grp];
    fsp = (const u32x4*)prm.sp_frag[grp];
  }
  // streamed blocks: sequence index b = 0..15 is block 15 - b of Pi, 16..31
  // block 31 - b of S'; thread t holds element t of the block's hi and lo parts
  // (NK * 64 = the workgroup's thread count) from its load to its LDS store.
  // Loads run two blocks ahead (register slots b & 1), so a block's wait at the
  // end of the one before it leaves the next block's loads in flight.
  constexpr int SBLK = 2 * NK * 64;  // u32x4 per streamed block
  u32x4 pend_h[2] = {}, pend_l[2] = {};
  auto stream_issue = [&](int bseq, int slot) {
    if constexpr (STREAM) {
      static_assert(NK * 64 == kQThreads, "one element of each part per thread");
      // buffer loads: one lane offset register for every block, the block's
      // offset in an SGPR (per-block 64-bit addresses would be hoisted and spilled)
      const buf_t r = make_buf(bseq < NQ ? fpi : fsp, FRAG_VECS * 16u);
      const int qb = bseq < NQ ? NQ - 1 - bseq : 2 * NQ - 1 - bseq;
      const uint4 h = ld128(r, 16u * threadIdx.x, (unsigned)((0 * NQ + qb) * NK * 64 * 16));
      const uint4 l = ld128(r, 16u * threadIdx.x, (unsigned)((1 * NQ + qb) * NK * 64 * 16));
      pend_h[slot] = u32x4{h.x, h.y, h.z, h.w};
      pend_l[slot] = u32x4{l.x, l.y, l.z, l.w};
    }
  };
  auto stream_store = [&](int buf) {  // block in register slot buf into LDS buffer buf
    if constexpr (STREAM) {
      smem_frag[buf * SBLK + threadIdx.x] = pend_h[buf];
      smem_frag[buf * SBLK + NK * 64 + threadIdx.x] = pend_l[buf];
      __syncthreads();
    }
  };
  if constexpr (STREAM) {
    stream_issue(0, 0);
    stream_issue(1, 1);
    stream_store(0);
  }
  // fragment (hilo, q, ks) of this lane
  auto frag = [&](const u32x4* base, int hl, int q, int ks) -> u32x4 {
    if constexpr (STREAM) {
      // the buffer of q's block: rotation block q is sequence 15 - q, projection
      // block q is 31 - q; both have the parity of q + 1
      return smem_frag[((q + 1) & 1) * SBLK + (hl * NK + ks) * 64 + lane];
    } else if constexpr (LDS_FRAG) {
      return base[((hl * QH + (q - q0)) * NK + ks) * 64 + lane];
    } else {
      // global: wave-uniform base and fragment offset in SGPRs, one lane offset
      // register for every fragment
      const buf_t r = make_buf(base, FRAG_VECS * 16u);
      const uint4 v = ld128(r, 16u * lane, (unsigned)(((hl * NQ + q) * NK + ks) * 64 * 16));
      return u32x4{v.x, v.y, v.z, v.w};
    }
  };

  for (; STREAM ? step - wave < steps : step < steps; step += stride) {
    // d = 256: the fragments stay in global memory. Opaque copies of their
    // addresses keep the compiler from hoisting every step-invariant fragment
    // load out of this loop (about a thousand registers, all spilled).
    const u32x4* fpi_l = fpi;
    const u32x4* fsp_l = fsp;
    if constexpr (!LDS_FRAG) asm volatile("" : "+s"(fpi_l), "+s"(fsp_l));
    const int64_t nstep = step + stride;
    if constexpr (PREF) {
      if (nstep < steps) load_step(nstep, nxt);
    }
    u32x4 xh[T][NK], xl[T][XF32 ? NK : 1];
    double ss[T];
    double ssp[FUSED ? T : 1][2];  // fused: |x|^2 over each part's channels
    // split: an opaque copy of the channel mask per step keeps the compiler from
    // holding every expanded word mask across the loop (register spills)
    unsigned cm_l = cm, cm0_l = cm0, cm1_l = cm1;
    if constexpr (SPLIT) asm volatile("" : "+v"(cm_l));
    if constexpr (FUSED) asm volatile("" : "+v"(cm0_l), "+v"(cm1_l));
#pragma unroll
    for (int t = 0; t < T; ++t) {
      if constexpr (SPLIT) mask_tile<D, XF32>(cur[t], cm_l);
      ss[t] = tile_operands<D, XF32>(cur[t], xh[t], xl[t]);
      if constexpr (FUSED) {
        // both parts' sums; the lanes' own part's goes on in ss
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          double a = sumsq_masked<D, XF32>(cur[t], k ? cm1_l : cm0_l, false);
          a += __shfl_xor(a, 16);
          a += __shfl_xor(a, 32);
          if constexpr (!XF32) {
            if (!(a >= kSumsqFastLo && a <= kSumsqFastHi)) {  // the vector's four lanes together
              a = sumsq_masked<D, XF32>(cur[t], k ? cm1_l : cm0_l, true);
              a += __shfl_xor(a, 16);
              a += __shfl_xor(a, 32);
            }
          }
          ssp[t][k] = a;
        }
        ss[t] = part ? ssp[t][1] : ssp[t][0];
        continue;
      }
      ss[t] += __shfl_xor(ss[t], 16);
      ss[t] += __shfl_xor(ss[t], 32);
      if constexpr (!XF32) {
        // the four lanes of a vector share ss, so they take this branch together
        if (!(ss[t] >= kSumsqFastLo && ss[t] <= kSumsqFastHi)) {
          ss[t] = sumsq_bf16_exact<D>(cur[t]);
          ss[t] += __shfl_xor(ss[t], 16);
          ss[t] += __shfl_xor(ss[t], 32);
        }
      }
    }
    const int64_t v0 = step * 16 * T;  // first vector of this step

    if constexpr (!BLK) {
      // ---- VECTOR layout: lane (vector r16 of tile t, g) holds coords Q4 g + 4q + i ----
      double nu[T];
      bool valid[T];
      float inv[T];
#pragma unroll
      for (int t = 0; t < T; ++t) {
        nu[t] = sqrt(ss[t]);
        valid[t] = nu[t] > 0.0;
        inv[t] = valid[t] ? (float)(1.0 / nu[t]) : 0.0f;
      }
      constexpr int WPLR = HALF ? 1 : WPL;  // plane words held per lane (a half holds word hq)
      unsigned pw[T][PP][WPLR];
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int p = 0; p < PP; ++p)
#pragma unroll
          for (int w = 0; w < WPLR; ++w) pw[t][p][w] = 0u;
      // prod: residual operands for the second contraction, K order = this lane's coords
      u32x4 eh[PROD ? T : 1][PROD ? NK : 1], el[PROD ? T : 1][PROD ? NK : 1];
      float eodd[PROD ? T : 1][4];
      float esq[T];
#pragma unroll
      for (int t = 0; t < T; ++t) esq[t] = 0.0f;

#pragma unroll
      for (int qq = QH - 1; qq >= 0; --qq) {
        const int q = q0 + qq;
        if constexpr (STREAM) stream_issue(NQ + 1 - q, (NQ - 1 - q) & 1);  // two blocks ahead
        f32x4 C[T];
#pragma unroll
        for (int t = 0; t < T; ++t) C[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) {
          const u32x4 ph = frag(fpi_l, 0, q, ks), pl = frag(fpi_l, 1, q, ks);
#pragma unroll
          for (int t = 0; t < T; ++t) {
            C[t] = mfma(ph, xh[t][ks], C[t]);
            C[t] = mfma(pl, xh[t][ks], C[t]);
            if constexpr (XF32) C[t] = mfma(ph, xl[t][ks], C[t]);
          }
        }
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const float y[4] = {C[t].x * inv[t], C[t].y * inv[t], C[t].z * inv[t], C[t].w * inv[t]};
          if constexpr (DBG) {
            const int64_t v = v0 + 16 * t + r16;
            if (r_rot && v < n && gv)
              *(float4*)(r_rot + (gbase + v) * RD + Q4 * gl + 4 * q) = float4{y[0], y[1], y[2], y[3]};
          }
          float e4[4];
          PlaneMasks<P> pm[4];
          if constexpr (P > 0) {
            if constexpr (SYM)
              nearest_planes_sym<P, 4>(y, tkey, pm);
            else
              nearest_planes<P, 4>(y, thr, pm);
#pragma unroll
            for (int p = 0; p < P; ++p)
#pragma unroll
              for (int i = 3; i >= 0; --i) {
                unsigned& w = pw[t][p][HALF ? 0 : (4 * qq + i) / 32];
                w = shift_in(w, pm[i].m[p]);
              }
          }
#pragma unroll
          for (int i = 3; i >= 0; --i) {
            if constexpr (PROD) {
              const float ej = (valid[t] && gv) ? y[i] - plane_centroid<P>(pm[i], cen) : 0.0f;
              e4[i] = ej;
              esq[t] = fmaf(ej, ej, esq[t]);
            }
          }
          if constexpr (PROD) {
            if (q & 1) {
#pragma unroll
              for (int i = 0; i < 4; ++i) eodd[t][i] = e4[i];
            } else {
              const float ev[8] = {e4[0], e4[1], e4[2], e4[3], eodd[t][0], eodd[t][1], eodd[t][2], eodd[t][3]};
              unsigned h[8], l[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                h[e] = bf16_part(ev[e], false);
                l[e] = bf16_part(ev[e], true);
              }
              eh[t][q / 2] = u32x4{pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7])};
              el[t][q / 2] = u32x4{pack2(l[0], l[1]), pack2(l[2], l[3]), pack2(l[4], l[5]), pack2(l[6], l[7])};
            }
          }
        }
        // keep the scheduler from hoisting every block's fragment reads (register spills)
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (STREAM) stream_store((NQ - q) & 1);
      }
      // bases of this step (wave-uniform unless fused), 32-bit lane offsets
      float* nbase = prm.norms + gbase + v0;
      uint8_t* cbase = r_codes + (gbase + v0) * (RP * RD / 8);
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const int rel = 16 * t + r16;
        if (v0 + rel < n) {
          if (g == 0 && hq == 0) nbase[rel] = (float)nu[t];
          if constexpr (FUSED) {
            if (g == G0) sx.norms1[gbase + v0 + rel] = (float)nu[t];
          }
          if (P > 0 && gv) {
            // 32-bit lane offset; opaque for a runtime record width, which keeps
            // the compiler from holding 64-bit addresses across the loop
            unsigned lo = (unsigned)rel * (unsigned)(RP * RD / 8) + (unsigned)(gl * (Q4 / 8));
            if constexpr (SPLIT) asm volatile("" : "+v"(lo));
#pragma unroll
            for (int p = 0; p < P; ++p) {
              if (FUSED && p >= RP) continue;  // the part's top planes (all zero) are not stored
              if constexpr (Q4 >= 32) {
#pragma unroll
                for (int w = 0; w < WPLR; ++w)
                  *(unsigned*)(cbase + lo + p * RD / 8 + 4 * (HALF ? hq : w)) = valid[t] ? pw[t][p][w] : 0u;
              } else {
                *(unsigned short*)(cbase + lo + p * RD / 8) = (unsigned short)(valid[t] ? pw[t][p][0] : 0u);
              }
            }
          }
        }
      }
      if constexpr (PROD) {
        // ---- second contraction: p = S' e, signs and |r| ----
        unsigned sw[T][WPL];
#pragma unroll
        for (int t = 0; t < T; ++t) {
          if constexpr (FUSED) {  // each part's residual over its own lane groups
            float e0 = part ? 0.0f : esq[t], e1 = part ? esq[t] : 0.0f;
            e0 += __shfl_xor(e0, 16);
            e1 += __shfl_xor(e1, 16);
            e0 += __shfl_xor(e0, 32);
            e1 += __shfl_xor(e1, 32);
            esq[t] = part ? e1 : e0;
          } else {
            esq[t] += __shfl_xor(esq[t], 16);
            esq[t] += __shfl_xor(esq[t], 32);
          }
#pragma unroll
          for (int w = 0; w < WPL; ++w) sw[t][w] = 0u;
        }
#pragma unroll
        for (int q = NQ - 1; q >= 0; --q) {
          if constexpr (STREAM) stream_issue((2 * NQ + 1 - q) % (2 * NQ), (2 * NQ - 1 - q) & 1);  // two blocks ahead (wraps to the next step's first two)
          f32x4 acc[T];
#pragma unroll
          for (int t = 0; t < T; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < NK; ++ks) {
            const u32x4 sh = frag(fsp_l, 0, q, ks), sl = frag(fsp_l, 1, q, ks);
#pragma unroll
            for (int t = 0; t < T; ++t) {
              acc[t] = mfma(sh, eh[t][ks], acc[t]);
              acc[t] = mfma(sl, eh[t][ks], acc[t]);
              acc[t] = mfma(sh, el[t][ks], acc[t]);
            }
          }
#pragma unroll
          for (int t = 0; t < T; ++t) {
            const float pv[4] = {acc[t].x, acc[t].y, acc[t].z, acc[t].w};
#pragma unroll
            for (int i = 3; i >= 0; --i) {
              // plain C here: the inline-asm helpers must not read MFMA results directly
              // (the compiler does not insert the MFMA-to-VALU wait states for asm operands)
              unsigned& w = sw[t][(4 * q + i) / 32];
              w = (w << 1) | (pv[i] >= 0.0f ? 1u : 0u);
            }
            if constexpr (DBG) {
              const int64_t v = v0 + 16 * t + r16;
              if (r_proj && v < n && gv)
                *(float4*)(r_proj + (gbase + v) * RD + Q4 * gl + 4 * q) = float4{pv[0], pv[1], pv[2], pv[3]};
            }
          }
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (STREAM) stream_store((2 * NQ - q) & 1);
        }
        float* rbase = prm.rnorms + gbase + v0;
        uint8_t* sbase = r_signs + (gbase + v0) * (RD / 8);
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const int rel = 16 * t + r16;
          if (v0 + rel < n) {
            if (g == 0) rbase[rel] = valid[t] ? sqrtf(esq[t]) : 0.0f;
            if constexpr (FUSED) {
              if (g == G0) sx.rnorms1[gbase + v0 + rel] = valid[t] ? sqrtf(esq[t]) : 0.0f;
            }
            uint8_t* dst = sbase + (unsigned)rel * (RD / 8);
            if constexpr (Q4 >= 32) {
              if (gv) {
                unsigned lo = (unsigned)rel * (unsigned)(RD / 8) + (unsigned)(gl * (Q4 / 8));
                if constexpr (SPLIT) asm volatile("" : "+v"(lo));
#pragma unroll
                for (int w = 0; w < WPL; ++w) *(unsigned*)(sbase + lo + 4 * w) = valid[t] ? sw[t][w] : 0u;
              }
            } else {
              *(unsigned short*)(dst + g * (Q4 / 8)) = (unsigned short)(valid[t] ? sw[t][0] : 0u);
            }
          }
        }
      }
    } else {
      // ---- BLOCK32 layout (mse): C = x Pi^T; lane (coord lane r16, g) holds vectors
      // 16t + 4g + k of out coord o = Q4 (r16/4) + 4q + (r16%4): word w = (D/16)(r16/4) + q,
      // bit 16t + 4 (r16%4) + k ----
      float inv[T][4];
      unsigned vmask[T];  // bit k: vector 16t + 4g + k has a nonzero norm
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const int64_t v = v0 + 16 * t + r16;
        vmask[t] = 0u;
        if constexpr (FUSED) {
          // vector 16t + r16's norm over each part; this lane takes its part's
          const double nu0 = sqrt(ssp[t][0]), nu1 = sqrt(ssp[t][1]);
          const float i0 = nu0 > 0.0 ? (float)(1.0 / nu0) : 0.0f, i1 = nu1 > 0.0 ? (float)(1.0 / nu1) : 0.0f;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float a = __shfl(i0, 4 * g + k), b = __shfl(i1, 4 * g + k);
            inv[t][k] = part ? b : a;
            vmask[t] |= (inv[t][k] > 0.0f ? 1u : 0u) << k;
          }
          if (g == 0 && v < n) prm.norms[gbase + v] = (float)nu0;
          if (g == 1 && v < n) sx.norms1[gbase + v] = (float)nu1;
          continue;
        }
        const double nu_own = sqrt(ss[t]);  // vector 16t + r16
        const float inv_own = nu_own > 0.0 ? (float)(1.0 / nu_own) : 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          inv[t][k] = __shfl(inv_own, 4 * g + k);
          vmask[t] |= (inv[t][k] > 0.0f ? 1u : 0u) << k;
        }
        if (g == 0 && hq == 0 && v < n) prm.norms[gbase + v] = (float)nu_own;
      }
      const int slot = r16 & 3;
      // this step's 32-vector block; 32-bit lane offset of word (p = 0, q = 0)
      // (split: a block of the part's records is 4 P d_p bytes, and lanes whose
      // coordinates lie beyond d_p store nothing)
      // (fused: each part's blocks in its own array, 4 P_p d_p bytes each; this
      // lane's coordinate group counted within its part)
      const buf_t blk = make_buf(prm.codes + ((gbase + v0) / 32) * (int64_t)(4 * P * RD), (unsigned)(4 * P * RD));
      buf_t blk0 = blk, blk1 = blk;
      if constexpr (FUSED) {
        const int b0 = 4 * sx.planes0 * sx.dp, b1 = 4 * sx.planes1 * sx.dp1;
        blk0 = make_buf(prm.codes + ((gbase + v0) / 32) * (int64_t)b0, (unsigned)b0);
        blk1 = make_buf(sx.codes1 + ((gbase + v0) / 32) * (int64_t)b1, (unsigned)b1);
      }
      const unsigned blk_lane = (unsigned)((g * (RD / 4) + (D / 16) * ((r16 >> 2) - (part ? G0 : 0))) * 4);
      const bool bv = FUSED || !SPLIT || (r16 >> 2) < RD / Q4;
#pragma unroll
      for (int qq = 0; qq < QH; ++qq) {
        const int q = q0 + qq;
        f32x4 C[T];
#pragma unroll
        for (int t = 0; t < T; ++t) C[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) {
          const u32x4 ph = frag(fpi_l, 0, q, ks), pl = frag(fpi_l, 1, q, ks);
#pragma unroll
          for (int t = 0; t < T; ++t) {
            C[t] = mfma(xh[t][ks], ph, C[t]);
            C[t] = mfma(xh[t][ks], pl, C[t]);
            if constexpr (XF32) C[t] = mfma(xl[t][ks], ph, C[t]);
          }
        }
        unsigned nib[T][PP];
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const float cv[4] = {C[t].x, C[t].y, C[t].z, C[t].w};
#pragma unroll
          for (int p = 0; p < PP; ++p) nib[t][p] = 0u;
          const float y[4] = {cv[0] * inv[t][0], cv[1] * inv[t][1], cv[2] * inv[t][2], cv[3] * inv[t][3]};
          PlaneMasks<P> pm[4];
          if constexpr (SYM)
            nearest_planes_sym<P, 4>(y, tkey, pm);
          else
            nearest_planes<P, 4>(y, thr, pm);
#pragma unroll
          for (int p = 0; p < P; ++p)
#pragma unroll
            for (int k = 3; k >= 0; --k) nib[t][p] = shift_in(nib[t][p], pm[k].m[p]);
          if constexpr (DBG) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const int64_t v = v0 + 16 * t + 4 * g + k;
              const int o = Q4 * ((r16 >> 2) - (part ? G0 : 0)) + 4 * q + slot;  // within the lane's part
              if (r_rot && v < n && bv) r_rot[(gbase + v) * RD + o] = y[k];
            }
          }
        }
        // word ((p, g), (D/16)(r16/4) + q) of the block
#pragma unroll
        for (int p = 0; p < P; ++p) {
          unsigned word = (nib[0][p] & vmask[0]) << (4 * slot);
          if constexpr (T > 1) word |= (nib[1][p] & vmask[1]) << (16 + 4 * slot);
          word = quad_or(word);
          if constexpr (FUSED) {
            if (slot == 0 && p < RP) {
              if (part)
                st32(blk1, word, blk_lane + (unsigned)(p * 4 * RD), (unsigned)(4 * q));
              else
                st32(blk0, word, blk_lane + (unsigned)(p * 4 * RD), (unsigned)(4 * q));
            }
          } else {
            if (slot == 0 && bv) st32(blk, word, blk_lane + (unsigned)(p * 4 * RD), (unsigned)(4 * q));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (PREF) {
      if (nstep < steps) {
#pragma unroll
        for (int t = 0; t < T; ++t) cur[t] = nxt[t];
      }
    } else if constexpr (STREAM) {
      load_step(nstep < steps ? nstep : steps - 1, cur);
    } else {
      if (nstep < steps) load_step(nstep, cur);
    }
  }
}

template <int D, int P, bool PROD, bool XF32, bool BLK, bool DBG, int SPLIT = 0>
__global__ __launch_bounds__(kQThreads, q_waves_per_simd(D, PROD, XF32, SPLIT == 2)) void quantize_kernel(
    QuantParams prm, std::conditional_t<SPLIT != 0, QuantSplitParams, QuantNoSplit> sx) {
  quantize_body<D, P, PROD, XF32, BLK, DBG, SPLIT>(prm, sx, (int)blockIdx.y);
}

// A layer's keys (VECTOR layout) and values (BLOCK32 layout) in one launch,
// both TurboQuant_mse with the same (d, bits): grid rows [0, rows_k) run the
// keys, the rest the values, so the two tensors share one launch's set-up and
// tail instead of paying each twice.
template <int D, int P, bool XF32>
__global__ __launch_bounds__(kQThreads, q_waves_per_simd(D, false, XF32)) void quantize_kv_kernel(
    QuantParams pk, QuantParams pv, int rows_k) {
  if ((int)blockIdx.y < rows_k)
    quantize_body<D, P, false, XF32, false, false>(pk, QuantNoSplit{}, (int)blockIdx.y);
  else
    quantize_body<D, P, false, XF32, true, false>(pv, QuantNoSplit{}, (int)blockIdx.y - rows_k);
}

// Keys of the magnitude search (nearest_planes_sym) for a codebook of P >= 3
// planes: TK[j] = 2 bits(t_u) + (1 unless the midpoint of centroids u and u+1
// is a float32), u = K/2 + j. The codebook is symmetric by construction
// (centroids rounded from a symmetric fp64 solution, middle midpoint 0); a
// codebook that is not is refused.
bool threshold_keys(const Codebook& cb, unsigned* tk) {
  const int K = 1 << cb.planes;
  if (cb.planes < 3) return true;
  for (int i = 0; i < K; ++i)
    if (cb.centroids[K - 1 - i] != -cb.centroids[i]) return false;
  if (cb.thresholds[K / 2 - 1] != 0.0f) return false;
  for (int j = 0; j < K / 2 - 1; ++j) {
    const int u = K / 2 + j;
    const double mid = ((double)cb.centroids[u] + (double)cb.centroids[u + 1]) / 2.0;  // exact in fp64
    unsigned b;
    std::memcpy(&b, &cb.thresholds[u], 4);
    tk[j] = 2u * b + ((double)(float)mid == mid ? 0u : 1u);
  }
  return true;
}

}  // namespace

tq_status launch_quantize(const QuantizeLaunch& a, hipStream_t stream) {
  const tq_quantizer* q0 = a.qz[0];
  const bool prod = q0->variant == TQ_PROD;
  const bool blk = a.layout == TQ_LAYOUT_BLOCK32;
  const bool xf32 = a.x_dtype == TQ_F32;
  const int P = q0->planes;
  for (int g0 = 0; g0 < a.n_groups; g0 += kMaxGroupsPerLaunch) {
    const int ng = a.n_groups - g0 < kMaxGroupsPerLaunch ? a.n_groups - g0 : kMaxGroupsPerLaunch;
    QuantParams prm{};
    prm.x = a.x;
    prm.x_row_bytes = a.x_stride * (xf32 ? 4 : 2);
    prm.n_per_group = a.n_per_group;
    prm.n_groups = ng;
    prm.group_base = g0;
    prm.codes = a.codes;
    prm.signs = a.signs;
    prm.norms = a.norms;
    prm.rnorms = a.rnorms;
    prm.rot_dbg = a.rot_dbg;
    prm.proj_dbg = a.proj_dbg;
    const int K = 1 << P;
    for (int i = 0; i + 1 < K; ++i) prm.thr[i] = q0->cb.thresholds[i];
    for (int i = 0; i < K; ++i) prm.cen[i] = q0->cb.centroids[i];
    if (!threshold_keys(q0->cb, prm.thr_key)) return set_error(TQ_ERR_UNSUPPORTED, "quantize: codebook is not symmetric");
    for (int g = 0; g < ng; ++g) {
      prm.pi_frag[g] = a.qz[g0 + g]->pi_frag;
      prm.sp_frag[g] = a.qz[g0 + g]->sp_frag;
    }
    const bool dbg = a.rot_dbg != nullptr || a.proj_dbg != nullptr;
    tq_status st = dispatch_dim(q0->d, [&](auto DC) -> tq_status {
      constexpr int D = decltype(DC)::value;
      // fragments in LDS: d <= 128 both matrices; d = 256 mse half of Pi per workgroup
      const bool half = D == 256 && !prod;
      // (d = 256 prod with bf16 input: two streamed 16-row blocks, hi and lo, 32 KB)
      const bool streamed = D == 256 && prod && !xf32;
      const size_t lds = D <= 128 ? (size_t)2 * D * D * 2 * (prod ? 2 : 1)
                         : half   ? (size_t)D * D * 2
                         : streamed ? (size_t)2 * 2 * (D / 32) * 64 * 16
                                  : 0;
      return dispatch_planes(P, [&](auto PC) -> tq_status {
        constexpr int PP = decltype(PC)::value;
        return dispatch_bool(prod, [&](auto PR) -> tq_status {
          constexpr bool PROD = decltype(PR)::value;
          return dispatch_bool(xf32, [&](auto XF) -> tq_status {
            constexpr bool XF32 = decltype(XF)::value;
            return dispatch_bool(blk, [&](auto BL) -> tq_status {
              constexpr bool BLK = decltype(BL)::value;
              if constexpr ((BLK && (PROD || PP == 0)) || (!PROD && PP == 0) || (PROD && PP > 3)) {
                return set_error(TQ_ERR_UNSUPPORTED, "quantize: unsupported (variant, planes, layout)");
              } else {
                return dispatch_bool(dbg, [&](auto DB) -> tq_status {
                  constexpr bool DBG = decltype(DB)::value;
                  auto kern = quantize_kernel<D, PP, PROD, XF32, BLK, DBG>;
                  if (lds > 64 * 1024) {
                    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
                    if (e != hipSuccess) return check_hip(e, "quantize: set LDS size");
                  }
                  // persistent workgroups: as many as fit on the device at once, split over the groups
                  constexpr int T = q_tiles(D, PROD, XF32, BLK);
                  const int by_waves = q_waves_per_simd(D, PROD, XF32) * 4 / kQWaves;
                  const int by_lds = lds ? (int)((160 * 1024) / lds) : by_waves;
                  const int per_cu = by_waves < by_lds ? by_waves : by_lds;
                  const int64_t steps = (a.n_per_group + 16 * T - 1) / (16 * T);
                  const int sets = half ? 2 * ng : ng;  // workgroup sets: (group, half of the rows) at d = 256 mse
                  int64_t want = ((int64_t)(per_cu > 0 ? per_cu : 1) * device_cus() + sets - 1) / sets;
                  const int64_t cap = (steps + kQWaves - 1) / kQWaves;
                  if (want > cap) want = cap;
                  if (want < 1) want = 1;
                  hipLaunchKernelGGL(kern, dim3((unsigned)want, (unsigned)sets), dim3(kQThreads), lds, stream, prm,
                                     QuantNoSplit{});
                  return launch_check("quantize: launch");
                });
              }
            });
          });
        });
      });
    });
    if (st != TQ_OK) return st;
  }
  return TQ_OK;
}

bool quantize_kv_fusable(const QuantizeLaunch& k, const QuantizeLaunch& v) {
  const tq_quantizer* a = k.qz[0];
  const tq_quantizer* b = v.qz[0];
  return a->variant == TQ_MSE && b->variant == TQ_MSE && a->d == b->d && a->bits == b->bits && a->d <= 256 &&
         k.layout == TQ_LAYOUT_VECTOR && v.layout == TQ_LAYOUT_BLOCK32 && k.x_dtype == v.x_dtype &&
         k.x_stride == a->d && v.x_stride == b->d && k.n_groups == v.n_groups && k.n_groups <= kMaxGroupsPerLaunch &&
         !k.rot_dbg && !v.rot_dbg && !k.proj_dbg && !v.proj_dbg;
}

tq_status launch_quantize_kv(const QuantizeLaunch& k, const QuantizeLaunch& v, hipStream_t stream) {
  const bool xf32 = k.x_dtype == TQ_F32;
  const int P = k.qz[0]->planes;
  const int ng = k.n_groups;
  auto params = [&](const QuantizeLaunch& a) {
    QuantParams prm{};
    prm.x = a.x;
    prm.x_row_bytes = a.x_stride * (xf32 ? 4 : 2);
    prm.n_per_group = a.n_per_group;
    prm.n_groups = ng;
    prm.group_base = 0;
    prm.codes = a.codes;
    prm.norms = a.norms;
    const tq_quantizer* q0 = a.qz[0];
    for (int i = 0; i + 1 < (1 << P); ++i) prm.thr[i] = q0->cb.thresholds[i];
    for (int i = 0; i < (1 << P); ++i) prm.cen[i] = q0->cb.centroids[i];
    for (int g = 0; g < ng; ++g) prm.pi_frag[g] = a.qz[g]->pi_frag;
    return prm;
  };
  QuantParams pk = params(k), pv = params(v);
  if (!threshold_keys(k.qz[0]->cb, pk.thr_key) || !threshold_keys(v.qz[0]->cb, pv.thr_key))
    return set_error(TQ_ERR_UNSUPPORTED, "quantize_kv: codebook is not symmetric");
  return dispatch_dim(k.qz[0]->d, [&](auto DC) -> tq_status {
    constexpr int D = decltype(DC)::value;
    constexpr bool HALF = D == 256;  // d = 256 mse: two workgroup rows per group, each half of Pi in LDS
    const size_t lds = D <= 128 ? (size_t)2 * D * D * 2 : (size_t)D * D * 2;
    return dispatch_planes(P, [&](auto PC) -> tq_status {
      constexpr int PP = decltype(PC)::value;
      if constexpr (PP == 0) {
        return set_error(TQ_ERR_UNSUPPORTED, "quantize_kv: mse needs code planes");
      } else {
        return dispatch_bool(xf32, [&](auto XF) -> tq_status {
          constexpr bool XF32 = decltype(XF)::value;
          auto kern = quantize_kv_kernel<D, PP, XF32>;
          if (lds > 64 * 1024) {
            hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return check_hip(e, "quantize_kv: set LDS size");
          }
          // persistent workgroups: as many as fit on the device at once, split over
          // the grid rows (each row walks the steps of one group, or half of one)
          constexpr int T = q_tiles(D, false, XF32, false);
          const int by_waves = q_waves_per_simd(D, false, XF32) * 4 / kQWaves;
          const int by_lds = (int)((160 * 1024) / lds);
          const int per_cu = by_waves < by_lds ? by_waves : by_lds;
          const int rows_k = HALF ? 2 * ng : ng;
          const int rows = 2 * rows_k;
          const int64_t n_max = k.n_per_group > v.n_per_group ? k.n_per_group : v.n_per_group;
          const int64_t steps = (n_max + 16 * T - 1) / (16 * T);
          int64_t want = ((int64_t)(per_cu > 0 ? per_cu : 1) * device_cus() + rows - 1) / rows;
          const int64_t cap = (steps + kQWaves - 1) / kQWaves;
          if (want > cap) want = cap;
          if (want < 1) want = 1;
          hipLaunchKernelGGL(kern, dim3((unsigned)want, (unsigned)rows), dim3(kQThreads), lds, stream, pk, pv, rows_k);
          return launch_check("quantize_kv: launch");
        });
      }
    });
  });
}

// In-place VECTOR -> BLOCK32 repack of the codes of 32-vector blocks (one
// workgroup per block): the block's 32 records, 4 planes d bytes together, are
// read into LDS, then every 32-bit block word is assembled from its 32 bits
// (word (p, g, w): bit 4r+k = plane p of coordinate 4w+r of block vector 4g+k,
// bit 16+4r+k the same for vector 16+4g+k) and written over the block.
constexpr int kRepackThreads = 256;
constexpr int kRepackMaxBytes = 4 * 4 * 512;  // 4 planes, d <= 512
__global__ __launch_bounds__(kRepackThreads) void repack_block32_kernel(uint8_t* codes, int planes, int d) {
  __shared__ unsigned rec[kRepackMaxBytes / 4];
  const int words = planes * d;  // 32-bit words per block (= 32 records of planes d / 8 bytes)
  unsigned* blk = (unsigned*)(codes + (int64_t)blockIdx.x * 4 * words);
  for (int i = threadIdx.x; i < words; i += kRepackThreads) rec[i] = blk[i];
  __syncthreads();
  const uint8_t* rb = (const uint8_t*)rec;
  const int rbytes = planes * d / 8;  // one record
  for (int i = threadIdx.x; i < words; i += kRepackThreads) {
    const int w = i % (d / 4), pg = i / (d / 4);
    const int g = pg & 3, p = pg >> 2;
    unsigned word = 0u;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int v = 16 * h + 4 * g + k, j = 4 * w + r;
          const unsigned bit = (rb[v * rbytes + p * (d / 8) + j / 8] >> (j % 8)) & 1u;
          word |= bit << (16 * h + 4 * r + k);
        }
    blk[i] = word;  // every read of the block happened before the barrier
  }
}

tq_status launch_repack_block32(uint8_t* codes, int64_t n_blocks, int planes, int d, hipStream_t stream) {
  if (n_blocks <= 0 || planes <= 0) return TQ_OK;
  if (d % 32 || 4 * planes * d > kRepackMaxBytes || n_blocks > 0x7FFFFFFF)
    return set_error(TQ_ERR_UNSUPPORTED, "block repack: d, planes or size out of range");
  hipLaunchKernelGGL(repack_block32_kernel, dim3((unsigned)n_blocks), dim3(kRepackThreads), 0, stream, codes, planes, d);
  return launch_check("block repack: launch");
}

bool quantize_split_fast(int dim, const tq_quantizer* q) {
  const bool prod = q->variant == TQ_PROD;
  // the kernel builds its fragments from pi32 and, for prod, sp32
  return dim == 128 && q->d % 32 == 0 && q->d <= 128 && q->pi32 != nullptr &&
         (prod ? q->planes <= 3 && q->sp32 != nullptr : q->planes >= 1);
}

bool quantize_split_fusable(int dim, const tq_quantizer* q0, const tq_quantizer* q1) {
  return quantize_split_fast(dim, q0) && quantize_split_fast(dim, q1) && q0->variant == q1->variant &&
         q0->d + q1->d == dim;
}

tq_status launch_quantize_split(const tq_quantizer* const* qz, const tq_quantizer* const* qz1, int n_groups,
                                int64_t n_per_group, const uint16_t* chan, const uint16_t* chan1, const void* x,
                                tq_dtype x_dtype, bool blk, const tq_records& out, const tq_records* out1,
                                hipStream_t stream) {
  constexpr int D = 128;
  const bool fused = qz1 != nullptr;
  const tq_quantizer* q0 = qz[0];
  const tq_quantizer* q1 = fused ? qz1[0] : nullptr;
  const int dp = q0->d;
  const bool prod = q0->variant == TQ_PROD;
  const bool xf32 = x_dtype == TQ_F32;
  const bool dbg = out.rot_dbg != nullptr || out.proj_dbg != nullptr ||
                   (fused && (out1->rot_dbg != nullptr || out1->proj_dbg != nullptr));
  const int P = fused && q1->planes > q0->planes ? q1->planes : q0->planes;
  const size_t lds = (size_t)2 * D * D * 2 * (prod ? 2 : 1);
  for (int g0 = 0; g0 < n_groups; g0 += kQSplitGroups) {
    const int ng = n_groups - g0 < kQSplitGroups ? n_groups - g0 : kQSplitGroups;
    QuantParams prm{};
    prm.x = x;
    prm.x_row_bytes = (int64_t)D * (xf32 ? 4 : 2);
    prm.n_per_group = n_per_group;
    prm.n_groups = ng;
    prm.group_base = g0;
    prm.codes = out.codes;
    prm.signs = out.signs;
    prm.norms = out.norms;
    prm.rnorms = out.rnorms;
    prm.rot_dbg = out.rot_dbg;
    prm.proj_dbg = out.proj_dbg;
    for (int i = 0; i + 1 < (1 << q0->planes); ++i) prm.thr[i] = q0->cb.thresholds[i];
    for (int i = 0; i < (1 << q0->planes); ++i) prm.cen[i] = q0->cb.centroids[i];
    QuantSplitParams sx{};
    sx.dp = dp;
    for (int g = 0; g < ng; ++g) {
      for (int k = 0; k < D; ++k) sx.inv[g][k] = kNoChannel;
      for (int part = 0; part < (fused ? 2 : 1); ++part) {
        const int d = part ? q1->d : dp;
        const uint16_t* c = (part ? chan1 : chan) + (size_t)(g0 + g) * d;
        unsigned(*mask)[4] = part ? sx.chan_mask1 : sx.chan_mask;
        for (int j = 0; j < d; ++j) {
          sx.inv[g][c[j]] = (uint8_t)((part << 7) | j);
          mask[g][c[j] / 32] |= 1u << (c[j] % 32);
        }
      }
      sx.pi[g] = qz[g0 + g]->pi32;
      sx.sp[g] = qz[g0 + g]->sp32;
      if (fused) {
        sx.pi1[g] = qz1[g0 + g]->pi32;
        sx.sp1[g] = qz1[g0 + g]->sp32;
      }
    }
    if (fused) {
      sx.dp1 = q1->d;
      sx.planes0 = q0->planes;
      sx.planes1 = q1->planes;
      // each part's thresholds and centroids on the P-plane search: a part with
      // fewer planes keeps its own below +inf, so its top planes come out 0
      for (int part = 0; part < 2; ++part) {
        const tq_quantizer* q = part ? q1 : q0;
        for (int i = 0; i < 15; ++i)
          sx.thr_e[part][i] = i + 1 < (1 << q->planes) ? q->cb.thresholds[i] : INFINITY;
        for (int i = 0; i < 16; ++i) sx.cen_e[part][i] = i < (1 << q->planes) ? q->cb.centroids[i] : 0.0f;
      }
      sx.codes1 = out1->codes;
      sx.signs1 = out1->signs;
      sx.norms1 = out1->norms;
      sx.rnorms1 = out1->rnorms;
      sx.rot1 = out1->rot_dbg;
      sx.proj1 = out1->proj_dbg;
    }
    tq_status st = dispatch_planes(P, [&](auto PC) -> tq_status {
      constexpr int PP = decltype(PC)::value;
      return dispatch_bool(prod, [&](auto PR) -> tq_status {
        constexpr bool PROD = decltype(PR)::value;
        if constexpr ((!PROD && PP == 0) || (PROD && PP > 3)) {
          return set_error(TQ_ERR_UNSUPPORTED, "split quantize: unsupported (variant, planes)");
        } else {
          return dispatch_bool(xf32, [&](auto XF) -> tq_status {
            constexpr bool XF32 = decltype(XF)::value;
            return dispatch_bool(dbg, [&](auto DB) -> tq_status {
              constexpr bool DBG = decltype(DB)::value;
              return dispatch_bool(blk, [&](auto BL) -> tq_status {
                constexpr bool BLK = decltype(BL)::value && !PROD;
                if (blk && !BLK) return set_error(TQ_ERR_UNSUPPORTED, "split quantize: BLOCK32 is for mse parts");
                return dispatch_bool(fused, [&](auto FU) -> tq_status {
                  constexpr int SPLIT = decltype(FU)::value ? 2 : 1;
                  auto kern = quantize_kernel<D, PP, PROD, XF32, BLK, DBG, SPLIT>;
                  hipError_t e =
                      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
                  if (e != hipSuccess) return check_hip(e, "split quantize: set LDS size");
                  constexpr int T = q_tiles(D, PROD, XF32, BLK);
                  const int by_waves = q_waves_per_simd(D, PROD, XF32, SPLIT == 2) * 4 / kQWaves;
                  const int by_lds = (int)((160 * 1024) / lds);
                  const int per_cu = by_waves < by_lds ? by_waves : by_lds;
                  const int64_t steps = (n_per_group + 16 * T - 1) / (16 * T);
                  int64_t want = ((int64_t)(per_cu > 0 ? per_cu : 1) * device_cus() + ng - 1) / ng;
                  const int64_t cap = (steps + kQWaves - 1) / kQWaves;
                  if (want > cap) want = cap;
                  if (want < 1) want = 1;
                  hipLaunchKernelGGL(kern, dim3((unsigned)want, (unsigned)ng), dim3(kQThreads), lds, stream, prm, sx);
                  return launch_check("split quantize: launch");
                });
              });
            });
          });
        }
      });
    });
    if (st != TQ_OK) return st;
  }
  return TQ_OK;
}

}  // namespace tq
