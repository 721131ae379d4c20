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
  const uint16_t* pi_frag[kMaxGroupsPerLaunch];
  const uint16_t* sp_frag[kMaxGroupsPerLaunch];
};

// 16-vector tiles per wave step (the block layout needs two: a block is 32 vectors)
__host__ __device__ constexpr int q_tiles(int D, bool prod, bool xf32, bool blk) {
  return (D == 256 && (prod || xf32) && !blk) ? 1 : 2;
}
__host__ __device__ constexpr int q_waves_per_simd(int D, bool prod) { return (D <= 128 && !prod) ? 4 : 2; }
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

// MFMA operands of a tile (K index 8g + e of k-step ks <-> coordinate
// g D/4 + 8 ks + e) and this lane's part of |x|^2 in fp64.
template <int D, bool XF32>
__device__ __forceinline__ double tile_operands(const XTile<D, XF32>& t, u32x4* xh, u32x4* xl) {
  constexpr int NK = D / 32;
  double acc = 0.0;
#pragma unroll
  for (int ks = 0; ks < NK; ++ks) {
    if constexpr (!XF32) {
      const u32x4 v = t.raw[ks];
      xh[ks] = v;
      const unsigned w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = bf16_val(w[e] & 0xFFFFu), b = bf16_val(w[e] >> 16);
        acc = fma((double)a, (double)a, acc);
        acc = fma((double)b, (double)b, acc);
      }
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

template <int D, int P, bool PROD, bool XF32, bool BLK, bool DBG>
__global__ __launch_bounds__(kQThreads, q_waves_per_simd(D, PROD)) void quantize_kernel(QuantParams prm) {
  constexpr int NQ = D / 16, NK = D / 32, Q4 = D / 4;
  constexpr int T = q_tiles(D, PROD, XF32, BLK);
  constexpr bool PREF = q_prefetch(D, XF32);
  constexpr int WPL = Q4 >= 32 ? Q4 / 32 : 1;  // 32-bit words per plane per lane (vector layout)
  constexpr int PP = P > 0 ? P : 1;
  constexpr bool LDS_FRAG = D <= 128;
  constexpr int FRAG_VECS = 2 * NQ * NK * 64;  // u32x4 per matrix (hi + lo)
  extern __shared__ u32x4 smem_frag[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int grp = blockIdx.y;
  const int64_t n = prm.n_per_group;
  const int64_t gbase = (prm.group_base + grp) * n;
  const int64_t steps = (n + 16 * T - 1) / (16 * T);
  constexpr int NTHR = P > 0 ? (1 << P) - 1 : 1;
  constexpr int NCEN = 1 << (P > 0 ? P : 0);
  float thr[NTHR], cen[NCEN];
#pragma unroll
  for (int i = 0; i < NTHR; ++i) thr[i] = opaque_vgpr(prm.thr[i]);
#pragma unroll
  for (int i = 0; i < NCEN; ++i) cen[i] = PROD ? opaque_vgpr(prm.cen[i]) : 0.0f;
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
  if (step < steps) load_step(step, cur);  // in flight while the fragments are staged

  const u32x4* fpi;
  const u32x4* fsp;
  if constexpr (LDS_FRAG) {
    const u32x4* src = (const u32x4*)prm.pi_frag[grp];
    for (int i = threadIdx.x; i < FRAG_VECS; i += kQThreads) smem_frag[i] = src[i];
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
  // fragment (hilo, q, ks) of this lane
  auto frag = [&](const u32x4* base, int hl, int q, int ks) -> u32x4 {
    return base[((hl * NQ + q) * NK + ks) * 64 + lane];
  };

  for (; step < steps; step += stride) {
    const int64_t nstep = step + stride;
    if constexpr (PREF) {
      if (nstep < steps) load_step(nstep, nxt);
    }
    u32x4 xh[T][NK], xl[T][XF32 ? NK : 1];
    double ss[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      ss[t] = tile_operands<D, XF32>(cur[t], xh[t], xl[t]);
      ss[t] += __shfl_xor(ss[t], 16);
      ss[t] += __shfl_xor(ss[t], 32);
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
      unsigned pw[T][PP][WPL];
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int p = 0; p < PP; ++p)
#pragma unroll
          for (int w = 0; w < WPL; ++w) pw[t][p][w] = 0u;
      // prod: residual operands for the second contraction, K order = this lane's coords
      u32x4 eh[PROD ? T : 1][PROD ? NK : 1], el[PROD ? T : 1][PROD ? NK : 1];
      float eodd[PROD ? T : 1][4];
      float esq[T];
#pragma unroll
      for (int t = 0; t < T; ++t) esq[t] = 0.0f;

#pragma unroll
      for (int q = NQ - 1; q >= 0; --q) {
        f32x4 C[T];
#pragma unroll
        for (int t = 0; t < T; ++t) C[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) {
          const u32x4 ph = frag(fpi, 0, q, ks), pl = frag(fpi, 1, q, ks);
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
            if (prm.rot_dbg && v < n)
              *(float4*)(prm.rot_dbg + (gbase + v) * D + Q4 * g + 4 * q) = float4{y[0], y[1], y[2], y[3]};
          }
          float e4[4];
          PlaneMasks<P> pm[4];
          if constexpr (P > 0) {
            nearest_planes<P, 4>(y, thr, pm);
#pragma unroll
            for (int p = 0; p < P; ++p)
#pragma unroll
              for (int i = 3; i >= 0; --i) {
                unsigned& w = pw[t][p][(4 * q + i) / 32];
                w = shift_in(w, pm[i].m[p]);
              }
          }
#pragma unroll
          for (int i = 3; i >= 0; --i) {
            if constexpr (PROD) {
              const float ej = valid[t] ? y[i] - plane_centroid<P>(pm[i], cen) : 0.0f;
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
      }
      // wave-uniform bases of this step, 32-bit lane offsets
      float* nbase = prm.norms + gbase + v0;
      uint8_t* cbase = prm.codes + (gbase + v0) * (P * D / 8);
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const int rel = 16 * t + r16;
        if (v0 + rel < n) {
          if (g == 0) nbase[rel] = (float)nu[t];
          if constexpr (P > 0) {
            uint8_t* dst = cbase + (unsigned)rel * (P * D / 8);
#pragma unroll
            for (int p = 0; p < P; ++p) {
              if constexpr (Q4 >= 32) {
#pragma unroll
                for (int w = 0; w < WPL; ++w)
                  *(unsigned*)(dst + p * D / 8 + g * (Q4 / 8) + 4 * w) = valid[t] ? pw[t][p][w] : 0u;
              } else {
                *(unsigned short*)(dst + p * D / 8 + g * (Q4 / 8)) = (unsigned short)(valid[t] ? pw[t][p][0] : 0u);
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
          esq[t] += __shfl_xor(esq[t], 16);
          esq[t] += __shfl_xor(esq[t], 32);
#pragma unroll
          for (int w = 0; w < WPL; ++w) sw[t][w] = 0u;
        }
#pragma unroll
        for (int q = NQ - 1; q >= 0; --q) {
          f32x4 acc[T];
#pragma unroll
          for (int t = 0; t < T; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < NK; ++ks) {
            const u32x4 sh = frag(fsp, 0, q, ks), sl = frag(fsp, 1, q, ks);
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
              if (prm.proj_dbg && v < n)
                *(float4*)(prm.proj_dbg + (gbase + v) * D + Q4 * g + 4 * q) = float4{pv[0], pv[1], pv[2], pv[3]};
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        float* rbase = prm.rnorms + gbase + v0;
        uint8_t* sbase = prm.signs + (gbase + v0) * (D / 8);
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const int rel = 16 * t + r16;
          if (v0 + rel < n) {
            if (g == 0) rbase[rel] = valid[t] ? sqrtf(esq[t]) : 0.0f;
            uint8_t* dst = sbase + (unsigned)rel * (D / 8);
            if constexpr (Q4 >= 32) {
#pragma unroll
              for (int w = 0; w < WPL; ++w) *(unsigned*)(dst + g * (Q4 / 8) + 4 * w) = valid[t] ? sw[t][w] : 0u;
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
        const double nu_own = sqrt(ss[t]);  // vector 16t + r16
        const float inv_own = nu_own > 0.0 ? (float)(1.0 / nu_own) : 0.0f;
        vmask[t] = 0u;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          inv[t][k] = __shfl(inv_own, 4 * g + k);
          vmask[t] |= (inv[t][k] > 0.0f ? 1u : 0u) << k;
        }
        const int64_t v = v0 + 16 * t + r16;
        if (g == 0 && v < n) prm.norms[gbase + v] = (float)nu_own;
      }
      const int slot = r16 & 3;
      uint8_t* blk = prm.codes + ((gbase + v0) / 32) * (int64_t)(4 * P * D);
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        f32x4 C[T];
#pragma unroll
        for (int t = 0; t < T; ++t) C[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) {
          const u32x4 ph = frag(fpi, 0, q, ks), pl = frag(fpi, 1, q, ks);
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
          nearest_planes<P, 4>(y, thr, pm);
#pragma unroll
          for (int p = 0; p < P; ++p)
#pragma unroll
            for (int k = 3; k >= 0; --k) nib[t][p] = shift_in(nib[t][p], pm[k].m[p]);
          if constexpr (DBG) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const int64_t v = v0 + 16 * t + 4 * g + k;
              const int o = Q4 * (r16 >> 2) + 4 * q + slot;
              if (prm.rot_dbg && v < n) prm.rot_dbg[(gbase + v) * D + o] = y[k];
            }
          }
        }
        const int w = (D / 16) * (r16 >> 2) + q;
#pragma unroll
        for (int p = 0; p < P; ++p) {
          unsigned word = (nib[0][p] & vmask[0]) << (4 * slot);
          if constexpr (T > 1) word |= (nib[1][p] & vmask[1]) << (16 + 4 * slot);
          word = quad_or(word);
          if (slot == 0) *(unsigned*)(blk + ((p * 4 + g) * (D / 4) + w) * 4) = word;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (PREF) {
      if (nstep < steps) {
#pragma unroll
        for (int t = 0; t < T; ++t) cur[t] = nxt[t];
      }
    } else {
      if (nstep < steps) load_step(nstep, cur);
    }
  }
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
    for (int g = 0; g < ng; ++g) {
      prm.pi_frag[g] = a.qz[g0 + g]->pi_frag;
      prm.sp_frag[g] = a.qz[g0 + g]->sp_frag;
    }
    const bool dbg = a.rot_dbg != nullptr || a.proj_dbg != nullptr;
    tq_status st = dispatch_dim(q0->d, [&](auto DC) -> tq_status {
      constexpr int D = decltype(DC)::value;
      const size_t lds = D <= 128 ? (size_t)2 * D * D * 2 * (prod ? 2 : 1) : 0;
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
                  const int by_waves = q_waves_per_simd(D, PROD) * 4 / kQWaves;
                  const int by_lds = lds ? (int)((160 * 1024) / lds) : by_waves;
                  const int per_cu = by_waves < by_lds ? by_waves : by_lds;
                  const int64_t steps = (a.n_per_group + 16 * T - 1) / (16 * T);
                  int64_t want = ((int64_t)(per_cu > 0 ? per_cu : 1) * device_cus() + ng - 1) / ng;
                  const int64_t cap = (steps + kQWaves - 1) / kQWaves;
                  if (want > cap) want = cap;
                  if (want < 1) want = 1;
                  hipLaunchKernelGGL(kern, dim3((unsigned)want, (unsigned)ng), dim3(kQThreads), lds, stream, prm);
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


}  // namespace tq
