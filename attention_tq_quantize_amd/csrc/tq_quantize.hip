// HIP kernels for gfx950 (CDNA4, wave64) and their launchers.
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
// fp32 accuracy for the dense rotations comes from splitting each operand into
// bf16 hi + lo parts (16 significant bits) and accumulating in fp32.
//
// Bit operands. A packed bit becomes a bf16 MFMA operand without unpacking:
// rotate the 32-bit word so that the wanted bit lands on exponent bit 4+k of a
// bf16 half and mask everything else; the half is then 0 or the exact power of
// two 2^(2^(4+k) - 127). The other operand carries the compensating factor
// 2^(E - e_k), so every product is exactly (weight * bit * 2^E). One rotate plus
// four ANDs turn a word into one MFMA operand (8 bits).
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
// One wave handles 32 vectors per iteration as two 16-vector MFMA tiles.
// ===========================================================================
struct QuantParams {
  const void* x;
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

template <int D, bool XF32>
__device__ __forceinline__ void load_x_frag(const QuantParams& prm, int64_t row, bool ok, int g,
                                            u32x4* xhi, u32x4* xlo, double* sumsq) {
  constexpr int NK = D / 32, Q4 = D / 4;
  double acc = 0.0;
#pragma unroll
  for (int ks = 0; ks < NK; ++ks) {
    if constexpr (!XF32) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (ok) v = *(const u32x4*)((const uint16_t*)prm.x + row * D + Q4 * g + 8 * ks);
      xhi[ks] = v;
      const unsigned w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = bf16_val(w[e] & 0xFFFFu), b = bf16_val(w[e] >> 16);
        acc += (double)(a * a) + (double)(b * b);  // bf16 squares are exact in fp32
      }
    } else {
      float f[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (ok) {
        const float4* src = (const float4*)((const float*)prm.x + row * D + Q4 * g + 8 * ks);
        const float4 a = src[0], b = src[1];
        f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
        f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
      }
      unsigned h[8], l[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        h[e] = bf16_part(f[e], false);
        l[e] = bf16_part(f[e], true);
        acc += (double)f[e] * (double)f[e];
      }
      xhi[ks] = u32x4{pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7])};
      xlo[ks] = u32x4{pack2(l[0], l[1]), pack2(l[2], l[3]), pack2(l[4], l[5]), pack2(l[6], l[7])};
    }
  }
  acc += __shfl_xor(acc, 16);
  acc += __shfl_xor(acc, 32);
  *sumsq = acc;
}

template <int D, int P, bool PROD, bool XF32, bool BLK>
__global__ __launch_bounds__(kThreads) void quantize_kernel(QuantParams prm) {
  constexpr int NQ = D / 16, NK = D / 32, Q4 = D / 4;
  constexpr bool LDS_FRAG = D <= 128;
  constexpr int FRAG_VECS = 2 * D * D / 8;  // u32x4 per matrix (hi + lo)
  extern __shared__ u32x4 smem_frag[];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int grp = blockIdx.y;
  const int64_t n = prm.n_per_group;
  const int64_t gbase = (prm.group_base + grp) * n;

  const u32x4* fpi;
  const u32x4* fsp;
  if constexpr (LDS_FRAG) {
    const u32x4* src = (const u32x4*)prm.pi_frag[grp];
    for (int i = threadIdx.x; i < FRAG_VECS; i += kThreads) smem_frag[i] = src[i];
    if constexpr (PROD) {
      const u32x4* s2 = (const u32x4*)prm.sp_frag[grp];
      for (int i = threadIdx.x; i < FRAG_VECS; i += kThreads) smem_frag[FRAG_VECS + i] = s2[i];
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

  const int64_t tiles = (n + 31) / 32;
  for (int64_t tile = (int64_t)blockIdx.x * 4 + wave; tile < tiles; tile += (int64_t)gridDim.x * 4) {
    u32x4 xh[2][NK], xl[2][NK];
    double ss[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int64_t v = tile * 32 + 16 * t + r16;
      load_x_frag<D, XF32>(prm, gbase + v, v < n, g, xh[t], xl[t], &ss[t]);
    }
    // y_raw = Pi x for both tiles
    f32x4 C[2][NQ];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int q = 0; q < NQ; ++q) C[t][q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        const u32x4 ph = frag(fpi, 0, q, ks), pl = frag(fpi, 1, q, ks);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          if constexpr (!BLK) {
            C[t][q] = mfma(ph, xh[t][ks], C[t][q]);
            C[t][q] = mfma(pl, xh[t][ks], C[t][q]);
            if constexpr (XF32) C[t][q] = mfma(ph, xl[t][ks], C[t][q]);
          } else {
            C[t][q] = mfma(xh[t][ks], ph, C[t][q]);
            C[t][q] = mfma(xh[t][ks], pl, C[t][q]);
            if constexpr (XF32) C[t][q] = mfma(xl[t][ks], ph, C[t][q]);
          }
        }
      }

    if constexpr (!BLK) {
      // ---- VECTOR layout: lane (vector r16 of tile t, g) holds out coords Q4*g + 4q + i ----
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int64_t v = tile * 32 + 16 * t + r16;
        const bool in = v < n;
        const double nu = sqrt(ss[t]);
        const bool valid = nu > 0.0;
        const float inv = valid ? (float)(1.0 / nu) : 0.0f;
        const int64_t row = gbase + v;
        float y[Q4];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          y[4 * q + 0] = C[t][q].x * inv;
          y[4 * q + 1] = C[t][q].y * inv;
          y[4 * q + 2] = C[t][q].z * inv;
          y[4 * q + 3] = C[t][q].w * inv;
        }
        constexpr int WPL = Q4 >= 32 ? Q4 / 32 : 1;   // words per plane per lane
        unsigned pw[P > 0 ? P : 1][WPL];
#pragma unroll
        for (int p = 0; p < (P > 0 ? P : 1); ++p)
#pragma unroll
          for (int w = 0; w < WPL; ++w) pw[p][w] = 0u;
        float e[PROD ? Q4 : 1];
        float esq = 0.0f;
#pragma unroll
        for (int j = 0; j < Q4; ++j) {
          bool bit[P > 0 ? P : 1];
          if constexpr (P > 0) search_bits<P>(y[j], prm.thr, bit);
#pragma unroll
          for (int p = 0; p < P; ++p) pw[p][j / 32] |= (bit[p] ? 1u : 0u) << (j % 32);
          if constexpr (PROD) {
            const float ej = valid ? y[j] - centroid_of<P>(bit, prm.cen) : 0.0f;
            e[j] = ej;
            esq += ej * ej;
          }
        }
        if (in) {
          if (g == 0) prm.norms[row] = (float)nu;
          if (prm.rot_dbg) {
#pragma unroll
            for (int j = 0; j < Q4; j += 4)
              *(float4*)(prm.rot_dbg + row * D + Q4 * g + j) = float4{y[j], y[j + 1], y[j + 2], y[j + 3]};
          }
          if constexpr (P > 0) {
            uint8_t* dst = prm.codes + row * (P * D / 8);
#pragma unroll
            for (int p = 0; p < P; ++p) {
              if constexpr (Q4 >= 32) {
#pragma unroll
                for (int w = 0; w < WPL; ++w)
                  *(unsigned*)(dst + p * D / 8 + g * (Q4 / 8) + 4 * w) = valid ? pw[p][w] : 0u;
              } else {
                *(unsigned short*)(dst + p * D / 8 + g * (Q4 / 8)) = (unsigned short)(valid ? pw[p][0] : 0u);
              }
            }
          }
        }
        if constexpr (PROD) {
          esq += __shfl_xor(esq, 16);
          esq += __shfl_xor(esq, 32);
          const float gamma = valid ? sqrtf(esq) : 0.0f;
          // residual fragments for the second contraction, K order = this lane's coords
          u32x4 eh[NK], el[NK];
#pragma unroll
          for (int ks = 0; ks < NK; ++ks) {
            unsigned h[8], l[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              h[i] = bf16_part(e[8 * ks + i], false);
              l[i] = bf16_part(e[8 * ks + i], true);
            }
            eh[ks] = u32x4{pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7])};
            el[ks] = u32x4{pack2(l[0], l[1]), pack2(l[2], l[3]), pack2(l[4], l[5]), pack2(l[6], l[7])};
          }
          unsigned sw[WPL];
#pragma unroll
          for (int w = 0; w < WPL; ++w) sw[w] = 0u;
#pragma unroll
          for (int q = 0; q < NQ; ++q) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NK; ++ks) {
              const u32x4 sh = frag(fsp, 0, q, ks), sl = frag(fsp, 1, q, ks);
              acc = mfma(sh, eh[ks], acc);
              acc = mfma(sl, eh[ks], acc);
              acc = mfma(sh, el[ks], acc);
            }
            const float pv[4] = {acc.x, acc.y, acc.z, acc.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int j = 4 * q + i;
              sw[j / 32] |= (pv[i] >= 0.0f ? 1u : 0u) << (j % 32);
            }
            if (in && prm.proj_dbg)
              *(float4*)(prm.proj_dbg + row * D + Q4 * g + 4 * q) = float4{pv[0], pv[1], pv[2], pv[3]};
          }
          if (in) {
            if (g == 0) prm.rnorms[row] = gamma;
            uint8_t* dst = prm.signs + row * (D / 8);
            if constexpr (Q4 >= 32) {
#pragma unroll
              for (int w = 0; w < WPL; ++w)
                *(unsigned*)(dst + g * (Q4 / 8) + 4 * w) = valid ? sw[w] : 0u;
            } else {
              *(unsigned short*)(dst + g * (Q4 / 8)) = (unsigned short)(valid ? sw[0] : 0u);
            }
          }
        }
      }
    } else {
      // ---- BLOCK32 layout (mse): lane (coord lane r16, g) holds vectors 16t + 4g + i of
      // out coord o = Q4*(r16/4) + 4q + (r16%4), i.e. word w = (D/16)(r16/4) + q, slot r = r16%4 ----
      double nu_own[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) nu_own[t] = sqrt(ss[t]);  // norm of vector 16t + r16
      float inv[2][4];
      bool valid[2][4];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const float inv_own = nu_own[t] > 0.0 ? (float)(1.0 / nu_own[t]) : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          inv[t][i] = __shfl(inv_own, 4 * g + i);
          valid[t][i] = inv[t][i] > 0.0f;
        }
        const int64_t v = tile * 32 + 16 * t + r16;
        if (g == 0 && v < n) prm.norms[gbase + v] = (float)nu_own[t];
      }
      unsigned part[P][NQ];
#pragma unroll
      for (int p = 0; p < P; ++p)
#pragma unroll
        for (int q = 0; q < NQ; ++q) part[p][q] = 0u;
      const int slot = r16 & 3;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          const float cv[4] = {C[t][q].x, C[t][q].y, C[t][q].z, C[t][q].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float y = cv[i] * inv[t][i];
            bool bit[P];
            search_bits<P>(y, prm.thr, bit);
#pragma unroll
            for (int p = 0; p < P; ++p)
              part[p][q] |= ((bit[p] && valid[t][i]) ? 1u : 0u) << (16 * t + 4 * slot + i);
            if (prm.rot_dbg) {
              const int64_t v = tile * 32 + 16 * t + 4 * g + i;
              const int o = Q4 * (r16 >> 2) + 4 * q + slot;
              if (v < n) prm.rot_dbg[(gbase + v) * D + o] = y;
            }
          }
        }
      // OR the four coordinate lanes of each word together
#pragma unroll
      for (int p = 0; p < P; ++p)
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          unsigned w = part[p][q];
          w |= __shfl_xor(w, 1);
          w |= __shfl_xor(w, 2);
          part[p][q] = w;
        }
      if (slot == 0) {
        uint8_t* blk = prm.codes + ((gbase + tile * 32) / 32) * (int64_t)(4 * P * D);
#pragma unroll
        for (int p = 0; p < P; ++p)
#pragma unroll
          for (int q = 0; q < NQ; ++q) {
            const int w = (D / 16) * (r16 >> 2) + q;
            *(unsigned*)(blk + ((p * 4 + g) * (D / 4) + w) * 4) = part[p][q];
          }
      }
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
    const int64_t tiles = (a.n_per_group + 31) / 32;
    int64_t want = (int64_t)2 * device_cus() / ng;  // about two workgroups per CU in total
    if (want < 1) want = 1;
    int64_t per = (tiles + 3) / 4;
    if (want > per) want = per;
    dim3 grid((unsigned)want, (unsigned)ng);
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
                auto kern = quantize_kernel<D, PP, PROD, XF32, BLK>;
                if (lds > 64 * 1024) {
                  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
                  if (e != hipSuccess) return check_hip(e, "quantize: set LDS size");
                }
                hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, stream, prm);
                return launch_check("quantize: launch");
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
