// Dequantize and inner-product kernels for gfx950 (CDNA4, wave64) and their
// launchers: the reference-speed library calls Q^-1 and <y, x~> on packed codes.
//
// What is computed follows [NIK] = S. Nikolenko, "Eternal mathematics of
// TurboQuant" (blog.sergeynikolenko.ru): "Step 2: optimal scalar quantization
// (Lloyd-Max)" (x~ = |x| Pi^T c[idx]), "QJL: a one-bit method" (the
// sqrt(pi/2)/d S^T z reconstruction) and "TurboQuant proper" (their sum for
// prod). Both kernels are plain fp32 VALU code over the quantizer's fp32 copies
// of Pi and S: they are not on the decode hot path, which reads the codes with
// matrix cores directly.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>

#include "tq_device.h"

namespace tq {
namespace {

// ===========================================================================
// Dequantize: [NIK] Step 2 (x~ = |x| Pi^T c[idx]); prod adds |r| sqrt(pi/2)/d S^T z.
// ===========================================================================
struct DequantParams {
  const uint8_t* codes;
  const uint8_t* signs;
  const float* norms;
  const float* rnorms;
  const float* pi;
  const float* s;
  float* out;
  int64_t n;
  float cen[16];
  float kappa;
};

template <int D, int P, bool PROD, bool BLK>
__global__ __launch_bounds__(kThreads) void dequantize_kernel(DequantParams prm) {
  constexpr int VB = 8;
  __shared__ float yc[VB][D];
  __shared__ float zs[VB][D];
  const int64_t v0 = (int64_t)blockIdx.x * VB;
  for (int e = threadIdx.x; e < VB * D; e += kThreads) {
    const int vi = e / D, j = e % D;
    const int64_t v = v0 + vi;
    float c = 0.f, z = 0.f;
    if (v < prm.n) {
      int idx = 0;
      if constexpr (P > 0) {
        if constexpr (!BLK) {
          const uint8_t* rec = prm.codes + v * (P * D / 8);
#pragma unroll
          for (int p = 0; p < P; ++p) idx |= ((rec[p * D / 8 + j / 8] >> (j % 8)) & 1) << p;
        } else {
          const int64_t blk = v / 32;
          const int u = (int)(v % 32), half = u / 16, gg = (u % 16) / 4, k = u % 4;
          const int w = j / 4, r = j % 4;
          const uint8_t* base = prm.codes + blk * (4 * P * D);
#pragma unroll
          for (int p = 0; p < P; ++p) {
            const unsigned word = *(const unsigned*)(base + ((p * 4 + gg) * (D / 4) + w) * 4);
            idx |= (int)((word >> (16 * half + 4 * r + k)) & 1u) << p;
          }
        }
      }
      c = prm.cen[idx];
      if constexpr (PROD) z = ((prm.signs[v * (D / 8) + j / 8] >> (j % 8)) & 1) ? 1.f : -1.f;
    }
    yc[vi][j] = c;
    zs[vi][j] = z;
  }
  __syncthreads();
  const int j = threadIdx.x;
  if (j < D) {
    for (int vi = 0; vi < VB; ++vi) {
      const int64_t v = v0 + vi;
      if (v >= prm.n) break;
      float a = 0.f, b = 0.f;
      for (int k = 0; k < D; ++k) {
        a += prm.pi[k * D + j] * yc[vi][k];
        if constexpr (PROD) b += prm.s[k * D + j] * zs[vi][k];
      }
      float r = a;
      if constexpr (PROD) r += prm.rnorms[v] * prm.kappa * b;
      prm.out[v * D + j] = prm.norms[v] * r;
    }
  }
}

// ===========================================================================
// Inner products <y, x~> = |x| (<Pi y, c[idx]> + |r| sqrt(pi/2)/d <S y, z>)
// ===========================================================================
struct IpParams {
  const float* y;
  const uint8_t* codes;
  const uint8_t* signs;
  const float* norms;
  const float* rnorms;
  const float* pi;
  const float* s;
  float* out;
  int64_t n;
  float cen[16];
  float kappa;
};

template <int D, int P, bool PROD>
__global__ __launch_bounds__(kThreads) void inner_products_kernel(IpParams prm) {
  constexpr int CHUNK = 1024;
  __shared__ float yq[D], yp[D], ys[D];
  const int64_t qi = blockIdx.y;
  for (int j = threadIdx.x; j < D; j += kThreads) yq[j] = prm.y[qi * D + j];
  __syncthreads();
  for (int j = threadIdx.x; j < D; j += kThreads) {
    float a = 0.f, b = 0.f;
    for (int k = 0; k < D; ++k) {
      a += prm.pi[j * D + k] * yq[k];
      if constexpr (PROD) b += prm.s[j * D + k] * yq[k];
    }
    yp[j] = a;
    ys[j] = b;
  }
  __syncthreads();
  const int64_t v_end = min(prm.n, (int64_t)(blockIdx.x + 1) * CHUNK);
  for (int64_t v = (int64_t)blockIdx.x * CHUNK + threadIdx.x; v < v_end; v += kThreads) {
    float a = 0.f, b = 0.f;
    const uint8_t* rec = prm.codes + v * (P * D / 8);
    for (int j8 = 0; j8 < D / 8; ++j8) {
      unsigned pb[P > 0 ? P : 1];
#pragma unroll
      for (int p = 0; p < P; ++p) pb[p] = rec[p * D / 8 + j8];
      unsigned sb = 0;
      if constexpr (PROD) sb = prm.signs[v * (D / 8) + j8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        int idx = 0;
#pragma unroll
        for (int p = 0; p < P; ++p) idx |= (int)((pb[p] >> i) & 1u) << p;
        a += yp[8 * j8 + i] * prm.cen[idx];
        if constexpr (PROD) b += ((sb >> i) & 1u) ? ys[8 * j8 + i] : -ys[8 * j8 + i];
      }
    }
    float r = a;
    if constexpr (PROD) r += prm.rnorms[v] * prm.kappa * b;
    prm.out[qi * prm.n + v] = prm.norms[v] * r;
  }
}

}  // namespace

tq_status launch_dequantize(const tq_quantizer* q, tq_layout layout, const uint8_t* codes,
                            const uint8_t* signs, const float* norms, const float* rnorms, int64_t n,
                            float* x_out, hipStream_t stream) {
  DequantParams prm{};
  prm.codes = codes;
  prm.signs = signs;
  prm.norms = norms;
  prm.rnorms = rnorms;
  prm.pi = q->pi32;
  prm.s = q->s32;
  prm.out = x_out;
  prm.n = n;
  for (int i = 0; i < (1 << q->planes); ++i) prm.cen[i] = q->cb.centroids[i];
  prm.kappa = (float)(std::sqrt(M_PI / 2.0) / q->d);
  const bool prod = q->variant == TQ_PROD, blk = layout == TQ_LAYOUT_BLOCK32;
  dim3 grid((unsigned)((n + 7) / 8));
  return dispatch_dim(q->d, [&](auto DC) -> tq_status {
    constexpr int D = decltype(DC)::value;
    return dispatch_planes(q->planes, [&](auto PC) -> tq_status {
      constexpr int PP = decltype(PC)::value;
      return dispatch_bool(prod, [&](auto PR) -> tq_status {
        constexpr bool PROD = decltype(PR)::value;
        return dispatch_bool(blk, [&](auto BL) -> tq_status {
          constexpr bool BLK = decltype(BL)::value;
          if constexpr ((BLK && PROD) || (PROD && PP > 3) || (!PROD && PP == 0)) {
            return set_error(TQ_ERR_UNSUPPORTED, "dequantize: unsupported (variant, planes, layout)");
          } else {
            hipLaunchKernelGGL((dequantize_kernel<D, PP, PROD, BLK>), grid, dim3(kThreads), 0, stream, prm);
            return launch_check("dequantize: launch");
          }
        });
      });
    });
  });
}

tq_status launch_inner_products(const tq_quantizer* q, const float* y, int64_t m, const uint8_t* codes,
                                const uint8_t* signs, const float* norms, const float* rnorms, int64_t n,
                                float* out, hipStream_t stream) {
  IpParams prm{};
  prm.y = y;
  prm.codes = codes;
  prm.signs = signs;
  prm.norms = norms;
  prm.rnorms = rnorms;
  prm.pi = q->pi32;
  prm.s = q->s32;
  prm.out = out;
  prm.n = n;
  for (int i = 0; i < (1 << q->planes); ++i) prm.cen[i] = q->cb.centroids[i];
  prm.kappa = (float)(std::sqrt(M_PI / 2.0) / q->d);
  const bool prod = q->variant == TQ_PROD;
  dim3 grid((unsigned)((n + 1023) / 1024), (unsigned)m);
  return dispatch_dim(q->d, [&](auto DC) -> tq_status {
    constexpr int D = decltype(DC)::value;
    return dispatch_planes(q->planes, [&](auto PC) -> tq_status {
      constexpr int PP = decltype(PC)::value;
      return dispatch_bool(prod, [&](auto PR) -> tq_status {
        constexpr bool PROD = decltype(PR)::value;
        if constexpr ((PROD && PP > 3) || (!PROD && PP == 0)) {
          return set_error(TQ_ERR_UNSUPPORTED, "inner_products: unsupported (variant, planes)");
        } else {
          hipLaunchKernelGGL((inner_products_kernel<D, PP, PROD>), grid, dim3(kThreads), 0, stream, prm);
          return launch_check("inner_products: launch");
        }
      });
    });
  });
}


}  // namespace tq
