// Quantize and inner products for large head dimensions (vector search,
// d = 512 .. 4096, multiples of 64): [NIK] "Step 0: normalization", "Step 1:
// random rotation", "Step 2: optimal scalar quantization", "QJL: a one-bit
// method" and "TurboQuant proper"; the vector-search workload of [NIK]
// "Experiments" (nearest neighbours at d = 1536 and 3072).
//
// At these sizes the rotation no longer fits the LDS-staged MFMA fragments of
// the d <= 256 kernels, so both kernels are plain fp32 code over the
// quantizer's fp32 Pi and S: a workgroup quantizes VB vectors at once, reading
// each row of Pi (and S) once for all VB vectors (VB dot products per matrix
// element fetched), with the vectors in LDS. The norm is accumulated in fp64.
#include <hip/hip_runtime.h>

#include "tq_device.h"

namespace tq {
namespace {

struct LargeQuantParams {
  const void* x;
  int64_t n_per_group;
  int d, planes, vb;
  bool prod, x_bf16;
  uint8_t* codes;
  uint8_t* signs;
  float* norms;
  float* rnorms;
  float* rot_dbg;
  float* proj_dbg;
  float thr[15];
  float cen[16];
  int64_t group_base;
  const float* pi[kMaxGroupsPerLaunch];
  const float* s[kMaxGroupsPerLaunch];
};

// out[v][i] = sum_j M[i][j] in[v][j] for the workgroup's nv vectors: thread t
// takes rows t, t + 256, ...; each row is read once (float4) for all vectors.
template <int VB>
__device__ void rows_times(const float* __restrict__ M, const float* in, float* out, int d, int nv) {
  for (int i = threadIdx.x; i < d; i += kThreads) {
    const float4* row = (const float4*)(M + (int64_t)i * d);
    float acc[VB];
#pragma unroll
    for (int v = 0; v < VB; ++v) acc[v] = 0.f;
    for (int j4 = 0; j4 < d / 4; ++j4) {
      const float4 m = row[j4];
#pragma unroll
      for (int v = 0; v < VB; ++v) {
        const float4 u = ((const float4*)(in + (size_t)v * d))[j4];
        acc[v] = fmaf(m.x, u.x, fmaf(m.y, u.y, fmaf(m.z, u.z, fmaf(m.w, u.w, acc[v]))));
      }
    }
#pragma unroll
    for (int v = 0; v < VB; ++v)
      if (v < nv) out[(size_t)v * d + i] = acc[v];
  }
}

// out[v][j] = sum_i M[i][j] in[v][i]: thread t takes columns t, t + 256, ...
// (consecutive threads read consecutive elements of a row)
template <int VB>
__device__ void cols_times(const float* __restrict__ M, const float* in, float* out, int d, int nv) {
  for (int j = threadIdx.x; j < d; j += kThreads) {
    float acc[VB];
#pragma unroll
    for (int v = 0; v < VB; ++v) acc[v] = 0.f;
    for (int i = 0; i < d; ++i) {
      const float m = M[(int64_t)i * d + j];
#pragma unroll
      for (int v = 0; v < VB; ++v) acc[v] = fmaf(m, in[(size_t)v * d + i], acc[v]);
    }
#pragma unroll
    for (int v = 0; v < VB; ++v)
      if (v < nv) out[(size_t)v * d + j] = acc[v];
  }
}

template <int VB>
__global__ __launch_bounds__(kThreads) void quantize_large_kernel(LargeQuantParams prm) {
  extern __shared__ float lds[];  // A[VB][d] (u, then r), B[VB][d] (y, then e), small arrays
  const int d = prm.d;
  float* A = lds;
  float* Bm = lds + (size_t)VB * d;
  float* nu_s = Bm + (size_t)VB * d;  // [VB]
  float* inv_s = nu_s + VB;           // [VB]
  float* gam_s = inv_s + VB;          // [VB]
  const int grp = blockIdx.y;
  const int64_t n = prm.n_per_group;
  const int64_t v0 = (int64_t)blockIdx.x * VB;
  const int nv = (int)min((int64_t)VB, n - v0);
  const int64_t gbase = (prm.group_base + grp) * n;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* pi = prm.pi[grp];
  // ---- norms (fp64) and unit vectors ----
  for (int v = wave; v < VB; v += kThreads / 64) {
    double acc = 0.0;
    if (v < nv) {
      const int64_t row = gbase + v0 + v;
      for (int j = lane; j < d; j += 64) {
        const float xv = prm.x_bf16 ? bf16_val(((const uint16_t*)prm.x)[row * d + j]) : ((const float*)prm.x)[row * d + j];
        A[(size_t)v * d + j] = xv;
        acc = fma((double)xv, (double)xv, acc);
      }
    } else {
      for (int j = lane; j < d; j += 64) A[(size_t)v * d + j] = 0.f;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    const double nu = sqrt(acc);
    if (lane == 0) {
      nu_s[v] = (float)nu;
      inv_s[v] = nu > 0.0 ? (float)(1.0 / nu) : 0.f;
    }
    __builtin_amdgcn_wave_barrier();
    const float inv = nu > 0.0 ? (float)(1.0 / nu) : 0.f;
    for (int j = lane; j < d; j += 64) A[(size_t)v * d + j] *= inv;
  }
  __syncthreads();
  // ---- y = Pi u ----
  rows_times<VB>(pi, A, Bm, d, VB);
  __syncthreads();
  // ---- nearest centroids, codes, residual ----
  const int K = 1 << prm.planes;
  for (int e = threadIdx.x; e < VB * d; e += kThreads) {
    const int v = e / d;
    const float y = Bm[e];
    if (prm.rot_dbg && v < nv) prm.rot_dbg[(gbase + v0 + v) * d + (e % d)] = y;
    int i = 0;
    for (int k = 0; k + 1 < K; ++k) i += y > prm.thr[k] ? 1 : 0;
    const bool zero = !(inv_s[v] > 0.f);
    if (zero) i = 0;
    A[e] = __int_as_float(i);            // A now holds the indices
    Bm[e] = zero ? 0.f : y - prm.cen[i];  // Bm now holds the residual e
  }
  __syncthreads();
  const int wpp = d / 32;
  const int P = prm.planes;
  for (int e = threadIdx.x; e < VB * P * wpp; e += kThreads) {
    const int v = e / (P * wpp), rest = e % (P * wpp), pl = rest / wpp, w = rest % wpp;
    if (v >= nv) continue;
    unsigned bits = 0u;
    for (int c = 0; c < 32; ++c) bits |= (unsigned)((__float_as_int(A[(size_t)v * d + 32 * w + c]) >> pl) & 1) << c;
    ((unsigned*)(prm.codes + (gbase + v0 + v) * (int64_t)(P * d / 8)))[pl * wpp + w] = bits;
  }
  if (threadIdx.x < VB && threadIdx.x < nv) prm.norms[gbase + v0 + threadIdx.x] = nu_s[threadIdx.x];
  if (!prm.prod) return;
  // ---- prod: |e|, r = Pi^T e, p = S r, sign bits ----
  for (int v = wave; v < VB; v += kThreads / 64) {
    double acc = 0.0;
    for (int j = lane; j < d; j += 64) {
      const float ev = Bm[(size_t)v * d + j];
      acc = fma((double)ev, (double)ev, acc);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    if (lane == 0) gam_s[v] = inv_s[v] > 0.f ? (float)sqrt(acc) : 0.f;
  }
  __syncthreads();  // the indices in A are no longer needed
  cols_times<VB>(pi, Bm, A, d, VB);
  __syncthreads();
  rows_times<VB>(prm.s[grp], A, Bm, d, VB);  // Bm = p
  __syncthreads();
  if (prm.proj_dbg)
    for (int e = threadIdx.x; e < VB * d; e += kThreads)
      if (e / d < nv) prm.proj_dbg[(gbase + v0 + e / d) * d + (e % d)] = Bm[e];
  for (int e = threadIdx.x; e < VB * wpp; e += kThreads) {
    const int v = e / wpp, w = e % wpp;
    if (v >= nv) continue;
    const bool zero = !(inv_s[v] > 0.f);
    unsigned bits = 0u;
    for (int c = 0; c < 32; ++c) bits |= (!zero && Bm[(size_t)v * d + 32 * w + c] >= 0.f ? 1u : 0u) << c;
    ((unsigned*)(prm.signs + (gbase + v0 + v) * (int64_t)(d / 8)))[w] = bits;
  }
  if (threadIdx.x < VB && threadIdx.x < nv) prm.rnorms[gbase + v0 + threadIdx.x] = gam_s[threadIdx.x];
}

// <y, x~> for large d: one workgroup per (query, 8192 vectors). The rotated
// query Pi y (and S y for prod) is formed once per workgroup in LDS; each
// thread then walks whole records, 8 coordinates per code byte.
struct LargeIpParams {
  const float* y;
  const uint8_t* codes;
  const uint8_t* signs;
  const float* norms;
  const float* rnorms;
  const float* pi;
  const float* s;
  float* out;
  int64_t n;
  int d, planes;
  bool prod;
  float cen[16];
  float kappa;
};

constexpr int kIpChunk = 8192;

__global__ __launch_bounds__(kThreads) void inner_products_large_kernel(LargeIpParams prm) {
  extern __shared__ float lds[];  // yq[d], yp[d], ys[d]
  const int d = prm.d;
  float* yq = lds;
  float* yp = lds + d;
  float* ys = lds + 2 * d;
  const int64_t qi = blockIdx.y;
  for (int j = threadIdx.x; j < d; j += kThreads) yq[j] = prm.y[qi * d + j];
  __syncthreads();
  rows_times<1>(prm.pi, yq, yp, d, 1);
  if (prm.prod) rows_times<1>(prm.s, yq, ys, d, 1);
  __syncthreads();
  const int P = prm.planes;
  const int64_t v_end = min(prm.n, (int64_t)(blockIdx.x + 1) * kIpChunk);
  for (int64_t v = (int64_t)blockIdx.x * kIpChunk + threadIdx.x; v < v_end; v += kThreads) {
    float a = 0.f, b = 0.f;
    const uint8_t* rec = prm.codes + v * (P * d / 8);
    const uint8_t* sg = prm.prod ? prm.signs + v * (d / 8) : nullptr;
    for (int j8 = 0; j8 < d / 8; ++j8) {
      unsigned pb[4] = {0u, 0u, 0u, 0u};
      for (int p = 0; p < P; ++p) pb[p] = rec[p * d / 8 + j8];
      const unsigned sb = prm.prod ? sg[j8] : 0u;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int idx = (int)(((pb[0] >> i) & 1u) | (((pb[1] >> i) & 1u) << 1) | (((pb[2] >> i) & 1u) << 2) |
                              (((pb[3] >> i) & 1u) << 3));
        a = fmaf(yp[8 * j8 + i], prm.cen[idx], a);
        if (prm.prod) b += ((sb >> i) & 1u) ? ys[8 * j8 + i] : -ys[8 * j8 + i];
      }
    }
    float r = a;
    if (prm.prod) r = fmaf(prm.rnorms[v] * prm.kappa, b, r);
    prm.out[qi * prm.n + v] = prm.norms[v] * r;
  }
}

}  // namespace

tq_status launch_quantize_large(const QuantizeLaunch& a, hipStream_t stream) {
  const tq_quantizer* q0 = a.qz[0];
  const int d = q0->d;
  if (a.layout != TQ_LAYOUT_VECTOR) return set_error(TQ_ERR_UNSUPPORTED, "quantize: d > 256 supports the vector layout only");
  const int vb = d <= 2048 ? 8 : 4;
  const size_t lds = ((size_t)2 * vb * d + 3 * vb) * sizeof(float);
  for (int g0 = 0; g0 < a.n_groups; g0 += kMaxGroupsPerLaunch) {
    const int ng = min(kMaxGroupsPerLaunch, a.n_groups - g0);
    LargeQuantParams prm{};
    prm.x = a.x;
    prm.n_per_group = a.n_per_group;
    prm.d = d;
    prm.planes = q0->planes;
    prm.vb = vb;
    prm.prod = q0->variant == TQ_PROD;
    prm.x_bf16 = a.x_dtype == TQ_BF16;
    prm.codes = a.codes;
    prm.signs = a.signs;
    prm.norms = a.norms;
    prm.rnorms = a.rnorms;
    prm.rot_dbg = a.rot_dbg;
    prm.proj_dbg = a.proj_dbg;
    const int K = 1 << q0->planes;
    for (int i = 0; i + 1 < K; ++i) prm.thr[i] = q0->cb.thresholds[i];
    for (int i = 0; i < K; ++i) prm.cen[i] = q0->cb.centroids[i];
    prm.group_base = g0;
    for (int g = 0; g < ng; ++g) {
      prm.pi[g] = a.qz[g0 + g]->pi32;
      prm.s[g] = a.qz[g0 + g]->s32;
    }
    const dim3 grid((unsigned)((a.n_per_group + vb - 1) / vb), (unsigned)ng);
    if (vb == 8) {
      hipError_t e = hipFuncSetAttribute((const void*)quantize_large_kernel<8>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return check_hip(e, "quantize: set LDS size");
      hipLaunchKernelGGL(quantize_large_kernel<8>, grid, dim3(kThreads), lds, stream, prm);
    } else {
      hipError_t e = hipFuncSetAttribute((const void*)quantize_large_kernel<4>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return check_hip(e, "quantize: set LDS size");
      hipLaunchKernelGGL(quantize_large_kernel<4>, grid, dim3(kThreads), lds, stream, prm);
    }
    tq_status st = launch_check("quantize (large d): launch");
    if (st != TQ_OK) return st;
  }
  return TQ_OK;
}

tq_status launch_inner_products_large(const tq_quantizer* q, const float* y, int64_t m, const uint8_t* codes,
                                      const uint8_t* signs, const float* norms, const float* rnorms, int64_t n,
                                      float* out, hipStream_t stream) {
  LargeIpParams prm{};
  prm.y = y;
  prm.codes = codes;
  prm.signs = signs;
  prm.norms = norms;
  prm.rnorms = rnorms;
  prm.pi = q->pi32;
  prm.s = q->s32;
  prm.out = out;
  prm.n = n;
  prm.d = q->d;
  prm.planes = q->planes;
  prm.prod = q->variant == TQ_PROD;
  for (int i = 0; i < (1 << q->planes); ++i) prm.cen[i] = q->cb.centroids[i];
  prm.kappa = (float)(std::sqrt(M_PI / 2.0) / q->d);
  if (prm.planes > 4) return set_error(TQ_ERR_UNSUPPORTED, "inner_products: planes");
  const size_t lds = (size_t)3 * q->d * sizeof(float);
  const dim3 grid((unsigned)((n + kIpChunk - 1) / kIpChunk), (unsigned)m);
  hipLaunchKernelGGL(inner_products_large_kernel, grid, dim3(kThreads), lds, stream, prm);
  return launch_check("inner_products (large d): launch");
}

}  // namespace tq
