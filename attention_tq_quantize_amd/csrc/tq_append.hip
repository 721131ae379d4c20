// Decode-step append: one workgroup per (batch, kv head) quantizes that head's
// new key and value vectors and writes them into the packed caches at the
// sequence's current length; the lengths the attention then reads (length + 1,
// at most max_ctx) are written beside them.
//
// This is the online use of the quantizer on one vector at a time ([NIK]
// "Step 0: normalization", "Step 1: random rotation", "Step 2"; prod keys also
// "TurboQuant proper": residual, |r| and sign(S r)). With a single vector per
// (batch, head) the dense rotations are fp32 matrix-vector products over the
// quantizer's fp32 copies of Pi and S' = S Pi^T (L2-resident across the batch:
// the residual stays in the rotated basis, S r = S' e); the norm is accumulated
// in fp64 and rounded to fp32 like the bulk kernel's. Keys and values of a
// (batch, head) are two workgroups.
#include <hip/hip_runtime.h>

#include "tq_device.h"

namespace tq {
namespace {

struct AppendParams {
  const int32_t* ctx_lens;  // [B] tokens already cached
  int32_t* lens_out;        // [B] tokens attended after the append
  int64_t max_ctx;
  int Hkv, d, k_planes, v_bits;
  bool k_prod, x_bf16;
  const void* k_new;  // [B][Hkv][d]
  const void* v_new;
  const float* k_pi[kMaxKvHeads];
  const float* k_sp[kMaxKvHeads];
  const float* v_pi[kMaxKvHeads];
  float k_thr[15], k_cen[16];
  float v_thr[15], v_cen[16];
  uint32_t* k_codes;  // [B][Hkv][max_ctx][k_planes * d / 32]
  uint32_t* k_signs;  // [B][Hkv][max_ctx][d / 32]
  float* k_norms;
  float* k_rnorms;
  uint32_t* v_codes;  // [B][Hkv][max_ctx / 32][v_bits * d] words (block layout)
  float* v_norms;
};

constexpr int kMaxD = 256;

struct Scratch {
  float x[kMaxD];  // input, then u
  float e[kMaxD];  // residual in the rotated basis
  float p[kMaxD];  // QJL projection
  int idx[kMaxD];
  double red[kThreads / 64];
};

__device__ __forceinline__ double block_sum(double v, Scratch& sh) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if ((threadIdx.x & 63) == 0) sh.red[threadIdx.x >> 6] = v;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) s += sh.red[w];
  __syncthreads();
  return s;
}

// a row of M (D floats, 16-byte aligned) dotted with v (shared memory); the
// row is read 64 floats at a time, each group's loads independent and in
// flight together
template <int D>
__device__ __forceinline__ float row_dot(const float* __restrict__ row, const float* v) {
  constexpr int G = D < 64 ? D / 4 : 16;  // float4 loads per group
  const float4* r4 = (const float4*)row;
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int j0 = 0; j0 < D / 4; j0 += G) {
    float4 m[G];
#pragma unroll
    for (int j = 0; j < G; ++j) m[j] = r4[j0 + j];
#pragma unroll
    for (int j = 0; j < G; j += 2) {
      const int c = 4 * (j0 + j);
      a0 = fmaf(m[j].x, v[c], fmaf(m[j].y, v[c + 1], fmaf(m[j].z, v[c + 2], fmaf(m[j].w, v[c + 3], a0))));
      a1 = fmaf(m[j + 1].x, v[c + 4], fmaf(m[j + 1].y, v[c + 5], fmaf(m[j + 1].z, v[c + 6], fmaf(m[j + 1].w, v[c + 7], a1))));
    }
  }
  return a0 + a1;
}

// One vector: norm, y = Pi u, nearest-centroid indices (count of y > t_k), and
// for prod e = y - c[idx], |e| and p = S' e. Leaves idx and p in shared memory.
template <int D>
__device__ void quantize_one(const void* src, bool bf16, const float* pi, const float* sp, int planes,
                             const float* thr, const float* cen, Scratch& sh, float& nu32, float& gamma) {
  const int t = threadIdx.x;
  float xv = 0.f;
  if (t < D) xv = bf16 ? bf16_val(((const uint16_t*)src)[t]) : ((const float*)src)[t];
  const double nu = sqrt(block_sum(t < D ? (double)xv * (double)xv : 0.0, sh));
  nu32 = (float)nu;
  const bool zero = !(nu > 0.0);
  if (t < D) sh.x[t] = zero ? 0.f : (float)((double)xv / nu);
  __syncthreads();
  float e = 0.f;
  if (t < D) {
    const float y = row_dot<D>(pi + (int64_t)t * D, sh.x);
    const int K = 1 << planes;
    int i = 0;
    for (int k = 0; k + 1 < K; ++k) i += y > thr[k] ? 1 : 0;
    if (zero) i = 0;
    sh.idx[t] = i;
    e = zero ? 0.f : y - cen[i];
    sh.e[t] = e;
  }
  gamma = 0.f;
  if (sp) {
    gamma = (float)sqrt(block_sum((double)e * (double)e, sh));  // also publishes e
    if (t < D) sh.p[t] = zero ? -1.f : row_dot<D>(sp + (int64_t)t * D, sh.e);  // zero vector: sign bits 0
  }
  __syncthreads();
}

template <int D>
__global__ __launch_bounds__(kThreads) void append_kernel(AppendParams p) {
  __shared__ Scratch sh;
  const int grp = blockIdx.x;
  const bool value = blockIdx.y == 1;
  const int b = grp / p.Hkv, h = grp % p.Hkv;
  const int tid = threadIdx.x;
  int64_t len = p.ctx_lens[b];
  len = len < 0 ? 0 : len;
  if (!value && h == 0 && tid == 0) p.lens_out[b] = (int32_t)(len < p.max_ctx ? len + 1 : p.max_ctx);
  if (len >= p.max_ctx) return;
  const int64_t slot = (int64_t)grp * p.max_ctx + len;  // (b, h, t) record index
  const size_t esz = p.x_bf16 ? 2 : 4;
  float nu, gamma;
  if (!value) {
    // ---- key: vector-layout record ----
    quantize_one<D>((const char*)p.k_new + (size_t)grp * D * esz, p.x_bf16, p.k_pi[h], p.k_prod ? p.k_sp[h] : nullptr,
                    p.k_planes, p.k_thr, p.k_cen, sh, nu, gamma);
    constexpr int wpp = D / 32;  // 32-bit words per plane of a record
    if (tid < p.k_planes * wpp) {
      const int pl = tid / wpp, w = tid % wpp;
      unsigned bits = 0u;
#pragma unroll
      for (int c = 0; c < 32; ++c) bits |= (unsigned)((sh.idx[32 * w + c] >> pl) & 1) << c;
      p.k_codes[slot * (p.k_planes * wpp) + tid] = bits;
    }
    if (p.k_prod && tid < wpp) {
      unsigned bits = 0u;
#pragma unroll
      for (int c = 0; c < 32; ++c) bits |= (sh.p[32 * tid + c] >= 0.f ? 1u : 0u) << c;
      p.k_signs[slot * wpp + tid] = bits;
    }
    if (tid == 0) {
      p.k_norms[slot] = nu;
      if (p.k_prod) p.k_rnorms[slot] = gamma;
    }
    return;
  }
  // ---- value: slot len % 32 of its block. Slot v is vector 4g + k (v < 16) or
  // 16 + 4g + k; plane pl, coordinate 4w + r sits at bit 4r + k (+16) of word
  // (pl*4 + g)*(d/4) + w of the block ----
  quantize_one<D>((const char*)p.v_new + (size_t)grp * D * esz, p.x_bf16, p.v_pi[h], nullptr, p.v_bits, p.v_thr,
                  p.v_cen, sh, nu, gamma);
  const int v = (int)(len % 32);
  const int hi = v >= 16 ? 16 : 0, g = (v % 16) / 4, k = v % 4;
  const unsigned keep = ~(0x1111u << (k + hi));
  constexpr int wq = D / 4;
  uint32_t* blk = p.v_codes + ((int64_t)grp * (p.max_ctx / 32) + len / 32) * (int64_t)(p.v_bits * D);
  for (int i = tid; i < p.v_bits * wq; i += kThreads) {
    const int pl = i / wq, w = i % wq;
    unsigned bits = 0u;
#pragma unroll
    for (int r = 0; r < 4; ++r) bits |= (unsigned)((sh.idx[4 * w + r] >> pl) & 1) << (4 * r + k + hi);
    uint32_t* word = blk + (pl * 4 + g) * wq + w;
    *word = (*word & keep) | bits;
  }
  if (tid == 0) p.v_norms[slot] = nu;
}

}  // namespace

tq_status launch_append(const AppendLaunch& a, hipStream_t stream) {
  if (a.d > 256 || a.n_kv_heads > kMaxKvHeads) return set_error(TQ_ERR_UNSUPPORTED, "append: shape");
  AppendParams p;
  p.ctx_lens = a.ctx_lens;
  p.lens_out = a.lens_out;
  p.max_ctx = a.max_ctx;
  p.Hkv = a.n_kv_heads;
  p.d = a.d;
  p.k_planes = a.kq[0]->planes;
  p.v_bits = a.vq[0]->bits;
  p.k_prod = a.kq[0]->variant == TQ_PROD;
  p.x_bf16 = a.x_dtype == TQ_BF16;
  p.k_new = a.k_new;
  p.v_new = a.v_new;
  for (int h = 0; h < a.n_kv_heads; ++h) {
    p.k_pi[h] = a.kq[h]->pi32;
    p.k_sp[h] = a.kq[h]->sp32;
    p.v_pi[h] = a.vq[h]->pi32;
  }
  const Codebook& kc = a.kq[0]->cb;
  const Codebook& vc = a.vq[0]->cb;
  for (int i = 0; i < 15; ++i) {
    p.k_thr[i] = i + 1 < (1 << kc.planes) ? kc.thresholds[i] : 0.f;
    p.v_thr[i] = i + 1 < (1 << vc.planes) ? vc.thresholds[i] : 0.f;
  }
  for (int i = 0; i < 16; ++i) {
    p.k_cen[i] = i < (1 << kc.planes) ? kc.centroids[i] : 0.f;
    p.v_cen[i] = i < (1 << vc.planes) ? vc.centroids[i] : 0.f;
  }
  p.k_codes = (uint32_t*)a.k_codes;
  p.k_signs = (uint32_t*)a.k_signs;
  p.k_norms = a.k_norms;
  p.k_rnorms = a.k_rnorms;
  p.v_codes = (uint32_t*)a.v_codes;
  p.v_norms = a.v_norms;
  const dim3 grid((unsigned)(a.batch * a.n_kv_heads), 2);
  return dispatch_dim(a.d, [&](auto dc) {
    constexpr int D = decltype(dc)::value;
    hipLaunchKernelGGL((append_kernel<D>), grid, dim3(kThreads), 0, stream, p);
    return launch_check("append");
  });
}

}  // namespace tq
