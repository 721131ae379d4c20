// Decode-step append: the new token's key and value, already quantized into
// per-(batch, kv head) staging records in the vector layout, are written into
// the packed caches at each sequence's current length, and the lengths the
// attention then reads (length + 1, at most max_ctx) are written beside them.
// The quantization itself is the regular quantize kernel ([NIK] "Step 0" to
// "Step 2", and "TurboQuant proper" for prod keys); this file only moves bits.
#include <hip/hip_runtime.h>

#include "tq_device.h"

namespace tq {
namespace {

struct AppendParams {
  const int32_t* ctx_lens;  // [B] tokens already cached
  int32_t* lens_out;        // [B] tokens attended after the append
  int64_t max_ctx;
  int Hkv, d, k_planes, v_bits;
  bool k_prod;
  // staging, one record per group g = b * Hkv + h (vector layout)
  const uint32_t* sk_codes;  // [G][k_planes * d / 32]
  const uint32_t* sk_signs;  // [G][d / 32]
  const float* sk_norms;
  const float* sk_rnorms;
  const uint32_t* sv_codes;  // [G][v_bits * d / 32]
  const float* sv_norms;
  // caches
  uint32_t* k_codes;  // [B][Hkv][max_ctx][k_planes * d / 32]
  uint32_t* k_signs;  // [B][Hkv][max_ctx][d / 32]
  float* k_norms;
  float* k_rnorms;
  uint32_t* v_codes;  // [B][Hkv][max_ctx / 32][4 * v_bits * d / 4] (block layout)
  float* v_norms;
};

// One workgroup per (batch, kv head); a sequence whose cache is full
// (length >= max_ctx) is not appended and keeps attending max_ctx tokens.
__global__ __launch_bounds__(kThreads) void append_scatter_kernel(AppendParams p) {
  const int grp = blockIdx.x;
  const int b = grp / p.Hkv;
  const int tid = threadIdx.x;
  int64_t len = p.ctx_lens[b];
  len = len < 0 ? 0 : len;
  if (grp % p.Hkv == 0 && tid == 0) p.lens_out[b] = (int32_t)(len < p.max_ctx ? len + 1 : p.max_ctx);
  if (len >= p.max_ctx) return;
  const int64_t slot = (int64_t)grp * p.max_ctx + len;  // (b, h, t) record index
  const int kw = p.k_planes * p.d / 32, sw = p.d / 32;
  for (int i = tid; i < kw; i += kThreads) p.k_codes[slot * kw + i] = p.sk_codes[(int64_t)grp * kw + i];
  if (p.k_prod)
    for (int i = tid; i < sw; i += kThreads) p.k_signs[slot * sw + i] = p.sk_signs[(int64_t)grp * sw + i];
  if (tid == 0) {
    p.k_norms[slot] = p.sk_norms[grp];
    if (p.k_prod) p.k_rnorms[slot] = p.sk_rnorms[grp];
    p.v_norms[slot] = p.sv_norms[grp];
  }
  // value bits: slot v of block t / 32 is vector 4g + k (v < 16) or 16 + 4g + k;
  // plane p, coordinate 4w + r sits at bit 4r + k (+16) of word (p*4 + g)*(d/4) + w
  const int v = (int)(len % 32);
  const int hi = v >= 16 ? 16 : 0, g = (v % 16) / 4, k = v % 4;
  const unsigned keep = ~(0x1111u << (k + hi));
  const int wpp = p.d / 4;  // words per (plane, group)
  uint32_t* blk = p.v_codes + ((int64_t)grp * (p.max_ctx / 32) + len / 32) * (int64_t)(p.v_bits * p.d);
  const uint32_t* src = p.sv_codes + (int64_t)grp * (p.v_bits * p.d / 32);
  for (int i = tid; i < p.v_bits * wpp; i += kThreads) {
    const int pl = i / wpp, w = i % wpp;
    const uint32_t plane_word = src[pl * (p.d / 32) + (4 * w) / 32];
    const unsigned nib = (plane_word >> ((4 * w) % 32)) & 0xFu;  // coordinates 4w .. 4w+3
    unsigned bits = 0u;
#pragma unroll
    for (int r = 0; r < 4; ++r) bits |= ((nib >> r) & 1u) << (4 * r + k + hi);
    uint32_t* word = blk + (pl * 4 + g) * wpp + w;
    *word = (*word & keep) | bits;
  }
}

}  // namespace

tq_status launch_append_scatter(const AppendScatter& a, hipStream_t stream) {
  AppendParams p;
  p.ctx_lens = a.ctx_lens;
  p.lens_out = a.lens_out;
  p.max_ctx = a.max_ctx;
  p.Hkv = a.n_kv_heads;
  p.d = a.d;
  p.k_planes = a.k_planes;
  p.v_bits = a.v_bits;
  p.k_prod = a.k_prod;
  p.sk_codes = (const uint32_t*)a.sk_codes;
  p.sk_signs = (const uint32_t*)a.sk_signs;
  p.sk_norms = a.sk_norms;
  p.sk_rnorms = a.sk_rnorms;
  p.sv_codes = (const uint32_t*)a.sv_codes;
  p.sv_norms = a.sv_norms;
  p.k_codes = (uint32_t*)a.k_codes;
  p.k_signs = (uint32_t*)a.k_signs;
  p.k_norms = a.k_norms;
  p.k_rnorms = a.k_rnorms;
  p.v_codes = (uint32_t*)a.v_codes;
  p.v_norms = a.v_norms;
  hipLaunchKernelGGL(append_scatter_kernel, dim3((unsigned)(a.batch * a.n_kv_heads)), dim3(kThreads), 0, stream, p);
  return launch_check("append scatter");
}

}  // namespace tq
