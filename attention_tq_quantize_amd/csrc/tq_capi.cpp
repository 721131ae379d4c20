// C ABI: argument validation, error reporting, quantizer handles.
// What each call computes is documented in include/tq.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "tq_internal.h"

namespace tq {

static thread_local std::string g_last_error;

tq_status set_error(tq_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

tq_status check_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return TQ_OK;
  std::string m = std::string(what) + ": " + hipGetErrorString(e);
  if (e == hipErrorOutOfMemory) return set_error(TQ_ERR_NO_MEMORY, m);
  return set_error(TQ_ERR_DEVICE, m);
}

namespace {

std::string fmt(const char* f, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, f);
  vsnprintf(buf, sizeof buf, f, ap);
  va_end(ap);
  return buf;
}

bool gpu_dim(int d) { return d == 64 || d == 128 || d == 256; }
bool misaligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) != 0; }
// head dimensions served by the generic kernels (quantize in the vector layout,
// inner products, channel splits): multiples of 32 up to 4096 other than 64,
// 128 and 256 (vector search at d = 1536 / 3072, the 32 / 96 channel parts of
// an outlier split)
bool large_dim(int d) { return d >= 32 && d <= 4096 && d % 32 == 0 && !gpu_dim(d); }

uint16_t bf16_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  uint32_t r = u + 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(r >> 16);
}

float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// MFMA fragments of a d x d matrix M for v_mfma_f32_16x16x32_bf16, as used by
// the quantize kernel: for output tile q, k-step ks and lane l = m + 16 g, the
// eight bf16 values M[row][col + i], row = (d/4)(m/4) + 4q + (m%4),
// col = (d/4) g + 8 ks. Stored [hilo][q][ks][lane][8]; hi = bf16(M),
// lo = bf16(M - hi).
void build_fragments(int d, const double* M, uint16_t* out) {
  const int nq = d / 16, nk = d / 32;
  const size_t per = (size_t)nq * nk * 64 * 8;
  for (int q = 0; q < nq; ++q)
    for (int ks = 0; ks < nk; ++ks)
      for (int l = 0; l < 64; ++l)
        for (int i = 0; i < 8; ++i) {
          const int m = l % 16, g = l / 16;
          const int row = (d / 4) * (m / 4) + 4 * q + (m % 4);
          const int col = (d / 4) * g + 8 * ks + i;
          const float v = (float)M[(size_t)row * d + col];
          const uint16_t hi = bf16_rne(v);
          const uint16_t lo = bf16_rne(v - bf16_to_f32(hi));
          const size_t off = (((size_t)q * nk + ks) * 64 + l) * 8 + i;
          out[off] = hi;
          out[per + off] = lo;
        }
}

}  // namespace
}  // namespace tq

using namespace tq;

extern "C" {

const char* tq_status_string(tq_status s) {
  switch (s) {
    case TQ_OK: return "ok";
    case TQ_ERR_INVALID_ARG: return "invalid argument";
    case TQ_ERR_UNSUPPORTED: return "unsupported";
    case TQ_ERR_NO_MEMORY: return "out of memory";
    case TQ_ERR_DEVICE: return "device error";
    case TQ_ERR_WORKSPACE: return "workspace too small";
  }
  return "unknown status";
}

const char* tq_last_error_message(void) { return g_last_error.c_str(); }

int tq_version(void) { return 2 * 10000 + 0 * 100 + 0; }

tq_status tq_codebook_build(int d, int bits, float* centroids, float* thresholds,
                            double* cost_per_coord) {
  if (d < 3 || d > 4096) return set_error(TQ_ERR_INVALID_ARG, fmt("codebook: d=%d outside [3, 4096]", d));
  if (bits < 0 || bits > 8) return set_error(TQ_ERR_INVALID_ARG, fmt("codebook: bits=%d outside [0, 8]", bits));
  if (!centroids) return set_error(TQ_ERR_INVALID_ARG, "codebook: centroids is NULL");
  const Codebook* cb = nullptr;
  tq_status st = get_codebook(d, bits, &cb);
  if (st != TQ_OK) return st;
  const int K = 1 << bits;
  std::memcpy(centroids, cb->centroids, sizeof(float) * K);
  if (thresholds && K > 1) std::memcpy(thresholds, cb->thresholds, sizeof(float) * (K - 1));
  if (cost_per_coord) *cost_per_coord = cb->cost;
  g_last_error.clear();
  return TQ_OK;
}

tq_status tq_quantizer_create(int d, int bits, tq_variant variant, const double* pi,
                              const double* s, tq_quantizer** out) {
  if (!out) return set_error(TQ_ERR_INVALID_ARG, "create: out is NULL");
  *out = nullptr;
  const bool large = large_dim(d);
  if (!gpu_dim(d) && !large)
    return set_error(TQ_ERR_UNSUPPORTED, fmt("create: d=%d (supported: 64, 128, 256; other multiples of 32 up to 4096 for quantize, inner products, search and channel splits)", d));
  if (bits < 1 || bits > kMaxBits) return set_error(TQ_ERR_UNSUPPORTED, fmt("create: bits=%d (supported: 1..4)", bits));
  if (variant != TQ_MSE && variant != TQ_PROD) return set_error(TQ_ERR_INVALID_ARG, "create: unknown variant");
  if (!pi) return set_error(TQ_ERR_INVALID_ARG, "create: pi is NULL");
  if (variant == TQ_PROD && !s) return set_error(TQ_ERR_INVALID_ARG, "create: prod needs the QJL matrix s");
  // Pi must be orthogonal (rows orthonormal) for Q^-1 = Pi^T to invert the rotation.
  double worst = 0.0;
  for (size_t i = 0; i < (size_t)d * d; ++i)
    if (!std::isfinite(pi[i])) return set_error(TQ_ERR_INVALID_ARG, "create: pi is not finite");
  if (!large) {
    for (int i = 0; i < d; ++i)
      for (int j = i; j < d; ++j) {
        double acc = 0.0;
        for (int k = 0; k < d; ++k) acc += pi[(size_t)i * d + k] * pi[(size_t)j * d + k];
        worst = std::fmax(worst, std::fabs(acc - (i == j ? 1.0 : 0.0)));
      }
  } else {
    // O(d^2) check instead of the O(d^3) Gram matrix: Pi^T Pi v = v for a few
    // fixed pseudo-random v (a matrix that is not orthogonal fails it for almost any v)
    std::vector<double> v(d), w(d), z(d);
    uint32_t st = 12345u;
    for (int rep = 0; rep < 4; ++rep) {
      for (int j = 0; j < d; ++j) {
        st = st * 1664525u + 1013904223u;
        v[j] = (double)(st >> 8) / 16777216.0 - 0.5;
      }
      for (int i = 0; i < d; ++i) {
        double acc = 0.0;
        for (int k = 0; k < d; ++k) acc += pi[(size_t)i * d + k] * v[k];
        w[i] = acc;
      }
      double nv = 0.0;
      for (int j = 0; j < d; ++j) {
        double acc = 0.0;
        for (int i = 0; i < d; ++i) acc += pi[(size_t)i * d + j] * w[i];
        z[j] = acc;
        nv = std::fmax(nv, std::fabs(v[j]));
      }
      for (int j = 0; j < d; ++j) worst = std::fmax(worst, std::fabs(z[j] - v[j]) / nv);
    }
  }
  if (worst > 1e-6) return set_error(TQ_ERR_INVALID_ARG, fmt("create: pi is not orthogonal (max |Pi Pi^T - I| = %.3g)", worst));
  if (variant == TQ_PROD)
    for (size_t i = 0; i < (size_t)d * d; ++i)
      if (!std::isfinite(s[i])) return set_error(TQ_ERR_INVALID_ARG, "create: s is not finite");

  tq_quantizer* q = new (std::nothrow) tq_quantizer();
  if (!q) return set_error(TQ_ERR_NO_MEMORY, "create: out of host memory");
  q->d = d;
  q->bits = bits;
  q->variant = variant;
  q->planes = variant == TQ_PROD ? bits - 1 : bits;
  const Codebook* cb = nullptr;
  tq_status st = get_codebook(d, q->planes, &cb);
  if (st != TQ_OK) {
    delete q;
    return st;
  }
  q->cb = *cb;
  tq_status hs = check_hip(hipGetDevice(&q->device), "create: hipGetDevice");
  if (hs != TQ_OK) {
    delete q;
    return hs;
  }

  const size_t dd = (size_t)d * d;
  // large d: fp32 Pi and S only (the MFMA fragments serve the d = 64, 128, 256
  // kernels). S' = S Pi^T is folded up to d = 256 (it also serves channel-split
  // parts of such sizes); beyond, the O(d^3) fold would dominate creation time.
  const size_t frag_bytes = large ? 0 : 2 * dd * sizeof(uint16_t);  // hi + lo
  const bool prod = variant == TQ_PROD;
  const bool fold = prod && d <= 256;
  // fp32 Pi is followed by its column sums (Pi^T 1, d floats); fp32 S by its
  // column sums (S^T 1) and its largest row norm (rounded up), 4 floats: the
  // decode query prep takes sum_j (Pi q)_j = (Pi^T 1) q, sum_j (S q)_j = (S^T 1) q,
  // max_j |(Pi q)_j| <= |q| and max_j |(S q)_j| <= |q| max_i |S_i| from them
  const size_t pi_tail = (size_t)d * sizeof(float), s_tail = ((size_t)d + 4) * sizeof(float);
  const size_t total = frag_bytes * (prod ? 2 : 1) + dd * sizeof(float) * (prod ? (fold ? 3 : 2) : 1) + pi_tail +
                       (prod ? s_tail : 0);
  std::vector<unsigned char> host(total);
  size_t off = 0;
  if (!large) build_fragments(d, pi, (uint16_t*)(host.data() + off));
  const size_t off_pi_frag = off;
  off += frag_bytes;
  size_t off_sp_frag = 0;
  std::vector<double> sp;
  if (fold) {
    // S' = S Pi^T, folded in fp64, so that S r = S' (Pi u - y~): the residual never
    // leaves the rotated space.
    sp.assign(dd, 0.0);
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < d; ++j) {
        double acc = 0.0;
        for (int k = 0; k < d; ++k) acc += s[(size_t)i * d + k] * pi[(size_t)j * d + k];
        sp[(size_t)i * d + j] = acc;
      }
  }
  if (prod && !large) {
    build_fragments(d, sp.data(), (uint16_t*)(host.data() + off));
    off_sp_frag = off;
    off += frag_bytes;
  }
  const size_t off_pi32 = off;
  for (size_t i = 0; i < dd; ++i) ((float*)(host.data() + off))[i] = (float)pi[i];
  off += dd * sizeof(float);
  for (int j = 0; j < d; ++j) {
    double acc = 0.0;
    for (int i = 0; i < d; ++i) acc += pi[(size_t)i * d + j];
    ((float*)(host.data() + off))[j] = (float)acc;
  }
  off += pi_tail;
  size_t off_s32 = 0, off_sp32 = 0;
  if (prod) {
    off_s32 = off;
    for (size_t i = 0; i < dd; ++i) ((float*)(host.data() + off))[i] = (float)s[i];
    off += dd * sizeof(float);
    float* tail = (float*)(host.data() + off);
    double rmax = 0.0;
    for (int j = 0; j < d; ++j) {
      double acc = 0.0, rn = 0.0;
      for (int i = 0; i < d; ++i) {
        acc += s[(size_t)i * d + j];
        rn += s[(size_t)j * d + i] * s[(size_t)j * d + i];
      }
      tail[j] = (float)acc;
      rmax = std::fmax(rmax, std::sqrt(rn));
    }
    tail[d] = (float)(rmax * (1.0 + 0x1p-20));
    tail[d + 1] = tail[d + 2] = tail[d + 3] = 0.0f;
    off += s_tail;
    if (fold) {
      off_sp32 = off;
      for (size_t i = 0; i < dd; ++i) ((float*)(host.data() + off))[i] = (float)sp[i];
      off += dd * sizeof(float);
    }
  }
  hs = check_hip(hipMalloc(&q->dev_block, total), "create: hipMalloc");
  if (hs != TQ_OK) {
    delete q;
    return hs;
  }
  hs = check_hip(hipMemcpy(q->dev_block, host.data(), total, hipMemcpyHostToDevice), "create: hipMemcpy");
  if (hs != TQ_OK) {
    (void)hipFree(q->dev_block);
    delete q;
    return hs;
  }
  unsigned char* base = (unsigned char*)q->dev_block;
  q->pi_frag = large ? nullptr : (const uint16_t*)(base + off_pi_frag);
  q->sp_frag = prod && !large ? (const uint16_t*)(base + off_sp_frag) : nullptr;
  q->pi32 = (const float*)(base + off_pi32);
  q->s32 = prod ? (const float*)(base + off_s32) : nullptr;
  q->sp32 = fold ? (const float*)(base + off_sp32) : nullptr;
  if (large) {
    hs = build_large_tables(q);
    if (hs != TQ_OK) {
      if (q->lq_block) (void)hipFree(q->lq_block);
      (void)hipFree(q->dev_block);
      delete q;
      return hs;
    }
  }
  *out = q;
  g_last_error.clear();
  return TQ_OK;
}

tq_status tq_quantizer_create_wht(int d, int bits, tq_variant variant, const double* signs,
                                  const double* s, tq_quantizer** out) {
  if (!out) return set_error(TQ_ERR_INVALID_ARG, "create_wht: out is NULL");
  *out = nullptr;
  if (!signs) return set_error(TQ_ERR_INVALID_ARG, "create_wht: signs is NULL");
  if (!gpu_dim(d) && !(large_dim(d) && (d & (d - 1)) == 0))
    return set_error(TQ_ERR_UNSUPPORTED, fmt("create_wht: d=%d (a supported power of two)", d));
  for (int j = 0; j < d; ++j)
    if (signs[j] != 1.0 && signs[j] != -1.0)
      return set_error(TQ_ERR_INVALID_ARG, fmt("create_wht: signs[%d] is not +-1", j));
  // Sylvester doubling: H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]
  std::vector<double> h((size_t)d * d, 0.0);
  h[0] = 1.0;
  for (int n = 1; n < d; n *= 2)
    for (int i = 0; i < n; ++i)
      for (int j = 0; j < n; ++j) {
        const double v = h[(size_t)i * d + j];
        h[(size_t)i * d + j + n] = v;
        h[(size_t)(i + n) * d + j] = v;
        h[(size_t)(i + n) * d + j + n] = -v;
      }
  const double inv = 1.0 / std::sqrt((double)d);
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) h[(size_t)i * d + j] *= signs[j] * inv;
  return tq_quantizer_create(d, bits, variant, h.data(), s, out);
}

tq_status tq_quantizer_destroy(tq_quantizer* q) {
  if (!q) return set_error(TQ_ERR_INVALID_ARG, "destroy: handle is NULL");
  tq_status st = TQ_OK;
  if (q->dev_block) st = check_hip(hipFree(q->dev_block), "destroy: hipFree");
  if (q->lq_block) {
    tq_status s2 = check_hip(hipFree(q->lq_block), "destroy: hipFree");
    if (st == TQ_OK) st = s2;
  }
  delete q;
  return st;
}

tq_status tq_quantizer_sizes(const tq_quantizer* q, size_t* code_bytes, size_t* sign_bytes) {
  if (!q) return set_error(TQ_ERR_INVALID_ARG, "sizes: handle is NULL");
  if (code_bytes) *code_bytes = (size_t)q->planes * q->d / 8;
  if (sign_bytes) *sign_bytes = q->variant == TQ_PROD ? (size_t)q->d / 8 : 0;
  return TQ_OK;
}

tq_status tq_quantizer_info(const tq_quantizer* q, int* d, int* bits, tq_variant* variant,
                            int* code_planes) {
  if (!q) return set_error(TQ_ERR_INVALID_ARG, "info: handle is NULL");
  if (d) *d = q->d;
  if (bits) *bits = q->bits;
  if (variant) *variant = q->variant;
  if (code_planes) *code_planes = q->planes;
  return TQ_OK;
}

// Argument checks of a quantize call; on TQ_OK *a describes the launch
// (n_per_group == 0 passes with nothing to launch).
static tq_status quantize_check(const tq_quantizer* const* qz, int n_groups, int64_t n_per_group,
                                const void* x, int64_t x_stride, tq_dtype x_dtype, tq_layout layout,
                                uint8_t* codes, uint8_t* signs, float* norms, float* rnorms, float* rot_dbg,
                                float* proj_dbg, QuantizeLaunch* a) {
  if (!qz) return set_error(TQ_ERR_INVALID_ARG, "quantize: qz is NULL");
  if (n_groups < 1) return set_error(TQ_ERR_INVALID_ARG, fmt("quantize: n_groups=%d < 1", n_groups));
  if (n_per_group < 0) return set_error(TQ_ERR_INVALID_ARG, "quantize: n_per_group < 0");
  const tq_quantizer* q0 = qz[0];
  if (!q0) return set_error(TQ_ERR_INVALID_ARG, "quantize: qz[0] is NULL");
  for (int g = 1; g < n_groups; ++g) {
    if (!qz[g]) return set_error(TQ_ERR_INVALID_ARG, fmt("quantize: qz[%d] is NULL", g));
    if (qz[g]->d != q0->d || qz[g]->bits != q0->bits || qz[g]->variant != q0->variant)
      return set_error(TQ_ERR_INVALID_ARG, "quantize: handles differ in (d, bits, variant)");
  }
  if (x_dtype != TQ_F32 && x_dtype != TQ_BF16) return set_error(TQ_ERR_INVALID_ARG, "quantize: unknown dtype");
  if (x_stride < q0->d) return set_error(TQ_ERR_INVALID_ARG, fmt("quantize: x_stride=%lld < d=%d", (long long)x_stride, q0->d));
  if ((x_stride * (x_dtype == TQ_F32 ? 4 : 2)) % 16)
    return set_error(TQ_ERR_INVALID_ARG, "quantize: x_stride must be a multiple of 16 bytes");
  if (layout != TQ_LAYOUT_VECTOR && layout != TQ_LAYOUT_BLOCK32) return set_error(TQ_ERR_INVALID_ARG, "quantize: unknown layout");
  if (layout == TQ_LAYOUT_BLOCK32) {
    if (q0->variant != TQ_MSE) return set_error(TQ_ERR_UNSUPPORTED, "quantize: BLOCK32 layout is for mse quantizers");
    if (n_per_group % kBlock) return set_error(TQ_ERR_INVALID_ARG, "quantize: BLOCK32 needs n_per_group % 32 == 0");
  }
  const bool prod = q0->variant == TQ_PROD;
  if (n_per_group == 0) {
    *a = QuantizeLaunch{qz, n_groups, 0, x, x_stride, x_dtype, layout, codes, signs, norms, rnorms, rot_dbg, proj_dbg};
    return TQ_OK;
  }
  if (!x) return set_error(TQ_ERR_INVALID_ARG, "quantize: x is NULL");
  if (q0->planes > 0 && !codes) return set_error(TQ_ERR_INVALID_ARG, "quantize: codes is NULL");
  if (!norms) return set_error(TQ_ERR_INVALID_ARG, "quantize: norms is NULL");
  if (prod && (!signs || !rnorms)) return set_error(TQ_ERR_INVALID_ARG, "quantize: prod needs signs and rnorms");
  if (!prod && proj_dbg) return set_error(TQ_ERR_INVALID_ARG, "quantize: proj_dbg is only for prod");
  if ((double)n_groups * (double)n_per_group > 4.0e9) return set_error(TQ_ERR_UNSUPPORTED, "quantize: more than 4e9 vectors");
  // the kernels load x in 16-byte vectors, store code and sign words and float4 debug rows
  if (misaligned(x, 16) || misaligned(codes, 4) || misaligned(signs, 4) || misaligned(rot_dbg, 16) ||
      misaligned(proj_dbg, 16))
    return set_error(TQ_ERR_INVALID_ARG, "quantize: x, rot_dbg and proj_dbg must be 16-byte aligned, codes and signs 4-byte aligned");
  *a = QuantizeLaunch{qz, n_groups, n_per_group, x, x_stride, x_dtype, layout, codes, signs, norms, rnorms, rot_dbg, proj_dbg};
  return TQ_OK;
}

static tq_status quantize_run(const QuantizeLaunch& a, void* stream) {
  if (a.n_per_group == 0) return TQ_OK;
  if (large_dim(a.qz[0]->d)) return launch_quantize_large(a, (hipStream_t)stream);
  return launch_quantize(a, (hipStream_t)stream);
}

static tq_status quantize_impl(const tq_quantizer* const* qz, int n_groups, int64_t n_per_group,
                               const void* x, int64_t x_stride, tq_dtype x_dtype, tq_layout layout,
                               uint8_t* codes, uint8_t* signs, float* norms, float* rnorms, float* rot_dbg,
                               float* proj_dbg, void* stream) {
  QuantizeLaunch a{};
  tq_status st = quantize_check(qz, n_groups, n_per_group, x, x_stride, x_dtype, layout, codes, signs, norms, rnorms,
                                rot_dbg, proj_dbg, &a);
  if (st != TQ_OK) return st;
  return quantize_run(a, stream);
}

tq_status tq_quantize_kv(const tq_quantizer* const* kqz, const tq_quantizer* const* vqz, int n_groups,
                         int64_t n_per_group, const void* xk, const void* xv, tq_dtype x_dtype, uint8_t* kcodes,
                         uint8_t* ksigns, float* knorms, float* krnorms, uint8_t* vcodes, float* vnorms,
                         void* stream) {
  if (!kqz || !kqz[0] || !vqz || !vqz[0]) return set_error(TQ_ERR_INVALID_ARG, "quantize_kv: kqz or vqz is NULL");
  if (vqz[0]->variant != TQ_MSE) return set_error(TQ_ERR_INVALID_ARG, "quantize_kv: value quantizers must be TQ_MSE");
  QuantizeLaunch k{}, v{};
  tq_status st = quantize_check(kqz, n_groups, n_per_group, xk, kqz[0]->d, x_dtype, TQ_LAYOUT_VECTOR, kcodes, ksigns,
                                knorms, krnorms, nullptr, nullptr, &k);
  if (st != TQ_OK) return st;
  st = quantize_check(vqz, n_groups, n_per_group, xv, vqz[0]->d, x_dtype, TQ_LAYOUT_BLOCK32, vcodes, nullptr, vnorms,
                      nullptr, nullptr, nullptr, &v);
  if (st != TQ_OK) return st;
  if (n_per_group == 0) return TQ_OK;
  if (quantize_kv_fusable(k, v)) return launch_quantize_kv(k, v, (hipStream_t)stream);
  st = quantize_run(k, stream);
  if (st != TQ_OK) return st;
  return quantize_run(v, stream);
}

tq_status tq_quantize(const tq_quantizer* const* qz, int n_groups, int64_t n_per_group,
                      const void* x, tq_dtype x_dtype, tq_layout layout, uint8_t* codes,
                      uint8_t* signs, float* norms, float* rnorms, float* rot_dbg,
                      float* proj_dbg, void* stream) {
  if (!qz || !qz[0]) return set_error(TQ_ERR_INVALID_ARG, "quantize: qz is NULL");
  return quantize_impl(qz, n_groups, n_per_group, x, qz[0]->d, x_dtype, layout, codes, signs, norms, rnorms,
                       rot_dbg, proj_dbg, stream);
}

tq_status tq_quantize_mse(const tq_quantizer* q, const void* x, tq_dtype x_dtype, int64_t n, int64_t x_stride,
                          uint8_t* codes, float* norms, float* rot_dbg, void* stream) {
  if (!q) return set_error(TQ_ERR_INVALID_ARG, "quantize_mse: handle is NULL");
  if (q->variant != TQ_MSE) return set_error(TQ_ERR_INVALID_ARG, "quantize_mse: handle is not TQ_MSE");
  return quantize_impl(&q, 1, n, x, x_stride, x_dtype, TQ_LAYOUT_VECTOR, codes, nullptr, norms, nullptr, rot_dbg,
                       nullptr, stream);
}

tq_status tq_quantize_prod(const tq_quantizer* q, const void* x, tq_dtype x_dtype, int64_t n, int64_t x_stride,
                           uint8_t* codes, uint8_t* signs, float* norms, float* rnorms,
                           float* rot_dbg, float* proj_dbg, void* stream) {
  if (!q) return set_error(TQ_ERR_INVALID_ARG, "quantize_prod: handle is NULL");
  if (q->variant != TQ_PROD) return set_error(TQ_ERR_INVALID_ARG, "quantize_prod: handle is not TQ_PROD");
  return quantize_impl(&q, 1, n, x, x_stride, x_dtype, TQ_LAYOUT_VECTOR, codes, signs, norms, rnorms, rot_dbg,
                       proj_dbg, stream);
}

tq_status tq_dequantize(const tq_quantizer* q, tq_layout layout, const uint8_t* codes,
                        const uint8_t* signs, const float* norms, const float* rnorms, int64_t n,
                        float* x_out, void* stream) {
  if (!q) return set_error(TQ_ERR_INVALID_ARG, "dequantize: handle is NULL");
  if (n < 0) return set_error(TQ_ERR_INVALID_ARG, "dequantize: n < 0");
  if (large_dim(q->d)) return set_error(TQ_ERR_UNSUPPORTED, "dequantize: d > 256 (quantize and inner products only)");
  if (layout != TQ_LAYOUT_VECTOR && layout != TQ_LAYOUT_BLOCK32) return set_error(TQ_ERR_INVALID_ARG, "dequantize: unknown layout");
  if (layout == TQ_LAYOUT_BLOCK32) {
    if (q->variant != TQ_MSE) return set_error(TQ_ERR_UNSUPPORTED, "dequantize: BLOCK32 layout is for mse quantizers");
    if (n % kBlock) return set_error(TQ_ERR_INVALID_ARG, "dequantize: BLOCK32 needs n % 32 == 0");
  }
  if (n == 0) return TQ_OK;
  if ((q->planes > 0 && !codes) || !norms || !x_out) return set_error(TQ_ERR_INVALID_ARG, "dequantize: NULL buffer");
  if (q->variant == TQ_PROD && (!signs || !rnorms)) return set_error(TQ_ERR_INVALID_ARG, "dequantize: prod needs signs and rnorms");
  if (n > (int64_t)1 << 31) return set_error(TQ_ERR_UNSUPPORTED, "dequantize: n > 2^31");
  return launch_dequantize(q, layout, codes, signs, norms, rnorms, n, x_out, (hipStream_t)stream);
}

tq_status tq_inner_products(const tq_quantizer* q, const float* y, int64_t m, const uint8_t* codes,
                            const uint8_t* signs, const float* norms, const float* rnorms, int64_t n,
                            float* out, void* stream) {
  if (!q) return set_error(TQ_ERR_INVALID_ARG, "inner_products: handle is NULL");
  if (m < 0 || n < 0) return set_error(TQ_ERR_INVALID_ARG, "inner_products: negative size");
  if (m == 0 || n == 0) return TQ_OK;
  if (!y || (q->planes > 0 && !codes) || !norms || !out) return set_error(TQ_ERR_INVALID_ARG, "inner_products: NULL buffer");
  if (q->variant == TQ_PROD && (!signs || !rnorms)) return set_error(TQ_ERR_INVALID_ARG, "inner_products: prod needs signs and rnorms");
  if (m > 65535 || n > (int64_t)1 << 31) return set_error(TQ_ERR_UNSUPPORTED, "inner_products: m > 65535 or n > 2^31");
  if (large_dim(q->d))
    return launch_inner_products_large(q, y, m, codes, signs, norms, rnorms, n, out, (hipStream_t)stream);
  return launch_inner_products(q, y, m, codes, signs, norms, rnorms, n, out, (hipStream_t)stream);
}

tq_status tq_search_workspace_size(const tq_quantizer* q, int64_t m, size_t* bytes) {
  if (!q || !bytes) return set_error(TQ_ERR_INVALID_ARG, "search_workspace_size: NULL argument");
  if (m < 0) return set_error(TQ_ERR_INVALID_ARG, "search_workspace_size: negative m");
  SearchPlan pl;
  tq_status st = search_plan(q, m, &pl);
  if (st != TQ_OK) return st;
  *bytes = pl.total;
  return TQ_OK;
}

tq_status tq_search_scores(const tq_quantizer* q, const float* y, int64_t m, const uint8_t* codes,
                           const uint8_t* signs, const float* norms, const float* rnorms, int64_t n, float* out,
                           void* workspace, size_t ws_bytes, void* stream) {
  if (!q) return set_error(TQ_ERR_INVALID_ARG, "search: handle is NULL");
  if (m < 0 || n < 0) return set_error(TQ_ERR_INVALID_ARG, "search: negative size");
  SearchPlan pl;
  tq_status st = search_plan(q, m, &pl);
  if (st != TQ_OK) return st;
  if (m == 0 || n == 0) return TQ_OK;
  if (!y || (q->planes > 0 && !codes) || !norms || !out) return set_error(TQ_ERR_INVALID_ARG, "search: NULL buffer");
  if (q->variant == TQ_PROD && (!signs || !rnorms)) return set_error(TQ_ERR_INVALID_ARG, "search: prod needs signs and rnorms");
  if (misaligned(y, 16) || misaligned(codes, 4) || misaligned(signs, 4))
    return set_error(TQ_ERR_INVALID_ARG, "search: y must be 16-byte aligned, codes and signs 4-byte aligned");
  if (m > 65535 || n > (int64_t)1 << 31) return set_error(TQ_ERR_UNSUPPORTED, "search: m > 65535 or n > 2^31");
  const size_t need = pl.total;
  if (!workspace || ws_bytes < need)
    return set_error(TQ_ERR_WORKSPACE, fmt("search: workspace needs %zu bytes, got %zu", need, workspace ? ws_bytes : (size_t)0));
  return launch_search(q, y, m, codes, signs, norms, rnorms, n, out, workspace, (hipStream_t)stream);
}

// ---- outlier-channel split ([NIK] "Experiments": separate quantizers for outlier and ordinary channels) ----
// qz [n_parts][n_groups], channels [n_parts][n_groups][d_p]: the handles of a
// part share d, bits and variant; every group's lists are in range and repeat
// no channel. chan receives the lists, off[p] the start of part p's block.
static tq_status check_split(const tq_quantizer* const* qz, int n_parts, int n_groups, const int32_t* channels,
                             int dim, std::vector<uint16_t>* chan, std::vector<int64_t>* off) {
  if (!qz || !channels) return set_error(TQ_ERR_INVALID_ARG, "split: qz or channels is NULL");
  if (n_parts < 1 || n_parts > 8) return set_error(TQ_ERR_INVALID_ARG, "split: n_parts outside [1, 8]");
  if (n_groups < 1) return set_error(TQ_ERR_INVALID_ARG, "split: n_groups < 1");
  if (dim < 1 || dim > kSplitMaxDim) return set_error(TQ_ERR_UNSUPPORTED, fmt("split: dim=%d outside [1, %d]", dim, kSplitMaxDim));
  int total = 0;
  off->assign(n_parts + 1, 0);
  for (int p = 0; p < n_parts; ++p) {
    const tq_quantizer* q0 = qz[(size_t)p * n_groups];
    if (!q0) return set_error(TQ_ERR_INVALID_ARG, fmt("split: part %d handle is NULL", p));
    if (q0->planes > 4) return set_error(TQ_ERR_UNSUPPORTED, "split: planes");
    for (int g = 1; g < n_groups; ++g) {
      const tq_quantizer* qg = qz[(size_t)p * n_groups + g];
      if (!qg || qg->d != q0->d || qg->bits != q0->bits || qg->variant != q0->variant)
        return set_error(TQ_ERR_INVALID_ARG, fmt("split: part %d handles differ across groups", p));
    }
    total += q0->d;
    (*off)[p + 1] = (int64_t)n_groups * total;
  }
  if (total > dim) return set_error(TQ_ERR_INVALID_ARG, fmt("split: parts cover %d channels, the rows have %d", total, dim));
  chan->resize((size_t)n_groups * total);
  for (int g = 0; g < n_groups; ++g) {
    std::vector<char> seen(dim, 0);
    for (int p = 0; p < n_parts; ++p) {
      const int dp = qz[(size_t)p * n_groups]->d;
      for (int j = 0; j < dp; ++j) {
        const int64_t at = (*off)[p] + (int64_t)g * dp + j;
        const int c = channels[at];
        if (c < 0 || c >= dim)
          return set_error(TQ_ERR_INVALID_ARG, fmt("split: channels[%lld]=%d (part %d, group %d) outside [0, %d)",
                                                   (long long)at, c, p, g, dim));
        if (seen[c]) return set_error(TQ_ERR_INVALID_ARG, fmt("split: group %d lists channel %d twice", g, c));
        seen[c] = 1;
        (*chan)[at] = (uint16_t)c;
      }
    }
  }
  return TQ_OK;
}

tq_status tq_quantize_split(const tq_quantizer* const* qz, int n_parts, int n_groups, const int32_t* channels, int dim,
                            const void* x, tq_dtype x_dtype, int64_t n_per_group, tq_layout layout,
                            const tq_records* out, void* stream) {
  std::vector<uint16_t> chan;
  std::vector<int64_t> off;
  tq_status st = check_split(qz, n_parts, n_groups, channels, dim, &chan, &off);
  if (st != TQ_OK) return st;
  if (!out) return set_error(TQ_ERR_INVALID_ARG, "split: out is NULL");
  if (n_per_group < 0) return set_error(TQ_ERR_INVALID_ARG, "split: negative n_per_group");
  if (x_dtype != TQ_F32 && x_dtype != TQ_BF16) return set_error(TQ_ERR_INVALID_ARG, "split: x_dtype");
  if (layout != TQ_LAYOUT_VECTOR && layout != TQ_LAYOUT_BLOCK32) return set_error(TQ_ERR_INVALID_ARG, "split: layout");
  if (layout == TQ_LAYOUT_BLOCK32) {
    if (n_per_group % 32) return set_error(TQ_ERR_INVALID_ARG, "split: BLOCK32 needs n_per_group % 32 == 0");
    for (int p = 0; p < n_parts; ++p)
      if (qz[(size_t)p * n_groups]->variant != TQ_MSE)
        return set_error(TQ_ERR_UNSUPPORTED, fmt("split: BLOCK32 is for mse parts (part %d is prod)", p));
  }
  if (n_per_group == 0) return TQ_OK;
  if (!x) return set_error(TQ_ERR_INVALID_ARG, "split: x is NULL");
  if ((int64_t)n_groups * n_per_group > (int64_t)1 << 31)
    return set_error(TQ_ERR_UNSUPPORTED, "split: n_groups * n_per_group > 2^31");
  for (int p = 0; p < n_parts; ++p) {
    const tq_records& r = out[p];
    const tq_quantizer* q0 = qz[(size_t)p * n_groups];
    const bool prod = q0->variant == TQ_PROD;
    if (!r.norms || (q0->planes > 0 && !r.codes) || (prod && (!r.signs || !r.rnorms)))
      return set_error(TQ_ERR_INVALID_ARG, fmt("split: part %d output buffer is NULL", p));
    if (misaligned(r.codes, 4) || misaligned(r.signs, 4))
      return set_error(TQ_ERR_INVALID_ARG, fmt("split: part %d codes and signs must be 4-byte aligned", p));
  }
  const size_t esize = x_dtype == TQ_F32 ? 4 : 2;
  if (n_parts == 2 && quantize_split_fusable(dim, qz[0], qz[n_groups])) {
    // both parts of a 128-channel head in one pass over the rows
    return launch_quantize_split(qz, qz + n_groups, n_groups, n_per_group, chan.data() + off[0], chan.data() + off[1],
                                 x, x_dtype, layout == TQ_LAYOUT_BLOCK32, out[0], &out[1], (hipStream_t)stream);
  }
  for (int p = 0; p < n_parts; ++p) {
    const tq_records& r = out[p];
    const tq_quantizer* const* qp = qz + (size_t)p * n_groups;
    const int dp = qp[0]->d;
    const int64_t cb = (int64_t)qp[0]->planes * dp / 8;
    // the generic kernels write the VECTOR layout; BLOCK32 repacks each 32-record block in place
    auto finish = [&]() -> tq_status {
      if (layout != TQ_LAYOUT_BLOCK32) return TQ_OK;
      return launch_repack_block32(r.codes, (int64_t)n_groups * n_per_group / 32, qp[0]->planes, dp,
                                   (hipStream_t)stream);
    };
    if (quantize_split_fast(dim, qp[0])) {  // writes either layout itself
      st = launch_quantize_split(qp, nullptr, n_groups, n_per_group, chan.data() + off[p], nullptr, x, x_dtype,
                                 layout == TQ_LAYOUT_BLOCK32, r, nullptr, (hipStream_t)stream);
      if (st != TQ_OK) return st;
      continue;
    }
    // generic fp32 kernels: one launch per group
    for (int g = 0; g < n_groups; ++g) {
      const int64_t v0 = (int64_t)g * n_per_group;
      const tq_quantizer* one[1] = {qp[g]};
      auto at = [&](auto* base, int64_t per) { return base ? base + v0 * per : base; };
      QuantizeLaunch a{one, 1, n_per_group, (const char*)x + v0 * dim * esize, dim, x_dtype, TQ_LAYOUT_VECTOR,
                       at(r.codes, cb), at(r.signs, (int64_t)dp / 8), at(r.norms, 1), at(r.rnorms, 1),
                       at(r.rot_dbg, dp), at(r.proj_dbg, dp)};
      st = launch_quantize_fp32(a, chan.data() + off[p] + (size_t)g * dp, dim, (hipStream_t)stream);
      if (st != TQ_OK) return st;
    }
    st = finish();
    if (st != TQ_OK) return st;
  }
  return TQ_OK;
}

tq_status tq_inner_products_split(const tq_quantizer* const* qz, int n_parts, const int32_t* channels, int dim,
                                  const float* y, int64_t m, const tq_records* recs, int64_t n, float* out,
                                  void* stream) {
  std::vector<uint16_t> chan;
  std::vector<int64_t> off;
  tq_status st = check_split(qz, n_parts, 1, channels, dim, &chan, &off);
  if (st != TQ_OK) return st;
  if (m < 0 || n < 0) return set_error(TQ_ERR_INVALID_ARG, "split inner products: negative size");
  if (m == 0 || n == 0) return TQ_OK;
  if (!y || !recs || !out) return set_error(TQ_ERR_INVALID_ARG, "split inner products: NULL buffer");
  if (m > 65535 || n > (int64_t)1 << 31) return set_error(TQ_ERR_UNSUPPORTED, "split inner products: m > 65535 or n > 2^31");
  for (int p = 0; p < n_parts; ++p) {
    const tq_records& r = recs[p];
    const bool prod = qz[p]->variant == TQ_PROD;
    if (!r.norms || (qz[p]->planes > 0 && !r.codes) || (prod && (!r.signs || !r.rnorms)))
      return set_error(TQ_ERR_INVALID_ARG, fmt("split inner products: part %d record buffer is NULL", p));
  }
  for (int p = 0; p < n_parts; ++p) {
    const tq_records& r = recs[p];
    st = launch_inner_products_fp32(qz[p], y, dim, chan.data() + off[p], p > 0, m, r.codes, r.signs, r.norms, r.rnorms,
                                    n, out, (hipStream_t)stream);
    if (st != TQ_OK) return st;
  }
  return TQ_OK;
}

// ---- decode attention over split caches ----
struct SplitPlan {
  int n_splits = 1;
  int64_t split_tokens = 0;
  int dk = 0, dv = 0;
  size_t bytes = 0;
};

static tq_status check_split_side(const tq_split_cache* c, const tq_attn_shape* s, bool values, SplitSide* side,
                                  int* total) {
  const char* what = values ? "split decode (values)" : "split decode (keys)";
  if (!c || !c->qz || !c->channels || !c->rec) return set_error(TQ_ERR_INVALID_ARG, fmt("%s: NULL cache description", what));
  if (c->n_parts < 1 || c->n_parts > kSplitMaxParts)
    return set_error(TQ_ERR_UNSUPPORTED, fmt("%s: n_parts outside [1, %d]", what, kSplitMaxParts));
  side->n_parts = c->n_parts;
  side->qz = c->qz;
  side->channels = c->channels;
  int off = 0;
  for (int p = 0; p < c->n_parts; ++p) {
    const tq_quantizer* q0 = c->qz[p * s->n_kv_heads];
    if (!q0) return set_error(TQ_ERR_INVALID_ARG, fmt("%s: part %d handle is NULL", what, p));
    for (int g = 1; g < s->n_kv_heads; ++g) {
      const tq_quantizer* qg = c->qz[p * s->n_kv_heads + g];
      if (!qg || qg->d != q0->d || qg->bits != q0->bits || qg->variant != q0->variant)
        return set_error(TQ_ERR_INVALID_ARG, fmt("%s: part %d handles differ across KV heads", what, p));
    }
    if (q0->d % 32) return set_error(TQ_ERR_UNSUPPORTED, fmt("%s: part %d dimension %d is not a multiple of 32", what, p, q0->d));
    if (q0->planes > 4) return set_error(TQ_ERR_UNSUPPORTED, fmt("%s: part %d planes", what, p));
    if (values && q0->variant != TQ_MSE) return set_error(TQ_ERR_UNSUPPORTED, fmt("%s: value parts must be mse", what));
    const tq_records& r = c->rec[p];
    const bool qjl = q0->variant == TQ_PROD;
    if (!r.norms || (q0->planes > 0 && !r.codes) || (qjl && (!r.signs || !r.rnorms)))
      return set_error(TQ_ERR_INVALID_ARG, fmt("%s: part %d record buffer is NULL", what, p));
    if (misaligned(r.codes, 4) || misaligned(r.signs, 4))
      return set_error(TQ_ERR_INVALID_ARG, fmt("%s: part %d codes and signs must be 4-byte aligned", what, p));
    side->codes[p] = r.codes;
    side->signs[p] = r.signs;
    side->norms[p] = r.norms;
    side->rnorms[p] = r.rnorms;
    off += q0->d;
  }
  if (off > s->head_dim) return set_error(TQ_ERR_INVALID_ARG, fmt("%s: parts cover %d channels of %d", what, off, s->head_dim));
  // channels [n_parts][n_kv_heads][d_p]: every KV head's lists over the parts
  // are in range and repeat no channel
  for (int g = 0; g < s->n_kv_heads; ++g) {
    std::vector<char> seen(s->head_dim, 0);
    int po = 0;
    for (int p = 0; p < c->n_parts; ++p) {
      const int dp = c->qz[p * s->n_kv_heads]->d;
      for (int j = 0; j < dp; ++j) {
        const int64_t at = (int64_t)s->n_kv_heads * po + (int64_t)g * dp + j;
        const int ch = c->channels[at];
        if (ch < 0 || ch >= s->head_dim)
          return set_error(TQ_ERR_INVALID_ARG, fmt("%s: channels[%lld]=%d (part %d, KV head %d) out of range", what,
                                                   (long long)at, ch, p, g));
        if (seen[ch])
          return set_error(TQ_ERR_INVALID_ARG, fmt("%s: KV head %d lists channel %d twice", what, g, ch));
        seen[ch] = 1;
      }
      po += dp;
    }
  }
  *total = off;
  return TQ_OK;
}

static tq_status plan_split_decode(const tq_attn_shape* s, const tq_split_cache* k, const tq_split_cache* v,
                                   SplitDecodeLaunch* L, SplitPlan* plan) {
  if (!s) return set_error(TQ_ERR_INVALID_ARG, "split decode: shape is NULL");
  if (s->batch < 1 || s->n_q_heads < 1 || s->n_kv_heads < 1 || s->max_ctx < 1)
    return set_error(TQ_ERR_INVALID_ARG, "split decode: empty shape");
  if (s->n_kv_heads > kSplitMaxKv) return set_error(TQ_ERR_UNSUPPORTED, fmt("split decode: more than %d KV heads", kSplitMaxKv));
  if (s->n_q_heads % s->n_kv_heads || s->n_q_heads / s->n_kv_heads > kSplitMaxGroup)
    return set_error(TQ_ERR_UNSUPPORTED, fmt("split decode: query heads per KV head must divide and be at most %d", kSplitMaxGroup));
  if (s->head_dim < 16 || s->head_dim > kSplitMaxDecodeDim)
    return set_error(TQ_ERR_UNSUPPORTED, fmt("split decode: head_dim outside [16, %d]", kSplitMaxDecodeDim));
  if (s->max_ctx > ((int64_t)1 << 31)) return set_error(TQ_ERR_UNSUPPORTED, "split decode: max_ctx > 2^31");
  if (s->max_ctx % 32)
    return set_error(TQ_ERR_INVALID_ARG, "split decode: max_ctx % 32 != 0 (value codes are in blocks of 32 tokens)");
  tq_status st = check_split_side(k, s, false, &L->k, &plan->dk);
  if (st != TQ_OK) return st;
  st = check_split_side(v, s, true, &L->v, &plan->dv);
  if (st != TQ_OK) return st;
  L->B = s->batch;
  L->Hq = s->n_q_heads;
  L->Hkv = s->n_kv_heads;
  L->dim = s->head_dim;
  L->max_ctx = s->max_ctx;
  // one wave per context split, as many splits as waves fit on the device at
  // once (a single round), splits a multiple of 32 tokens
  const int64_t bg = (int64_t)s->batch * s->n_kv_heads;
  int64_t ns = split_decode_resident_waves(*L) / bg;
  const int64_t chunks = (s->max_ctx + 31) / 32;
  if (ns > chunks) ns = chunks;
  if (ns < 1) ns = 1;
  int64_t per = (s->max_ctx + ns - 1) / ns;
  per = (per + 31) / 32 * 32;
  ns = (s->max_ctx + per - 1) / per;
  if (ns > 65535) return set_error(TQ_ERR_UNSUPPORTED, "split decode: too many splits");
  plan->n_splits = (int)ns;
  plan->split_tokens = per;
  L->n_splits = plan->n_splits;
  L->split_tokens = per;
  plan->bytes = split_decode_workspace_bytes(*L, plan->dk, plan->dv);
  return TQ_OK;
}

tq_status tq_decode_split_workspace_size(const tq_attn_shape* shape, const tq_split_cache* k, const tq_split_cache* v,
                                         size_t* bytes) {
  if (!bytes) return set_error(TQ_ERR_INVALID_ARG, "split decode workspace: bytes is NULL");
  SplitDecodeLaunch L{};
  SplitPlan plan;
  tq_status st = plan_split_decode(shape, k, v, &L, &plan);
  if (st != TQ_OK) return st;
  *bytes = plan.bytes;
  return TQ_OK;
}

tq_status tq_decode_attention_split(const tq_attn_shape* shape, const void* q, const tq_split_cache* k,
                                    const tq_split_cache* v, const int32_t* ctx_lens, float scale, float* out,
                                    void* workspace, size_t ws_bytes, void* stream) {
  SplitDecodeLaunch L{};
  SplitPlan plan;
  tq_status st = plan_split_decode(shape, k, v, &L, &plan);
  if (st != TQ_OK) return st;
  if (!q || !ctx_lens || !out) return set_error(TQ_ERR_INVALID_ARG, "split decode: q, ctx_lens or out is NULL");
  if (!std::isfinite(scale)) return set_error(TQ_ERR_INVALID_ARG, "split decode: scale is not finite");
  if (!workspace || ws_bytes < plan.bytes)
    return set_error(TQ_ERR_WORKSPACE, fmt("split decode: workspace needs %zu bytes, got %zu", plan.bytes, workspace ? ws_bytes : (size_t)0));
  L.q = q;
  L.lens = ctx_lens;
  L.scale = scale;
  L.out = out;
  L.workspace = workspace;
  return launch_split_decode(L, (hipStream_t)stream);
}

static tq_status check_decode(const tq_attn_shape* s, const tq_packed_kv* k, const tq_packed_kv* v,
                              DecodePlan* plan) {
  if (!s || !k || !v) return set_error(TQ_ERR_INVALID_ARG, "decode: NULL shape or cache");
  if (s->batch < 1 || s->n_q_heads < 1 || s->n_kv_heads < 1)
    return set_error(TQ_ERR_INVALID_ARG, "decode: batch and head counts must be >= 1");
  if (s->n_kv_heads > kMaxKvHeads) return set_error(TQ_ERR_UNSUPPORTED, fmt("decode: n_kv_heads > %d", kMaxKvHeads));
  if (s->n_q_heads % s->n_kv_heads) return set_error(TQ_ERR_INVALID_ARG, "decode: n_q_heads % n_kv_heads != 0");
  const int group = s->n_q_heads / s->n_kv_heads;
  if (group > 8 && group % 8) return set_error(TQ_ERR_UNSUPPORTED, "decode: group size > 8 must be a multiple of 8");
  if (s->max_ctx < 32 || s->max_ctx % 32) return set_error(TQ_ERR_INVALID_ARG, "decode: max_ctx must be a positive multiple of 32");
  if (s->max_ctx > ((int64_t)1 << 30)) return set_error(TQ_ERR_UNSUPPORTED, "decode: max_ctx > 2^30");
  if (!k->qz || !v->qz) return set_error(TQ_ERR_INVALID_ARG, "decode: quantizer arrays are NULL");
  const tq_quantizer* k0 = k->qz[0];
  const tq_quantizer* v0 = v->qz[0];
  if (!k0 || !v0) return set_error(TQ_ERR_INVALID_ARG, "decode: NULL quantizer handle");
  if (k0->d != s->head_dim || v0->d != s->head_dim) return set_error(TQ_ERR_INVALID_ARG, "decode: head_dim differs from the quantizers' d");
  for (int h = 0; h < s->n_kv_heads; ++h) {
    const tq_quantizer* kh = k->qz[h];
    const tq_quantizer* vh = v->qz[h];
    if (!kh || !vh) return set_error(TQ_ERR_INVALID_ARG, fmt("decode: NULL handle for kv head %d", h));
    if (kh->d != k0->d || kh->bits != k0->bits || kh->variant != k0->variant)
      return set_error(TQ_ERR_INVALID_ARG, "decode: key handles differ in (d, bits, variant)");
    if (vh->d != v0->d || vh->bits != v0->bits || vh->variant != v0->variant)
      return set_error(TQ_ERR_INVALID_ARG, "decode: value handles differ in (d, bits, variant)");
  }
  if (v0->variant != TQ_MSE) return set_error(TQ_ERR_UNSUPPORTED, "decode: values must use TQ_MSE quantizers");
  if ((k0->planes > 0 && !k->codes) || !k->norms) return set_error(TQ_ERR_INVALID_ARG, "decode: key cache buffers are NULL");
  if (k0->variant == TQ_PROD && (!k->signs || !k->rnorms)) return set_error(TQ_ERR_INVALID_ARG, "decode: prod keys need signs and rnorms");
  if (!v->codes || !v->norms) return set_error(TQ_ERR_INVALID_ARG, "decode: value cache buffers are NULL");
  return plan_decode(s, k0, v0, plan);
}

tq_status tq_decode_workspace_size(const tq_attn_shape* shape, const tq_packed_kv* k,
                                   const tq_packed_kv* v, size_t* bytes) {
  if (!bytes) return set_error(TQ_ERR_INVALID_ARG, "decode_workspace_size: bytes is NULL");
  DecodePlan p;
  tq_status st = check_decode(shape, k, v, &p);
  if (st != TQ_OK) return st;
  *bytes = p.total_bytes;
  return TQ_OK;
}

tq_status tq_decode_attention(const tq_attn_shape* shape, const void* q, const tq_packed_kv* k,
                              const tq_packed_kv* v, const int32_t* ctx_lens, float scale,
                              float* out, float* scores_dbg, void* workspace, size_t ws_bytes,
                              void* stream) {
  DecodePlan p;
  tq_status st = check_decode(shape, k, v, &p);
  if (st != TQ_OK) return st;
  if (!q || !ctx_lens || !out) return set_error(TQ_ERR_INVALID_ARG, "decode: q, ctx_lens or out is NULL");
  if (!std::isfinite(scale)) return set_error(TQ_ERR_INVALID_ARG, "decode: scale is not finite");
  if (!workspace || ws_bytes < p.total_bytes)
    return set_error(TQ_ERR_WORKSPACE, fmt("decode: workspace needs %zu bytes, got %zu", p.total_bytes, workspace ? ws_bytes : (size_t)0));
  return launch_decode(p, q, k, v, ctx_lens, scale, out, scores_dbg, workspace, (hipStream_t)stream);
}

tq_status tq_decode_attention_noalloc(const tq_attn_shape* shape, const void* q, const tq_packed_kv* k,
                                      const tq_packed_kv* v, const int32_t* ctx_lens, float scale,
                                      float* out, float* scores_dbg, void* stream) {
  DecodePlan p;
  tq_status st = check_decode(shape, k, v, &p);
  if (st != TQ_OK) return st;
  if (!q || !ctx_lens || !out) return set_error(TQ_ERR_INVALID_ARG, "decode_noalloc: q, ctx_lens or out is NULL");
  if (!std::isfinite(scale)) return set_error(TQ_ERR_INVALID_ARG, "decode_noalloc: scale is not finite");
  if (p.total_bytes > kNoAllocScratchBytes)
    return set_error(TQ_ERR_WORKSPACE, fmt("decode_noalloc: the call needs %zu bytes of scratch, the static scratch "
                                           "holds %zu; use tq_decode_attention with a workspace",
                                           p.total_bytes, kNoAllocScratchBytes));
  void* ws = nullptr;
  st = noalloc_scratch(&ws);
  if (st != TQ_OK) return st;
  return launch_decode(p, q, k, v, ctx_lens, scale, out, scores_dbg, ws, (hipStream_t)stream);
}

// Append workspace: the same as the plain decode's (the new records go straight
// into the caches; the attended length is formed in the main kernel)
static size_t append_workspace(const DecodePlan& p) { return p.total_bytes; }

tq_status tq_decode_append_workspace_size(const tq_attn_shape* shape, const tq_packed_kv* k,
                                          const tq_packed_kv* v, size_t* bytes) {
  if (!bytes) return set_error(TQ_ERR_INVALID_ARG, "decode_append_workspace_size: bytes is NULL");
  DecodePlan p;
  tq_status st = check_decode(shape, k, v, &p);
  if (st != TQ_OK) return st;
  *bytes = append_workspace(p);
  return TQ_OK;
}

tq_status tq_decode_append_attention(const tq_attn_shape* shape, const void* q, const void* k_new,
                                     const void* v_new, tq_dtype kv_dtype, const tq_packed_kv* k,
                                     const tq_packed_kv* v, const int32_t* ctx_lens, float scale,
                                     float* out, const tq_append_debug* dbg, void* workspace,
                                     size_t ws_bytes, void* stream) {
  DecodePlan p;
  tq_status st = check_decode(shape, k, v, &p);
  if (st != TQ_OK) return st;
  if (!q || !ctx_lens || !out) return set_error(TQ_ERR_INVALID_ARG, "decode_append: q, ctx_lens or out is NULL");
  if (!k_new || !v_new) return set_error(TQ_ERR_INVALID_ARG, "decode_append: k_new or v_new is NULL");
  if (kv_dtype != TQ_F32 && kv_dtype != TQ_BF16) return set_error(TQ_ERR_INVALID_ARG, "decode_append: unknown kv_dtype");
  if (!std::isfinite(scale)) return set_error(TQ_ERR_INVALID_ARG, "decode_append: scale is not finite");
  if (p.d > 256) return set_error(TQ_ERR_UNSUPPORTED, "decode_append: head_dim > 256");
  const size_t need = append_workspace(p);
  if (!workspace || ws_bytes < need)
    return set_error(TQ_ERR_WORKSPACE, fmt("decode_append: workspace needs %zu bytes, got %zu", need, workspace ? ws_bytes : (size_t)0));
  AppendLaunch a;
  a.k_new = k_new;
  a.v_new = v_new;
  a.x_dtype = kv_dtype;
  a.rot_dbg = dbg ? dbg->rot : nullptr;
  a.proj_dbg = dbg ? dbg->proj : nullptr;
  return launch_decode(p, q, k, v, ctx_lens, scale, out, nullptr, workspace, (hipStream_t)stream, &a);
}

}  // extern "C"
