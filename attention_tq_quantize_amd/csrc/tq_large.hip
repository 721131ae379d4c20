// Quantize, inner products and scoring for the head dimensions outside the
// d = 64 / 128 / 256 kernels: vector search (d = 1536, 3072; [NIK]
// "Experiments", nearest neighbours) and the parts of an outlier-channel split
// (d = 32, 96; [NIK] "Experiments", KV cache), following [NIK] "Step 0:
// normalization", "Step 1: random rotation", "Step 2: optimal scalar
// quantization", "QJL: a one-bit method" and "TurboQuant proper".
//
// Three families of kernels live here:
// * generic fp32 kernels for any d that is a multiple of 32 (with an optional
//   channel map for splits): a workgroup quantizes VB vectors at once, reading
//   each row of Pi (and S) once for all VB vectors, with the vectors in LDS;
//   the norm is accumulated in fp64;
// * the matrix-core GEMM quantize for d a multiple of 128 above 256;
// * the matrix-core scoring of a packed database (tq_search_scores).
#include <hip/hip_runtime.h>

#include "tq_device.h"

namespace tq {
namespace {

constexpr int kMaxSplitDim = 512;  // channel maps travel in the kernel arguments

struct LargeQuantParams {
  const void* x;
  int64_t x_stride;       // elements per input row (d, or the full width of a channel split)
  bool chan_map;          // coordinate j of the quantized vector is input channel chan[j]
  uint16_t chan[kMaxSplitDim];
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

// out[v][i] = sum_j M[i][j] in[v][j] for the workgroup's nv vectors. The work
// items are (row, group of VG vectors), spread over the threads so that small d
// still uses them all; each item reads its row once (float4) for its vectors.
template <int VB, int VG = VB>
__device__ void rows_times(const float* __restrict__ M, const float* in, float* out, int d, int nv) {
  static_assert(VB % VG == 0, "vector groups");
  for (int e = threadIdx.x; e < d * (VB / VG); e += kThreads) {
    const int i = e % d, g0 = (e / d) * VG;
    const float4* row = (const float4*)(M + (int64_t)i * d);
    float acc[VG];
#pragma unroll
    for (int v = 0; v < VG; ++v) acc[v] = 0.f;
    for (int j4 = 0; j4 < d / 4; ++j4) {
      const float4 m = row[j4];
#pragma unroll
      for (int v = 0; v < VG; ++v) {
        const float4 u = ((const float4*)(in + (size_t)(g0 + v) * d))[j4];
        acc[v] = fmaf(m.x, u.x, fmaf(m.y, u.y, fmaf(m.z, u.z, fmaf(m.w, u.w, acc[v]))));
      }
    }
#pragma unroll
    for (int v = 0; v < VG; ++v)
      if (g0 + v < nv) out[(size_t)(g0 + v) * d + i] = acc[v];
  }
}

// out[v][j] = sum_i M[i][j] in[v][i]: work items (column, group of VG vectors);
// consecutive threads read consecutive elements of a row
template <int VB, int VG = VB>
__device__ void cols_times(const float* __restrict__ M, const float* in, float* out, int d, int nv) {
  static_assert(VB % VG == 0, "vector groups");
  for (int e = threadIdx.x; e < d * (VB / VG); e += kThreads) {
    const int j = e % d, g0 = (e / d) * VG;
    float acc[VG];
#pragma unroll
    for (int v = 0; v < VG; ++v) acc[v] = 0.f;
    for (int i = 0; i < d; ++i) {
      const float m = M[(int64_t)i * d + j];
#pragma unroll
      for (int v = 0; v < VG; ++v) acc[v] = fmaf(m, in[(size_t)(g0 + v) * d + i], acc[v]);
    }
#pragma unroll
    for (int v = 0; v < VG; ++v)
      if (g0 + v < nv) out[(size_t)(g0 + v) * d + j] = acc[v];
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
  // ---- inputs of all the workgroup's vectors (every load in flight at once) ----
  for (int e = threadIdx.x; e < VB * d; e += kThreads) {
    const int v = e / d, j = e - v * d;
    float xv = 0.f;
    if (v < nv) {
      const int64_t src = (gbase + v0 + v) * prm.x_stride + (prm.chan_map ? prm.chan[j] : j);
      xv = prm.x_bf16 ? bf16_val(((const uint16_t*)prm.x)[src]) : ((const float*)prm.x)[src];
    }
    A[e] = xv;
  }
  __syncthreads();
  // ---- norms (fp64) and unit vectors ----
  for (int v = wave; v < VB; v += kThreads / 64) {
    double acc = 0.0;
    for (int j = lane; j < d; j += 64) {
      const float xv = A[(size_t)v * d + j];
      acc = fma((double)xv, (double)xv, acc);
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
  rows_times<VB, (VB < 8 ? VB : 8)>(pi, A, Bm, d, VB);
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
  cols_times<VB, (VB < 8 ? VB : 8)>(pi, Bm, A, d, VB);
  __syncthreads();
  rows_times<VB, (VB < 8 ? VB : 8)>(prm.s[grp], A, Bm, d, VB);  // Bm = p
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
  int64_t y_stride;       // elements per query row
  bool chan_map;          // coordinate j of the query is its channel chan[j]
  bool accumulate;        // add into out (the parts of a channel split)
  uint16_t chan[kMaxSplitDim];
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
  for (int j = threadIdx.x; j < d; j += kThreads) yq[j] = prm.y[qi * prm.y_stride + (prm.chan_map ? prm.chan[j] : j)];
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
    float* o = prm.out + qi * prm.n + v;
    *o = prm.accumulate ? *o + prm.norms[v] * r : prm.norms[v] * r;
  }
}


// ===========================================================================
// Scoring on the matrix cores (tq_search_scores): the key-side contraction of
// the decode kernel applied to a database. For a group of 8 queries the 16
// MFMA columns hold each query's rotated vector (hi, lo fp16 parts, one
// exponent per query); the records' bit planes are the other operand (shifted
// onto fp16 bits 8-11 and masked, bit_operand). With sigma = 2 bit - 1 and the
// odd Walsh expansion c[idx] = sum_s a_s prod_{i in s} sigma_i, a product over
// an odd subset being 2 xor(bits) - 1,
//   <y, x~> = |x| (sum_s 2 a_s <Pi y, xor_s> - (sum_s a_s) sum_j (Pi y)_j
//                  + |r| sqrt(pi/2)/d (2 <S y, z> - sum_j (S y)_j)),
// so a record is scored with (odd subsets + 1 sign plane) x d/32 MFMAs per
// 16 records and 16 columns, without unpacking.
// Coordinates: 32-bit word u of a plane holds coordinates 32u .. 32u+31 (LSB
// first); lane quarter g reads the words u = 4w + g, w < d/128, so the four
// quarters of a record read 16 contiguous bytes. Within the word, bit
// 16 half + 4 r + k is MFMA k-slot 2k + half of step r.
// Fragments: [query group][4 W + r][64 lanes] u32x4, W = s (d/128) + w for
// Walsh subset s (then the sign words, s = number of subsets).
// ===========================================================================
constexpr int kSearchConsts = 48;     // per query group: [0,16) mse init, [16,32) qjl init, [32,48) 2^(10-E)
constexpr int kSearchMaxFragKB = 144;  // LDS for one coordinate slice's fragments
constexpr int kSearchThreads = 512;

constexpr int kProjRows = 16;  // rows of Pi (or S) per projection workgroup

struct SearchProjParams {
  const float* y;
  int64_t m;
  int d;
  const float* pi;
  const float* s;
  float* qp;  // [groups * 8][d]: Pi y
  float* qq;  // [groups * 8][d]: S y
};

// grid (d / kProjRows, query groups, 1 + qjl): rows [i0, i0 + kProjRows) of Pi
// (z = 0) or S (z = 1) times the group's 8 queries, so each matrix is read once
// per query group, spread over the chip
__global__ __launch_bounds__(kThreads) void search_project_kernel(SearchProjParams prm) {
  extern __shared__ float4 ylds[];  // [8][d / 4]
  const int d = prm.d, d4 = d / 4;
  const int64_t qg = blockIdx.y;
  const int nq = (int)min((int64_t)8, prm.m - 8 * qg);
  for (int e = threadIdx.x; e < 8 * d4; e += kThreads) {
    const int h = e / d4, j = e % d4;
    ylds[e] = h < nq ? ((const float4*)(prm.y + (qg * 8 + h) * d))[j] : float4{0.f, 0.f, 0.f, 0.f};
  }
  __syncthreads();
  const float* M = blockIdx.z ? prm.s : prm.pi;
  float* out = blockIdx.z ? prm.qq : prm.qp;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int ri = wave; ri < kProjRows; ri += kThreads / 64) {
    const int i = blockIdx.x * kProjRows + ri;
    const float4* row = (const float4*)(M + (int64_t)i * d);
    float acc[8];
#pragma unroll
    for (int h = 0; h < 8; ++h) acc[h] = 0.f;
    for (int j = lane; j < d4; j += 64) {
      const float4 pv = row[j];
#pragma unroll
      for (int h = 0; h < 8; ++h) {
        const float4 yv = ylds[h * d4 + j];
        acc[h] = fmaf(pv.x, yv.x, fmaf(pv.y, yv.y, fmaf(pv.z, yv.z, fmaf(pv.w, yv.w, acc[h]))));
      }
    }
#pragma unroll
    for (int h = 0; h < 8; ++h) {
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) acc[h] += __shfl_xor(acc[h], o);
      if (lane == h && h < nq) out[(qg * 8 + h) * d + i] = acc[h];
    }
  }
}

struct SearchPrepParams {
  int64_t m;
  int d, wk, wpp;
  bool qjl;
  const float* qp;
  const float* qq;
  u32x4* frag;
  float* consts;
  int nf;
  float kappa;
  float kcoef[8];
};

// one workgroup per query: from q' = Pi y and q'' = S y, the query's fragment columns and constants
__global__ __launch_bounds__(kThreads) void search_prep_kernel(SearchPrepParams prm) {
  extern __shared__ float lds[];  // qp[d], qq[d]
  __shared__ float red[4][kThreads / 64];
  const int d = prm.d;
  float* qp = lds;
  float* qq = lds + d;
  const int64_t qi = blockIdx.x;
  const int64_t qg = qi / 8;
  const int h = (int)(qi % 8);
  const int nq = (int)min((int64_t)8, prm.m - 8 * qg);
  for (int j = threadIdx.x; j < d; j += kThreads) {
    qp[j] = prm.qp[qi * d + j];
    if (prm.qjl) qq[j] = prm.qq[qi * d + j];
  }
  __syncthreads();
  float sp = 0.f, sq = 0.f, mp = 0.f, mq = 0.f;
  for (int j = threadIdx.x; j < d; j += kThreads) {
    sp += qp[j];
    mp = fmaxf(mp, fabsf(qp[j]));
    if (prm.qjl) {
      sq += qq[j];
      mq = fmaxf(mq, fabsf(qq[j]));
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    sp += __shfl_xor(sp, o);
    sq += __shfl_xor(sq, o);
    mp = fmaxf(mp, __shfl_xor(mp, o));
    mq = fmaxf(mq, __shfl_xor(mq, o));
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[0][wave] = sp;
    red[1][wave] = sq;
    red[2][wave] = mp;
    red[3][wave] = mq;
  }
  __syncthreads();
  float sum_p = 0.f, sum_q = 0.f, max_p = 0.f, max_q = 0.f;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    sum_p += red[0][w];
    sum_q += red[1][w];
    max_p = fmaxf(max_p, red[2][w]);
    max_q = fmaxf(max_q, red[3][w]);
  }
  float amax = 0.f, asum = 0.f;
  for (int s = 0; s < prm.wk; ++s) {
    amax = fmaxf(amax, fabsf(prm.kcoef[s]));
    asum += prm.kcoef[s];
  }
  // one exponent for both terms: every fragment entry |v| 2^E < 1
  const int E = range_exp(fmaxf(2.f * amax * max_p, prm.qjl ? 2.f * prm.kappa * max_q : 0.f));
  float* cst = prm.consts + qg * kSearchConsts;
  if (threadIdx.x < 2) {
    const int row = 2 * h + threadIdx.x;  // hi column carries the constant, lo column 0
    cst[row] = threadIdx.x == 0 ? -asum * sum_p * ldexpf(1.0f, E - 10) : 0.f;
    cst[16 + row] = threadIdx.x == 0 && prm.qjl ? -prm.kappa * sum_q * ldexpf(1.0f, E - 10) : 0.f;
    cst[32 + row] = ldexpf(1.0f, 10 - E);
  }
  // the group's first query also fills the columns of absent queries (partial last group)
  if (h == 0 && nq < 8 && threadIdx.x >= 2 * nq && threadIdx.x < 16) {
    cst[threadIdx.x] = 0.f;
    cst[16 + threadIdx.x] = 0.f;
    cst[32 + threadIdx.x] = 1.f;
  }
  const int nwm = prm.wk * prm.wpp;
  u32x4* frag = prm.frag + qg * (int64_t)prm.nf * 64;
  for (int e = threadIdx.x; e < prm.nf * 8; e += kThreads) {
    const int f = e / 8, g = (e / 2) % 4, lo = e % 2;
    const int W = f / 4, r = f % 4;
    const int lane = 16 * g + 2 * h + lo;
    unsigned hv[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int k = it / 2, half = it % 2;
      const int beta = 16 * half + 4 * r + k;  // bit of the lane's word
      float val;
      if (W < nwm) {
        const int sub = W / prm.wpp, w = W % prm.wpp;
        val = 2.f * prm.kcoef[sub] * qp[32 * (4 * w + g) + beta];
      } else {
        const int w = W - nwm;
        val = 2.f * prm.kappa * qq[32 * (4 * w + g) + beta];
      }
      // the bit reads as 2^(operand_pos(k) - 24); raw scores come out x 2^(E - 10)
      val *= ldexpf(1.0f, E + 14 - operand_pos(k));
      hv[it] = f16_part(val, lo);
    }
    frag[(int64_t)f * 64 + lane] =
        u32x4{pack2(hv[0], hv[1]), pack2(hv[2], hv[3]), pack2(hv[4], hv[5]), pack2(hv[6], hv[7])};
  }
  if (h == 0 && nq < 8)
    for (int e = threadIdx.x; e < prm.nf * 64; e += kThreads)
      if ((e % 16) >= 2 * nq) frag[e] = u32x4{0u, 0u, 0u, 0u};
}

struct SearchParams {
  const u32x4* frag;
  const float* consts;
  const uint8_t* codes;
  const uint8_t* signs;
  const float* norms;
  const float* rnorms;
  float* out;
  int64_t n, m;
  int d, wpp, nf;
  int w0, ws;  // this launch scores word groups [w0, w0 + ws) of every record
  bool first;  // first slice: starts from the constants and writes (later slices add)
};

// Persistent workgroups of 8 waves; the slice's fragments sit in LDS; a wave
// scores 32 records (two 16-record tiles) per step for one group of 8 queries.
template <int PK, bool QJL>
__global__ __launch_bounds__(kSearchThreads, 1) void search_score_kernel(SearchParams prm) {
  extern __shared__ u32x4 sfrag[];
  constexpr int WK = n_walsh(PK);
  constexpr int NS = WK + (QJL ? 1 : 0);  // operand kinds per word: Walsh subsets, then signs
  constexpr int NW = kSearchThreads / 64;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int64_t qg = blockIdx.y;
  const int d = prm.d, wpp = prm.wpp, w0 = prm.w0, ws = prm.ws;
  {
    // local fragment 4 (s ws + w - w0) + r <- global 4 (s wpp + w) + r
    const u32x4* src = prm.frag + qg * (int64_t)prm.nf * 64;
    for (int e = threadIdx.x; e < NS * ws * 4 * 64; e += kSearchThreads) {
      const int fl = e / 64, ln = e % 64;
      const int Wl = fl / 4, r = fl % 4;
      const int W = (Wl / ws) * wpp + w0 + Wl % ws;
      sfrag[e] = src[(int64_t)(4 * W + r) * 64 + ln];
    }
  }
  __syncthreads();
  const float* cst = prm.consts + qg * kSearchConsts;
  const float cm0 = prm.first ? cst[r16] : 0.f;
  const float cq0 = prm.first ? cst[16 + r16] : 0.f;
  const float isc = cst[32 + r16];
  const int nq = (int)min((int64_t)8, prm.m - 8 * qg);
  const int h = r16 >> 1;
  const bool writer = !(r16 & 1) && h < nq;
  const int plane_bytes = d / 8;
  const int64_t n = prm.n;
  const int64_t steps = (n + 31) / 32;
  for (int64_t step = (int64_t)blockIdx.x * NW + wave; step < steps; step += (int64_t)gridDim.x * NW) {
    const int64_t v0 = step * 32;
    f32x4 cm[2], cq[2];
    const uint8_t* crec[2];
    const uint8_t* srec[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      cm[t] = f32x4{cm0, cm0, cm0, cm0};
      cq[t] = f32x4{cq0, cq0, cq0, cq0};
      const int64_t v = min(v0 + 16 * t + r16, n - 1);  // rows past the end repeat the last record
      crec[t] = prm.codes + v * (PK * plane_bytes) + 4 * g;
      srec[t] = QJL ? prm.signs + v * plane_bytes + 4 * g : nullptr;
    }
    for (int wl = 0; wl < ws; ++wl) {
      const int off = 16 * (w0 + wl);
      unsigned pw[2][PK > 0 ? PK : 1], sw[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int p = 0; p < PK; ++p) pw[t][p] = *(const unsigned*)(crec[t] + p * plane_bytes + off);
        if constexpr (QJL) sw[t] = *(const unsigned*)(srec[t] + off);
      }
#pragma unroll
      for (int sub = 0; sub < NS; ++sub) {
        unsigned word[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          if (sub < WK) {
            unsigned x = 0u;
#pragma unroll
            for (int p = 0; p < PK; ++p)
              if (walsh_mask(PK, sub) >> p & 1) x ^= pw[t][p];
            word[t] = x;
          } else {
            word[t] = sw[t];
          }
        }
        const u32x4* fb = sfrag + 4 * (sub * ws + wl) * 64 + lane;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const u32x4 bf = fb[r * 64];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            if (sub < WK)
              cm[t] = mfma16(bit_operand(word[t], r), bf, cm[t]);
            else
              cq[t] = mfma16(bit_operand(word[t], r), bf, cq[t]);
          }
        }
      }
    }
    // lane (column r16, quarter g) holds rows 4 g + i: records v0 + 16 t + 4 g + i
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float cmv[4] = {cm[t].x, cm[t].y, cm[t].z, cm[t].w};
      const float cqv[4] = {cq[t].x, cq[t].y, cq[t].z, cq[t].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = cmv[i] + swap_pair(cmv[i]);  // hi + lo columns
        const float b = QJL ? cqv[i] + swap_pair(cqv[i]) : 0.f;
        const int64_t v = v0 + 16 * t + 4 * g + i;
        if (writer && v < n) {
          const float gam = QJL ? prm.rnorms[v] : 0.f;
          const float sc = prm.norms[v] * fmaf(gam, b, a) * isc;
          float* o = prm.out + (qg * 8 + h) * n + v;
          *o = prm.first ? sc : *o + sc;
        }
      }
    }
  }
}

}  // namespace

tq_status search_plan(const tq_quantizer* q, int64_t m, SearchPlan* pl) {
  const int d = q->d;
  if (d % 128 || d < 128 || d > 4096) return set_error(TQ_ERR_UNSUPPORTED, "search: d must be a multiple of 128 in [128, 4096]");
  const bool qjl = q->variant == TQ_PROD;
  const int pk = q->planes;
  if (pk > 4 || (!qjl && pk == 0)) return set_error(TQ_ERR_UNSUPPORTED, "search: planes");
  const int wk = pk > 0 ? 1 << (pk - 1) : 0;
  const int wpp = d / 128;
  pl->nf = 4 * (wk + (qjl ? 1 : 0)) * wpp;
  const size_t groups = (size_t)((m + 7) / 8);
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  pl->frag_off = 0;
  pl->const_off = up(groups * (size_t)pl->nf * 64 * sizeof(u32x4));
  pl->qp_off = pl->const_off + up(groups * kSearchConsts * sizeof(float));
  pl->qq_off = pl->qp_off + up(groups * 8 * (size_t)d * sizeof(float));
  pl->total = pl->qq_off + (qjl ? up(groups * 8 * (size_t)d * sizeof(float)) : 0);
  return TQ_OK;
}

tq_status launch_search(const tq_quantizer* q, const float* y, int64_t m, const uint8_t* codes, const uint8_t* signs,
                        const float* norms, const float* rnorms, int64_t n, float* out, void* workspace,
                        hipStream_t stream) {
  SearchPlan pl;
  tq_status st = search_plan(q, m, &pl);
  if (st != TQ_OK) return st;
  const int d = q->d, pk = q->planes, wpp = d / 128, nf = pl.nf;
  const bool qjl = q->variant == TQ_PROD;
  const int wk = pk > 0 ? 1 << (pk - 1) : 0;
  char* base = (char*)workspace;
  u32x4* frag = (u32x4*)(base + pl.frag_off);
  float* consts = (float*)(base + pl.const_off);
  float* qp = (float*)(base + pl.qp_off);
  float* qq = qjl ? (float*)(base + pl.qq_off) : nullptr;
  const int64_t groups = (m + 7) / 8;
  {
    SearchProjParams pj{y, m, d, q->pi32, q->s32, qp, qq};
    const size_t lds = (size_t)8 * d * sizeof(float);
    hipError_t e = hipFuncSetAttribute((const void*)search_project_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return check_hip(e, "search: set LDS size");
    hipLaunchKernelGGL(search_project_kernel, dim3((unsigned)(d / kProjRows), (unsigned)groups, qjl ? 2u : 1u),
                       dim3(kThreads), lds, stream, pj);
    st = launch_check("search: projection launch");
    if (st != TQ_OK) return st;
  }
  SearchPrepParams pp{};
  pp.m = m;
  pp.d = d;
  pp.wk = wk;
  pp.wpp = wpp;
  pp.qjl = qjl;
  pp.qp = qp;
  pp.qq = qq;
  pp.frag = frag;
  pp.consts = consts;
  pp.nf = nf;
  pp.kappa = (float)(std::sqrt(M_PI / 2.0) / d);
  for (int s = 0; s < wk; ++s) pp.kcoef[s] = q->cb.walsh_coef[s];
  hipLaunchKernelGGL(search_prep_kernel, dim3((unsigned)m), dim3(kThreads), (size_t)2 * d * sizeof(float), stream, pp);
  st = launch_check("search: prep launch");
  if (st != TQ_OK) return st;
  // coordinate slices whose fragments fit the LDS budget
  const int per_word = 4 * (wk + (qjl ? 1 : 0));  // fragments per word index
  int ws = (kSearchMaxFragKB * 1024) / (per_word * 64 * (int)sizeof(u32x4));
  if (ws > wpp) ws = wpp;
  if (ws < 1) return set_error(TQ_ERR_UNSUPPORTED, "search: fragments exceed the LDS budget");
  SearchParams sp{};
  sp.frag = frag;
  sp.consts = consts;
  sp.codes = codes;
  sp.signs = signs;
  sp.norms = norms;
  sp.rnorms = rnorms;
  sp.out = out;
  sp.n = n;
  sp.m = m;
  sp.d = d;
  sp.wpp = wpp;
  sp.nf = nf;
  const int64_t steps = (n + 31) / 32;
  int64_t gx = (device_cus() + groups - 1) / groups;
  const int64_t cap = (steps + kSearchThreads / 64 - 1) / (kSearchThreads / 64);
  if (gx > cap) gx = cap;
  if (gx < 1) gx = 1;
  for (int w0 = 0; w0 < wpp; w0 += ws) {
    sp.w0 = w0;
    sp.ws = min(ws, wpp - w0);
    sp.first = w0 == 0;
    const size_t lds = (size_t)per_word * sp.ws * 64 * sizeof(u32x4);
    st = dispatch_planes(pk, [&](auto PC) -> tq_status {
      constexpr int PK = decltype(PC)::value;
      return dispatch_bool(qjl, [&](auto QC) -> tq_status {
        constexpr bool QJL = decltype(QC)::value;
        if constexpr (!QJL && PK == 0) {
          return set_error(TQ_ERR_UNSUPPORTED, "search: planes");
        } else {
          auto kern = search_score_kernel<PK, QJL>;
          hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
          if (e != hipSuccess) return check_hip(e, "search: set LDS size");
          hipLaunchKernelGGL(kern, dim3((unsigned)gx, (unsigned)groups), dim3(kSearchThreads), lds, stream, sp);
          return launch_check("search: score launch");
        }
      });
    });
    if (st != TQ_OK) return st;
  }
  return TQ_OK;
}

namespace {

// ===========================================================================
// Quantize on the matrix cores for d a multiple of 128 (the indexing half of
// vector search). The rotation y = Pi u over a batch of vectors is a dense
// GEMM: a workgroup computes 128 coordinates x 256 vectors, Pi (and S' = S
// Pi^T for the QJL stage) as bf16 hi/lo fragments, fp32 inputs split into
// bf16 hi/lo when staged through LDS (hi*hi + lo*hi + hi*lo, ~16 significant
// bits per operand, fp32 accumulation). The matrix rows are ordered so that
// lane quarter g of the MFMA output owns coordinates 32 g .. 32 g + 31 of
// the block: every plane's 32-bit word is built in one lane's registers.
// The norm is accumulated in fp64 while the input is staged. prod runs a
// second GEMM, p = S' e, over the fp32 residuals e = y - c[idx] of the first
// (stream-ordered scratch); its staging accumulates |e|^2.
// ===========================================================================
constexpr int kLqCoords = 128;                           // coordinates per workgroup
constexpr int kLqWaves = 4;
constexpr int kLqTiles = 4;                              // 16-vector tiles per wave
constexpr int kLqVecs = kLqWaves * kLqTiles * 16;        // vectors per workgroup (256)
constexpr int kLqThreads = kLqWaves * 64;
constexpr int kLqMatFrag = 8 * 2 * 64;                   // u32x4 per k-step of a coordinate block (16 KB)
constexpr int kLqVecFrag = kLqVecs / 16 * 2 * 64;        // u32x4 per k-step of a vector block (32 KB)
static_assert(kLqVecs == kLqThreads, "one staged vector per thread");

struct LqParams {
  const void* x;          // MODE 0: inputs; MODE 1: residuals (fp32)
  int64_t xg0, xgs, xoff; // input row of vector v of group grp: (grp + xg0) * xgs + v - xoff
  int64_t x_stride;       // elements from one input row to the next
  int64_t n_per_group;    // outputs: row (group_base + grp) * n_per_group + v
  int64_t group_base;
  int64_t v_begin, v_end; // vectors of this launch, in every group
  int d;
  float* resid;           // MODE 0 prod: residual out, row grp * cap + v - v_begin
  int64_t cap;
  uint8_t* codes;
  uint8_t* signs;
  float* norms;
  float* rnorms;
  float* rot_dbg;
  float* proj_dbg;
  float thr[15];
  float cen[16];
  const u32x4* mat[kMaxGroupsPerLaunch];  // fragment-ordered Pi (MODE 0) or S' (MODE 1)
};

__device__ __forceinline__ float opaque_f(float v) {
  asm volatile("" : "+v"(v));
  return v;
}

template <int P, int MODE, bool XF32, bool PROD>
__global__ __launch_bounds__(kLqThreads, 2) void lq_kernel(LqParams prm) {
  extern __shared__ u32x4 lq_lds[];  // matrix fragments [kLqMatFrag], vector fragments [kLqVecFrag]
  __shared__ float vsc[kLqVecs];     // per staged vector: 1/|x| (MODE 0) or |e| (MODE 1)
  constexpr int XB = XF32 ? 4 : 2;   // input bytes per element
  constexpr int XR = XF32 ? 8 : 4;   // u32x4 per 32 staged elements
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int d = prm.d, NKS = d / 32, NCB = d / kLqCoords;
  // XCD-aware order: consecutive workgroup ids go to different XCDs, so give each
  // XCD a contiguous range of (vector block, coordinate block) pairs with the
  // coordinate block fastest: the blocks of one vector block share its inputs in L2
  const int64_t total = (int64_t)gridDim.x, total8 = total & ~(int64_t)7;
  int64_t L = blockIdx.x;
  if (L < total8) L = (L & 7) * (total8 >> 3) + (L >> 3);
  const int cb = (int)(L % NCB);
  const int64_t v0 = prm.v_begin + (L / NCB) * kLqVecs;
  const int grp = blockIdx.y;
  // staging: thread tid brings in vector v0 + tid (clamped to the last one)
  const int64_t sv = min(v0 + tid, prm.v_end - 1);
  const uint8_t* xsrc = (const uint8_t*)prm.x + ((grp + prm.xg0) * prm.xgs + sv - prm.xoff) * prm.x_stride * XB;
  const u32x4* msrc = prm.mat[grp] + (int64_t)cb * NKS * kLqMatFrag;
  u32x4* ldsm = lq_lds;
  u32x4* ldsx = lq_lds + kLqMatFrag;
  const int tv = tid >> 4, rv = tid & 15;  // the staged vector's tile and row
  u32x4 xr[XR], mr[kLqMatFrag / kLqThreads];
  auto gload = [&](int ks) {
    const u32x4* xs = (const u32x4*)(xsrc + (int64_t)ks * 32 * XB);
#pragma unroll
    for (int j = 0; j < XR; ++j) xr[j] = xs[j];
    const u32x4* ms = msrc + (int64_t)ks * kLqMatFrag;
#pragma unroll
    for (int j = 0; j < kLqMatFrag / kLqThreads; ++j) mr[j] = ms[tid + kLqThreads * j];
  };
  double ss = 0.0;
  auto lstore = [&]() {
#pragma unroll
    for (int j = 0; j < kLqMatFrag / kLqThreads; ++j) ldsm[tid + kLqThreads * j] = mr[j];
#pragma unroll
    for (int sg = 0; sg < 4; ++sg) {  // 8 elements of K segment sg -> lane 16 sg + rv
      if constexpr (XF32) {
        const u32x4 u0 = xr[2 * sg], u1 = xr[2 * sg + 1];
        const float f[8] = {__uint_as_float(u0.x), __uint_as_float(u0.y), __uint_as_float(u0.z), __uint_as_float(u0.w),
                            __uint_as_float(u1.x), __uint_as_float(u1.y), __uint_as_float(u1.z), __uint_as_float(u1.w)};
        unsigned h[8], l[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          h[e] = bf16_part(f[e], false);
          l[e] = bf16_part(f[e], true);
          ss = fma((double)f[e], (double)f[e], ss);
        }
        ldsx[(tv * 2) * 64 + 16 * sg + rv] = u32x4{pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7])};
        ldsx[(tv * 2 + 1) * 64 + 16 * sg + rv] = u32x4{pack2(l[0], l[1]), pack2(l[2], l[3]), pack2(l[4], l[5]), pack2(l[6], l[7])};
      } else {
        const u32x4 v = xr[sg];
        const unsigned w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a = bf16_val(w[e] & 0xFFFFu), b = bf16_val(w[e] >> 16);
          ss = fma((double)a, (double)a, ss);
          ss = fma((double)b, (double)b, ss);
        }
        ldsx[(tv * 2) * 64 + 16 * sg + rv] = v;
      }
    }
  };
  f32x4 acc[8][kLqTiles];
#pragma unroll
  for (int q = 0; q < 8; ++q)
#pragma unroll
    for (int t = 0; t < kLqTiles; ++t) acc[q][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  gload(0);
  for (int ks = 0; ks < NKS; ++ks) {
    __syncthreads();  // the previous step's fragments are consumed
    lstore();
    __syncthreads();
    gload(min(ks + 1, NKS - 1));  // next step in flight during this step's MFMAs
    u32x4 xh[kLqTiles], xl[kLqTiles];
#pragma unroll
    for (int t = 0; t < kLqTiles; ++t) {
      xh[t] = ldsx[((wave * kLqTiles + t) * 2) * 64 + lane];
      if constexpr (XF32) xl[t] = ldsx[((wave * kLqTiles + t) * 2 + 1) * 64 + lane];
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const u32x4 ph = ldsm[(q * 2) * 64 + lane], pl = ldsm[(q * 2 + 1) * 64 + lane];
#pragma unroll
      for (int t = 0; t < kLqTiles; ++t) {
        acc[q][t] = mfma(ph, xh[t], acc[q][t]);
        acc[q][t] = mfma(pl, xh[t], acc[q][t]);
        if constexpr (XF32) acc[q][t] = mfma(ph, xl[t], acc[q][t]);
      }
    }
  }
  // per-vector scale from the staging thread's sum of squares
  {
    const double nrm = sqrt(ss);
    const int64_t v = v0 + tid;
    const int64_t orow = (prm.group_base + grp) * prm.n_per_group + v;
    if constexpr (MODE == 0) {
      vsc[tid] = nrm > 0.0 ? (float)(1.0 / nrm) : 0.f;
      if (cb == 0 && v < prm.v_end) prm.norms[orow] = (float)nrm;
    } else {
      vsc[tid] = (float)nrm;
      if (cb == 0 && v < prm.v_end) prm.rnorms[orow] = prm.norms[orow] > 0.f ? (float)nrm : 0.f;
    }
  }
  __syncthreads();
  constexpr int NT = P > 0 ? (1 << P) - 1 : 1;
  float thr[NT], cen[1 << (P > 0 ? P : 0)];
#pragma unroll
  for (int i = 0; i < NT; ++i) thr[i] = opaque_f(prm.thr[i]);
#pragma unroll
  for (int i = 0; i < (1 << (P > 0 ? P : 0)); ++i) cen[i] = opaque_f(prm.cen[i]);
  const int c0 = kLqCoords * cb + 32 * g;  // this lane's 32 coordinates
#pragma unroll
  for (int t = 0; t < kLqTiles; ++t) {
    const int vl = wave * (16 * kLqTiles) + 16 * t + r16;
    const int64_t v = v0 + vl;
    if (v >= prm.v_end) continue;
    const int64_t orow = (prm.group_base + grp) * prm.n_per_group + v;
    if constexpr (MODE == 0) {
      const float inv = vsc[vl];
      const bool valid = inv > 0.f;
      unsigned w[P > 0 ? P : 1];
#pragma unroll
      for (int p = 0; p < P; ++p) w[p] = 0u;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float y[4] = {acc[q][t].x * inv, acc[q][t].y * inv, acc[q][t].z * inv, acc[q][t].w * inv};
        float e[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bool b[P > 0 ? P : 1];
          if constexpr (P > 0) {
            search_bits<P>(y[i], thr, b);
#pragma unroll
            for (int p = 0; p < P; ++p) w[p] |= (b[p] ? 1u : 0u) << (4 * q + i);
          }
          if constexpr (PROD) e[i] = valid ? y[i] - centroid_of<P>(b, cen) : 0.f;
        }
        if (prm.rot_dbg) *(float4*)(prm.rot_dbg + orow * d + c0 + 4 * q) = float4{y[0], y[1], y[2], y[3]};
        if constexpr (PROD)
          *(float4*)(prm.resid + ((int64_t)grp * prm.cap + v - prm.v_begin) * d + c0 + 4 * q) = float4{e[0], e[1], e[2], e[3]};
      }
      if constexpr (P > 0) {
        uint8_t* rec = prm.codes + orow * (int64_t)(P * d / 8) + c0 / 8;
#pragma unroll
        for (int p = 0; p < P; ++p) *(unsigned*)(rec + p * (d / 8)) = valid ? w[p] : 0u;
      }
    } else {
      const bool valid = prm.norms[orow] > 0.f;
      unsigned w = 0u;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const f32x4 pv = acc[q][t];
        w |= (pv.x >= 0.f ? 1u : 0u) << (4 * q);
        w |= (pv.y >= 0.f ? 1u : 0u) << (4 * q + 1);
        w |= (pv.z >= 0.f ? 1u : 0u) << (4 * q + 2);
        w |= (pv.w >= 0.f ? 1u : 0u) << (4 * q + 3);
        if (prm.proj_dbg) *(float4*)(prm.proj_dbg + orow * d + c0 + 4 * q) = float4{pv.x, pv.y, pv.z, pv.w};
      }
      *(unsigned*)(prm.signs + orow * (int64_t)(d / 8) + c0 / 8) = valid ? w : 0u;
    }
  }
}

// ---- tables of the GEMM path, built once per quantizer ----
// C = A B^T for d x d fp32 matrices (S' = S Pi^T), 64 x 64 output per workgroup
__global__ __launch_bounds__(256) void abt_kernel(const float* __restrict__ A, const float* __restrict__ B, float* C, int d) {
  __shared__ float As[64][33], Bs[64][33];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int j0 = blockIdx.y * 64, k0 = blockIdx.x * 64;
  float acc[4][4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[u][v] = 0.f;
  for (int i0 = 0; i0 < d; i0 += 32) {
    for (int e = threadIdx.x; e < 64 * 32; e += 256) {
      const int r = e >> 5, c = e & 31;
      As[r][c] = A[(int64_t)(j0 + r) * d + i0 + c];
      Bs[r][c] = B[(int64_t)(k0 + r) * d + i0 + c];
    }
    __syncthreads();
#pragma unroll 8
    for (int c = 0; c < 32; ++c) {
      float a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = As[ty + 16 * u][c];
        b[u] = Bs[tx + 16 * u][c];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = fmaf(a[u], b[v], acc[u][v]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) C[(int64_t)(j0 + ty + 16 * u) * d + k0 + tx + 16 * v] = acc[u][v];
}

// Fragment order of a d x d fp32 matrix M for lq_kernel: entry
// ((cb * d/32 + ks) * 8 + q) * 2 + hl) * 64 + lane, lane = r + 16 g, holds
// M[128 cb + 32 (r / 4) + 4 q + r % 4][32 ks + 8 g .. + 7] as bf16 (hl = 0 hi, 1 lo).
__global__ __launch_bounds__(256) void frag_order_kernel(const float* __restrict__ M, u32x4* out, int d) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)d * d / 4) return;
  const int lane = (int)(e & 63), hl = (int)((e >> 6) & 1), q = (int)((e >> 7) & 7);
  const int64_t rest = e >> 10;
  const int nks = d / 32;
  const int ks = (int)(rest % nks), cb = (int)(rest / nks);
  const int r = lane & 15, g = lane >> 4;
  const int row = kLqCoords * cb + 32 * (r >> 2) + 4 * q + (r & 3);
  const float* src = M + (int64_t)row * d + 32 * ks + 8 * g;
  unsigned h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = bf16_part(src[i], hl == 1);
  out[e] = u32x4{pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7])};
}

}  // namespace

bool lq_supported(int d) { return d > 256 && d <= 4096 && d % kLqCoords == 0; }

tq_status build_large_tables(tq_quantizer* q) {
  const int d = q->d;
  if (!lq_supported(d)) return TQ_OK;
  const size_t mat = (size_t)d * d * sizeof(u32x4) / 4;  // d^2 / 4 u32x4 = hi + lo bf16
  const bool prod = q->variant == TQ_PROD;
  tq_status st = check_hip(hipMalloc(&q->lq_block, mat * (prod ? 2 : 1)), "create: hipMalloc (GEMM tables)");
  if (st != TQ_OK) return st;
  u32x4* pif = (u32x4*)q->lq_block;
  const unsigned nb = (unsigned)(((int64_t)d * d / 4 + 255) / 256);
  hipLaunchKernelGGL(frag_order_kernel, dim3(nb), dim3(256), 0, nullptr, q->pi32, pif, d);
  st = launch_check("create: fragment order");
  if (st == TQ_OK && prod) {
    float* sp = nullptr;
    st = check_hip(hipMalloc(&sp, (size_t)d * d * sizeof(float)), "create: hipMalloc (S')");
    if (st == TQ_OK) {
      hipLaunchKernelGGL(abt_kernel, dim3(d / 64, d / 64), dim3(256), 0, nullptr, q->s32, q->pi32, sp, d);
      st = launch_check("create: S' = S Pi^T");
      if (st == TQ_OK) {
        hipLaunchKernelGGL(frag_order_kernel, dim3(nb), dim3(256), 0, nullptr, sp, pif + mat / sizeof(u32x4), d);
        st = launch_check("create: fragment order (S')");
      }
      if (st == TQ_OK) st = check_hip(hipDeviceSynchronize(), "create: GEMM tables");
      tq_status fs = check_hip(hipFree(sp), "create: hipFree (S')");
      if (st == TQ_OK) st = fs;
    }
  } else if (st == TQ_OK) {
    st = check_hip(hipDeviceSynchronize(), "create: GEMM tables");
  }
  if (st == TQ_OK) {
    q->lq_pi = pif;
    q->lq_sp = prod ? pif + mat / sizeof(u32x4) : nullptr;
  }
  return st;
}

static tq_status launch_lq(const QuantizeLaunch& a, hipStream_t stream) {
  const tq_quantizer* q0 = a.qz[0];
  const int d = q0->d, P = q0->planes;
  const bool prod = q0->variant == TQ_PROD;
  const bool xf32 = a.x_dtype == TQ_F32;
  const int64_t n = a.n_per_group;
  for (int g0 = 0; g0 < a.n_groups; g0 += kMaxGroupsPerLaunch) {
    const int ng = min(kMaxGroupsPerLaunch, a.n_groups - g0);
    // prod: stream-ordered scratch for the fp32 residuals, at most 1 GiB per chunk of vectors
    int64_t cap = n;
    float* resid = nullptr;
    if (prod) {
      const int64_t lim = ((int64_t)1 << 30) / ((int64_t)ng * d * 4);
      cap = min(n, max((int64_t)kLqVecs, lim / kLqVecs * kLqVecs));
      tq_status st = check_hip(hipMallocAsync((void**)&resid, (size_t)ng * cap * d * sizeof(float), stream),
                               "quantize: hipMallocAsync (residual scratch)");
      if (st != TQ_OK) return st;
    }
    tq_status st = TQ_OK;
    for (int64_t vb = 0; vb < n && st == TQ_OK; vb += cap) {
      LqParams prm{};
      prm.x = a.x;
      prm.xg0 = g0;
      prm.xgs = n;
      prm.xoff = 0;
      prm.x_stride = a.x_stride;
      prm.n_per_group = n;
      prm.group_base = g0;
      prm.v_begin = vb;
      prm.v_end = min(n, vb + cap);
      prm.d = d;
      prm.resid = resid;
      prm.cap = cap;
      prm.codes = a.codes;
      prm.signs = a.signs;
      prm.norms = a.norms;
      prm.rnorms = a.rnorms;
      prm.rot_dbg = a.rot_dbg;
      prm.proj_dbg = a.proj_dbg;
      const int K = 1 << P;
      for (int i = 0; i + 1 < K; ++i) prm.thr[i] = q0->cb.thresholds[i];
      for (int i = 0; i < K; ++i) prm.cen[i] = q0->cb.centroids[i];
      for (int g = 0; g < ng; ++g) prm.mat[g] = (const u32x4*)a.qz[g0 + g]->lq_pi;
      const int64_t nvb = (prm.v_end - vb + kLqVecs - 1) / kLqVecs;
      const dim3 grid((unsigned)(nvb * (d / kLqCoords)), (unsigned)ng);
      const size_t lds = (size_t)(kLqMatFrag + kLqVecFrag) * sizeof(u32x4);
      st = dispatch_planes(P, [&](auto PC) -> tq_status {
        constexpr int PP = decltype(PC)::value;
        return dispatch_bool(xf32, [&](auto XC) -> tq_status {
          constexpr bool XF = decltype(XC)::value;
          return dispatch_bool(prod, [&](auto RC) -> tq_status {
            constexpr bool PR = decltype(RC)::value;
            if constexpr (!PR && PP == 0) {
              return set_error(TQ_ERR_UNSUPPORTED, "quantize: planes");
            } else {
              hipLaunchKernelGGL((lq_kernel<PP, 0, XF, PR>), grid, dim3(kLqThreads), lds, stream, prm);
              return launch_check("quantize (GEMM): rotation launch");
            }
          });
        });
      });
      if (st != TQ_OK || !prod) continue;
      LqParams p2 = prm;
      p2.x = resid;
      p2.xg0 = 0;
      p2.xgs = cap;
      p2.xoff = vb;
      p2.x_stride = d;
      for (int g = 0; g < ng; ++g) p2.mat[g] = (const u32x4*)a.qz[g0 + g]->lq_sp;
      hipLaunchKernelGGL((lq_kernel<0, 1, true, true>), grid, dim3(kLqThreads), lds, stream, p2);
      st = launch_check("quantize (GEMM): QJL launch");
    }
    if (resid) {
      tq_status fs = check_hip(hipFreeAsync(resid, stream), "quantize: hipFreeAsync (residual scratch)");
      if (st == TQ_OK) st = fs;
    }
    if (st != TQ_OK) return st;
  }
  return TQ_OK;
}

tq_status launch_quantize_large(const QuantizeLaunch& a, hipStream_t stream) {
  const tq_quantizer* q0 = a.qz[0];
  const int d = q0->d;
  bool gemm = a.layout == TQ_LAYOUT_VECTOR;
  for (int g = 0; g < a.n_groups && gemm; ++g) gemm = a.qz[g]->lq_pi != nullptr;
  if (gemm) return launch_lq(a, stream);
  if (a.layout != TQ_LAYOUT_VECTOR) return set_error(TQ_ERR_UNSUPPORTED, "quantize: d > 256 supports the vector layout only");
  return launch_quantize_fp32(a, nullptr, a.x_stride, stream);
}

tq_status launch_quantize_fp32(const QuantizeLaunch& a, const uint16_t* chan, int64_t x_stride, hipStream_t stream) {
  const tq_quantizer* q0 = a.qz[0];
  const int d = q0->d;
  // vectors per workgroup: 32 for d <= 128 (the matrix rows are then read once
  // per 32 vectors and every thread has work), 8 up to 2048, 4 beyond
  const int vb = d <= 128 ? 32 : (d <= 2048 ? 8 : 4);
  const size_t lds = ((size_t)2 * vb * d + 3 * vb) * sizeof(float);
  for (int g0 = 0; g0 < a.n_groups; g0 += kMaxGroupsPerLaunch) {
    const int ng = min(kMaxGroupsPerLaunch, a.n_groups - g0);
    LargeQuantParams prm{};
    prm.x = a.x;
    prm.x_stride = x_stride;
    prm.chan_map = chan != nullptr;
    if (chan)
      for (int j = 0; j < d; ++j) prm.chan[j] = chan[j];
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
    if (vb == 32) {
      hipError_t e = hipFuncSetAttribute((const void*)quantize_large_kernel<32>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return check_hip(e, "quantize: set LDS size");
      hipLaunchKernelGGL(quantize_large_kernel<32>, grid, dim3(kThreads), lds, stream, prm);
    } else if (vb == 8) {
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
  return launch_inner_products_fp32(q, y, q->d, nullptr, false, m, codes, signs, norms, rnorms, n, out, stream);
}

tq_status launch_inner_products_fp32(const tq_quantizer* q, const float* y, int64_t y_stride, const uint16_t* chan,
                                     bool accumulate, int64_t m, const uint8_t* codes, const uint8_t* signs,
                                     const float* norms, const float* rnorms, int64_t n, float* out,
                                     hipStream_t stream) {
  LargeIpParams prm{};
  prm.y = y;
  prm.y_stride = y_stride;
  prm.chan_map = chan != nullptr;
  prm.accumulate = accumulate;
  if (chan)
    for (int j = 0; j < q->d; ++j) prm.chan[j] = chan[j];
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
