// Decode attention over a KV cache quantized with an outlier-channel split
// ([NIK] "Experiments", KV cache: outlier channels at more bits than the
// others; every part is TurboQuant in its own dimension with its own rotation,
// norm, codebook and, for prod keys, QJL matrix). For each batch b and query
// head h (KV head g = h / (Hq / Hkv)):
//   s_t = scale * sum_p <q restricted to part p's channels, k~_{p,t}>,  t < len_b
//   out = sum_t softmax(s)_t v~_t, each value part written back to its channels
// (channels no value part keeps come out 0).
//
// Generic fp32 code for part dimensions that are multiples of 32 (the 32 / 96
// split of a 128-channel head): a workgroup takes one (batch, KV head, token
// split) and all query heads of the group. Each block of 256 tokens first
// copies every part's records (contiguous per part) into LDS with coalesced
// 32-bit loads; threads then read their token's bits from LDS. The query parts are rotated into
// each part's basis once per workgroup (q' = Pi_p q_p, q'' = S_p q_p, scale and
// the QJL factor folded in), so a score is a sum over code bits with no
// inverse rotation; values are accumulated in each part's rotated basis and
// rotated back once, in the combine. Tokens go in blocks of 256, one per
// thread, with an online softmax per block; the value sum stages 16
// dequantized coordinates of the block's tokens in LDS at a time, token-major
// so both the weights and the values are read four tokens per access. Splits are
// merged by log-sum-exp in a second kernel (deterministic, no atomics).
#include <hip/hip_runtime.h>

#include "tq_device.h"

namespace tq {
namespace {

constexpr int kSdBlock = 256;  // tokens per block = threads per workgroup
constexpr int kSdChunk = 16;   // value coordinates staged per pass
static_assert(kSdBlock == 2 * kSplitMaxGroup * kSdChunk, "two threads per (head, coordinate) pair in the value sum");

struct SdPart {
  int d, planes, off;  // part dimension, MSE-stage planes, offset in the concatenated channel list
  int lds_codes, lds_signs;  // 32-bit word offsets of the part's staged records in dynamic LDS
  bool qjl;
  const uint8_t* codes;  // [B][Hkv][T][planes*d/8]
  const uint8_t* signs;  // [B][Hkv][T][d/8] (qjl)
  const float* norms;    // [B][Hkv][T]
  const float* rnorms;   // [B][Hkv][T] (qjl)
  float cen[16];
  float kappa;  // sqrt(pi/2) / d
  const float* pi[kSplitMaxKv];
  const float* s[kSplitMaxKv];
};

struct SdParams {
  int Hq, Hkv, G, dim, nk, nv, dk, dv, n_splits;
  int64_t T, split_tokens;
  const uint16_t* q;  // bf16 [B][Hq][dim]
  const int32_t* lens;
  float scale;
  float* part;  // [B][Hq][n_splits][dv + 2]
  float* out;   // [B][Hq][dim]
  uint8_t kchan[kSplitMaxDecodeDim], vchan[kSplitMaxDecodeDim];
  SdPart kp[kSplitMaxParts], vp[kSplitMaxParts];
};

// plane bytes jb of a record (coordinates 8 jb .. 8 jb + 7)
__device__ __forceinline__ void plane_bytes(const uint8_t* rec, int planes, int d, int jb, unsigned* pb) {
#pragma unroll
  for (int pl = 0; pl < 4; ++pl) pb[pl] = pl < planes ? rec[pl * (d / 8) + jb] : 0u;
}
__device__ __forceinline__ int bit_index(const unsigned* pb, int bit) {
  return (int)(((pb[0] >> bit) & 1u) | (((pb[1] >> bit) & 1u) << 1) | (((pb[2] >> bit) & 1u) << 2) |
               (((pb[3] >> bit) & 1u) << 3));
}

__device__ float block_reduce(float v, bool is_max, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float u = __shfl_xor(v, o);
    v = is_max ? fmaxf(v, u) : v + u;
  }
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kSdBlock / 64; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
  return r;
}

// the records of up to 256 consecutive tokens of one part: nt * bytes contiguous
// bytes (a multiple of 4) copied to LDS with coalesced 32-bit loads
__device__ __forceinline__ void stage(const uint8_t* src, uint32_t* dst, int nt, int bytes) {
  const uint32_t* s = (const uint32_t*)src;
  for (int e = threadIdx.x; e < nt * bytes / 4; e += kSdBlock) dst[e] = s[e];
}

__global__ __launch_bounds__(kSdBlock) void split_decode_kernel(SdParams prm) {
  extern __shared__ uint32_t rec_lds[];  // staged key and value records of the current block
  __shared__ float qk[kSplitMaxGroup][kSplitMaxDecodeDim];  // q' per head, key parts' bases
  __shared__ float qs[kSplitMaxGroup][kSplitMaxDecodeDim];  // q'' per head (QJL parts)
  __shared__ float acc[kSplitMaxGroup][kSplitMaxDecodeDim];  // value sums, value parts' bases
  __shared__ float wts[kSplitMaxGroup][kSdBlock];            // block scores, then weights
  __shared__ float vt[kSdChunk][kSdBlock];                   // dequantized value coordinates, [coordinate][token]
  __shared__ float vhalf[kSplitMaxGroup * kSdChunk];           // second half of the token sum
  __shared__ float mrow[kSplitMaxGroup], lrow[kSplitMaxGroup], resc[kSplitMaxGroup];
  __shared__ float red[kSdBlock / 64];
  __shared__ float cenk[kSplitMaxParts][16], cenv[kSplitMaxParts][16];
  const int tid = threadIdx.x;
  const int b = blockIdx.x / prm.Hkv, g = blockIdx.x % prm.Hkv, split = blockIdx.y;
  if (tid < kSplitMaxParts * 16) {
    cenk[tid / 16][tid % 16] = prm.kp[tid / 16].cen[tid % 16];
    cenv[tid / 16][tid % 16] = prm.vp[tid / 16].cen[tid % 16];
  }
  const int G = prm.G;
  const int64_t len = min(max((int64_t)prm.lens[b], (int64_t)0), prm.T);  // lengths beyond the cache attend all of it
  const int64_t t0 = (int64_t)split * prm.split_tokens;
  const int64_t t1 = min(len, t0 + prm.split_tokens);
  const int64_t bg = (int64_t)b * prm.Hkv + g;

  // ---- query parts in the key parts' bases (acc is scratch for the raw queries) ----
  for (int e = tid; e < G * prm.dim; e += kSdBlock) {
    const int h = e / prm.dim, j = e % prm.dim;
    acc[h][j] = __uint_as_float((unsigned)prm.q[((int64_t)b * prm.Hq + g * G + h) * prm.dim + j] << 16);
  }
  __syncthreads();
  for (int p = 0; p < prm.nk; ++p) {
    const SdPart& P = prm.kp[p];
    for (int e = tid; e < G * P.d; e += kSdBlock) {
      const int h = e / P.d, i = e % P.d;
      const float* prow = P.pi[g] + (int64_t)i * P.d;
      const float* srow = P.qjl ? P.s[g] + (int64_t)i * P.d : nullptr;
      float a = 0.f, c = 0.f;
      for (int j = 0; j < P.d; ++j) {
        const float qv = acc[h][prm.kchan[P.off + j]];
        a = fmaf(prow[j], qv, a);
        if (P.qjl) c = fmaf(srow[j], qv, c);
      }
      qk[h][P.off + i] = prm.scale * a;
      qs[h][P.off + i] = P.qjl ? prm.scale * P.kappa * c : 0.f;
    }
  }
  __syncthreads();
  for (int e = tid; e < G * prm.dv; e += kSdBlock) acc[e / prm.dv][e % prm.dv] = 0.f;
  if (tid < G) {
    mrow[tid] = -INFINITY;
    lrow[tid] = 0.f;
  }
  __syncthreads();

  for (int64_t tb = t0; tb < t1; tb += kSdBlock) {
    const int64_t t = tb + tid;
    const bool valid = t < t1;
    {
      const int nt = (int)min((int64_t)kSdBlock, t1 - tb);
      const int64_t r0 = bg * prm.T + tb;
      for (int p = 0; p < prm.nk; ++p) {
        const SdPart& P = prm.kp[p];
        if (P.planes) stage(P.codes + r0 * (P.planes * P.d / 8), rec_lds + P.lds_codes, nt, P.planes * P.d / 8);
        if (P.qjl) stage(P.signs + r0 * (P.d / 8), rec_lds + P.lds_signs, nt, P.d / 8);
      }
      for (int p = 0; p < prm.nv; ++p) {
        const SdPart& P = prm.vp[p];
        stage(P.codes + r0 * (P.planes * P.d / 8), rec_lds + P.lds_codes, nt, P.planes * P.d / 8);
      }
      __syncthreads();
    }
    // ---- scores of this thread's token for every head of the group ----
    float sc[kSplitMaxGroup];
#pragma unroll
    for (int h = 0; h < kSplitMaxGroup; ++h) sc[h] = 0.f;
    if (valid) {
      for (int p = 0; p < prm.nk; ++p) {
        const SdPart& P = prm.kp[p];
        const int64_t r = bg * prm.T + t;
        const uint8_t* rec = (const uint8_t*)(rec_lds + P.lds_codes) + tid * (P.planes * P.d / 8);
        const uint8_t* sg = (const uint8_t*)(rec_lds + P.lds_signs) + tid * (P.d / 8);
        float a[kSplitMaxGroup], c[kSplitMaxGroup];
#pragma unroll
        for (int h = 0; h < kSplitMaxGroup; ++h) a[h] = c[h] = 0.f;
        for (int jb = 0; jb < P.d / 8; ++jb) {
          // 8 coordinates per byte: centroid values, then float4 broadcasts of q' (q'')
          unsigned pb[4];
          plane_bytes(rec, P.planes, P.d, jb, pb);
          float cv[8];
#pragma unroll
          for (int bit = 0; bit < 8; ++bit) cv[bit] = cenk[p][bit_index(pb, bit)];
          const int j0 = P.off + 8 * jb;
#pragma unroll
          for (int h = 0; h < kSplitMaxGroup; ++h)
            if (h < G) {
              const float4 u0 = *(const float4*)&qk[h][j0], u1 = *(const float4*)&qk[h][j0 + 4];
              a[h] = fmaf(u0.x, cv[0], fmaf(u0.y, cv[1], fmaf(u0.z, cv[2], fmaf(u0.w, cv[3], a[h]))));
              a[h] = fmaf(u1.x, cv[4], fmaf(u1.y, cv[5], fmaf(u1.z, cv[6], fmaf(u1.w, cv[7], a[h]))));
            }
          if (P.qjl) {
            const unsigned zb = sg[jb];
            float z[8];
#pragma unroll
            for (int bit = 0; bit < 8; ++bit) z[bit] = ((zb >> bit) & 1u) ? 1.f : -1.f;
#pragma unroll
            for (int h = 0; h < kSplitMaxGroup; ++h)
              if (h < G) {
                const float4 u0 = *(const float4*)&qs[h][j0], u1 = *(const float4*)&qs[h][j0 + 4];
                c[h] = fmaf(u0.x, z[0], fmaf(u0.y, z[1], fmaf(u0.z, z[2], fmaf(u0.w, z[3], c[h]))));
                c[h] = fmaf(u1.x, z[4], fmaf(u1.y, z[5], fmaf(u1.z, z[6], fmaf(u1.w, z[7], c[h]))));
              }
          }
        }
        const float nu = P.norms[r], gam = P.qjl ? P.rnorms[r] : 0.f;
#pragma unroll
        for (int h = 0; h < kSplitMaxGroup; ++h) sc[h] = fmaf(nu, fmaf(gam, c[h], a[h]), sc[h]);
      }
    }
    // ---- online softmax over the block ----
#pragma unroll
    for (int h = 0; h < kSplitMaxGroup; ++h) {
      if (h >= G) break;  // uniform: every thread leaves together
      const float bmax = block_reduce(valid ? sc[h] : -INFINITY, true, red);
      const float mnew = fmaxf(mrow[h], bmax);
      const float w = valid ? __expf(sc[h] - mnew) : 0.f;
      wts[h][tid] = w;
      const float bsum = block_reduce(w, false, red);
      if (tid == 0) {
        resc[h] = __expf(mrow[h] - mnew);  // 0 on the first block (mrow = -inf)
        lrow[h] = lrow[h] * resc[h] + bsum;
        mrow[h] = mnew;
      }
    }
    __syncthreads();
    for (int e = tid; e < G * prm.dv; e += kSdBlock) acc[e / prm.dv][e % prm.dv] *= resc[e / prm.dv];
    // ---- values: acc[h][j] += sum_t w[h][t] * nu_t * c[idx_{t,j}], 16 coordinates at a time ----
    for (int p = 0; p < prm.nv; ++p) {
      const SdPart& P = prm.vp[p];
      const int64_t r = bg * prm.T + t;
      for (int c0 = 0; c0 < P.d; c0 += kSdChunk) {
        __syncthreads();  // vt of the previous pass consumed; acc rescale done
        if (valid) {
          const uint8_t* rec = (const uint8_t*)(rec_lds + P.lds_codes) + tid * (P.planes * P.d / 8);
          const float nu = P.norms[r];
#pragma unroll
          for (int half = 0; half < kSdChunk / 8; ++half) {
            unsigned pb[4];
            plane_bytes(rec, P.planes, P.d, c0 / 8 + half, pb);
#pragma unroll
            for (int bit = 0; bit < 8; ++bit) vt[8 * half + bit][tid] = nu * cenv[p][bit_index(pb, bit)];
          }
        } else {
#pragma unroll
          for (int k = 0; k < kSdChunk; ++k) vt[k][tid] = 0.f;
        }
        __syncthreads();
        // pair (h, k) sums its token half; the two halves are added in a fixed order
        const int pair = tid % (kSplitMaxGroup * kSdChunk), th = tid / (kSplitMaxGroup * kSdChunk);
        const int h = pair / kSdChunk, k = pair % kSdChunk;
        float sum = 0.f;
        if (h < G) {
          const float4* wv = (const float4*)&wts[h][th * (kSdBlock / 2)];
          const float4* vv = (const float4*)&vt[k][th * (kSdBlock / 2)];
          for (int i = 0; i < kSdBlock / 8; ++i) {
            const float4 a4 = wv[i], b4 = vv[i];
            sum = fmaf(a4.x, b4.x, fmaf(a4.y, b4.y, fmaf(a4.z, b4.z, fmaf(a4.w, b4.w, sum))));
          }
          if (th == 1) vhalf[pair] = sum;
        }
        __syncthreads();
        if (th == 0 && h < G) acc[h][P.off + c0 + k] += sum + vhalf[pair];
      }
    }
    __syncthreads();
  }
  // ---- partials: acc[dv], m, l per head ----
  for (int e = tid; e < G * (prm.dv + 2); e += kSdBlock) {
    const int h = e / (prm.dv + 2), j = e % (prm.dv + 2);
    const float v = j < prm.dv ? acc[h][j] : (j == prm.dv ? mrow[h] : lrow[h]);
    prm.part[(((int64_t)b * prm.Hq + g * G + h) * prm.n_splits + split) * (prm.dv + 2) + j] = v;
  }
}

// one workgroup per (batch, query head): log-sum-exp merge of the splits, then
// each value part rotated back (Pi_p^T) and written to its channels
__global__ __launch_bounds__(kSdBlock) void split_combine_kernel(SdParams prm) {
  __shared__ float a[kSplitMaxDecodeDim];
  __shared__ float ml[2];
  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.x;
  const int hq = (int)(bh % prm.Hq);
  const int g = hq / prm.G;
  const float* src = prm.part + bh * prm.n_splits * (prm.dv + 2);
  if (tid == 0) {
    float M = -INFINITY;
    for (int s = 0; s < prm.n_splits; ++s) M = fmaxf(M, src[s * (prm.dv + 2) + prm.dv]);
    float L = 0.f;
    if (M > -INFINITY)
      for (int s = 0; s < prm.n_splits; ++s)
        L += src[s * (prm.dv + 2) + prm.dv + 1] * __expf(src[s * (prm.dv + 2) + prm.dv] - M);
    ml[0] = M;
    ml[1] = L;
  }
  __syncthreads();
  const float M = ml[0], L = ml[1];
  for (int j = tid; j < prm.dv; j += kSdBlock) {
    float v = 0.f;
    if (L > 0.f) {
      for (int s = 0; s < prm.n_splits; ++s) {
        const float ms = src[s * (prm.dv + 2) + prm.dv];
        if (ms > -INFINITY) v = fmaf(src[s * (prm.dv + 2) + j], __expf(ms - M), v);
      }
      v /= L;
    }
    a[j] = v;
  }
  __syncthreads();
  float* o = prm.out + bh * prm.dim;
  for (int j = tid; j < prm.dim; j += kSdBlock) o[j] = 0.f;  // channels no value part keeps
  __syncthreads();
  for (int p = 0; p < prm.nv; ++p) {
    const SdPart& P = prm.vp[p];
    for (int j = tid; j < P.d; j += kSdBlock) {
      float v = 0.f;
      for (int i = 0; i < P.d; ++i) v = fmaf(P.pi[g][(int64_t)i * P.d + j], a[P.off + i], v);
      o[prm.vchan[P.off + j]] = v;
    }
  }
}

}  // namespace

tq_status launch_split_decode(const SplitDecodeLaunch& L, hipStream_t stream) {
  SdParams prm{};
  prm.Hq = L.Hq;
  prm.Hkv = L.Hkv;
  prm.G = L.Hq / L.Hkv;
  prm.dim = L.dim;
  prm.T = L.max_ctx;
  prm.q = (const uint16_t*)L.q;
  prm.lens = L.lens;
  prm.scale = L.scale;
  prm.out = L.out;
  prm.part = (float*)L.workspace;
  prm.n_splits = L.n_splits;
  prm.split_tokens = L.split_tokens;
  int lds_words = 0;  // dynamic LDS: every part's records of one 256-token block
  for (int side = 0; side < 2; ++side) {
    const SplitSide& S = side == 0 ? L.k : L.v;
    SdPart* dst = side == 0 ? prm.kp : prm.vp;
    uint8_t* chan = side == 0 ? prm.kchan : prm.vchan;
    int off = 0;
    for (int p = 0; p < S.n_parts; ++p) {
      const tq_quantizer* q0 = S.qz[p * L.Hkv];
      SdPart& P = dst[p];
      P.d = q0->d;
      P.planes = q0->planes;
      P.off = off;
      P.qjl = q0->variant == TQ_PROD;
      P.lds_codes = lds_words;
      lds_words += kSdBlock * (P.planes * P.d / 8) / 4;
      P.lds_signs = lds_words;
      if (side == 0 && P.qjl) lds_words += kSdBlock * (P.d / 8) / 4;
      P.codes = S.codes[p];
      P.signs = S.signs[p];
      P.norms = S.norms[p];
      P.rnorms = S.rnorms[p];
      for (int i = 0; i < (1 << q0->planes); ++i) P.cen[i] = q0->cb.centroids[i];
      P.kappa = (float)(std::sqrt(M_PI / 2.0) / q0->d);
      for (int g = 0; g < L.Hkv; ++g) {
        P.pi[g] = S.qz[p * L.Hkv + g]->pi32;
        P.s[g] = S.qz[p * L.Hkv + g]->s32;
      }
      for (int j = 0; j < P.d; ++j) chan[off + j] = (uint8_t)S.channels[off + j];
      off += P.d;
    }
    if (side == 0) {
      prm.nk = S.n_parts;
      prm.dk = off;
    } else {
      prm.nv = S.n_parts;
      prm.dv = off;
    }
  }
  const size_t lds = (size_t)lds_words * 4;
  hipError_t e = hipFuncSetAttribute((const void*)split_decode_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return check_hip(e, "split decode: set LDS size");
  hipLaunchKernelGGL(split_decode_kernel, dim3((unsigned)(L.B * L.Hkv), (unsigned)L.n_splits), dim3(kSdBlock), lds,
                     stream, prm);
  tq_status st = launch_check("split decode: main launch");
  if (st != TQ_OK) return st;
  hipLaunchKernelGGL(split_combine_kernel, dim3((unsigned)(L.B * L.Hq)), dim3(kSdBlock), 0, stream, prm);
  return launch_check("split decode: combine launch");
}

}  // namespace tq
