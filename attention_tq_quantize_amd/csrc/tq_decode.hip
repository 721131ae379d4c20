// Decode attention over a packed KV cache, HIP for gfx950 (CDNA4, wave64).
//
// What is computed follows [NIK] = S. Nikolenko, "Eternal mathematics of
// TurboQuant" (blog.sergeynikolenko.ru), problem statement (attention scores
// are inner products of the query with every cached key) and the sections
// "Step 2" (dequantization c[idx] rotated back by Pi^T), "QJL" and "TurboQuant
// proper" (prod keys add |r| sqrt(pi/2)/d S^T z); [NAH] = "What exactly
// TurboQuant showed" (nahornyi.ai): prod keys need a dedicated attention kernel.
//
// Matrix cores: v_mfma_f32_16x16x32_f16. For C = A*B + C with A 16x32, B 32x16
// and lane l = r + 16*g (r in 0..15, g in 0..3):
//   A: lane l holds A[r][8g .. 8g+7];  B: lane l holds B[8g .. 8g+7][r];
//   C: lane l holds C[4g .. 4g+3][r].
// 16 rows = 8 query heads of a GQA group x (hi, lo) fp16 parts of each head's
// weights, so every MFMA row is used and weights carry 22 significant bits.
//
// Bit operands. A packed cache bit becomes an fp16 MFMA operand without
// unpacking: shift the 32-bit word so the wanted nibble lands on bits 8-11 of
// each fp16 half and mask one bit per element (bit_operand); the half is then
// 0 or the exact power of two 2^(k - 16) for slot k. The other operand carries
// the compensating power of two, so each product is exactly
// weight * bit * 2^E for a per-row exponent E chosen to keep the weights in
// fp16 range. One shift (none for the third nibble) plus four ANDs make one
// MFMA operand (8 bits). Positions 8-11 keep the matrix cores' products exact
// in their sums; deeper subnormal positions would lose low product bits.
//
// Both contractions use 0/1 bits. With sigma = 2 bit - 1 and the odd Walsh
// expansion of the symmetric codebook, c[idx] = sum_s a_s prod_{i in s} sigma_i,
// so sum_j w_j c[idx_j] = sum_s a_s (2 sum_j w_j bit_{s,j} - sum_j w_j) where
// bit_{s,j} is the XOR of the planes in subset s.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>

#include "tq_device.h"

namespace tq {
namespace {

// ===========================================================================
//   prep   : per (batch, kv head, head chunk): q' = Pi_K q, q'' = S_K q, packed
//            into the fp16 hi/lo operands of the score contraction.
//   main   : one wave per (batch, kv head, head chunk, context split): streams
//            packed keys and values, scores 8 query heads against the key bits,
//            runs an online softmax and accumulates values in the value
//            rotation's space.
//   combine: log-sum-exp merge of the splits, then out = Pi_V^T acc / l.
// Scores are kept in log2 units (scale * log2 e folded into the operands).
// ===========================================================================
// Value operands: a set bit of the value bit operand in slot k (token 4g + k of
// a lane's group) is 2^(k - 16) = 2^(vslot_exp(k) - 2); the weight of that token
// carries 2^(ev - vslot_exp(k)), so every product is w 2^(ev - 2).
__host__ __device__ constexpr int vslot_exp(int k) { return k - 14; }

// Append of the new token (online quantization of one vector per (batch, KV
// head) and tensor: [NIK] "Step 0" to "Step 2", prod keys also "TurboQuant
// proper"). The vector is normalized with its norm accumulated in fp64, rotated
// with the quantizer's fp32 Pi (prod: the residual e = y - c[idx] stays in the
// rotated basis and is projected with S' = S Pi^T, so S r = S' e), and its
// record is written at the sequence's current length; the value goes into its
// slot of the 32-token block (the other slots are kept).
struct AppendArgs {
  const int32_t* ctx_lens;
  int64_t max_ctx;
  int k_planes, v_bits;
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
  float* rot_dbg;   // optional [B][Hkv][2][d]: rotated unit vectors (key, value)
  float* proj_dbg;  // optional [B][Hkv][d]: S r of the key (prod)
};

struct DecPrepParams {
  const uint16_t* q;
  const float* pk[kMaxKvHeads];
  const float* sk[kMaxKvHeads];
  u32x4* frag;
  float* consts;
  int Hq, Hkv, group, chunk_heads, n_chunks, n_units;
  float scale_log2e;
  float kappa;
  float kcoef[kMaxWalsh];
  AppendArgs app;  // used by the blocks past n_units (2 per (batch, KV head))
};

// K-side operand words, for lane group g: the odd Walsh combinations of the
// stored key planes over the coordinate quarter [g D/4, (g+1) D/4), then the
// QJL sign plane. D >= 128: D/128 words per vector; D = 64: two vectors share a
// word (low / high 16 bits), the QJL plane has its own word (high half zero).
template <int D, int PK, bool QJL>
struct KWords {
  static constexpr int WK = n_walsh(PK);
  static constexpr int NWM = PK == 0 ? 0 : (D >= 128 ? WK * (D / 128) : (WK + 1) / 2);
  static constexpr int NWQ = QJL ? (D >= 128 ? D / 128 : 1) : 0;
  static constexpr int NW = NWM + NWQ;
  static constexpr int NF = 4 * NW;
};

// consts per (batch, kv head, chunk): [0,16) mse init, [16,32) qjl init,
// [32,48) 2^(10-E_mse), [48,64) 2^(10-E_qjl) (raw scores are score x 2^(E-10)),
// one value per MFMA row.
constexpr int kConstsPerUnit = 64;

template <int NTH>
__device__ __forceinline__ double block_sum_f64(double v, double* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int w = 0; w < NTH / 64; ++w) s += red[w];
  __syncthreads();
  return s;
}

// a row of M (D floats, 16-byte aligned) dotted with v (shared memory); groups
// of up to 16 float4 loads in flight
template <int D>
__device__ __forceinline__ float row_dot(const float* __restrict__ row, const float* v) {
  constexpr int G = D < 64 ? D / 4 : 16;
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

// The append role: one block per (batch, kv head, tensor); thread t < D owns coordinate t.
template <int D, int NTH>
__device__ void append_one(const AppendArgs& p, int grp, bool value, int Hkv) {
  __shared__ float sx[D], se[D], sp[D];
  __shared__ int sidx[D];
  __shared__ double red[NTH / 64];
  const int t = threadIdx.x;
  const int b = grp / Hkv, h = grp % Hkv;
  int64_t len = p.ctx_lens[b];
  len = len < 0 ? 0 : len;
  if (len >= p.max_ctx) return;  // block-uniform: a full cache is not appended
  const int64_t slot = (int64_t)grp * p.max_ctx + len;
  const void* src = (const char*)(value ? p.v_new : p.k_new) + (size_t)grp * D * (p.x_bf16 ? 2 : 4);
  const float* pi = value ? p.v_pi[h] : p.k_pi[h];
  const float* spm = (!value && p.k_prod) ? p.k_sp[h] : nullptr;
  const int planes = value ? p.v_bits : p.k_planes;
  const float* thr = value ? p.v_thr : p.k_thr;
  const float* cen = value ? p.v_cen : p.k_cen;
  float xv = 0.f;
  if (t < D) xv = p.x_bf16 ? bf16_val(((const uint16_t*)src)[t]) : ((const float*)src)[t];
  const double nu = sqrt(block_sum_f64<NTH>(t < D ? (double)xv * (double)xv : 0.0, red));
  const float nu32 = (float)nu;
  const bool zero = !(nu > 0.0);
  if (t < D) sx[t] = zero ? 0.f : (float)((double)xv / nu);
  __syncthreads();
  float e = 0.f;
  if (t < D) {
    const float y = row_dot<D>(pi + (int64_t)t * D, sx);
    const int K = 1 << planes;
    int i = 0;
    for (int k = 0; k + 1 < K; ++k) i += y > thr[k] ? 1 : 0;
    if (zero) i = 0;
    sidx[t] = i;
    e = zero ? 0.f : y - cen[i];
    se[t] = e;
    if (p.rot_dbg) p.rot_dbg[((int64_t)grp * 2 + (value ? 1 : 0)) * D + t] = y;
  }
  float gamma = 0.f;
  if (spm) {
    gamma = (float)sqrt(block_sum_f64<NTH>((double)e * (double)e, red));  // also publishes se
    if (t < D) {
      const float pr = row_dot<D>(spm + (int64_t)t * D, se);
      sp[t] = zero ? -1.f : pr;  // zero vector: sign bits 0
      if (p.proj_dbg) p.proj_dbg[(int64_t)grp * D + t] = pr;
    }
  }
  __syncthreads();
  if (!value) {
    constexpr int wpp = D / 32;  // 32-bit words per plane of a record
    if (t < p.k_planes * wpp) {
      const int pl = t / wpp, w = t % wpp;
      unsigned bits = 0u;
#pragma unroll
      for (int c = 0; c < 32; ++c) bits |= (unsigned)((sidx[32 * w + c] >> pl) & 1) << c;
      p.k_codes[slot * (p.k_planes * wpp) + t] = bits;
    }
    if (p.k_prod && t < wpp) {
      unsigned bits = 0u;
#pragma unroll
      for (int c = 0; c < 32; ++c) bits |= (sp[32 * t + c] >= 0.f ? 1u : 0u) << c;
      p.k_signs[slot * wpp + t] = bits;
    }
    if (t == 0) {
      p.k_norms[slot] = nu32;
      if (p.k_prod) p.k_rnorms[slot] = gamma;
    }
    return;
  }
  // value: slot len % 32 of its block. Slot v is vector 4g + k (v < 16) or 16 + 4g + k;
  // plane pl, coordinate 4w + r sits at bit 4r + k (+16) of word (pl*4 + g)*(d/4) + w
  const int v = (int)(len % 32);
  const int hi = v >= 16 ? 16 : 0, g = (v % 16) / 4, k = v % 4;
  const unsigned keep = ~(0x1111u << (k + hi));
  constexpr int wq = D / 4;
  uint32_t* blk = p.v_codes + ((int64_t)grp * (p.max_ctx / 32) + len / 32) * (int64_t)(p.v_bits * D);
  for (int i = t; i < p.v_bits * wq; i += NTH) {
    const int pl = i / wq, w = i % wq;
    unsigned bits = 0u;
#pragma unroll
    for (int r = 0; r < 4; ++r) bits |= (unsigned)((sidx[4 * w + r] >> pl) & 1) << (4 * r + k + hi);
    uint32_t* word = blk + (pl * 4 + g) * wq + w;
    *word = (*word & keep) | bits;
  }
  if (t == 0) p.v_norms[slot] = nu32;
}

// One launch before the main loop. Blocks [0, n_units): one per (batch, kv
// head, head chunk): threads 2j and 2j + 1 take the two halves of row j of
// Pi_K (j < D) or of S_K (j >= D) and dot them with every head of the chunk
// (each matrix row is read once for all of them, every load of a thread in
// flight at once); then the block writes the chunk's score-operand fragments
// (fp16 hi/lo of 2 a_s (Pi_K q)_j and 2 kappa (S_K q)_j with the bit-position
// powers of two) and the per-row constants. Blocks past n_units (decode with
// append): the new token's key and value records.
// Query prep of one (batch, KV head, head chunk) unit, in kPrepSlices
// workgroups: slice s owns coordinates [s D/4, (s+1) D/4) of q' = Pi_K q and
// q'' = S_K q, which are exactly the K elements of lane group s in every score
// fragment, so a workgroup reads only its D/4 rows of each matrix and writes
// the fragment lanes of its group. The per-head operand exponent comes from
// bounds that every slice has at hand: |q'_j| <= |q| (Pi's rows are unit
// vectors) and |q''_j| <= |q| max_i |S_i|; the constant parts of the scores
// use sum_j q'_j = (Pi^T 1) q and sum_j q''_j = (S^T 1) q (slice 0).
constexpr int kPrepSlices = 4;

template <int D, int PK, bool QJL>
__global__ __launch_bounds__(4 * D) void decode_prep_kernel(DecPrepParams prm) {
  using KW = KWords<D, PK, QJL>;
  constexpr int NTH = 4 * D;
  constexpr int RS = D / kPrepSlices;  // rows of each matrix per slice
  if ((int)blockIdx.x >= prm.n_units * kPrepSlices) {
    const int a = blockIdx.x - prm.n_units * kPrepSlices;
    append_one<D, NTH>(prm.app, a >> 1, a & 1, prm.Hkv);
    return;
  }
  __shared__ float qs[8][D];            // the unit's queries
  __shared__ float qp[8][RS], qq[8][RS];  // this slice's coordinates of Pi_K q and S_K q
  __shared__ float qn[8], qsp[8], qsq[8];  // |q|, (Pi^T 1) q, (S^T 1) q per head
  __shared__ float opscale[8][4];
  const int unit = blockIdx.x / kPrepSlices, slice = blockIdx.x % kPrepSlices;
  const int chunk = unit % prm.n_chunks, bh = unit / prm.n_chunks;
  const int b = bh / prm.Hkv, hkv = bh % prm.Hkv;
  const int nh = prm.chunk_heads;
  const int hq0 = hkv * prm.group + chunk * nh;
  const int t = threadIdx.x;
  // thread t: eighth (t % 8) of row pair t / 8; pairs [0, RS) are rows of Pi_K,
  // [RS, 2 RS) rows of S_K, both within this slice
  const int pair = t >> 3, part = t & 7;
  const bool s_row = pair >= RS;
  const int row = slice * RS + pair % RS;
  const bool m_active = !s_row || QJL;
  constexpr int NE = D / 8;  // row elements per thread
  constexpr int NV = NE / 4;
  const float* mrow = (s_row ? prm.sk[hkv] : prm.pk[hkv]) + (int64_t)row * D + part * NE;
  float4 mv[NV];
  if (m_active) {
#pragma unroll
    for (int k = 0; k < NV; ++k) mv[k] = ((const float4*)mrow)[k];
  }
  for (int i = t; i < nh * D; i += NTH)
    qs[i / D][i % D] = bf16_val(prm.q[((int64_t)b * prm.Hq + hq0 + i / D) * D + i % D]);
  // slice 0: the column sums Pi^T 1 and S^T 1 (stored after each matrix), and S's row-norm bound
  __shared__ float colsum[2][D + 1];
  if (slice == 0)
    for (int i = t; i < 2 * D; i += NTH) {
      const int m = i / D, j = i % D;
      if (m == 0 || QJL) colsum[m][j] = (m ? prm.sk[hkv] : prm.pk[hkv])[D * D + j];
    }
  if (QJL && t == 0) colsum[1][D] = prm.sk[hkv][D * D + D];
  __syncthreads();
  {
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (m_active) {
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const int c = part * NE + 4 * k;
#pragma unroll
        for (int h = 0; h < 8; ++h)
          if (h < nh)
            a[h] = fmaf(mv[k].x, qs[h][c], fmaf(mv[k].y, qs[h][c + 1], fmaf(mv[k].z, qs[h][c + 2], fmaf(mv[k].w, qs[h][c + 3], a[h]))));
      }
    }
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      a[h] += __shfl_xor(a[h], 1);
      a[h] += __shfl_xor(a[h], 2);
      a[h] += __shfl_xor(a[h], 4);
    }
    if (part == 0 && m_active) {
      float(*dst)[RS] = s_row ? qq : qp;
#pragma unroll
      for (int h = 0; h < 8; ++h)
        if (h < nh) dst[h][pair % RS] = a[h];
    }
  }
  // |q| per head, and on slice 0 the sums of q' and q'' (one wave per head)
  {
    const int wave = t >> 6, lane = t & 63;
    for (int h = wave; h < nh; h += NTH / 64) {
      float s2 = 0.f, s_p = 0.f, s_q = 0.f;
      for (int j = lane; j < D; j += 64) {
        s2 = fmaf(qs[h][j], qs[h][j], s2);
        if (slice == 0) {
          s_p = fmaf(colsum[0][j], qs[h][j], s_p);
          if (QJL) s_q = fmaf(colsum[1][j], qs[h][j], s_q);
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        s2 += __shfl_xor(s2, o);
        s_p += __shfl_xor(s_p, o);
        s_q += __shfl_xor(s_q, o);
      }
      if (lane == 0) {
        qn[h] = sqrtf(s2);
        qsp[h] = s_p;
        qsq[h] = s_q;
      }
    }
  }
  __syncthreads();
  float amax = 0.f, asum = 0.f;
  for (int s = 0; s < KW::WK; ++s) {
    amax = fmaxf(amax, fabsf(prm.kcoef[s]));
    asum += prm.kcoef[s];
  }
  const float smax = QJL ? colsum[1][D] : 0.f;
  // one exponent per head for both score parts (the main loop scales their sum
  // once), and each head's operand scale per slot k: scale log2 e 2^(E + 14 - pos(k));
  // slice 0 writes the unit's constants
  float* cst = prm.consts + (int64_t)unit * kConstsPerUnit;
  if (t < 16) {
    const int h = t >> 1, lo = t & 1;
    if (h < nh) {
      // the bound on |q|: the rounding of the fp32 products and sums stays far
      // below the factor 2 of headroom range_exp leaves
      const int em = range_exp(fmaxf(2.f * amax * qn[h], QJL ? 2.f * prm.kappa * qn[h] * smax : 0.f) *
                               prm.scale_log2e);
      if (slice == 0) {
        cst[t] = lo ? 0.f : -asum * qsp[h] * prm.scale_log2e * ldexpf(1.0f, em - 10);
        cst[16 + t] = lo ? 0.f : (QJL ? -prm.kappa * qsq[h] * prm.scale_log2e * ldexpf(1.0f, em - 10) : 0.f);
        cst[32 + t] = ldexpf(1.0f, 10 - em);
        cst[48 + t] = ldexpf(1.0f, 10 - em);
      }
      if (!lo)
        for (int k = 0; k < 4; ++k) opscale[h][k] = prm.scale_log2e * ldexpf(1.0f, em + 14 - operand_pos(k));
    } else {
      if (slice == 0) {
        cst[t] = 0.f;
        cst[16 + t] = 0.f;
        cst[32 + t] = 1.f;
        cst[48 + t] = 1.f;
      }
      if (!lo)
        for (int k = 0; k < 4; ++k) opscale[h][k] = 0.f;
    }
  }
  __syncthreads();
  // fragment (f, lane) of lane group g = slice: row r16 = 2 h + lo of the MFMA,
  // K elements 8 g .. 8 g + 7
  const int g = slice;
  for (int e = t; e < KW::NF * 16; e += NTH) {
    const int f = e / 16, r16 = e % 16;
    const int h = r16 >> 1, lo = r16 & 1;
    const int W = f / 4, r = f % 4;
    unsigned hv[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int k = it / 2, half = it % 2;
      const int beta = 16 * half + 4 * r + k;  // bit of the lane's word
      float val = 0.f;
      if (h < nh) {
        if (W < KW::NWM) {
          int s, jl;  // Walsh subset and the coordinate within this slice
          if constexpr (D >= 128) {
            s = W / (D / 128);
            jl = 32 * (W % (D / 128)) + beta;
          } else {
            s = 2 * W + half;
            jl = beta % 16;
          }
          if (s < KW::WK) val = 2.f * prm.kcoef[s] * qp[h][jl];
        } else {
          const int Wq = W - KW::NWM;
          if constexpr (D >= 128) {
            val = 2.f * prm.kappa * qq[h][32 * Wq + beta];
          } else {
            if (half == 0) val = 2.f * prm.kappa * qq[h][beta];
          }
        }
        // the lane's bit reads as 2^(operand_pos(k) - 24); raw scores come out x 2^(E - 10)
        val *= opscale[h][k];
      }
      hv[it] = f16_part(val, lo);
    }
    prm.frag[((int64_t)unit * KW::NF + f) * 64 + 16 * g + r16] =
        u32x4{pack2(hv[0], hv[1]), pack2(hv[2], hv[3]), pack2(hv[4], hv[5]), pack2(hv[6], hv[7])};
  }
}

struct DecMainParams {
  const u32x4* frag;
  const float* consts;
  const uint8_t* kcodes;
  const uint8_t* ksigns;
  const float* knorms;
  const float* krnorms;
  const uint8_t* vcodes;
  const float* vnorms;
  const int* ctx_lens;
  int len_add;  // 1 when the step appended a token at ctx_lens[b]
  float* part_acc;
  float* part_ml;
  float* scores_dbg;
  int64_t max_ctx;
  int64_t split_tokens;
  int n_splits;
  int Hq, Hkv, group, chunk_heads, n_chunks;
  float vrho[kMaxWalsh];   // per value subset: a_s / a_lead of its set (1 for leads)
  float vlead[kMaxWalsh];  // per set: the lead subset's coefficient
  float vcoef_sum;         // sum of all value subset coefficients
};

// two floats to fp16 (round toward zero) packed into one dword, a in the low half
__device__ __forceinline__ unsigned pack_rtz(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(a, b));
}

// fp16 hi (nsel = -0) or lo (nsel = -1) parts of x0 and x1 packed in one dword:
// h = RNE_f16(x); the result is RNE_f16(x + nsel * h). x - h is exact in fp32,
// so hi + lo carries 22 significant bits. The inputs are ordinary VALU results.
__device__ __forceinline__ unsigned split_pair(float x0, float x1, float nsel) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  const unsigned h = __builtin_bit_cast(unsigned, __builtin_convertvector((f2){x0, x1}, h2));
  unsigned r;
  asm("v_fma_mixlo_f16 %0, %1, %2, %3 op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixhi_f16 %0, %1, %2, %4 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
      : "=&v"(r)
      : "v"(h), "v"(nsel), "v"(x0), "v"(x1));
  return r;
}

// RNE fp16 of x0 (low half) and x1 (high half): the hi parts of split_pair
__device__ __forceinline__ unsigned f16_pair_rne(float x0, float x1) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f2){x0, x1}, h2));
}

// max of three floats as one v_max3_f32 (fmaxf chains pick up NaN
// canonicalisations in IEEE mode); the inputs are ordinary VALU results
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max8f(const float (&v)[2][4]) {
  return max3f(max3f(v[0][0], v[0][1], v[0][2]), max3f(v[0][3], v[1][0], v[1][1]), max3f(v[1][2], v[1][3], v[1][3]));
}
// max of non-negative floats through their bit patterns (same order as the values)
__device__ __forceinline__ unsigned max8_nonneg_bits(const float (&v)[2][4]) {
  unsigned m = 0u;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) m = max(m, __float_as_uint(v[t][i]));
  return m;
}


// Value accumulator sets. The odd Walsh subsets of the VB value planes are
// split into NSET sets; set j accumulates sum_t w_t (bits of its lead subset)
// plus, for its other subsets s, sum_t (w_t rho_s)(bits of s) with
// rho_s = a_s / a_lead <= 1. The lead of set j is the single top plane
// {VB-1-j} (the largest coefficients of a symmetric Lloyd-Max codebook); with
// NSET = 2^(VB-1) every subset is its own lead.
__host__ __device__ constexpr int value_sets(int D, int VB) {
  // at most 64 accumulator registers (D/4 per set), and single-plane leads
  const int wv = n_walsh(VB);
  int n = 64 / (D / 4);
  if (n >= wv) return wv;
  if (n > VB) n = VB;
  return n < 1 ? 1 : n;
}
__host__ __device__ constexpr bool walsh_is_lead(int VB, int NSET, int s) {
  if (NSET == n_walsh(VB)) return true;
  for (int j = 0; j < NSET; ++j)
    if (walsh_mask(VB, s) == (1 << (VB - 1 - j))) return true;
  return false;
}
__host__ __device__ constexpr int walsh_set(int VB, int NSET, int s) {
  if (NSET == n_walsh(VB)) return s;
  for (int j = 0; j < NSET; ++j)
    if (walsh_mask(VB, s) == (1 << (VB - 1 - j))) return j;
  int k = 0;
  for (int t = 0; t < s; ++t)
    if (!walsh_is_lead(VB, NSET, t)) ++k;
  return k % NSET;
}

// Largest value-weight operand the loop accepts before it lowers the row's
// value exponent (fp16 holds up to 65504; the weights are kept below 2^14).
constexpr float kWeightOperandMax = 32768.0f;
// "value exponent not chosen yet"
constexpr int kEvUnset = 40;

// Main loop. One wave per (batch, kv head, head chunk, context split); 32
// tokens (two 16-token tiles) per iteration.
//
// Scores: C[row][token] over 16 rows = 8 query heads x (hi, lo) fp16 parts of
// the score operands (the MFMA's A operand, held in registers for the whole
// split) against the key bit planes (B operand). Lane (n, g) holds rows
// 4g .. 4g+3 of token n of each tile, i.e. heads 2g and 2g + 1 with both their
// parts, so a head's score is one add per part and the softmax runs once per
// (head, token) in the lane that owns the token.
//
// Values: C[row][coord] with A[row][token] = the hi (even rows) or lo (odd rows)
// fp16 part of the weight w = p * |v| times 2^(ev - e_k), e_k = vslot_exp(k),
// for the token in slot k of the value bit operand (the K order of the value
// cache block layout puts token 16t + 4g + k in slot k; its bit reads as
// 2^(k - 16), and the leftover 2^-2 is removed after the loop). The factor is
// folded into the exp2 argument. The weights reach the A-operand lanes through
// a per-wave LDS transpose: each token lane splits its two heads' weights of
// both tiles into fp16 hi and lo pairs (for the lead subsets and, scaled by
// a_s / a_lead, for every other subset: see value_sets) and writes them into
// the rows the value lanes read as whole operands. Each set's lead coefficient
// and the 0/1-to-sign correction are applied once, after the loop.
constexpr int kWRow = 40;  // dwords per (version, head) row: hi pairs [0,16), lo pairs [16,32), padding

// Raw cache bytes of one 32-token chunk of one (batch, kv head) as the main loop
// stages them in LDS: key codes, QJL signs, key norms, residual norms, value
// norms (128 bytes each) and the 32-token value block, each contiguous in HBM.
// DEPTH chunks per wave are in flight (buffer-to-LDS loads, no registers held);
// the depth is the largest of 3, 2, 1 that leaves room for two workgroups per
// CU next to the score fragments and the weight transpose, else 0 (registers,
// one chunk ahead).
// Score fragments held in registers for the whole split instead of re-read
// from LDS every chunk: chosen for the shapes where that still compiles
// without spills at two waves per SIMD.
__host__ __device__ constexpr bool frag_in_regs(int D, int PK, bool QJL, int VB) {
  return D == 128 && PK <= 2 && (VB == 3 || (VB == 4 && (QJL || PK < 2)));
}

template <int D, int PK, bool QJL, int VB, int NSET>
struct DecRing {
  static constexpr int KREC = PK * D / 8, SREC = D / 8;
  static constexpr int OFF_S = 32 * KREC;
  static constexpr int OFF_NK = OFF_S + (QJL ? 32 * SREC : 0);
  static constexpr int OFF_GM = OFF_NK + 128;
  static constexpr int OFF_NV = OFF_GM + (QJL ? 128 : 0);
  static constexpr int OFF_V = OFF_NV + 128;
  static constexpr int BYTES = OFF_V + 4 * VB * D;
  static constexpr int WAVES = kThreads / 64;
  static constexpr int FIXED = (frag_in_regs(D, PK, QJL, VB) ? 0 : KWords<D, PK, QJL>::NF * 64 * 16) +
                               WAVES * (1 + n_walsh(VB) - NSET) * 8 * kWRow * 4;
  static constexpr int kBudget = 80 * 1024;  // bytes per workgroup: two per CU
  static constexpr int fits(int r) { return FIXED + r * WAVES * BYTES <= kBudget; }
  static constexpr int DEPTH = fits(3) ? 3 : fits(2) ? 2 : fits(1) ? 1 : 0;
  // 16-byte buffer-to-LDS loads per chunk (each segment a multiple of 128 bytes)
  static constexpr int segs(int bytes) { return (bytes + 1023) / 1024; }
  static constexpr int LOADS = (PK > 0 ? segs(32 * KREC) : 0) + (QJL ? segs(32 * SREC) + 1 : 0) + 2 + segs(4 * VB * D);
};

template <int D, int PK, bool QJL, int VB, int NSET>
__global__ __launch_bounds__(kThreads, 2) void decode_main_kernel(DecMainParams prm) {
  using KW = KWords<D, PK, QJL>;
  constexpr int WV = n_walsh(VB);
  constexpr int NT = D / 16;   // value N-tiles (16 coordinates each)
  constexpr int VWL = D / 64;  // value words per lane per plane
  constexpr int NACC = NSET;
  static_assert(NSET == WV || NSET <= VB, "accumulator sets need single-plane leads");
  constexpr int KREC = PK * D / 8;
  constexpr int SREC = D / 8;
  constexpr int VBLK = 4 * VB * D;  // bytes of one 32-token value block
  constexpr int WPP = D >= 128 ? D / 128 : 1;
  constexpr bool KF_REG = frag_in_regs(D, PK, QJL, VB);  // score fragments in registers (else LDS)

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int bhc = blockIdx.y;
  const int chunk = bhc % prm.n_chunks;
  const int bh = bhc / prm.n_chunks;
  const int b = bh / prm.Hkv, hkv = bh % prm.Hkv;
  __shared__ u32x4 kf_lds[KF_REG ? 1 : KW::NF * 64];
  constexpr int NVER = 1 + (WV - NSET);  // weight versions: the leads, then one per other subset
  __shared__ unsigned wt_lds[kThreads / 64][NVER][8][kWRow];
  const u32x4* fsrc = prm.frag + (int64_t)bhc * KW::NF * 64;
  u32x4 kf[KF_REG ? KW::NF : 1];
  if constexpr (KF_REG) {
#pragma unroll
    for (int f = 0; f < KW::NF; ++f) kf[f] = fsrc[f * 64 + lane];
  } else {
    for (int i = threadIdx.x; i < KW::NF * 64; i += kThreads) kf_lds[i] = fsrc[i];
    __syncthreads();
  }
  auto kfrag = [&](int f) -> u32x4 {
    if constexpr (KF_REG) return kf[f];
    else return kf_lds[f * 64 + lane];
  };
  const int split = blockIdx.x * 4 + wave;
  if (split >= prm.n_splits) return;
  int64_t ctx = prm.ctx_lens[b];
  ctx = ctx < 0 ? 0 : ctx + prm.len_add;
  ctx = ctx > prm.max_ctx ? prm.max_ctx : ctx;
  const int64_t t0 = (int64_t)split * prm.split_tokens;
  const int64_t t1 = min(t0 + prm.split_tokens, ctx);
  const int hq0 = hkv * prm.group + chunk * prm.chunk_heads;

  // constants of this lane's rows 4g .. 4g+3 (heads 2g, 2g + 1; hi and lo parts)
  const float* cst = prm.consts + bhc * kConstsPerUnit;
  float cm_init[4], cq_init[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    cm_init[i] = cst[4 * g + i];
    cq_init[i] = cst[16 + 4 * g + i];
  }
  const float isc[2] = {cst[32 + 4 * g], cst[32 + 4 * g + 2]};  // 2^-E of the two heads' score operands

  // buffer resources over this split's part of each cache array; per-lane 32-bit offsets
  const int64_t grp = (int64_t)b * prm.Hkv + hkv;
  const int64_t tok0 = grp * prm.max_ctx + t0;
  const unsigned span = (unsigned)((t1 > t0 ? t1 - t0 : 0) + 31) & ~31u;  // tokens read by this split
  const buf_t rk = make_buf(prm.kcodes + tok0 * KREC, span * KREC);
  const buf_t rs = make_buf(QJL ? prm.ksigns + tok0 * SREC : prm.kcodes, QJL ? span * SREC : 0u);
  const buf_t rn = make_buf(prm.knorms + tok0, span * 4);
  const buf_t rr = make_buf(QJL ? prm.krnorms + tok0 : prm.knorms, QJL ? span * 4 : 0u);
  const buf_t rvn = make_buf(prm.vnorms + tok0, span * 4);
  const buf_t rv = make_buf(prm.vcodes + (grp * (prm.max_ctx / 32) + t0 / 32) * (int64_t)VBLK, (span / 32) * VBLK);
  const unsigned k_off = (unsigned)(r16 * KREC + g * (D / 32));
  const unsigned s_off = (unsigned)(r16 * SREC + g * (D / 32));
  const unsigned v_off = (unsigned)((g * (D / 4) + VWL * r16) * 4);
  const unsigned n_off = (unsigned)r16 * 4;
  // value slot of this lane's tokens (16 t + r16 sits in slot r16 % 4 of its block group)
  const float e_slot = (float)vslot_exp(r16 & 3);

  // online softmax state of the lane's two heads (identical across the 16 token lanes of group g)
  float m_run[2] = {-INFINITY, -INFINITY};  // running max (log2 units)
  float m_thr[2] = {-INFINITY, -INFINITY};  // (m_run + slack) 2^E: raise the max above this raw score
  int ev[2] = {kEvUnset, kEvUnset};          // value exponent of the head's rows
  float mk[2] = {-INFINITY, -INFINITY};      // m_run - (ev - e_slot): exp2(s - mk) = p * 2^(ev - e_slot)
  float lsum[2] = {0.f, 0.f};                // sum of p * 2^(ev - e_slot) over this lane's tokens
  f32x4 acc[NACC][NT];
#pragma unroll
  for (int a = 0; a < NACC; ++a)
#pragma unroll
    for (int q = 0; q < NT; ++q) acc[a][q] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 wacc = {0.f, 0.f, 0.f, 0.f};  // sum of w 2^ev per row (every column)
  const u32x4 ones = {pos_mask(8), pos_mask(9), pos_mask(10), pos_mask(11)};  // slot k: 2^(k - 16)

  // Raw cache data of one 32-token chunk for this lane: its key and value bit
  // words, and the norms of its two tokens (16 t + r16).
  struct Chunk {
    unsigned kpl[2][PK > 0 ? PK : 1][WPP];
    unsigned ksg[2][KW::NWQ > 0 ? KW::NWQ : 1];
    unsigned vp[VB][VWL];
    float nk[2], gm[2], nv[2];
    // an empty asm per register: a chunk that runs again after a rescale is
    // not loop-invariant to the compiler, which would otherwise hoist every
    // value derived from it out of the rerun loop (and spill them)
    __device__ void opaque() {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int p = 0; p < (PK > 0 ? PK : 1); ++p)
#pragma unroll
          for (int w = 0; w < WPP; ++w) asm volatile("" : "+v"(kpl[t][p][w]));
#pragma unroll
        for (int w = 0; w < (KW::NWQ > 0 ? KW::NWQ : 1); ++w) asm volatile("" : "+v"(ksg[t][w]));
        asm volatile("" : "+v"(nk[t]), "+v"(gm[t]), "+v"(nv[t]));
      }
#pragma unroll
      for (int p = 0; p < VB; ++p)
#pragma unroll
        for (int w = 0; w < VWL; ++w) asm volatile("" : "+v"(vp[p][w]));
    }
  };
  auto load_chunk = [&](unsigned rel, Chunk& c) {  // rel = chunk start - t0 (multiple of 32)
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      if constexpr (PK > 0) {
#pragma unroll
        for (int p = 0; p < PK; ++p)
#pragma unroll
          for (int w = 0; w < WPP; ++w) {
            const unsigned o = k_off + 16 * tile * KREC + p * (D / 8) + 4 * w;
            const unsigned x = ld32(rk, o & ~3u, rel * KREC);
            c.kpl[tile][p][w] = (D >= 128) ? x : ((o & 2u) ? (x >> 16) : (x & 0xFFFFu));
          }
      }
      if constexpr (QJL) {
#pragma unroll
        for (int Wq = 0; Wq < KW::NWQ; ++Wq) {
          const unsigned o = s_off + 16 * tile * SREC + 4 * Wq;
          const unsigned x = ld32(rs, o & ~3u, rel * SREC);
          c.ksg[tile][Wq] = (D >= 128) ? x : ((o & 2u) ? (x >> 16) : (x & 0xFFFFu));
        }
      }
      c.nk[tile] = __uint_as_float(ld32(rn, n_off + 64 * tile, rel * 4));
      c.gm[tile] = QJL ? __uint_as_float(ld32(rr, n_off + 64 * tile, rel * 4)) : 0.f;
      c.nv[tile] = __uint_as_float(ld32(rvn, n_off + 64 * tile, rel * 4));
    }
#pragma unroll
    for (int p = 0; p < VB; ++p) {
      const unsigned o = p * (4 * (D / 4) * 4) + v_off;
      const unsigned so = (rel / 32) * VBLK;
      if constexpr (VWL == 1) {
        c.vp[p][0] = ld32(rv, o, so);
      } else if constexpr (VWL == 2) {
        const uint2 t = ld64(rv, o, so);
        c.vp[p][0] = t.x;
        c.vp[p][1] = t.y;
      } else {
        const uint4 t = ld128(rv, o, so);
        c.vp[p][0] = t.x;
        c.vp[p][1] = t.y;
        c.vp[p][2] = t.z;
        c.vp[p][3] = t.w;
      }
    }
  };

  const unsigned n_rel = (unsigned)(t1 > t0 ? t1 - t0 : 0);

  using RG = DecRing<D, PK, QJL, VB, NSET>;
  constexpr int DEPTH = RG::DEPTH;
  // the wave's ring of DEPTH staged chunks
  __shared__ __attribute__((aligned(16))) uint8_t ring[RG::WAVES][DEPTH > 0 ? DEPTH : 1][DEPTH > 0 ? RG::BYTES : 16];
  // ring loads: byte ranges of each cache array over this split
  const i32x4 qk = make_rsrc4(prm.kcodes + tok0 * KREC, span * KREC);
  const i32x4 qs = make_rsrc4(QJL ? prm.ksigns + tok0 * SREC : prm.kcodes, QJL ? span * SREC : 0u);
  const i32x4 qn = make_rsrc4(prm.knorms + tok0, span * 4);
  const i32x4 qr = make_rsrc4(QJL ? prm.krnorms + tok0 : prm.knorms, QJL ? span * 4 : 0u);
  const i32x4 qvn = make_rsrc4(prm.vnorms + tok0, span * 4);
  const i32x4 qv = make_rsrc4(prm.vcodes + (grp * (prm.max_ctx / 32) + t0 / 32) * (int64_t)VBLK, (span / 32) * VBLK);
  // bytes [off, off + n) of r into dst, 16 bytes per lane per load; lane 0 is
  // active in every load, so each counts once in vmcnt (RG::LOADS per chunk)
  auto dma = [&](const i32x4& r, unsigned off, uint8_t* dst, auto NC) {
    constexpr int n = decltype(NC)::value;
    const unsigned lds = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(lds_ptr)dst);
#pragma unroll
    for (int i = 0; i < n; i += 1024) {
      if (n - i >= 1024 || lane < (n - i) / 16) lds_load16(r, off + (unsigned)(i + 16 * lane), lds + i);
    }
  };
  auto issue_chunk = [&](unsigned rel, uint8_t* dst) {
    if constexpr (PK > 0) dma(qk, rel * KREC, dst, std::integral_constant<int, 32 * KREC>{});
    if constexpr (QJL) dma(qs, rel * SREC, dst + RG::OFF_S, std::integral_constant<int, 32 * SREC>{});
    dma(qn, rel * 4, dst + RG::OFF_NK, std::integral_constant<int, 128>{});
    if constexpr (QJL) dma(qr, rel * 4, dst + RG::OFF_GM, std::integral_constant<int, 128>{});
    dma(qvn, rel * 4, dst + RG::OFF_NV, std::integral_constant<int, 128>{});
    dma(qv, (rel / 32) * VBLK, dst + RG::OFF_V, std::integral_constant<int, VBLK>{});
  };
  // this lane's words of a staged chunk (the same offsets load_chunk reads in HBM)
  auto read_chunk = [&](const uint8_t* src, Chunk& c) {
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      if constexpr (PK > 0) {
#pragma unroll
        for (int p = 0; p < PK; ++p)
#pragma unroll
          for (int w = 0; w < WPP; ++w) {
            const unsigned o = k_off + 16 * tile * KREC + p * (D / 8) + 4 * w;
            const unsigned x = *(const unsigned*)(src + (o & ~3u));
            c.kpl[tile][p][w] = (D >= 128) ? x : ((o & 2u) ? (x >> 16) : (x & 0xFFFFu));
          }
      }
      if constexpr (QJL) {
#pragma unroll
        for (int Wq = 0; Wq < KW::NWQ; ++Wq) {
          const unsigned o = s_off + 16 * tile * SREC + 4 * Wq;
          const unsigned x = *(const unsigned*)(src + RG::OFF_S + (o & ~3u));
          c.ksg[tile][Wq] = (D >= 128) ? x : ((o & 2u) ? (x >> 16) : (x & 0xFFFFu));
        }
      }
      c.nk[tile] = *(const float*)(src + RG::OFF_NK + n_off + 64 * tile);
      c.gm[tile] = QJL ? *(const float*)(src + RG::OFF_GM + n_off + 64 * tile) : 0.f;
      c.nv[tile] = *(const float*)(src + RG::OFF_NV + n_off + 64 * tile);
    }
#pragma unroll
    for (int p = 0; p < VB; ++p) {
      const uint8_t* vsrc = src + RG::OFF_V + p * (4 * D) + v_off;
      if constexpr (VWL == 1) {
        c.vp[p][0] = *(const unsigned*)vsrc;
      } else if constexpr (VWL == 2) {
        const uint2 t = *(const uint2*)vsrc;
        c.vp[p][0] = t.x;
        c.vp[p][1] = t.y;
      } else {
        const uint4 t = *(const uint4*)vsrc;
        c.vp[p][0] = t.x;
        c.vp[p][1] = t.y;
        c.vp[p][2] = t.z;
        c.vp[p][3] = t.w;
      }
    }
  };

  int pend = 0;                       // 1: raise the running max; 2: lower the value exponent
  float pend_val[2] = {0.f, 0.f};     // lane values per head that triggered it
  unsigned (*wrow)[8][kWRow] = wt_lds[wave];

  // One chunk: 0 = accumulated, otherwise the pend code (nothing accumulated).
  // mask_c: the chunk runs past the context (only a split's last chunk can);
  // mid() runs once per chunk (first pass), after the key phase has consumed
  // the chunk's key words
  auto step = [&](unsigned rel, Chunk& cur, auto mask_c, bool first, auto&& mid) -> int {
    constexpr bool MASK = decltype(mask_c)::value;
    cur.opaque();
    // ---------------- scores: two tiles of 16 tokens ----------------
    f32x4 cm[2], cq[2];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      cm[tile] = f32x4{cm_init[0], cm_init[1], cm_init[2], cm_init[3]};
      cq[tile] = f32x4{cq_init[0], cq_init[1], cq_init[2], cq_init[3]};
    }
    // key words of fragment group W (one Walsh subset / the sign plane) for both tiles
    auto key_words = [&](int W, unsigned (&word)[2]) {
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) {
        if (W >= KW::NWM) {
          if constexpr (QJL) word[tile] = cur.ksg[tile][W - KW::NWM];
        } else if constexpr (PK > 0) {
          if constexpr (D >= 128) {
            const int s = W / (D / 128), w = W % (D / 128);
            const int mask = walsh_mask(PK, s);
            word[tile] = 0u;
#pragma unroll
            for (int p = 0; p < PK; ++p)
              if (mask >> p & 1) word[tile] ^= cur.kpl[tile][p][w];
          } else {
            unsigned lo16 = 0u, hi16 = 0u;
            const int s0 = 2 * W, s1 = 2 * W + 1;
            const int m0 = walsh_mask(PK, s0);
            const int m1 = s1 < KW::WK ? walsh_mask(PK, s1) : 0;
#pragma unroll
            for (int p = 0; p < PK; ++p) {
              if (m0 >> p & 1) lo16 ^= cur.kpl[tile][p][0];
              if (m1 >> p & 1) hi16 ^= cur.kpl[tile][p][0];
            }
            word[tile] = (lo16 & 0xFFFFu) | (hi16 << 16);
          }
        }
      }
    };
    unsigned kw[KW::NW][2];
#pragma unroll
    for (int W = 0; W < KW::NW; ++W) key_words(W, kw[W]);
    // fragment f = 4 W + r scores both tiles: word W, nibble r. The two bit operands
    // of fragment f + 1 are built while fragment f's MFMAs run, so no MFMA waits on
    // the VALU that wrote its operand
    u32x4 kop_next[2] = {bit_operand(kw[0][0], 0), bit_operand(kw[0][1], 0)};
#pragma unroll
    for (int f = 0; f < KW::NF; ++f) {
      const u32x4 op0 = kop_next[0], op1 = kop_next[1];
      if (f + 1 < KW::NF) {
        kop_next[0] = bit_operand(kw[(f + 1) / 4][0], (f + 1) % 4);
        kop_next[1] = bit_operand(kw[(f + 1) / 4][1], (f + 1) % 4);
      }
      const u32x4 bf = kfrag(f);
      if (f / 4 < KW::NWM) {
        cm[0] = mfma16(bf, op0, cm[0]);
        cm[1] = mfma16(bf, op1, cm[1]);
      } else {
        cq[0] = mfma16(bf, op0, cq[0]);
        cq[1] = mfma16(bf, op1, cq[1]);
      }
      // keep the operand construction next to its MFMAs (hoisting it all costs registers)
      __builtin_amdgcn_sched_barrier(0);
    }
    if (first) mid();
    // this lane: token 16 t + r16 of the chunk, heads 2g (rows 4g, 4g+1) and 2g + 1 (rows 4g+2, 4g+3);
    // raw scores sr = score 2^E (the operand exponent is applied in the exp2 argument)
    float sr[2][2];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      const float cmv[4] = {cm[tile].x, cm[tile].y, cm[tile].z, cm[tile].w};
      const float cqv[4] = {cq[tile].x, cq[tile].y, cq[tile].z, cq[tile].w};
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float sc = cmv[2 * hh] + cmv[2 * hh + 1];
        if constexpr (QJL) sc = fmaf(cur.gm[tile], cqv[2 * hh] + cqv[2 * hh + 1], sc);
        sr[tile][hh] = cur.nk[tile] * sc;
        if constexpr (MASK) {
          if (rel + 16 * tile + r16 >= n_rel) sr[tile][hh] = -INFINITY;
        }
      }
    }
    // ---------------- online softmax: lane-local checks, no cross-lane work ----------------
    const float mx0 = fmaxf(sr[0][0], sr[1][0]), mx1 = fmaxf(sr[0][1], sr[1][1]);
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(mx0 > m_thr[0] || mx1 > m_thr[1]) != 0, 0)) {
      pend_val[0] = mx0 * isc[0];
      pend_val[1] = mx1 * isc[1];
      return 1;
    }
    float wv[2][2], pk[2][2];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        pk[tile][hh] = __builtin_amdgcn_exp2f(fmaf(sr[tile][hh], isc[hh], -mk[hh]));  // p 2^(ev - e_slot)
        float w = pk[tile][hh] * cur.nv[tile];
        if constexpr (MASK) w = pk[tile][hh] > 0.f ? w : 0.f;  // masked tokens may hold garbage norms
        wv[tile][hh] = w;
      }
    const float wm0 = fmaxf(wv[0][0], wv[1][0]), wm1 = fmaxf(wv[0][1], wv[1][1]);
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(fmaxf(wm0, wm1) >= kWeightOperandMax) != 0, 0)) {
      // largest unscaled weight of this lane per head: w 2^(e_slot - ev); nothing accumulated
      pend_val[0] = wm0 * exp2f(e_slot - (float)ev[0]);
      pend_val[1] = wm1 * exp2f(e_slot - (float)ev[1]);
      return 2;
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) lsum[hh] += pk[0][hh] + pk[1][hh];
    if (prm.scores_dbg) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int h = 2 * g + hh;
        if (h < prm.chunk_heads) {
          float* dst = prm.scores_dbg + ((int64_t)b * prm.Hq + hq0 + h) * prm.max_ctx + t0;
#pragma unroll
          for (int tile = 0; tile < 2; ++tile) {
            const unsigned tt = rel + 16 * tile + r16;
            if (tt < n_rel) dst[tt] = sr[tile][hh] * isc[hh] * kLn2;
          }
        }
      }
    }
    // ---------------- weights: token lanes -> row lanes through LDS ----------------
    // dword r16 of row (version, head) holds (tile 0, tile 1) of token r16 as fp16 hi
    // parts, dword 16 + r16 the lo parts: K elements 2k, 2k + 1 of value lane group
    // g' are tokens 4g' + k and 16 + 4g' + k, so a value lane reads 4 whole dwords
#pragma unroll
    for (int v = 0; v < NVER; ++v) {
      float rho = 1.0f;
#pragma unroll
      for (int s = 0, n = 0; s < WV; ++s)
        if (!walsh_is_lead(VB, NSET, s)) {
          if (++n == v) rho = prm.vrho[s];
        }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const float x0 = v ? wv[0][hh] * rho : wv[0][hh], x1 = v ? wv[1][hh] * rho : wv[1][hh];
        unsigned* row = wrow[v][2 * g + hh];
        row[r16] = f16_pair_rne(x0, x1);
        row[16 + r16] = split_pair(x0, x1, -1.0f);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // ---------------- values ----------------
    // A operand of version v: the hi (even rows) or lo (odd rows) parts of head r16 / 2
    auto a_operand = [&](int v) -> u32x4 {
      return *(const u32x4*)&wrow[v][r16 >> 1][16 * (r16 & 1) + 4 * g];
    };
    const u32x4 a_lead = a_operand(0);
    u32x4 af[NVER];
    af[0] = a_lead;
#pragma unroll
    for (int v = 1; v < NVER; ++v) af[v] = a_operand(v);
    // value words of every subset (XORs of the planes), then MFMA i: subset i / (4 VWL),
    // word (i / 4) % VWL, nibble i % 4, operands built one MFMA ahead
    unsigned vw[WV][VWL];
#pragma unroll
    for (int s = 0; s < WV; ++s)
#pragma unroll
      for (int w = 0; w < VWL; ++w) {
        unsigned word = 0u;
#pragma unroll
        for (int p = 0; p < VB; ++p)
          if (walsh_mask(VB, s) >> p & 1) word ^= cur.vp[p][w];
        vw[s][w] = word;
      }
    constexpr int NVI = 4 * VWL * WV;
    auto vop = [&](int i) { return bit_operand(vw[i / (4 * VWL)][(i / 4) % VWL], i % 4); };
    u32x4 vop_next[2] = {vop(0), vop(1)};  // operands two MFMAs ahead
#pragma unroll
    for (int i = 0; i < NVI; ++i) {
      const int s = i / (4 * VWL), q = i % (4 * VWL);
      const u32x4 op = vop_next[i % 2];
      if (i + 2 < NVI) vop_next[i % 2] = vop(i + 2);
      int ver = 0;  // weight version of subset s: 0 for a lead, else its rank among the others
#pragma unroll
      for (int t = 0; t <= s; ++t)
        if (!walsh_is_lead(VB, NSET, t)) ++ver;
      if (walsh_is_lead(VB, NSET, s)) ver = 0;
      const int set = walsh_set(VB, NSET, s);
      acc[set][q] = mfma16(af[ver], op, acc[set][q]);
      __builtin_amdgcn_sched_barrier(0);
    }
    wacc = mfma16(a_lead, ones, wacc);
    return 0;
  };

  // The hot loop touches the accumulators only with MFMAs. When a chunk needs
  // the running max raised or the value exponent lowered, it is not
  // accumulated: the state is rescaled here and the chunk runs again.
  auto rescale = [&]() {
    // group-wide maxima over the 16 token lanes of this lane group (heads 2g, 2g + 1)
    float f[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      float v = pend_val[hh];
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
      f[hh] = 1.0f;
      if (pend == 1) {
        const float m_new = fmaxf(m_run[hh], v);
        // 0 on the first chunk (m_run = -inf); the state is still zero then
        if (m_new > -INFINITY) f[hh] = exp2f(m_run[hh] - m_new);
        m_run[hh] = m_new;
      } else {
        const int e_need = range_exp(v);  // v: the head's largest weight in this chunk
        const int ev_new = e_need < ev[hh] ? e_need : ev[hh];
        f[hh] = ldexpf(1.0f, ev_new - ev[hh]);
        ev[hh] = ev_new;
      }
      m_thr[hh] = (m_run[hh] + kRescaleSlack) / isc[hh];
      mk[hh] = m_run[hh] - ((float)ev[hh] - e_slot);
      lsum[hh] *= f[hh];
    }
    // value rows 4g .. 4g+3 of every lane in this group are heads 2g (x, y) and 2g + 1 (z, w)
#pragma unroll
    for (int a = 0; a < NACC; ++a)
#pragma unroll
      for (int q = 0; q < NT; ++q) {
        acc[a][q].x *= f[0];
        acc[a][q].y *= f[0];
        acc[a][q].z *= f[1];
        acc[a][q].w *= f[1];
      }
    wacc.x *= f[0];
    wacc.y *= f[0];
    wacc.z *= f[1];
    wacc.w *= f[1];
  };
  auto run = [&](unsigned rel, Chunk& cur, auto mask_c, auto&& mid) {
    bool first = true;
    while ((pend = step(rel, cur, mask_c, first, mid)) != 0) {
      rescale();
      first = false;
    }
  };
  // chunks [0, n_full) lie inside the context; a last partial chunk runs masked
  const unsigned n_full = n_rel & ~31u;
  if constexpr (DEPTH == 0) {
    // registers: the next chunk loads while this one computes, then moves in
    Chunk cur, nxt;
    if (n_rel > 0) load_chunk(0, cur);
    unsigned rel = 0;
    for (; rel < n_full; rel += 32) {
      if (rel + 32 < n_rel) load_chunk(rel + 32, nxt);
      run(rel, cur, std::false_type{}, [] {});
      cur = nxt;
    }
    if (rel < n_rel) run(rel, cur, std::true_type{}, [] {});
  } else {
    // LDS ring: chunk c sits in slot c % DEPTH. Before a chunk is read, the
    // loads of the (up to DEPTH - 1) chunks issued after it may stay in
    // flight; once its key phase has run, its slot is refilled with chunk
    // c + DEPTH. One chunk per loop iteration keeps the register allocation
    // of a single step.
    for (int j = 0; j < DEPTH; ++j)
      if (32u * j < n_rel) issue_chunk(32u * j, ring[wave][j]);
    const unsigned last = (n_rel - 1) / 32;  // index of the split's last chunk
    int slot = 0;
    auto body = [&](unsigned rel, auto mask_c) {
      uint8_t* sb = ring[wave][slot];
      // the debug score stores also count in vmcnt, so that mode waits for all
      const unsigned ahead = min(last - rel / 32, (unsigned)(DEPTH - 1));
      if (prm.scores_dbg || ahead == 0) wait_vmcnt<0>();
      else if (ahead == 1) wait_vmcnt<RG::LOADS>();
      else wait_vmcnt<(DEPTH > 2 ? 2 : 1) * RG::LOADS>();
      Chunk cur;
      read_chunk(sb, cur);
      run(rel, cur, mask_c, [&] {
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // the slot's reads have landed
        if (rel + 32u * DEPTH < n_rel) issue_chunk(rel + 32u * DEPTH, sb);
      });
      slot = slot + 1 == DEPTH ? 0 : slot + 1;
    };
    unsigned rel = 0;
    for (; rel < n_full; rel += 32) body(rel, std::false_type{});
    if (rel < n_rel) body(rel, std::true_type{});
  }

  // ---------------- write this split's partial state ----------------
  // softmax denominator per head: sum over the 16 token lanes of lsum 2^(e_slot - ev)
  float l_acc[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    float l = lsum[hh] * exp2f(e_slot - (float)ev[hh]);
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) l += __shfl_xor(l, o);
    l_acc[hh] = l;
  }
  const int64_t hq_base = (int64_t)b * prm.Hq + hq0;
  if (r16 == 0) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int h = 2 * g + hh;
      if (h < prm.chunk_heads) {
        float* ml = prm.part_ml + ((hq_base + h) * prm.n_splits + split) * 2;
        ml[0] = m_run[hh];
        ml[1] = l_acc[hh];
      }
    }
  }
  // sum of w 2^ev per head, in the value lanes' row order (rows 4g .. 4g+3)
  const float wt[2] = {wacc.x + wacc.y, wacc.z + wacc.w};
  // value lanes: coordinate lane r16 (coords (D/16) r16 + q), rows 4g .. 4g+3 = heads 2g, 2g+1 (hi, lo)
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int h = 2 * g + hh;
    if (h >= prm.chunk_heads) continue;
    const float unscale = ldexpf(1.0f, -ev[hh]);
    const float wh = wt[hh] * 4.0f;  // the ones operand reads 2^(k - 16) against 2^(14 - k)
    float outv[NT];
#pragma unroll
    for (int q = 0; q < NT; ++q) {
      // sum_t w_t c[idx_t] = sum_s a_s (2 sum_t w_t bit_s - sum_t w_t)
      float v = -wh * prm.vcoef_sum;
#pragma unroll
      for (int j = 0; j < NSET; ++j) {
        const float c2 = (hh ? (acc[j][q].z + acc[j][q].w) : (acc[j][q].x + acc[j][q].y)) * 4.0f;
        v = fmaf(2.f * prm.vlead[j], c2, v);
      }
      outv[q] = v * unscale;
    }
    float* dst = prm.part_acc + ((hq_base + h) * prm.n_splits + split) * D + (D / 16) * r16;
#pragma unroll
    for (int q = 0; q < NT; q += 4) *(float4*)(dst + q) = float4{outv[q], outv[q + 1], outv[q + 2], outv[q + 3]};
  }
}

struct DecCombineParams {
  const float* part_acc;
  const float* part_ml;
  const float* pv[kMaxKvHeads];
  float* out;
  int n_splits, Hq, Hkv, group, chunk_heads, n_chunks;
};

// One block of 512 threads per (batch, query head): the weights 2^(m_s - M) / L
// of every split (block reductions), the merged rotated-space accumulator
// (thread (quad, phase) sums phase, phase + P, ... of its four coordinates with
// 16-byte loads, then the phases are added in LDS), and out = Pi_V^T acc.
constexpr int kCombineThreads = 512;
template <int D>
__global__ __launch_bounds__(kCombineThreads) void decode_combine_kernel(DecCombineParams prm) {
  extern __shared__ float wsplit[];  // [n_splits]
  constexpr int NQ = D / 4;                   // coordinate quads
  constexpr int P = kCombineThreads / NQ;     // split phases
  __shared__ float4 part[P][NQ];
  __shared__ float o[D];
  __shared__ float red[2][kCombineThreads / 64];
  const int64_t bhq = blockIdx.x;
  const int hq = (int)(bhq % prm.Hq);
  const int hkv = hq / prm.group;
  const int ns = prm.n_splits;
  const float* ml = prm.part_ml + bhq * ns * 2;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // this thread's column entries of Pi_V for the final out = Pi_V^T acc, in
  // flight while the splits are merged: thread (i, phase) holds rows phase,
  // phase + R, ... of column i
  constexpr int R = kCombineThreads / D;
  constexpr int NJ = D / R;
  const float* Pv = prm.pv[hkv];
  const int i = t % D, pr = t / D;
  float pvv[NJ];
#pragma unroll
  for (int u = 0; u < NJ; ++u) pvv[u] = Pv[(int64_t)(pr + u * R) * D + i];
  float mx = -INFINITY;
  for (int s = t; s < ns; s += kCombineThreads)
    if (ml[2 * s + 1] > 0.f) mx = fmaxf(mx, ml[2 * s]);
#pragma unroll
  for (int o2 = 32; o2 > 0; o2 >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o2));
  if (lane == 0) red[0][wave] = mx;
  __syncthreads();
  float M = red[0][0];
#pragma unroll
  for (int w = 1; w < kCombineThreads / 64; ++w) M = fmaxf(M, red[0][w]);
  float lsum = 0.f;
  for (int s = t; s < ns; s += kCombineThreads) {
    const float l = ml[2 * s + 1];
    const float w = l > 0.f ? exp2f(ml[2 * s] - M) : 0.f;
    wsplit[s] = w;
    lsum += w * l;
  }
#pragma unroll
  for (int o2 = 32; o2 > 0; o2 >>= 1) lsum += __shfl_xor(lsum, o2);
  if (lane == 0) red[1][wave] = lsum;
  __syncthreads();  // also publishes wsplit
  float L = red[1][0];
#pragma unroll
  for (int w = 1; w < kCombineThreads / 64; ++w) L += red[1][w];
  const float invL = L > 0.f ? 1.0f / L : 0.f;
  const int quad = t % NQ, ph = t / NQ;
  const float4* acc = (const float4*)(prm.part_acc + bhq * (int64_t)ns * D) + quad;
  float4 a[4] = {};
  int s = ph;
  for (; s + 3 * P < ns; s += 4 * P) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float w = wsplit[s + u * P];
      const float4 v = acc[(int64_t)(s + u * P) * NQ];
      a[u].x = fmaf(w, v.x, a[u].x);
      a[u].y = fmaf(w, v.y, a[u].y);
      a[u].z = fmaf(w, v.z, a[u].z);
      a[u].w = fmaf(w, v.w, a[u].w);
    }
  }
  for (; s < ns; s += P) {
    const float w = wsplit[s];
    const float4 v = acc[(int64_t)s * NQ];
    a[0].x = fmaf(w, v.x, a[0].x);
    a[0].y = fmaf(w, v.y, a[0].y);
    a[0].z = fmaf(w, v.z, a[0].z);
    a[0].w = fmaf(w, v.w, a[0].w);
  }
  part[ph][quad] = float4{(a[0].x + a[1].x) + (a[2].x + a[3].x), (a[0].y + a[1].y) + (a[2].y + a[3].y),
                          (a[0].z + a[1].z) + (a[2].z + a[3].z), (a[0].w + a[1].w) + (a[2].w + a[3].w)};
  __syncthreads();
  if (t < D) {
    float v = 0.f;
#pragma unroll
    for (int p = 0; p < P; ++p) v += ((const float*)part[p])[t];
    o[t] = v * invL;
  }
  __syncthreads();
  // out[i] = sum_j Pi_V[j][i] o[j]: thread (i, phase) sums rows phase, phase + R, ...
  float b4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < NJ; ++u) b4[u & 3] = fmaf(pvv[u], o[pr + u * R], b4[u & 3]);
  float* pb = (float*)part;
  pb[pr * D + i] = (b4[0] + b4[1]) + (b4[2] + b4[3]);
  __syncthreads();
  if (t < D) {
    float v = 0.f;
#pragma unroll
    for (int p = 0; p < R; ++p) v += pb[p * D + t];
    prm.out[bhq * D + t] = v;
  }
}

}  // namespace

tq_status plan_decode(const tq_attn_shape* s, const tq_quantizer* k0, const tq_quantizer* v0,
                      DecodePlan* p) {
  p->batch = s->batch;
  p->n_q_heads = s->n_q_heads;
  p->n_kv_heads = s->n_kv_heads;
  p->d = s->head_dim;
  p->group = s->n_q_heads / s->n_kv_heads;
  p->chunk_heads = p->group < 8 ? p->group : 8;
  p->n_chunks = p->group / p->chunk_heads;
  p->max_ctx = s->max_ctx;
  p->k_planes = k0->planes;
  p->k_qjl = k0->variant == TQ_PROD;
  p->k_walsh = k0->planes > 0 ? 1 << (k0->planes - 1) : 0;
  p->v_bits = v0->bits;
  p->v_walsh = 1 << (v0->bits - 1);
  const int d = p->d;
  const int nwm = p->k_planes == 0 ? 0 : (d >= 128 ? p->k_walsh * (d / 128) : (p->k_walsh + 1) / 2);
  const int nwq = p->k_qjl ? (d >= 128 ? d / 128 : 1) : 0;
  p->k_words = nwm + nwq;
  const int64_t units = (int64_t)p->batch * p->n_kv_heads * p->n_chunks;
  // one round of waves (the main kernel holds 8 per CU), splits of at least 256 tokens
  const int64_t target = (int64_t)8 * device_cus();
  int64_t ns = (target + units - 1) / units;
  const int64_t max_splits = (p->max_ctx + 255) / 256;
  if (ns > max_splits) ns = max_splits;
  if (ns > 4096) ns = 4096;  // the combine keeps one weight per split in LDS
  if (ns < 1) ns = 1;
  int64_t st = (p->max_ctx + ns - 1) / ns;
  st = (st + 31) / 32 * 32;
  ns = (p->max_ctx + st - 1) / st;
  p->n_splits = (int)ns;
  p->split_tokens = st;
  p->frag_bytes = (size_t)units * 4 * p->k_words * 64 * 16;
  p->const_bytes = (size_t)units * kConstsPerUnit * sizeof(float);
  p->partial_bytes = (size_t)p->batch * p->n_q_heads * ns * (d + 2) * sizeof(float);
  auto align = [](size_t x) { return (x + 255) / 256 * 256; };
  p->total_bytes = align(p->frag_bytes) + align(p->const_bytes) + align(p->partial_bytes);
  return TQ_OK;
}

tq_status launch_decode(const DecodePlan& p, const void* q, const tq_packed_kv* k, const tq_packed_kv* v,
                        const int32_t* ctx_lens, float scale, float* out, float* scores_dbg,
                        void* workspace, hipStream_t stream, const AppendLaunch* app) {
  auto align = [](size_t x) { return (x + 255) / 256 * 256; };
  unsigned char* ws = (unsigned char*)workspace;
  u32x4* frag = (u32x4*)ws;
  float* consts = (float*)(ws + align(p.frag_bytes));
  float* part_acc = (float*)(ws + align(p.frag_bytes) + align(p.const_bytes));
  float* part_ml = part_acc + (size_t)p.batch * p.n_q_heads * p.n_splits * p.d;
  const tq_quantizer* k0 = k->qz[0];
  const tq_quantizer* v0 = v->qz[0];
  const int units = p.batch * p.n_kv_heads * p.n_chunks;

  DecPrepParams pp{};
  pp.q = (const uint16_t*)q;
  for (int h = 0; h < p.n_kv_heads; ++h) {
    pp.pk[h] = k->qz[h]->pi32;
    pp.sk[h] = k->qz[h]->s32;
  }
  pp.frag = frag;
  pp.consts = consts;
  pp.Hq = p.n_q_heads;
  pp.Hkv = p.n_kv_heads;
  pp.group = p.group;
  pp.chunk_heads = p.chunk_heads;
  pp.n_chunks = p.n_chunks;
  pp.n_units = units;

  pp.scale_log2e = scale * kLog2e;
  pp.kappa = (float)(std::sqrt(M_PI / 2.0) / p.d);
  for (int s = 0; s < k0->cb.n_walsh; ++s) pp.kcoef[s] = k0->cb.walsh_coef[s];
  if (app) {
    AppendArgs& a = pp.app;
    a.ctx_lens = ctx_lens;
    a.max_ctx = p.max_ctx;
    a.k_planes = k0->planes;
    a.v_bits = v0->bits;
    a.k_prod = k0->variant == TQ_PROD;
    a.x_bf16 = app->x_dtype == TQ_BF16;
    a.k_new = app->k_new;
    a.v_new = app->v_new;
    for (int h = 0; h < p.n_kv_heads; ++h) {
      a.k_pi[h] = k->qz[h]->pi32;
      a.k_sp[h] = k->qz[h]->sp32;
      a.v_pi[h] = v->qz[h]->pi32;
    }
    const Codebook& kc = k0->cb;
    const Codebook& vc = v0->cb;
    for (int i = 0; i < 15; ++i) {
      a.k_thr[i] = i + 1 < (1 << kc.planes) ? kc.thresholds[i] : 0.f;
      a.v_thr[i] = i + 1 < (1 << vc.planes) ? vc.thresholds[i] : 0.f;
    }
    for (int i = 0; i < 16; ++i) {
      a.k_cen[i] = i < (1 << kc.planes) ? kc.centroids[i] : 0.f;
      a.v_cen[i] = i < (1 << vc.planes) ? vc.centroids[i] : 0.f;
    }
    a.k_codes = (uint32_t*)const_cast<uint8_t*>(k->codes);
    a.k_signs = (uint32_t*)const_cast<uint8_t*>(k->signs);
    a.k_norms = const_cast<float*>(k->norms);
    a.k_rnorms = const_cast<float*>(k->rnorms);
    a.v_codes = (uint32_t*)const_cast<uint8_t*>(v->codes);
    a.v_norms = const_cast<float*>(v->norms);
    a.rot_dbg = app->rot_dbg;
    a.proj_dbg = app->proj_dbg;
  }
  const int prep_blocks = units * kPrepSlices + (app ? 2 * p.batch * p.n_kv_heads : 0);

  DecMainParams mp{};
  mp.frag = frag;
  mp.consts = consts;
  mp.kcodes = k->codes;
  mp.ksigns = k->signs;
  mp.knorms = k->norms;
  mp.krnorms = k->rnorms;
  mp.vcodes = v->codes;
  mp.vnorms = v->norms;
  mp.ctx_lens = ctx_lens;
  mp.len_add = app ? 1 : 0;
  mp.part_acc = part_acc;
  mp.part_ml = part_ml;
  mp.scores_dbg = scores_dbg;
  mp.max_ctx = p.max_ctx;
  mp.split_tokens = p.split_tokens;
  mp.n_splits = p.n_splits;
  mp.Hq = p.n_q_heads;
  mp.Hkv = p.n_kv_heads;
  mp.group = p.group;
  mp.chunk_heads = p.chunk_heads;
  mp.n_chunks = p.n_chunks;
  // value subsets: sets, leads and ratios (a_s / a_lead must not exceed 1)
  const int vb = v0->bits;
  const int nset = value_sets(p.d, vb);
  float csum = 0.f;
  for (int s = 0; s < v0->cb.n_walsh; ++s) csum += v0->cb.walsh_coef[s];
  mp.vcoef_sum = csum;
  for (int s = 0; s < v0->cb.n_walsh; ++s) {
    if (walsh_is_lead(vb, nset, s)) mp.vlead[walsh_set(vb, nset, s)] = v0->cb.walsh_coef[s];
  }
  for (int s = 0; s < v0->cb.n_walsh; ++s) {
    const float lead = mp.vlead[walsh_set(vb, nset, s)];
    const float rho = walsh_is_lead(vb, nset, s) ? 1.0f : v0->cb.walsh_coef[s] / lead;
    if (!(std::fabs(rho) <= 1.0f)) return set_error(TQ_ERR_UNSUPPORTED, "decode: value codebook coefficients out of order");
    mp.vrho[s] = rho;
  }

  DecCombineParams cp{};
  cp.part_acc = part_acc;
  cp.part_ml = part_ml;
  for (int h = 0; h < p.n_kv_heads; ++h) cp.pv[h] = v->qz[h]->pi32;
  cp.out = out;
  cp.n_splits = p.n_splits;
  cp.Hq = p.n_q_heads;
  cp.Hkv = p.n_kv_heads;
  cp.group = p.group;
  cp.chunk_heads = p.chunk_heads;
  cp.n_chunks = p.n_chunks;

  return dispatch_dim(p.d, [&](auto DC) -> tq_status {
    constexpr int D = decltype(DC)::value;
    return dispatch_planes(p.k_planes, [&](auto KPC) -> tq_status {
      constexpr int PK = decltype(KPC)::value;
      return dispatch_bool(p.k_qjl, [&](auto QC) -> tq_status {
        constexpr bool QJL = decltype(QC)::value;
        if constexpr ((!QJL && PK == 0) || (QJL && PK > 3)) {
          return set_error(TQ_ERR_UNSUPPORTED, "decode: unsupported key quantizer");
        } else {
          hipLaunchKernelGGL((decode_prep_kernel<D, PK, QJL>), dim3((unsigned)prep_blocks), dim3(4 * D), 0, stream, pp);
          tq_status st = launch_check("decode: prep launch");
          if (st != TQ_OK) return st;
          st = dispatch_planes(p.v_bits, [&](auto VBC) -> tq_status {
            constexpr int VB = decltype(VBC)::value;
            if constexpr (VB == 0) {
              return set_error(TQ_ERR_UNSUPPORTED, "decode: value bits");
            } else {
              constexpr int NSET = value_sets(D, VB);
              dim3 grid((unsigned)((p.n_splits + 3) / 4), (unsigned)units);
              hipLaunchKernelGGL((decode_main_kernel<D, PK, QJL, VB, NSET>), grid, dim3(kThreads), 0, stream, mp);
              return launch_check("decode: main launch");
            }
          });
          if (st != TQ_OK) return st;
          hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((unsigned)(p.batch * p.n_q_heads)),
                             dim3(kCombineThreads), (size_t)p.n_splits * sizeof(float), stream, cp);
          return launch_check("decode: combine launch");
        }
      });
    });
  });
}


// ---------------------------------------------------------------------------
// Scratch of tq_decode_attention_noalloc: the decode workspace (score
// fragments, constants and split partials) as a file-scope device array, for
// callers that cannot allocate. Each GPU the library runs on holds its own
// copy until the process ends. In host code "scratch" names a host-side
// stand-in; the device address comes from hipGetSymbolAddress, looked up once
// per device with that device current, and only that address is used.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];
}  // namespace

tq_status noalloc_scratch(void** ptr) {
  int dev = -1;
  tq_status st = check_hip(hipGetDevice(&dev), "noalloc: hipGetDevice");
  if (st != TQ_OK) return st;
  if (dev < 0 || dev >= kMaxScratchDevices)
    return set_error(TQ_ERR_UNSUPPORTED, "noalloc: device index " + std::to_string(dev) + " out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    st = check_hip(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "noalloc: hipGetSymbolAddress(scratch)");
    if (st != TQ_OK) return st;
    if (!p) return set_error(TQ_ERR_DEVICE, "noalloc: scratch has no device address");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return TQ_OK;
}

}  // namespace tq
