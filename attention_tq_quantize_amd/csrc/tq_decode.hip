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

struct DecPrepParams {
  const uint16_t* q;
  const float* pk[kMaxKvHeads];
  const float* sk[kMaxKvHeads];
  u32x4* frag;
  float* consts;
  int Hq, Hkv, group, chunk_heads, n_chunks;
  float scale_log2e;
  float kappa;
  float kcoef[kMaxWalsh];
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

// One workgroup of D threads per (batch, query head): thread j computes
// q'_j = (Pi_K q)_j and q''_j = (S_K q)_j, then the workgroup writes this head's
// two MFMA rows (hi, lo) of every score-operand fragment and of the constants.
// The workgroup of the chunk's first head also zero-fills unused rows.
template <int D, int PK, bool QJL>
__global__ __launch_bounds__(D) void decode_prep_kernel(DecPrepParams prm) {
  using KW = KWords<D, PK, QJL>;
  __shared__ float qs[D], qp[D], qq[D];
  __shared__ float red[4][D / 64];
  const int bhq = blockIdx.x;
  const int b = bhq / prm.Hq, hq = bhq % prm.Hq;
  const int hkv = hq / prm.group;
  const int in_group = hq % prm.group;
  const int chunk = in_group / prm.chunk_heads, h = in_group % prm.chunk_heads;
  const int bhc = (b * prm.Hkv + hkv) * prm.n_chunks + chunk;
  const int j = threadIdx.x;
  qs[j] = bf16_val(prm.q[(int64_t)bhq * D + j]);
  __syncthreads();
  const float4* prow = (const float4*)(prm.pk[hkv] + (int64_t)j * D);
  const float4* srow = QJL ? (const float4*)(prm.sk[hkv] + (int64_t)j * D) : nullptr;
  float a0 = 0.f, a1 = 0.f, c0 = 0.f, c1 = 0.f;
#pragma unroll 4
  for (int k = 0; k < D / 4; k += 2) {
    const float4 p0 = prow[k], p1 = prow[k + 1];
    a0 += p0.x * qs[4 * k] + p0.y * qs[4 * k + 1] + p0.z * qs[4 * k + 2] + p0.w * qs[4 * k + 3];
    a1 += p1.x * qs[4 * k + 4] + p1.y * qs[4 * k + 5] + p1.z * qs[4 * k + 6] + p1.w * qs[4 * k + 7];
    if constexpr (QJL) {
      const float4 s0 = srow[k], s1 = srow[k + 1];
      c0 += s0.x * qs[4 * k] + s0.y * qs[4 * k + 1] + s0.z * qs[4 * k + 2] + s0.w * qs[4 * k + 3];
      c1 += s1.x * qs[4 * k + 4] + s1.y * qs[4 * k + 5] + s1.z * qs[4 * k + 6] + s1.w * qs[4 * k + 7];
    }
  }
  const float vp = a0 + a1, vq = c0 + c1;
  qp[j] = vp;
  qq[j] = vq;
  // per-head sums and maxima (wave reductions, then across the D/64 waves)
  float s_p = vp, s_q = vq, m_p = fabsf(vp), m_q = fabsf(vq);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    s_p += __shfl_xor(s_p, o);
    s_q += __shfl_xor(s_q, o);
    m_p = fmaxf(m_p, __shfl_xor(m_p, o));
    m_q = fmaxf(m_q, __shfl_xor(m_q, o));
  }
  if ((j & 63) == 0) {
    red[0][j / 64] = s_p;
    red[1][j / 64] = s_q;
    red[2][j / 64] = m_p;
    red[3][j / 64] = m_q;
  }
  __syncthreads();
  float sum_p = 0.f, sum_q = 0.f, max_p = 0.f, max_q = 0.f;
#pragma unroll
  for (int w = 0; w < D / 64; ++w) {
    sum_p += red[0][w];
    sum_q += red[1][w];
    max_p = fmaxf(max_p, red[2][w]);
    max_q = fmaxf(max_q, red[3][w]);
  }
  float amax = 0.f, asum = 0.f;
  for (int s = 0; s < KW::WK; ++s) {
    amax = fmaxf(amax, fabsf(prm.kcoef[s]));
    asum += prm.kcoef[s];
  }
  // one exponent for both score parts: the main loop scales their sum once
  const int em = range_exp(fmaxf(2.f * amax * max_p, QJL ? 2.f * prm.kappa * max_q : 0.f) * prm.scale_log2e);
  const int eq = em;
  float* cst = prm.consts + (int64_t)bhc * kConstsPerUnit;
  if (j < 2) {
    const int row = 2 * h + j;
    cst[row] = j == 0 ? -asum * sum_p * prm.scale_log2e * ldexpf(1.0f, em - 10) : 0.f;
    cst[16 + row] = j == 0 ? (QJL ? -prm.kappa * sum_q * prm.scale_log2e * ldexpf(1.0f, eq - 10) : 0.f) : 0.f;
    cst[32 + row] = ldexpf(1.0f, 10 - em);
    cst[48 + row] = ldexpf(1.0f, 10 - eq);
  }
  if (h == 0 && prm.chunk_heads < 8 && j >= 2 * prm.chunk_heads && j < 16) {
    cst[j] = 0.f;
    cst[16 + j] = 0.f;
    cst[32 + j] = 1.f;
    cst[48 + j] = 1.f;
  }
  // fragment elements of this head's rows: (fragment f, lane group g, hi/lo) per thread
  for (int e = j; e < KW::NF * 4 * 2; e += D) {
    const int f = e / 8, g = (e / 2) % 4, lo = e % 2;
    const int W = f / 4, r = f % 4;
    const int lane = 16 * g + 2 * h + lo;
    unsigned hv[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int k = it / 2, half = it % 2;
      const int beta = 16 * half + 4 * r + k;  // bit of the lane's word
      float val = 0.f;
      int E;
      if (W < KW::NWM) {
        int s, jj;
        if constexpr (D >= 128) {
          s = W / (D / 128);
          jj = g * (D / 4) + 32 * (W % (D / 128)) + beta;
        } else {
          s = 2 * W + half;
          jj = g * (D / 4) + (beta % 16);
        }
        if (s < KW::WK) val = 2.f * prm.kcoef[s] * qp[jj];
        E = em;
      } else {
        const int Wq = W - KW::NWM;
        if constexpr (D >= 128) {
          val = 2.f * prm.kappa * qq[g * (D / 4) + 32 * Wq + beta];
        } else {
          if (half == 0) val = 2.f * prm.kappa * qq[g * (D / 4) + beta];
        }
        E = eq;
      }
      // the lane's bit reads as 2^(operand_pos(k) - 24); raw scores come out x 2^(E - 10)
      val *= prm.scale_log2e * ldexpf(1.0f, E + 14 - operand_pos(k));
      hv[it] = f16_part(val, lo);
    }
    prm.frag[((int64_t)bhc * KW::NF + f) * 64 + lane] =
        u32x4{pack2(hv[0], hv[1]), pack2(hv[2], hv[3]), pack2(hv[4], hv[5]), pack2(hv[6], hv[7])};
  }
  if (h == 0 && prm.chunk_heads < 8) {
    for (int e = j; e < KW::NF * 64; e += D) {
      const int lane = e % 64, row = lane % 16;
      if (row >= 2 * prm.chunk_heads) prm.frag[(int64_t)bhc * KW::NF * 64 + e] = u32x4{0u, 0u, 0u, 0u};
    }
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
// Scores: C[token][row] over 16 rows = 8 query heads x (hi, lo) fp16 parts of
// the score operands; lane (r, g) holds tokens 16t + 4g + i of row r, and the
// hi and lo lanes of a head (r, r ^ 1) add their parts with one DPP exchange.
//
// Values: A[row][token] holds the hi (even rows) or lo (odd rows) fp16 part of
// the weight w = p * |v| times 2^(ev - e_k), e_k = vslot_exp(k), for the token
// in slot k = i of the value bit operand (the K order of the value cache block
// layout puts token 16t + 4g + k in slot k; its bit reads as 2^(k - 16), and
// the leftover 2^-2 is removed after the loop). The factor is
// folded into the exp2 argument, so the weights need no extra multiply. The
// value subsets accumulate in NSET sets (see value_sets); each set's lead
// coefficient and the 0/1-to-sign correction are applied once, after the loop.
template <int D, int PK, bool QJL, int VB, int NSET, bool SCORES>
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

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int bhc = blockIdx.y;
  const int chunk = bhc % prm.n_chunks;
  const int bh = bhc / prm.n_chunks;
  const int b = bh / prm.Hkv, hkv = bh % prm.Hkv;
  // score operands of this (batch, kv head, chunk), shared by the workgroup's waves
  __shared__ u32x4 kf_lds[KW::NF * 64];
  // per wave: the norms of the chunk in flight, [0, 32) |k|, [32, 64) |r|, [64, 96) |v|
  __shared__ float4 nrm_lds[kThreads / 64][24];
  {
    const u32x4* src = prm.frag + (int64_t)bhc * KW::NF * 64;
    for (int i = threadIdx.x; i < KW::NF * 64; i += kThreads) kf_lds[i] = src[i];
  }
  __syncthreads();
  auto kfrag = [&](int f) -> u32x4 { return kf_lds[f * 64 + lane]; };
  const int split = blockIdx.x * 4 + wave;
  if (split >= prm.n_splits) return;
  int64_t ctx = prm.ctx_lens[b];
  ctx = ctx < 0 ? 0 : (ctx > prm.max_ctx ? prm.max_ctx : ctx);
  const int64_t t0 = (int64_t)split * prm.split_tokens;
  const int64_t t1 = min(t0 + prm.split_tokens, ctx);
  const int hq0 = hkv * prm.group + chunk * prm.chunk_heads;

  const float* cst = prm.consts + bhc * kConstsPerUnit;
  const float cm0 = cst[r16], cq0 = cst[16 + r16];
  const float isc = cst[32 + r16];  // 2^-E of this row's score operands

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
  const bool lo_row = r16 & 1;
  const float nsel = lo_row ? -1.0f : -0.0f;  // x + nsel * hi(x): the lo part on odd rows

  float m_run = -INFINITY;  // running max of this row's scores (log2 units)
  float m_thr = -INFINITY;  // (m_run + slack) 2^E: raise the max above this raw score
  int ev = kEvUnset;        // value exponent of this row
  float mk[4];              // m_run - (ev - e_k): exp2(s - mk[k]) = p * 2^(ev - e_k)
  float lsum[4];            // per slot: sum of p * 2^(ev - e_k)
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    mk[k] = -INFINITY;
    lsum[k] = 0.f;
  }
  f32x4 acc[NACC][NT];
#pragma unroll
  for (int a = 0; a < NACC; ++a)
#pragma unroll
    for (int q = 0; q < NT; ++q) acc[a][q] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 wacc = {0.f, 0.f, 0.f, 0.f};  // sum of w 2^ev per row (every column)
  const u32x4 ones = {pos_mask(8), pos_mask(9), pos_mask(10), pos_mask(11)};  // slot k: 2^(k - 16)

  // Raw cache data of one 32-token chunk for this lane: its key and value bit
  // words, and one norm (lanes 0..31: |k| of token lane, 32..63: |r|; nb: |v|)
  // that goes through LDS to the lanes that use it.
  struct Chunk {
    unsigned kpl[2][PK > 0 ? PK : 1][WPP];
    unsigned ksg[2][KW::NWQ > 0 ? KW::NWQ : 1];
    unsigned vp[VB][VWL];
    float na, nb;
  };
  const unsigned ln4 = (unsigned)(lane & 31) * 4;
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
    if (lane < 32) {
      c.na = __uint_as_float(ld32(rn, ln4, rel * 4));
      c.nb = __uint_as_float(ld32(rvn, ln4, rel * 4));
    } else {
      c.na = QJL ? __uint_as_float(ld32(rr, ln4, rel * 4)) : 0.f;
      c.nb = 0.f;
    }
  };

  const unsigned n_rel = (unsigned)(t1 > t0 ? t1 - t0 : 0);
  int pend = 0;           // 1: raise the running max; 2: lower the value exponent
  float pend_val = 0.f;   // lane maximum that triggered it

  // One chunk: 0 = accumulated, otherwise the pend code (nothing accumulated).
  auto step = [&](unsigned rel, const Chunk& cur, auto mask_c) -> int {
    constexpr bool MASK = decltype(mask_c)::value;  // the chunk runs past the context
    {
      float* nl = (float*)nrm_lds[wave];
      nl[lane] = cur.na;
      if (lane < 32) nl[64 + lane] = cur.nb;
    }
    // ---------------- scores: two tiles of 16 tokens ----------------
    f32x4 cm[2], cq[2];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      cm[tile] = f32x4{cm0, cm0, cm0, cm0};
      cq[tile] = f32x4{cq0, cq0, cq0, cq0};
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
    // fragments are read from LDS one step ahead of their MFMAs
    u32x4 bf_next = kfrag(0);
#pragma unroll
    for (int W = 0; W < KW::NW; ++W) {
      unsigned word[2];
      key_words(W, word);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int f = 4 * W + r;
        const u32x4 bf = bf_next;
        if (f + 1 < KW::NF) bf_next = kfrag(f + 1);
        if (W < KW::NWM) {
          cm[0] = mfma16(bit_operand(word[0], r), bf, cm[0]);
          cm[1] = mfma16(bit_operand(word[1], r), bf, cm[1]);
        } else {
          cq[0] = mfma16(bit_operand(word[0], r), bf, cq[0]);
          cq[1] = mfma16(bit_operand(word[1], r), bf, cq[1]);
        }
        // keep the bit operands next to their MFMAs (hoisting them all costs registers)
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // this lane: row r16 (head r16/2, hi or lo part), tokens rel + 16 tile + 4g + i;
    // raw scores sr = score 2^E (the row's operand exponent is applied in the exp2 argument)
    float sr[2][4];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      const float4 nk4 = nrm_lds[wave][4 * tile + g];
      const float4 gm4 = QJL ? nrm_lds[wave][8 + 4 * tile + g] : float4{0.f, 0.f, 0.f, 0.f};
      const float nkv[4] = {nk4.x, nk4.y, nk4.z, nk4.w};
      const float gmv[4] = {gm4.x, gm4.y, gm4.z, gm4.w};
      const float cmv[4] = {cm[tile].x, cm[tile].y, cm[tile].z, cm[tile].w};
      const float cqv[4] = {cq[tile].x, cq[tile].y, cq[tile].z, cq[tile].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // hi row + lo row of the same head live in lanes r16 and r16 ^ 1
        float sc = cmv[i] + swap_pair(cmv[i]);
        if constexpr (QJL) sc = fmaf(gmv[i], cqv[i] + swap_pair(cqv[i]), sc);
        sr[tile][i] = nkv[i] * sc;
      }
      if constexpr (MASK) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (rel + 16 * tile + 4 * g + i >= n_rel) sr[tile][i] = -INFINITY;
      }
    }
    // ---------------- online softmax: lane-local checks, no cross-lane work ----------------
    const float mx = max8f(sr);
    if (__builtin_expect(__any(mx > m_thr), 0)) {
      pend_val = mx * isc;
      return 1;
    }
    float wv[2][4], pk[2][4];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      const float4 nv4 = nrm_lds[wave][16 + 4 * tile + g];
      const float nvv[4] = {nv4.x, nv4.y, nv4.z, nv4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pk[tile][i] = __builtin_amdgcn_exp2f(fmaf(sr[tile][i], isc, -mk[i]));  // p 2^(ev - e_i)
        float w = pk[tile][i] * nvv[i];
        if constexpr (MASK) w = pk[tile][i] > 0.f ? w : 0.f;  // masked tokens may hold garbage norms
        wv[tile][i] = w;
      }
    }
    const unsigned wm = max8_nonneg_bits(wv);
    if (__builtin_expect(__any(wm >= __float_as_uint(kWeightOperandMax)), 0)) {
      // largest unscaled weight of this lane: wv 2^(e_k - ev)
      float u = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) u = fmaxf(u, fmaxf(wv[0][i], wv[1][i]) * ldexpf(1.0f, vslot_exp(i) - ev));
      pend_val = u;
      return 2;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) lsum[i] += pk[0][i] + pk[1][i];
    if constexpr (SCORES) {
      const int h = r16 >> 1;
      if (!lo_row && h < prm.chunk_heads) {
        float* dst = prm.scores_dbg + ((int64_t)b * prm.Hq + hq0 + h) * prm.max_ctx + t0;
#pragma unroll
        for (int tile = 0; tile < 2; ++tile)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const unsigned tt = rel + 16 * tile + 4 * g + i;
            if (tt < n_rel) dst[tt] = sr[tile][i] * isc * kLn2;
          }
      }
    }
    // ---------------- values ----------------
    // A operand for weights x: the hi (even rows) or lo (odd rows) fp16 part
    auto a_operand = [&](float rho, bool scaled) -> u32x4 {
      unsigned d4[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        d4[k] = split_pair(scaled ? wv[0][k] * rho : wv[0][k], scaled ? wv[1][k] * rho : wv[1][k], nsel);
      return u32x4{d4[0], d4[1], d4[2], d4[3]};
    };
    const u32x4 a_lead = a_operand(1.0f, false);
#pragma unroll
    for (int s = 0; s < WV; ++s) {
      const int mask = walsh_mask(VB, s);
      const bool lead = walsh_is_lead(VB, NSET, s);
      const int set = walsh_set(VB, NSET, s);
      const u32x4 af = lead ? a_lead : a_operand(prm.vrho[s], true);
#pragma unroll
      for (int w = 0; w < VWL; ++w) {
        unsigned word = 0u;
#pragma unroll
        for (int p = 0; p < VB; ++p)
          if (mask >> p & 1) word ^= cur.vp[p][w];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int q = 4 * w + r;
          acc[set][q] = mfma16(af, bit_operand(word, r), acc[set][q]);
          if (r & 1) __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    wacc = mfma16(a_lead, ones, wacc);
    return 0;
  };

  // The hot loop touches the accumulators only with MFMAs. When a chunk needs
  // the running max raised or the value exponent lowered, it is not
  // accumulated: the state is rescaled here and the chunk runs again.
  unsigned rel = 0;
  while (true) {
    if (pend) {
      // row-wide maximum of the lane values (lanes 16 apart hold the same row)
      float v = pend_val;
      v = fmaxf(v, __shfl_xor(v, 16));
      v = fmaxf(v, __shfl_xor(v, 32));
      float f = 1.0f;
      if (pend == 1) {
        const float m_new = fmaxf(m_run, v);
        f = exp2f(m_run - m_new);  // 0 on the first chunk (m_run = -inf); the state is still zero
        m_run = m_new;
      } else {
        const int e_need = range_exp(v);  // v: the row's largest weight in this chunk
        const int ev_new = e_need < ev ? e_need : ev;
        f = ldexpf(1.0f, ev_new - ev);
        ev = ev_new;
      }
      m_thr = (m_run + kRescaleSlack) / isc;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        mk[k] = m_run - (float)(ev - vslot_exp(k));
        lsum[k] *= f;
      }
      float fr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) fr[i] = __shfl(f, 4 * g + i);
#pragma unroll
      for (int a = 0; a < NACC; ++a)
#pragma unroll
        for (int q = 0; q < NT; ++q) {
          acc[a][q].x *= fr[0];
          acc[a][q].y *= fr[1];
          acc[a][q].z *= fr[2];
          acc[a][q].w *= fr[3];
        }
      wacc.x *= fr[0];
      wacc.y *= fr[1];
      wacc.z *= fr[2];
      wacc.w *= fr[3];
      pend = 0;
    }
    if (rel >= n_rel) break;
    // ping-pong buffers: the next chunk loads while this one computes
    const unsigned n_full = n_rel & ~31u;  // chunks that lie inside the context
    Chunk ca, cb;
    load_chunk(rel, ca);
    while (rel < n_full) {
      if (rel + 32 < n_rel) load_chunk(rel + 32, cb);
      pend = step(rel, ca, std::false_type{});
      if (pend) break;
      rel += 32;
      if (rel >= n_full) {
        ca = cb;  // the tail chunk, if any
        break;
      }
      if (rel + 32 < n_rel) load_chunk(rel + 32, ca);
      pend = step(rel, cb, std::false_type{});
      if (pend) break;
      rel += 32;
    }
    if (!pend && rel < n_rel) {
      pend = step(rel, ca, std::true_type{});
      if (!pend) rel += 32;
    }
  }

  // ---------------- write this split's partial state ----------------
  // softmax denominator of this row: sum_k lsum[k] 2^(e_k - ev), over the 4 lane groups
  float l_acc = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) l_acc += lsum[k] * ldexpf(1.0f, vslot_exp(k) - ev);
  l_acc += __shfl_xor(l_acc, 16);
  l_acc += __shfl_xor(l_acc, 32);
  const int64_t hq_base = (int64_t)b * prm.Hq + hq0;
  if (g == 0 && !lo_row && (r16 >> 1) < prm.chunk_heads) {
    float* ml = prm.part_ml + ((hq_base + (r16 >> 1)) * prm.n_splits + split) * 2;
    ml[0] = m_run;
    ml[1] = l_acc;
  }
  // sum of w 2^ev per head, in the value lanes' row order (rows 4g .. 4g+3)
  const float wt[2] = {wacc.x + wacc.y, wacc.z + wacc.w};
  // value lanes: coordinate lane r16 (coords (D/16) r16 + q), rows 4g .. 4g+3 = heads 2g, 2g+1 (hi, lo)
  const int ev_h0 = __shfl(ev, 4 * g);
  const int ev_h1 = __shfl(ev, 4 * g + 2);
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int h = 2 * g + hh;
    if (h >= prm.chunk_heads) continue;
    const float unscale = ldexpf(1.0f, -(hh ? ev_h1 : ev_h0));
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
  int n_splits, Hq, group;
};

// One workgroup per (batch, query head): weights 2^(m_s - M) / L of every
// split, the merged rotated-space accumulator, then out = Pi_V^T acc.
template <int D>
__global__ __launch_bounds__(kThreads) void decode_combine_kernel(DecCombineParams prm) {
  extern __shared__ float wsplit[];  // [n_splits]
  __shared__ float red[2][kThreads / 64];
  __shared__ float part[kThreads / D][D];
  __shared__ float o[D];
  const int64_t bhq = blockIdx.x;
  const int hq = (int)(bhq % prm.Hq);
  const int hkv = hq / prm.group;
  const int ns = prm.n_splits;
  const float* ml = prm.part_ml + bhq * ns * 2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // block reductions: within each wave by shuffles, then across the waves
  float mx = -INFINITY;
  for (int s = threadIdx.x; s < ns; s += kThreads)
    if (ml[2 * s + 1] > 0.f) mx = fmaxf(mx, ml[2 * s]);
#pragma unroll
  for (int o2 = 32; o2 > 0; o2 >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o2));
  if (lane == 0) red[0][wave] = mx;
  __syncthreads();
  float M = red[0][0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) M = fmaxf(M, red[0][w]);
  float lsum = 0.f;
  for (int s = threadIdx.x; s < ns; s += kThreads) {
    const float l = ml[2 * s + 1];
    const float wgt = l > 0.f ? exp2f(ml[2 * s] - M) : 0.f;
    wsplit[s] = wgt;
    lsum += wgt * l;
  }
#pragma unroll
  for (int o2 = 32; o2 > 0; o2 >>= 1) lsum += __shfl_xor(lsum, o2);
  if (lane == 0) red[1][wave] = lsum;
  __syncthreads();  // also publishes wsplit
  float L = red[1][0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) L += red[1][w];
  const float invL = L > 0.f ? 1.0f / L : 0.f;
  // merged accumulator: thread (j, phase) sums splits phase, phase + P, ...
  constexpr int P = kThreads / D;
  const int j = threadIdx.x % D, ph = threadIdx.x / D;
  const float* acc = prm.part_acc + bhq * (int64_t)ns * D + j;
  float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};  // eight loads in flight
  int s = ph;
  for (; s + 7 * P < ns; s += 8 * P) {
#pragma unroll
    for (int u = 0; u < 8; ++u) a[u] += wsplit[s + u * P] * acc[(int64_t)(s + u * P) * D];
  }
  for (; s < ns; s += P) a[0] += wsplit[s] * acc[(int64_t)s * D];
  part[ph][j] = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
  __syncthreads();
  if (threadIdx.x < D) {
    float t = 0.f;
#pragma unroll
    for (int p = 0; p < P; ++p) t += part[p][threadIdx.x];
    o[threadIdx.x] = t * invL;
  }
  __syncthreads();
  // out[j] = sum_i Pi_V[i][j] o[i]
  const float* Pv = prm.pv[hkv];
  float bq[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};  // eight rows in flight
  for (int i = ph * 8; i < D; i += 8 * P) {
#pragma unroll
    for (int u = 0; u < 8; ++u) bq[u] += Pv[(int64_t)(i + u) * D + j] * o[i + u];
  }
  part[ph][j] = ((bq[0] + bq[1]) + (bq[2] + bq[3])) + ((bq[4] + bq[5]) + (bq[6] + bq[7]));
  __syncthreads();
  if (threadIdx.x < D) {
    float t = 0.f;
#pragma unroll
    for (int p = 0; p < P; ++p) t += part[p][threadIdx.x];
    prm.out[bhq * D + threadIdx.x] = t;
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
  // aim for about 16 waves per CU in total, splits of at least 256 tokens
  const int64_t target = (int64_t)16 * device_cus();
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
                        void* workspace, hipStream_t stream) {
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
  pp.scale_log2e = scale * kLog2e;
  pp.kappa = (float)(std::sqrt(M_PI / 2.0) / p.d);
  for (int s = 0; s < k0->cb.n_walsh; ++s) pp.kcoef[s] = k0->cb.walsh_coef[s];

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
  cp.group = p.group;

  return dispatch_dim(p.d, [&](auto DC) -> tq_status {
    constexpr int D = decltype(DC)::value;
    return dispatch_planes(p.k_planes, [&](auto KPC) -> tq_status {
      constexpr int PK = decltype(KPC)::value;
      return dispatch_bool(p.k_qjl, [&](auto QC) -> tq_status {
        constexpr bool QJL = decltype(QC)::value;
        if constexpr ((!QJL && PK == 0) || (QJL && PK > 3)) {
          return set_error(TQ_ERR_UNSUPPORTED, "decode: unsupported key quantizer");
        } else {
          hipLaunchKernelGGL((decode_prep_kernel<D, PK, QJL>), dim3((unsigned)(p.batch * p.n_q_heads)), dim3(D), 0, stream, pp);
          tq_status st = launch_check("decode: prep launch");
          if (st != TQ_OK) return st;
          st = dispatch_planes(p.v_bits, [&](auto VBC) -> tq_status {
            constexpr int VB = decltype(VBC)::value;
            if constexpr (VB == 0) {
              return set_error(TQ_ERR_UNSUPPORTED, "decode: value bits");
            } else {
              constexpr int NSET = value_sets(D, VB);
              return dispatch_bool(scores_dbg != nullptr, [&](auto SC) -> tq_status {
                constexpr bool SCORES = decltype(SC)::value;
                dim3 grid((unsigned)((p.n_splits + 3) / 4), (unsigned)units);
                hipLaunchKernelGGL((decode_main_kernel<D, PK, QJL, VB, NSET, SCORES>), grid, dim3(kThreads), 0, stream,
                                   mp);
                return launch_check("decode: main launch");
              });
            }
          });
          if (st != TQ_OK) return st;
          hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((unsigned)(p.batch * p.n_q_heads)), dim3(kThreads),
                             (size_t)p.n_splits * sizeof(float), stream, cp);
          return launch_check("decode: combine launch");
        }
      });
    });
  });
}


}  // namespace tq
