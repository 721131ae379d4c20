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
// unpacking: rotate the 32-bit word so the wanted bit lands on exponent bit k
// of an fp16 half (bit position 10+k or 26+k) and mask everything else; the
// half is then 0 or the exact power of two 2^(2^k - 15). The weight operand
// carries the compensating power of two, so each product is exactly
// weight * bit * 2^E for a per-row exponent E chosen to keep the weights in
// fp16 range. One rotate plus four ANDs make one MFMA operand (8 bits).
//
// Both contractions use 0/1 bits. With sigma = 2 bit - 1 and the odd Walsh
// expansion of the symmetric codebook, c[idx] = sum_s a_s prod_{i in s} sigma_i,
// so sum_j w_j c[idx_j] = sum_s a_s (2 sum_j w_j bit_{s,j} - sum_j w_j) where
// bit_{s,j} is the XOR of the planes in subset s.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>

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
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                0, 0, 0);
}
__device__ __forceinline__ unsigned f16_bits(float v) {
  return (unsigned)__builtin_bit_cast(unsigned short, (_Float16)v);
}
__device__ __forceinline__ float f16_val(unsigned h) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(h & 0xFFFFu));
}
// hi (lo = false) or lo (lo = true) fp16 part of v; hi + lo carries 22 significant bits
__device__ __forceinline__ unsigned f16_part(float v, bool lo) {
  const unsigned hi = f16_bits(v);
  return lo ? f16_bits(v - f16_val(hi)) : hi;
}
// fp16 value of an operand bit in slot pair k: exponent bit k set, 2^((1 << k) - 15)
__host__ __device__ constexpr int slot_exp16(int k) { return (1 << k) - 15; }
// exponent E such that |w| <= wmax keeps |w| 2^(E + 14) < 2^14 (the largest
// compensation is 2^14), so every scaled weight and its lo part stay normal fp16
// down to about 2^-10 of the largest weight
__device__ __forceinline__ int range_exp(float wmax) {
  if (!(wmax > 0.f)) return 0;
  int e;
  frexpf(wmax, &e);  // wmax < 2^e
  return -e;
}

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
// [32,48) 2^-E_mse, [48,64) 2^-E_qjl, one value per MFMA row.
constexpr int kConstsPerUnit = 64;

template <int D, int PK, bool QJL>
__global__ __launch_bounds__(kThreads) void decode_prep_kernel(DecPrepParams prm) {
  using KW = KWords<D, PK, QJL>;
  __shared__ float qs[8][D], qp[8][D], qq[8][D];
  __shared__ float red[2][8][kThreads / 8];
  __shared__ int em_s[8], eq_s[8];
  const int bhc = blockIdx.x;
  const int chunk = bhc % prm.n_chunks;
  const int bh = bhc / prm.n_chunks;
  const int b = bh / prm.Hkv, hkv = bh % prm.Hkv;
  const int hq0 = hkv * prm.group + chunk * prm.chunk_heads;
  for (int e = threadIdx.x; e < 8 * D; e += kThreads) {
    const int h = e / D, j = e % D;
    float v = 0.f;
    if (h < prm.chunk_heads) v = bf16_val(prm.q[((int64_t)b * prm.Hq + hq0 + h) * D + j]);
    qs[h][j] = v;
  }
  __syncthreads();
  const float* P = prm.pk[hkv];
  const float* S = prm.sk[hkv];
  for (int e = threadIdx.x; e < 8 * D; e += kThreads) {
    const int h = e / D, j = e % D;
    float a = 0.f, c = 0.f;
    if (h < prm.chunk_heads) {
      for (int k = 0; k < D; ++k) {
        a += P[j * D + k] * qs[h][k];
        if constexpr (QJL) c += S[j * D + k] * qs[h][k];
      }
    }
    qp[h][j] = a;
    qq[h][j] = c;
  }
  __syncthreads();
  // per-head max |q'| and |q''|: 32 threads per head
  {
    const int h = threadIdx.x / 32, t = threadIdx.x % 32;
    float mp = 0.f, mq = 0.f;
    for (int j = t; j < D; j += 32) {
      mp = fmaxf(mp, fabsf(qp[h][j]));
      mq = fmaxf(mq, fabsf(qq[h][j]));
    }
    red[0][h][t] = mp;
    red[1][h][t] = mq;
  }
  __syncthreads();
  if (threadIdx.x < 8) {
    const int h = threadIdx.x;
    float mp = 0.f, mq = 0.f;
    for (int t = 0; t < 32; ++t) {
      mp = fmaxf(mp, red[0][h][t]);
      mq = fmaxf(mq, red[1][h][t]);
    }
    float amax = 0.f;
    for (int s = 0; s < KW::WK; ++s) amax = fmaxf(amax, fabsf(prm.kcoef[s]));
    em_s[h] = range_exp(2.f * amax * mp * prm.scale_log2e);
    eq_s[h] = range_exp(2.f * prm.kappa * mq * prm.scale_log2e);
  }
  __syncthreads();
  // constants: hi rows carry -(sum_s a_s sum_j q'_j) and -kappa sum_j q''_j, x scale log2e 2^E
  if (threadIdx.x < 64) {
    const int which = threadIdx.x / 16, row = threadIdx.x % 16, h = row / 2;
    float v = 0.f;
    if (h < prm.chunk_heads) {
      const int E = (which == 0 || which == 2) ? em_s[h] : eq_s[h];
      if (which < 2) {
        if ((row & 1) == 0) {
          float sq = 0.f;
          for (int j = 0; j < D; ++j) sq += which == 0 ? qp[h][j] : qq[h][j];
          float coef = 0.f;
          if (which == 0) {
            for (int s = 0; s < KW::WK; ++s) coef += prm.kcoef[s];
          } else {
            coef = QJL ? prm.kappa : 0.f;
          }
          v = -coef * sq * prm.scale_log2e * ldexpf(1.0f, E);
        }
      } else {
        v = ldexpf(1.0f, -E);
      }
    } else if (which >= 2) {
      v = 1.0f;
    }
    prm.consts[bhc * kConstsPerUnit + which * 16 + row] = v;
  }
  // operand fragments
  for (int e = threadIdx.x; e < KW::NF * 64; e += kThreads) {
    const int f = e / 64, lane = e % 64;
    const int W = f / 4, r = f % 4;
    const int row = lane % 16, g = lane / 16, h = row / 2;
    const bool lo = row & 1;
    unsigned hv[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int k = it / 2, half = it % 2;
      const int beta = 16 * half + 4 * r + k;  // bit of the lane's word
      float val = 0.f;
      int E = 0;
      if (h < prm.chunk_heads) {
        if (W < KW::NWM) {
          int s, j;
          if constexpr (D >= 128) {
            s = W / (D / 128);
            j = g * (D / 4) + 32 * (W % (D / 128)) + beta;
          } else {
            s = 2 * W + half;
            j = g * (D / 4) + (beta % 16);
          }
          if (s < KW::WK) val = 2.f * prm.kcoef[s] * qp[h][j];
          E = em_s[h];
        } else {
          const int Wq = W - KW::NWM;
          if constexpr (D >= 128) {
            const int j = g * (D / 4) + 32 * Wq + beta;
            val = 2.f * prm.kappa * qq[h][j];
          } else {
            if (half == 0) val = 2.f * prm.kappa * qq[h][g * (D / 4) + beta];
          }
          E = eq_s[h];
        }
        val *= prm.scale_log2e * ldexpf(1.0f, E - slot_exp16(k));
      }
      hv[it] = f16_part(val, lo);
    }
    prm.frag[((int64_t)bhc * KW::NF + f) * 64 + lane] =
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
  float* part_acc;
  float* part_ml;
  float* scores_dbg;
  int64_t max_ctx;
  int64_t split_tokens;
  int n_splits;
  int Hq, Hkv, group, chunk_heads, n_chunks;
  float vcoef[kMaxWalsh];
  float vcoef_sum;
};

template <int D, int PK>
__device__ __forceinline__ unsigned load_plane_chunk(const uint8_t* rec, int p, int g, int w) {
  // D/4 bits of plane p for coordinate quarter g; word w of them (D = 64: 16 bits)
  if constexpr (D >= 128) {
    return *(const unsigned*)(rec + p * (D / 8) + g * (D / 32) + 4 * w);
  } else {
    return *(const unsigned short*)(rec + p * (D / 8) + g * (D / 32));
  }
}

template <int D, int PK, bool QJL, int VB, bool FOLD, bool SCORES>
__global__ __launch_bounds__(kThreads) void decode_main_kernel(DecMainParams prm) {
  using KW = KWords<D, PK, QJL>;
  constexpr int WV = n_walsh(VB);
  constexpr int NT = D / 16;   // value N-tiles (16 coordinates each)
  constexpr int VWL = D / 64;  // value words per lane per plane
  constexpr int NACC = FOLD ? 1 : WV;
  constexpr int KREC = PK * D / 8;
  constexpr bool KF_REG = KW::NF <= 24;  // keep the score operands in registers

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int bhc = blockIdx.y;
  const int chunk = bhc % prm.n_chunks;
  const int bh = bhc / prm.n_chunks;
  const int b = bh / prm.Hkv, hkv = bh % prm.Hkv;
  const int split = blockIdx.x * 4 + wave;
  if (split >= prm.n_splits) return;
  int64_t ctx = prm.ctx_lens[b];
  ctx = ctx < 0 ? 0 : (ctx > prm.max_ctx ? prm.max_ctx : ctx);
  const int64_t t0 = (int64_t)split * prm.split_tokens;
  const int64_t t1 = min(t0 + prm.split_tokens, ctx);
  const int hq0 = hkv * prm.group + chunk * prm.chunk_heads;

  const u32x4* kfg = prm.frag + (int64_t)bhc * KW::NF * 64 + lane;
  u32x4 kf[KF_REG ? KW::NF : 1];
  if constexpr (KF_REG) {
#pragma unroll
    for (int f = 0; f < KW::NF; ++f) kf[f] = kfg[f * 64];
  }
  auto kfrag = [&](int f) -> u32x4 {
    if constexpr (KF_REG) return kf[f];
    else return kfg[f * 64];
  };
  const float* cst = prm.consts + bhc * kConstsPerUnit;
  const float cm0 = cst[r16], cq0 = cst[16 + r16];
  const float ism = cst[32 + r16], isq = cst[48 + r16];

  const int64_t grp = (int64_t)b * prm.Hkv + hkv;
  const uint8_t* kc = prm.kcodes + grp * prm.max_ctx * KREC;
  const uint8_t* ksg = QJL ? prm.ksigns + grp * prm.max_ctx * (D / 8) : nullptr;
  const float* kn = prm.knorms + grp * prm.max_ctx;
  const float* kr = QJL ? prm.krnorms + grp * prm.max_ctx : nullptr;
  const uint8_t* vc = prm.vcodes + grp * (prm.max_ctx / 32) * (int64_t)(4 * VB * D);
  const float* vn = prm.vnorms + grp * prm.max_ctx;
  const bool lo_row = r16 & 1;

  float m_run = -INFINITY, l_acc = 0.f, w_acc = 0.f;
  int ev = 64;  // value accumulator exponent of this row (64 = unset)
  f32x4 acc[NACC][NT];
#pragma unroll
  for (int a = 0; a < NACC; ++a)
#pragma unroll
    for (int q = 0; q < NT; ++q) acc[a][q] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t tc = t0; tc < t1; tc += 32) {
    // ---------------- scores: two tiles of 16 tokens ----------------
    f32x4 cm[2], cq[2];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      const int64_t tok = tc + 16 * tile + r16;  // always < max_ctx (32-aligned chunks)
      cm[tile] = f32x4{cm0, cm0, cm0, cm0};
      cq[tile] = f32x4{cq0, cq0, cq0, cq0};
      if constexpr (PK > 0) {
        const uint8_t* rec = kc + tok * KREC;
        constexpr int WPP = D >= 128 ? D / 128 : 1;
        unsigned pl[PK][WPP];
#pragma unroll
        for (int p = 0; p < PK; ++p)
#pragma unroll
          for (int w = 0; w < WPP; ++w) pl[p][w] = load_plane_chunk<D, PK>(rec, p, g, w);
#pragma unroll
        for (int W = 0; W < KW::NWM; ++W) {
          unsigned word;
          if constexpr (D >= 128) {
            const int s = W / (D / 128), w = W % (D / 128);
            const int mask = walsh_mask(PK, s);
            word = 0u;
#pragma unroll
            for (int p = 0; p < PK; ++p)
              if (mask >> p & 1) word ^= pl[p][w];
          } else {
            unsigned lo16 = 0u, hi16 = 0u;
            const int s0 = 2 * W, s1 = 2 * W + 1;
            const int m0 = walsh_mask(PK, s0);
            const int m1 = s1 < KW::WK ? walsh_mask(PK, s1) : 0;
#pragma unroll
            for (int p = 0; p < PK; ++p) {
              if (m0 >> p & 1) lo16 ^= pl[p][0];
              if (m1 >> p & 1) hi16 ^= pl[p][0];
            }
            word = (lo16 & 0xFFFFu) | (hi16 << 16);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) cm[tile] = mfma16(bit_operand(word, r), kfrag(4 * W + r), cm[tile]);
        }
      }
      if constexpr (QJL) {
        const uint8_t* srec = ksg + tok * (D / 8);
#pragma unroll
        for (int Wq = 0; Wq < KW::NWQ; ++Wq) {
          unsigned word;
          if constexpr (D >= 128) word = *(const unsigned*)(srec + g * (D / 32) + 4 * Wq);
          else word = *(const unsigned short*)(srec + g * (D / 32));
#pragma unroll
          for (int r = 0; r < 4; ++r)
            cq[tile] = mfma16(bit_operand(word, r), kfrag(4 * (KW::NWM + Wq) + r), cq[tile]);
        }
      }
    }
    // this lane: row r16 (head r16/2, hi or lo part), tokens tc + 16 tile + 4g + i
    float s2[2][4];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      const int64_t tb = tc + 16 * tile + 4 * g;
      const float4 nk = *(const float4*)(kn + tb);
      float4 gm = float4{0.f, 0.f, 0.f, 0.f};
      if constexpr (QJL) gm = *(const float4*)(kr + tb);
      const float nkv[4] = {nk.x, nk.y, nk.z, nk.w};
      const float gmv[4] = {gm.x, gm.y, gm.z, gm.w};
      const float cmv[4] = {cm[tile].x, cm[tile].y, cm[tile].z, cm[tile].w};
      const float cqv[4] = {cq[tile].x, cq[tile].y, cq[tile].z, cq[tile].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // hi row + lo row of the same head live in lanes r16 and r16 ^ 1
        float sc = (cmv[i] + __shfl_xor(cmv[i], 1)) * ism;
        if constexpr (QJL) sc += gmv[i] * (cqv[i] + __shfl_xor(cqv[i], 1)) * isq;
        const float v = nkv[i] * sc;
        s2[tile][i] = (tb + i < t1) ? v : -INFINITY;
      }
      if constexpr (SCORES) {
        const int h = r16 >> 1;
        if (!lo_row && h < prm.chunk_heads) {
          float* dst = prm.scores_dbg + ((int64_t)b * prm.Hq + hq0 + h) * prm.max_ctx;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (tb + i < t1) dst[tb + i] = s2[tile][i] * kLn2;
        }
      }
    }
    // ---------------- online softmax ----------------
    float cmax = s2[0][0];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile)
#pragma unroll
      for (int i = 0; i < 4; ++i) cmax = fmaxf(cmax, s2[tile][i]);
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
    float alpha = 1.0f;
    if (__any(cmax > m_run + kRescaleSlack)) {
      const float m_new = fmaxf(m_run, cmax);
      alpha = exp2f(m_run - m_new);
      l_acc *= alpha;
      w_acc *= alpha;
      m_run = m_new;
    }
    float wv[2][4];
    float wmax = 0.f;
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      const int64_t tb = tc + 16 * tile + 4 * g;
      const float4 nv = *(const float4*)(vn + tb);
      const float nvv[4] = {nv.x, nv.y, nv.z, nv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = exp2f(s2[tile][i] - m_run);
        l_acc += p;
        const float w = p > 0.f ? p * nvv[i] : 0.f;
        w_acc += w;
        wv[tile][i] = w;
        wmax = fmaxf(wmax, w);
      }
    }
    wmax = fmaxf(wmax, __shfl_xor(wmax, 16));
    wmax = fmaxf(wmax, __shfl_xor(wmax, 32));
    // keep w 2^(ev + 14) below 2^14: lower the row exponent when a chunk brings larger weights
    const int e_need = range_exp(wmax);
    const bool lower = wmax > 0.f && e_need < ev;
    if (__any(lower || alpha != 1.0f)) {
      const int ev_new = lower ? e_need : ev;
      const float f = alpha * ldexpf(1.0f, ev_new - ev);
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
      ev = ev_new;
    }
    // ---------------- values ----------------
    float sc_v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) sc_v[k] = ldexpf(1.0f, ev - slot_exp16(k));
    u32x4 af[FOLD ? WV : 1];
#pragma unroll
    for (int a = 0; a < (FOLD ? WV : 1); ++a) {
      const float cf = FOLD ? prm.vcoef[a] : 1.0f;
      unsigned d4[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const unsigned h0 = f16_part(wv[0][k] * cf * sc_v[k], lo_row);
        const unsigned h1 = f16_part(wv[1][k] * cf * sc_v[k], lo_row);
        d4[k] = pack2(h0, h1);
      }
      af[a] = u32x4{d4[0], d4[1], d4[2], d4[3]};
    }
    const uint8_t* vblk = vc + (tc / 32) * (int64_t)(4 * VB * D);
    unsigned vp[VB][VWL];
#pragma unroll
    for (int p = 0; p < VB; ++p) {
      const uint8_t* src = vblk + ((p * 4 + g) * (D / 4) + VWL * r16) * 4;
      if constexpr (VWL == 1) {
        vp[p][0] = *(const unsigned*)src;
      } else if constexpr (VWL == 2) {
        const uint2 t = *(const uint2*)src;
        vp[p][0] = t.x;
        vp[p][1] = t.y;
      } else {
        const uint4 t = *(const uint4*)src;
        vp[p][0] = t.x;
        vp[p][1] = t.y;
        vp[p][2] = t.z;
        vp[p][3] = t.w;
      }
    }
#pragma unroll
    for (int s = 0; s < WV; ++s) {
      const int mask = walsh_mask(VB, s);
#pragma unroll
      for (int w = 0; w < VWL; ++w) {
        unsigned word = 0u;
#pragma unroll
        for (int p = 0; p < VB; ++p)
          if (mask >> p & 1) word ^= vp[p][w];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int q = 4 * w + r;
          acc[FOLD ? 0 : s][q] = mfma16(af[FOLD ? s : 0], bit_operand(word, r), acc[FOLD ? 0 : s][q]);
        }
      }
    }
  }

  // ---------------- write this split's partial state ----------------
  l_acc += __shfl_xor(l_acc, 16);
  l_acc += __shfl_xor(l_acc, 32);
  w_acc += __shfl_xor(w_acc, 16);
  w_acc += __shfl_xor(w_acc, 32);
  const int64_t hq_base = (int64_t)b * prm.Hq + hq0;
  if (g == 0 && !lo_row && (r16 >> 1) < prm.chunk_heads) {
    float* ml = prm.part_ml + ((hq_base + (r16 >> 1)) * prm.n_splits + split) * 2;
    ml[0] = m_run;
    ml[1] = l_acc;
  }
  // value lanes: coordinate lane r16 (coords (D/16) r16 + q), rows 4g .. 4g+3 = heads 2g, 2g+1 (hi, lo)
  const float w_h0 = __shfl(w_acc, 4 * g);
  const float w_h1 = __shfl(w_acc, 4 * g + 2);
  const int ev_h0 = __shfl(ev, 4 * g);
  const int ev_h1 = __shfl(ev, 4 * g + 2);
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int h = 2 * g + hh;
    if (h >= prm.chunk_heads) continue;
    const float wh = hh ? w_h1 : w_h0;
    const float unscale = 2.f * ldexpf(1.0f, -(hh ? ev_h1 : ev_h0));
    float outv[NT];
#pragma unroll
    for (int q = 0; q < NT; ++q) {
      float v = 0.f;
      if constexpr (FOLD) {
        const float c2 = hh ? (acc[0][q].z + acc[0][q].w) : (acc[0][q].x + acc[0][q].y);
        v = unscale * c2 - wh * prm.vcoef_sum;
      } else {
#pragma unroll
        for (int s = 0; s < WV; ++s) {
          const float c2 = hh ? (acc[s][q].z + acc[s][q].w) : (acc[s][q].x + acc[s][q].y);
          v += prm.vcoef[s] * (unscale * c2 - wh);
        }
      }
      outv[q] = v;
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

template <int D>
__global__ __launch_bounds__(kThreads) void decode_combine_kernel(DecCombineParams prm) {
  __shared__ float red[kThreads];
  __shared__ float o[D];
  __shared__ float M_s, L_s;
  const int64_t bhq = blockIdx.x;
  const int hq = (int)(bhq % prm.Hq);
  const int hkv = hq / prm.group;
  const float* ml = prm.part_ml + bhq * prm.n_splits * 2;
  float mx = -INFINITY;
  for (int s = threadIdx.x; s < prm.n_splits; s += kThreads)
    if (ml[2 * s + 1] > 0.f) mx = fmaxf(mx, ml[2 * s]);
  red[threadIdx.x] = mx;
  __syncthreads();
  for (int st = kThreads / 2; st > 0; st >>= 1) {
    if (threadIdx.x < st) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + st]);
    __syncthreads();
  }
  if (threadIdx.x == 0) M_s = red[0];
  __syncthreads();
  const float M = M_s;
  float lsum = 0.f;
  for (int s = threadIdx.x; s < prm.n_splits; s += kThreads)
    if (ml[2 * s + 1] > 0.f) lsum += exp2f(ml[2 * s] - M) * ml[2 * s + 1];
  red[threadIdx.x] = lsum;
  __syncthreads();
  for (int st = kThreads / 2; st > 0; st >>= 1) {
    if (threadIdx.x < st) red[threadIdx.x] += red[threadIdx.x + st];
    __syncthreads();
  }
  if (threadIdx.x == 0) L_s = red[0];
  __syncthreads();
  const float L = L_s;
  for (int j = threadIdx.x; j < D; j += kThreads) {
    float a = 0.f;
    if (L > 0.f) {
      for (int s = 0; s < prm.n_splits; ++s) {
        if (ml[2 * s + 1] > 0.f) a += exp2f(ml[2 * s] - M) * prm.part_acc[(bhq * prm.n_splits + s) * D + j];
      }
      a /= L;
    }
    o[j] = a;
  }
  __syncthreads();
  const float* P = prm.pv[hkv];
  for (int j = threadIdx.x; j < D; j += kThreads) {
    float a = 0.f;
    for (int i = 0; i < D; ++i) a += P[i * D + j] * o[i];
    prm.out[bhq * D + j] = a;
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
  float csum = 0.f;
  for (int s = 0; s < v0->cb.n_walsh; ++s) {
    mp.vcoef[s] = v0->cb.walsh_coef[s];
    csum += v0->cb.walsh_coef[s];
  }
  mp.vcoef_sum = csum;

  DecCombineParams cp{};
  cp.part_acc = part_acc;
  cp.part_ml = part_ml;
  for (int h = 0; h < p.n_kv_heads; ++h) cp.pv[h] = v->qz[h]->pi32;
  cp.out = out;
  cp.n_splits = p.n_splits;
  cp.Hq = p.n_q_heads;
  cp.group = p.group;

  const bool fold = (size_t)p.v_walsh * (p.d / 16) * 4 > 128;  // per-plane accumulators must fit in 128 regs
  return dispatch_dim(p.d, [&](auto DC) -> tq_status {
    constexpr int D = decltype(DC)::value;
    return dispatch_planes(p.k_planes, [&](auto KPC) -> tq_status {
      constexpr int PK = decltype(KPC)::value;
      return dispatch_bool(p.k_qjl, [&](auto QC) -> tq_status {
        constexpr bool QJL = decltype(QC)::value;
        if constexpr ((!QJL && PK == 0) || (QJL && PK > 3)) {
          return set_error(TQ_ERR_UNSUPPORTED, "decode: unsupported key quantizer");
        } else {
          hipLaunchKernelGGL((decode_prep_kernel<D, PK, QJL>), dim3(units), dim3(kThreads), 0, stream, pp);
          tq_status st = launch_check("decode: prep launch");
          if (st != TQ_OK) return st;
          st = dispatch_planes(p.v_bits, [&](auto VBC) -> tq_status {
            constexpr int VB = decltype(VBC)::value;
            if constexpr (VB == 0) {
              return set_error(TQ_ERR_UNSUPPORTED, "decode: value bits");
            } else {
              return dispatch_bool(fold, [&](auto FC) -> tq_status {
                constexpr bool FOLD = decltype(FC)::value;
                constexpr bool fits = (n_walsh(VB) * (D / 16) * 4 <= 128);
                if constexpr (!FOLD && !fits) {
                  return set_error(TQ_ERR_UNSUPPORTED, "decode: accumulator mode");
                } else {
                  return dispatch_bool(scores_dbg != nullptr, [&](auto SC) -> tq_status {
                    constexpr bool SCORES = decltype(SC)::value;
                    dim3 grid((unsigned)((p.n_splits + 3) / 4), (unsigned)units);
                    hipLaunchKernelGGL((decode_main_kernel<D, PK, QJL, VB, FOLD, SCORES>), grid, dim3(kThreads), 0,
                                       stream, mp);
                    return launch_check("decode: main launch");
                  });
                }
              });
            }
          });
          if (st != TQ_OK) return st;
          hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((unsigned)(p.batch * p.n_q_heads)), dim3(kThreads), 0,
                             stream, cp);
          return launch_check("decode: combine launch");
        }
      });
    });
  });
}


}  // namespace tq
