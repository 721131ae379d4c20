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
  const int em = range_exp(2.f * amax * max_p * prm.scale_log2e);
  const int eq = range_exp(2.f * prm.kappa * max_q * prm.scale_log2e);
  float* cst = prm.consts + (int64_t)bhc * kConstsPerUnit;
  if (j < 2) {
    const int row = 2 * h + j;
    cst[row] = j == 0 ? -asum * sum_p * prm.scale_log2e * ldexpf(1.0f, em) : 0.f;
    cst[16 + row] = j == 0 ? (QJL ? -prm.kappa * sum_q * prm.scale_log2e * ldexpf(1.0f, eq) : 0.f) : 0.f;
    cst[32 + row] = ldexpf(1.0f, -em);
    cst[48 + row] = ldexpf(1.0f, -eq);
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
      val *= prm.scale_log2e * ldexpf(1.0f, E - slot_exp16(k));
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

// lanes l and l ^ 1 exchange a value (DPP quad permutation [1, 0, 3, 2])
__device__ __forceinline__ float swap_pair(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true));
}
// two fp16 bit patterns (in the low 16 bits of each argument) packed into one dword
__device__ __forceinline__ unsigned pack_f16x2(unsigned lo_half, unsigned hi_half) {
  return __builtin_amdgcn_perm(hi_half, lo_half, 0x05040100u);
}

template <int D, int PK, bool QJL, int VB, bool FOLD, bool SCORES, bool PREFETCH>
__global__ __launch_bounds__(kThreads, FOLD ? 2 : 1) void decode_main_kernel(DecMainParams prm) {
  using KW = KWords<D, PK, QJL>;
  constexpr int WV = n_walsh(VB);
  constexpr int NT = D / 16;   // value N-tiles (16 coordinates each)
  constexpr int VWL = D / 64;  // value words per lane per plane
  constexpr int NACC = FOLD ? 1 : WV;
  constexpr int NAF = FOLD ? WV : 1;
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
  const float ism = cst[32 + r16], isq = cst[48 + r16];

  // wave-uniform bases of this split; per-lane 32-bit offsets below
  const int64_t grp = (int64_t)b * prm.Hkv + hkv;
  const int64_t tok0 = grp * prm.max_ctx + t0;
  const uint8_t* kc = prm.kcodes + tok0 * KREC;
  const uint8_t* ksg = QJL ? prm.ksigns + tok0 * SREC : nullptr;
  const float* kn = prm.knorms + tok0;
  const float* kr = QJL ? prm.krnorms + tok0 : nullptr;
  const float* vn = prm.vnorms + tok0;
  const uint8_t* vc = prm.vcodes + (grp * (prm.max_ctx / 32) + t0 / 32) * (int64_t)VBLK;
  const unsigned k_off = (unsigned)(r16 * KREC + g * (D / 32));
  const unsigned s_off = (unsigned)(r16 * SREC + g * (D / 32));
  const unsigned n_off = (unsigned)(4 * g);
  const unsigned v_off = (unsigned)((g * (D / 4) + VWL * r16) * 4);
  const bool lo_row = r16 & 1;

  float m_run = -INFINITY, l_acc = 0.f, w_acc = 0.f;
  int ev = 64;  // value accumulator exponent of this row (64 = unset)
  float wsc[NAF][4];  // per-slot weight multipliers: coefficient (fold) * 2^(ev - e_k)
#pragma unroll
  for (int a = 0; a < NAF; ++a)
#pragma unroll
    for (int k = 0; k < 4; ++k) wsc[a][k] = 0.f;
  f32x4 acc[NACC][NT];
#pragma unroll
  for (int a = 0; a < NACC; ++a)
#pragma unroll
    for (int q = 0; q < NT; ++q) acc[a][q] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Raw cache data of one 32-token chunk for this lane.
  struct Chunk {
    unsigned kpl[2][PK > 0 ? PK : 1][WPP];
    unsigned ksg[2][KW::NWQ > 0 ? KW::NWQ : 1];
    float4 nk[2], gm[2], nv[2];
    unsigned vp[VB][VWL];
  };
  auto load_chunk = [&](unsigned rel, Chunk& c) {  // rel = chunk start - t0 (multiple of 32)
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      const unsigned tt = rel + 16 * tile;
      if constexpr (PK > 0) {
#pragma unroll
        for (int p = 0; p < PK; ++p)
#pragma unroll
          for (int w = 0; w < WPP; ++w) {
            const unsigned o = tt * KREC + k_off + p * (D / 8) + 4 * w;
            if constexpr (D >= 128) c.kpl[tile][p][w] = *(const unsigned*)(kc + o);
            else c.kpl[tile][p][w] = *(const unsigned short*)(kc + o);
          }
      }
      if constexpr (QJL) {
#pragma unroll
        for (int Wq = 0; Wq < KW::NWQ; ++Wq) {
          const unsigned o = tt * SREC + s_off + 4 * Wq;
          if constexpr (D >= 128) c.ksg[tile][Wq] = *(const unsigned*)(ksg + o);
          else c.ksg[tile][Wq] = *(const unsigned short*)(ksg + o);
        }
      }
      c.nk[tile] = *(const float4*)(kn + tt + n_off);
      if constexpr (QJL) c.gm[tile] = *(const float4*)(kr + tt + n_off);
      else c.gm[tile] = float4{0.f, 0.f, 0.f, 0.f};
      c.nv[tile] = *(const float4*)(vn + tt + n_off);
    }
    const uint8_t* vblk = vc + (size_t)(rel / 32) * VBLK;
#pragma unroll
    for (int p = 0; p < VB; ++p) {
      const uint8_t* src = vblk + p * (4 * (D / 4) * 4) + v_off;
      if constexpr (VWL == 1) {
        c.vp[p][0] = *(const unsigned*)src;
      } else if constexpr (VWL == 2) {
        const uint2 t = *(const uint2*)src;
        c.vp[p][0] = t.x;
        c.vp[p][1] = t.y;
      } else {
        const uint4 t = *(const uint4*)src;
        c.vp[p][0] = t.x;
        c.vp[p][1] = t.y;
        c.vp[p][2] = t.z;
        c.vp[p][3] = t.w;
      }
    }
  };

  const unsigned n_rel = (unsigned)(t1 > t0 ? t1 - t0 : 0);
  // The hot loop touches the value accumulators only with MFMAs. When a chunk
  // needs the running max raised (online softmax) or the value exponent lowered,
  // the loop exits before accumulating that chunk; the accumulators are rescaled
  // out here and the chunk is processed again.
  unsigned rel = 0;
  float pend_cmax = -INFINITY, pend_wmax = 0.f;
  int pend = 0;  // 1: raise the max to pend_cmax; 2: lower the exponent for pend_wmax
  while (true) {
    if (pend) {
      float f = 1.0f;
      if (pend == 1) {
        const float m_new = fmaxf(m_run, pend_cmax);
        f = exp2f(m_run - m_new);
        l_acc *= f;
        w_acc *= f;
        m_run = m_new;
      } else {
        const int e_need = range_exp(pend_wmax);
        const int ev_new = e_need < ev ? e_need : ev;
        f = ldexpf(1.0f, ev_new - ev);
        ev = ev_new;
#pragma unroll
        for (int a = 0; a < NAF; ++a)
#pragma unroll
          for (int k = 0; k < 4; ++k) wsc[a][k] = (FOLD ? prm.vcoef[a] : 1.0f) * ldexpf(1.0f, ev - slot_exp16(k));
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
      pend = 0;
    }
    if (rel >= n_rel) break;
    Chunk cur, nxt;
    load_chunk(rel, cur);
    for (; rel < n_rel; rel += 32) {
      if constexpr (PREFETCH) {
        if (rel + 32 < n_rel) load_chunk(rel + 32, nxt);
      }
      // ---------------- scores: two tiles of 16 tokens ----------------
      f32x4 cm[2], cq[2];
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) {
        cm[tile] = f32x4{cm0, cm0, cm0, cm0};
        cq[tile] = f32x4{cq0, cq0, cq0, cq0};
      }
      if constexpr (PK > 0) {
#pragma unroll
        for (int W = 0; W < KW::NWM; ++W) {
          unsigned word[2];
#pragma unroll
          for (int tile = 0; tile < 2; ++tile) {
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
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const u32x4 bf = kfrag(4 * W + r);
            cm[0] = mfma16(bit_operand(word[0], r), bf, cm[0]);
            cm[1] = mfma16(bit_operand(word[1], r), bf, cm[1]);
          }
        }
      }
      if constexpr (QJL) {
#pragma unroll
        for (int Wq = 0; Wq < KW::NWQ; ++Wq) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const u32x4 bf = kfrag(4 * (KW::NWM + Wq) + r);
            cq[0] = mfma16(bit_operand(cur.ksg[0][Wq], r), bf, cq[0]);
            cq[1] = mfma16(bit_operand(cur.ksg[1][Wq], r), bf, cq[1]);
          }
        }
      }
      // this lane: row r16 (head r16/2, hi or lo part), tokens rel + 16 tile + 4g + i
      const bool full = rel + 32 <= n_rel;
      float s2[2][4];
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) {
        const float nkv[4] = {cur.nk[tile].x, cur.nk[tile].y, cur.nk[tile].z, cur.nk[tile].w};
        const float gmv[4] = {cur.gm[tile].x, cur.gm[tile].y, cur.gm[tile].z, cur.gm[tile].w};
        const float cmv[4] = {cm[tile].x, cm[tile].y, cm[tile].z, cm[tile].w};
        const float cqv[4] = {cq[tile].x, cq[tile].y, cq[tile].z, cq[tile].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // hi row + lo row of the same head live in lanes r16 and r16 ^ 1
          float sc = (cmv[i] + swap_pair(cmv[i])) * ism;
          if constexpr (QJL) sc += gmv[i] * (cqv[i] + swap_pair(cqv[i])) * isq;
          s2[tile][i] = nkv[i] * sc;
        }
        if (!full) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (rel + 16 * tile + 4 * g + i >= n_rel) s2[tile][i] = -INFINITY;
        }
      }
      // ---------------- online softmax ----------------
      float cmax = fmaxf(fmaxf(fmaxf(s2[0][0], s2[0][1]), fmaxf(s2[0][2], s2[0][3])),
                         fmaxf(fmaxf(s2[1][0], s2[1][1]), fmaxf(s2[1][2], s2[1][3])));
      cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
      cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
      if (__any(cmax > m_run + kRescaleSlack)) {
        pend = 1;
        pend_cmax = cmax;
        break;
      }
      float wv[2][4];
      float psum = 0.f, wsum = 0.f, wmax = 0.f;
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) {
        const float nvv[4] = {cur.nv[tile].x, cur.nv[tile].y, cur.nv[tile].z, cur.nv[tile].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(s2[tile][i] - m_run);
          psum += p;
          float w = p * nvv[i];
          if (!full) w = p > 0.f ? w : 0.f;  // masked tokens may hold garbage norms
          wsum += w;
          wv[tile][i] = w;
          wmax = fmaxf(wmax, w);
        }
      }
      wmax = fmaxf(wmax, __shfl_xor(wmax, 16));
      wmax = fmaxf(wmax, __shfl_xor(wmax, 32));
      // keep w 2^(ev + 14) below 2^14: lower the row exponent when a chunk brings larger weights
      if (__any(wmax > 0.f && range_exp(wmax) < ev)) {
        pend = 2;
        pend_wmax = wmax;
        break;
      }
      l_acc += psum;
      w_acc += wsum;
      if constexpr (SCORES) {
        const int h = r16 >> 1;
        if (!lo_row && h < prm.chunk_heads) {
          float* dst = prm.scores_dbg + ((int64_t)b * prm.Hq + hq0 + h) * prm.max_ctx + t0;
#pragma unroll
          for (int tile = 0; tile < 2; ++tile)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const unsigned tt = rel + 16 * tile + 4 * g + i;
              if (tt < n_rel) dst[tt] = s2[tile][i] * kLn2;
            }
        }
      }
      // ---------------- values ----------------
      u32x4 af[NAF];
#pragma unroll
      for (int a = 0; a < NAF; ++a) {
        unsigned d4[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const unsigned h0 = f16_part(wv[0][k] * wsc[a][k], lo_row);
          const unsigned h1 = f16_part(wv[1][k] * wsc[a][k], lo_row);
          d4[k] = pack_f16x2(h0, h1);
        }
        af[a] = u32x4{d4[0], d4[1], d4[2], d4[3]};
      }
#pragma unroll
      for (int s = 0; s < WV; ++s) {
        const int mask = walsh_mask(VB, s);
#pragma unroll
        for (int w = 0; w < VWL; ++w) {
          unsigned word = 0u;
#pragma unroll
          for (int p = 0; p < VB; ++p)
            if (mask >> p & 1) word ^= cur.vp[p][w];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int q = 4 * w + r;
            acc[FOLD ? 0 : s][q] = mfma16(af[FOLD ? s : 0], bit_operand(word, r), acc[FOLD ? 0 : s][q]);
          }
        }
      }
      if constexpr (PREFETCH) cur = nxt;
      else if (rel + 32 < n_rel) load_chunk(rel + 32, cur);
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

// One workgroup per (batch, query head): weights 2^(m_s - M) / L of every
// split, the merged rotated-space accumulator, then out = Pi_V^T acc.
template <int D>
__global__ __launch_bounds__(kThreads) void decode_combine_kernel(DecCombineParams prm) {
  extern __shared__ float wsplit[];  // [n_splits]
  __shared__ float red[kThreads];
  __shared__ float part[kThreads / D][D];
  __shared__ float o[D];
  const int64_t bhq = blockIdx.x;
  const int hq = (int)(bhq % prm.Hq);
  const int hkv = hq / prm.group;
  const int ns = prm.n_splits;
  const float* ml = prm.part_ml + bhq * ns * 2;
  float mx = -INFINITY;
  for (int s = threadIdx.x; s < ns; s += kThreads)
    if (ml[2 * s + 1] > 0.f) mx = fmaxf(mx, ml[2 * s]);
  red[threadIdx.x] = mx;
  __syncthreads();
  for (int st = kThreads / 2; st > 0; st >>= 1) {
    if (threadIdx.x < st) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + st]);
    __syncthreads();
  }
  const float M = red[0];
  __syncthreads();
  float lsum = 0.f;
  for (int s = threadIdx.x; s < ns; s += kThreads) {
    const float l = ml[2 * s + 1];
    const float wgt = l > 0.f ? exp2f(ml[2 * s] - M) : 0.f;
    wsplit[s] = wgt;
    lsum += wgt * l;
  }
  red[threadIdx.x] = lsum;
  __syncthreads();
  for (int st = kThreads / 2; st > 0; st >>= 1) {
    if (threadIdx.x < st) red[threadIdx.x] += red[threadIdx.x + st];
    __syncthreads();
  }
  const float L = red[0];
  const float invL = L > 0.f ? 1.0f / L : 0.f;
  // merged accumulator: thread (j, phase) sums splits phase, phase + P, ...
  constexpr int P = kThreads / D;
  const int j = threadIdx.x % D, ph = threadIdx.x / D;
  const float* acc = prm.part_acc + bhq * (int64_t)ns * D + j;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  int s = ph;
  for (; s + 3 * P < ns; s += 4 * P) {
    a0 += wsplit[s] * acc[(int64_t)s * D];
    a1 += wsplit[s + P] * acc[(int64_t)(s + P) * D];
    a2 += wsplit[s + 2 * P] * acc[(int64_t)(s + 2 * P) * D];
    a3 += wsplit[s + 3 * P] * acc[(int64_t)(s + 3 * P) * D];
  }
  for (; s < ns; s += P) a0 += wsplit[s] * acc[(int64_t)s * D];
  part[ph][j] = (a0 + a1) + (a2 + a3);
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
  float b0 = 0.f, b1 = 0.f, b2 = 0.f, b3 = 0.f;
  for (int i = ph * 4; i < D; i += 4 * P) {
    b0 += Pv[(int64_t)i * D + j] * o[i];
    b1 += Pv[(int64_t)(i + 1) * D + j] * o[i + 1];
    b2 += Pv[(int64_t)(i + 2) * D + j] * o[i + 2];
    b3 += Pv[(int64_t)(i + 3) * D + j] * o[i + 3];
  }
  part[ph][j] = (b0 + b1) + (b2 + b3);
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

  // Value accumulators: one folded set (two waves per SIMD; measured faster on
  // MI355X) or one set per Walsh plane (fewer VALU ops, one wave per SIMD).
  // TQ_DECODE_VARIANT selects explicitly: "fold" / "planes", optionally ",prefetch".
  bool fold = true;
  bool prefetch = false;
  if (const char* env = std::getenv("TQ_DECODE_VARIANT")) {
    const std::string v(env);
    if (v.find("fold") != std::string::npos) fold = true;
    if (v.find("planes") != std::string::npos && (size_t)p.v_walsh * (p.d / 16) * 4 <= 128) fold = false;
    prefetch = v.find("prefetch") != std::string::npos;
  }
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
              return dispatch_bool(fold, [&](auto FC) -> tq_status {
                constexpr bool FOLD = decltype(FC)::value;
                constexpr bool fits = (n_walsh(VB) * (D / 16) * 4 <= 128);
                if constexpr (!FOLD && !fits) {
                  return set_error(TQ_ERR_UNSUPPORTED, "decode: accumulator mode");
                } else {
                  return dispatch_bool(scores_dbg != nullptr, [&](auto SC) -> tq_status {
                    constexpr bool SCORES = decltype(SC)::value;
                    return dispatch_bool(prefetch, [&](auto PF) -> tq_status {
                      constexpr bool PREF = decltype(PF)::value;
                      dim3 grid((unsigned)((p.n_splits + 3) / 4), (unsigned)units);
                      hipLaunchKernelGGL((decode_main_kernel<D, PK, QJL, VB, FOLD, SCORES, PREF>), grid, dim3(kThreads),
                                         0, stream, mp);
                      return launch_check("decode: main launch");
                    });
                  });
                }
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
