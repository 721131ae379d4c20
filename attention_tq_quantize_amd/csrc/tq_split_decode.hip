// Decode attention over a KV cache quantized with an outlier-channel split
// ([NIK] "Experiments", KV cache: outlier channels at more bits than the
// others; every part is TurboQuant in its own dimension with its own rotation,
// norm, codebook and, for prod keys, QJL matrix). For each batch b and query
// head h (KV head g = h / (Hq / Hkv)):
//   s_t = scale * sum_p <q restricted to part p's channels, k~_{p,t}>,  t < len_b
//   out = sum_t softmax(s)_t v~_t, each value part written back to its channels
// (channels no value part keeps come out 0).
//
// Matrix-core design for part dimensions that are multiples of 32 (the 32 / 96
// split of a 128-channel head), in three kernels:
//  1. prep, one workgroup per (batch, KV head): the query parts rotated into
//     each key part's basis (q' = scale Pi_p q_p, q'' = scale sqrt(pi/2)/d_p
//     S_p q_p), a power-of-two scale per head, and the fp16 hi/lo MFMA
//     fragments (rows = 8 heads x {hi, lo}, K = 32 coordinates), written to the
//     workspace;
//  2. main, one wave per context split (as many splits as waves fit on the
//     device at once). Each wave walks its split in chunks of 32 tokens:
//      * the chunk's records of every part are copied straight from HBM into
//        the wave's LDS staging buffer (global_load_lds, double-buffered);
//      * scores: per key part and 32-coordinate step, each lane turns the
//        coordinates of one token into exact fp16 hi/lo centroid operands with
//        one bit-field extract per plane and one table read per four
//        coordinates (parts of one or two planes: quad tables) or per two
//        (pair tables), the QJL signs into +-1 per four from a nibble table,
//        and the matrix cores form <q', c~> and <q'', z> for 16 tokens x 8
//        heads per instruction;
//      * an online softmax per head over the chunk (16-lane DPP reductions);
//      * values: the probabilities times each value part's norms become the
//        fp16 hi/lo weight operand (rows = 8 heads x {hi, lo}, K = 32 tokens in
//        the BLOCK32 token order); the value codes are BLOCK32, so one word per
//        plane holds a lane's coordinate for all eight of its tokens, and each
//        lane turns four (quad tables) or two (pair tables) tokens at a time
//        into the centroid operand; the matrix cores
//        accumulate 16 coordinates x 8 heads per instruction in the part's
//        rotated basis (a running power-of-two exponent per part keeps the
//        weights in fp16 range);
//  3. combine, one workgroup per (batch, query head): log-sum-exp merge of the
//     splits, each value part rotated back (Pi_p^T) and scattered to its
//     channels (deterministic, no atomics).
#include <hip/hip_runtime.h>

#include <mutex>
#include <type_traits>
#include <vector>

#include "tq_device.h"

namespace tq {
namespace {

constexpr int kSmWaves = 4;                 // waves per workgroup, one context split each
constexpr int kSmThreads = 64 * kSmWaves;
constexpr int kSmChunk = 32;                // tokens per step
constexpr int kSmMaxSeg = 6 * kSplitMaxParts;
constexpr int kSmEvUnset = -1000;
constexpr int kSmSplitsCached = 1024;  // split weights the combine keeps in LDS

struct SmPart {
  int d, planes, off, qjl;
  int rec;                                   // code bytes per token: planes * d / 8
  int st_codes, st_signs, st_norms, st_rnorms;  // byte offsets in a staging buffer
  int ptab;                                  // byte offset of its quad or pair table from the tables' start
  float kappa;                               // sqrt(pi/2) / d
  unsigned tab[16];                          // centroid i as fp16 hi | lo << 16
  const float* pi[kSplitMaxKv];
  const float* s[kSplitMaxKv];
};

struct SmSeg {  // one per-token array of one part: elem bytes per token, [B * Hkv][T][elem]
  const uint8_t* base;
  int elem, lds;
  int blocked;  // BLOCK32 codes: a chunk is one whole block (no per-token clamp)
};

struct SmParams {
  int Hq, Hkv, G, dim, nk, nv, dk, dv, n_splits, n_seg;
  int64_t T, split_tokens;
  const uint16_t* q;  // bf16 [B][Hq][dim]
  const int32_t* lens;
  float scale;
  float* part;  // [B][Hq][n_splits][dv + 2]
  float* out;   // [B][Hq][dim]
  u32x4* qfrag;  // [B * Hkv][dk / 32][{mse, qjl}][64 lanes]: score operand fragments
  int* qexp;     // [B * Hkv][2][8]: their power-of-two scales per (kind, head)
  int stage_bytes, tab_off, wave_off, wave_bytes;  // LDS layout (bytes); fragments at 0
  int prep_rows;  // matrix rows the prep kernel stages per block
  uint8_t kchan[kSplitMaxKv][kSplitMaxDecodeDim], vchan[kSplitMaxKv][kSplitMaxDecodeDim];  // per KV head
  uint8_t vword_part[kSplitMaxDecodeDim / 32];  // value part of each 32-coordinate word
  SmPart kp[kSplitMaxParts], vp[kSplitMaxParts];
  SmSeg seg[kSmMaxSeg];
};


__device__ __forceinline__ unsigned lds_u32(const uint8_t* p) { return *(const unsigned*)p; }

// w >> off (off a VGPR) masked to W bits, as one v_bfe_u32: plain ALU, the
// compiler otherwise splits constant-offset extracts into a shift and a mask
template <int W>
__device__ __forceinline__ unsigned bfe(unsigned w, unsigned off) {
  unsigned r;
  asm("v_bfe_u32 %0, %1, %2, %3" : "=v"(r) : "v"(w), "v"(off), "n"(W));
  return r;
}

// Pair tables: entry (a, b) of a part with PL planes, a and b the code indices of
// two coordinates, holds their centroids as fp16 (hi_a | hi_b << 16, lo_a | lo_b
// << 16), i.e. one dword of each MFMA operand. The entry index interleaves the
// planes: bits 2 pl and 2 pl + 1 are plane pl of a and of b.
// Parts with one or two planes use quad tables instead: entry e of a part with
// PL planes holds four coordinates' centroids (hi_0 | hi_1 << 16, hi_2 | hi_3 <<
// 16, lo_0 | lo_1 << 16, lo_2 | lo_3 << 16), two dwords of each operand from
// one 16-byte read; bits 4 pl .. 4 pl + 3 of e are plane pl of the four. Both
// kinds sit in LDS, 16-byte aligned, at the part's table offset.
__host__ __device__ constexpr bool quad_table(int PL) { return PL == 1 || PL == 2; }
__host__ __device__ constexpr int table_entries(int PL) { return quad_table(PL) ? 1 << (4 * PL) : 1 << (2 * PL); }
__host__ __device__ constexpr int table_bytes(int PL) {
  return PL == 0 ? 0 : quad_table(PL) ? 16 * table_entries(PL) : (8 * table_entries(PL) + 15) / 16 * 16;
}
// QJL sign nibbles: entry e holds four fp16 +-1 (bit set: +1), two dwords
constexpr int kSignTableBytes = 16 * 8;

// Reductions over each row of 16 lanes with DPP permutations (no LDS round
// trip): swap neighbours, then pairs of a quad, then mirror the half rows and
// the row; every step combines two partials that the partner lane combines in
// the other order, so all 16 lanes end with the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_perm(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float group16_max(float v) {
  v = fmaxf(v, dpp_perm<0xB1>(v));   // quad_perm [1, 0, 3, 2]
  v = fmaxf(v, dpp_perm<0x4E>(v));   // quad_perm [2, 3, 0, 1]
  v = fmaxf(v, dpp_perm<0x141>(v));  // row_half_mirror
  return fmaxf(v, dpp_perm<0x140>(v));  // row_mirror
}
__device__ __forceinline__ float group16_sum(float v) {
  v += dpp_perm<0xB1>(v);
  v += dpp_perm<0x4E>(v);
  v += dpp_perm<0x141>(v);
  return v + dpp_perm<0x140>(v);
}
// maximum over the wave: the rows' maxima, then the four rows' through readlane
__device__ __forceinline__ float wave_max(float v) {
  v = group16_max(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// One workgroup per (batch, KV head): the query parts rotated into each key
// part's basis (q' = scale Pi_p q_p, q'' = scale sqrt(pi/2)/d_p S_p q_p, fp32),
// a power-of-two scale per (kind, head) with |x| 2^S < 2^14, and the fp16 hi/lo
// MFMA fragments (rows = 8 heads x {hi, lo}, K = 32 coordinates). The matrices
// are staged through LDS in blocks of rows (padded against bank conflicts).
__global__ __launch_bounds__(kSmThreads) void split_prep_kernel(SmParams prm) {
  extern __shared__ __align__(16) float sm[];
  __shared__ int sexp[2][kSplitMaxGroup];
  const int tid = threadIdx.x;
  const int bgi = blockIdx.x;
  const int b = bgi / prm.Hkv, g = bgi % prm.Hkv;
  const int G = prm.G;
  float* qraw = sm;                     // [G][dk]: q in the key parts' channel order
  float* qr = qraw + G * prm.dk;        // [G][dk]  q'
  float* qs = qr + G * prm.dk;          // [G][dk]  q''
  float* mat = qs + G * prm.dk;         // [2][prep_rows][d + 1] rows of Pi and S
  for (int e = tid; e < G * prm.dk; e += kSmThreads) {
    const int h = e / prm.dk, j = e % prm.dk;
    qraw[e] = __uint_as_float((unsigned)prm.q[((int64_t)b * prm.Hq + g * G + h) * prm.dim + prm.kchan[g][j]] << 16);
  }
  for (int p = 0; p < prm.nk; ++p) {
    const SmPart& P = prm.kp[p];
    const int d = P.d, ld = d + 1;
    for (int i0 = 0; i0 < d; i0 += prm.prep_rows) {
      const int nr = min(prm.prep_rows, d - i0);
      __syncthreads();  // previous block consumed (and qraw written)
      {  // eight loads in flight per thread and matrix, then the LDS stores
        const float* pg = P.pi[g] + (int64_t)i0 * d;
        const float* sg = P.qjl ? P.s[g] + (int64_t)i0 * d : pg;
        const int n = nr * d;
        for (int e0 = tid; e0 < n; e0 += 8 * kSmThreads) {
          float vp[8], vs[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int e = e0 + u * kSmThreads;
            vp[u] = e < n ? pg[e] : 0.f;
            vs[u] = e < n ? sg[e] : 0.f;
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int e = e0 + u * kSmThreads;
            if (e < n) {
              const int i = e / d, j = e - i * d;
              mat[i * ld + j] = vp[u];
              if (P.qjl) mat[prm.prep_rows * ld + i * ld + j] = vs[u];
            }
          }
        }
      }
      __syncthreads();
      for (int e = tid; e < G * nr; e += kSmThreads) {
        const int h = e / nr, i = e % nr;
        const float* pr = mat + i * ld;
        const float* sr = mat + prm.prep_rows * ld + i * ld;
        float a = 0.f, c = 0.f;
        const float* qp = qraw + h * prm.dk + P.off;
        if (P.qjl) {
#pragma unroll 8
          for (int j = 0; j < d; ++j) {
            a = fmaf(pr[j], qp[j], a);
            c = fmaf(sr[j], qp[j], c);
          }
        } else {
#pragma unroll 8
          for (int j = 0; j < d; ++j) a = fmaf(pr[j], qp[j], a);
        }
        qr[h * prm.dk + P.off + i0 + i] = prm.scale * a;
        qs[h * prm.dk + P.off + i0 + i] = P.qjl ? prm.scale * P.kappa * c : 0.f;
      }
    }
  }
  __syncthreads();
  {  // 16 threads per (kind, head): largest |x|, then its power-of-two scale
    const int kind = tid / 128, h = (tid / 16) % kSplitMaxGroup, l16 = tid % 16;
    const float* src = kind ? qs : qr;
    float mx = 0.f;
    if (h < G)
      for (int j = l16; j < prm.dk; j += 16) mx = fmaxf(mx, fabsf(src[h * prm.dk + j]));
    mx = group16_max(mx);
    if (l16 == 0) {
      int e = 0;
      frexpf(mx, &e);  // mx < 2^e
      sexp[kind][h] = mx > 0.f ? min(14 - e, 100) : 0;
      prm.qexp[bgi * 2 * kSplitMaxGroup + kind * kSplitMaxGroup + h] = sexp[kind][h];
    }
  }
  __syncthreads();
  u32x4* dst = prm.qfrag + (int64_t)bgi * (prm.dk / 32) * 2 * 64;
  for (int f = tid; f < (prm.dk / 32) * 2 * 64; f += kSmThreads) {
    const int ks = f / 128, kind = (f / 64) & 1, ln = f % 64;
    const int row = ln % 16, h = row >> 1, kb = ks * 32 + 8 * (ln / 16);
    const bool lo = row & 1;
    const float* src = kind ? qs : qr;
    u32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float x0 = 0.f, x1 = 0.f;
      if (h < G) {
        x0 = ldexpf(src[h * prm.dk + kb + 2 * e], sexp[kind][h]);
        x1 = ldexpf(src[h * prm.dk + kb + 2 * e + 1], sexp[kind][h]);
      }
      v[e] = f16_part(x0, lo) | (f16_part(x1, lo) << 16);
    }
    dst[f] = v;
  }
}

// Part configurations of the main kernel. SmDyn reads every part's shape from
// the kernel arguments at run time; SmPages fixes the pages' split of a
// 128-channel head (32 outlier channels, then 96; keys prod, values mse, each
// part with its own plane count) at compile time, so the part loops, the
// staging copies and every record offset fold into constants.
struct SmDyn {
  static constexpr bool fixed = false;
  static constexpr int nk = 0, nv = 0, dv = 0, nseg = 0;
  static constexpr int kd[1] = {0}, kpl[1] = {0}, vd[1] = {0}, vpl[1] = {0};
  __host__ __device__ static constexpr int koff(int) { return 0; }
  __host__ __device__ static constexpr int voff(int) { return 0; }
  __host__ __device__ static constexpr int vpart(int) { return 0; }
  __host__ __device__ static constexpr int seg_elem(int) { return 0; }
  __host__ __device__ static constexpr bool seg_blocked(int) { return false; }
  __host__ __device__ static constexpr int seg_lds(int) { return 0; }
  static constexpr int stage_bytes = 0, dma_rounds = 0;
  static constexpr int vnorm_seg[1] = {0};
};
template <int KP0, int KP1, int VP0, int VP1>
struct SmPages {
  static_assert(KP0 > 0 && KP1 > 0 && VP0 > 0 && VP1 > 0, "every part has code planes");
  static constexpr bool fixed = true;
  static constexpr int nk = 2, nv = 2, dv = 128, nseg = 12;
  static constexpr int kd[2] = {32, 96}, kpl[2] = {KP0, KP1}, vd[2] = {32, 96}, vpl[2] = {VP0, VP1};
  __host__ __device__ static constexpr int koff(int p) { return p ? 32 : 0; }
  __host__ __device__ static constexpr int voff(int p) { return p ? 32 : 0; }
  __host__ __device__ static constexpr int vpart(int np) { return np ? 1 : 0; }
  // staging segments, in the order the host adds them: per key part its codes,
  // signs, norms and residual norms; per value part its codes (BLOCK32) and norms
  __host__ __device__ static constexpr int seg_elem(int si) {
    return si == 0 ? 4 * KP0 : si == 4 ? 12 * KP1 : si == 8 ? 4 * VP0 : si == 10 ? 12 * VP1 : si == 5 ? 12 : 4;
  }
  __host__ __device__ static constexpr bool seg_blocked(int si) { return si == 8 || si == 10; }
  // staging offset of segment si (each 32-token segment padded to 16 bytes, as the host lays them)
  __host__ __device__ static constexpr int seg_lds(int si) {
    int at = 0;
    for (int i = 0; i < si; ++i) at += (kSmChunk * seg_elem(i) + 15) / 16 * 16;
    return at;
  }
  static constexpr int stage_bytes = seg_lds(nseg);
  static constexpr int dma_rounds = (stage_bytes + 1023) / 1024;  // 16 bytes x 64 lanes per copy
  static constexpr int vnorm_seg[2] = {9, 11};                     // value parts' norm segments
};

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

template <int NW, class C>  // NW: 32-coordinate words of the value vector, at most
__global__ __launch_bounds__(kSmThreads) __attribute__((amdgpu_waves_per_eu(C::fixed ? 3 : (NW == 4 ? 4 : 3)))) void split_main_kernel(SmParams prm) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ int sexp[2][kSplitMaxGroup];
  __shared__ __align__(16) float wts_s[kSmWaves][kSplitMaxGroup * kSmChunk];
  __shared__ int evs_s[kSmWaves][kSplitMaxParts];
  __shared__ float fix_s[kSmWaves][kSplitMaxParts];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g4 = lane >> 4;
  const int bgi = blockIdx.y;
  const int b = bgi / prm.Hkv, g = bgi % prm.Hkv;
  const int G = prm.G;
  u32x4* frag = (u32x4*)lds;  // [dk / 32][{mse, qjl}][64 lanes]
  unsigned* tabs = (unsigned*)(lds + prm.tab_off);

  // ---- tables: QJL sign nibbles (+-1 fp16), then a quad or pair table per key and value part ----
  if (tid < 32) {
    const int e = tid >> 1, h = tid & 1;  // dword h of entry e: signs of bits 2h, 2h + 1
    const unsigned s0 = (e >> (2 * h)) & 1 ? 0x3C00u : 0xBC00u, s1 = (e >> (2 * h + 1)) & 1 ? 0x3C00u : 0xBC00u;
    tabs[tid] = s0 | (s1 << 16);
  }
  for (int side = 0; side < 2; ++side) {
    const int np = side ? prm.nv : prm.nk;
    for (int p = 0; p < np; ++p) {
      const SmPart& P = side ? prm.vp[p] : prm.kp[p];
      if (quad_table(P.planes)) {
        u32x4* qt = (u32x4*)(lds + prm.tab_off + P.ptab);
        for (int e = tid; e < table_entries(P.planes); e += kSmThreads) {
          unsigned t[4];
          for (int i = 0; i < 4; ++i) {
            unsigned c = 0;
            for (int pl = 0; pl < P.planes; ++pl) c |= ((e >> (4 * pl + i)) & 1) << pl;
            t[i] = P.tab[c];
          }
          qt[e] = u32x4{(t[0] & 0xFFFFu) | (t[1] << 16), (t[2] & 0xFFFFu) | (t[3] << 16),
                        (t[0] >> 16) | (t[1] & 0xFFFF0000u), (t[2] >> 16) | (t[3] & 0xFFFF0000u)};
        }
      } else if (P.planes > 0) {
        uint2* pt = (uint2*)(lds + prm.tab_off + P.ptab);
        for (int e = tid; e < table_entries(P.planes); e += kSmThreads) {
          unsigned ia = 0, ib = 0;
          for (int pl = 0; pl < P.planes; ++pl) {
            ia |= ((e >> (2 * pl)) & 1) << pl;
            ib |= ((e >> (2 * pl + 1)) & 1) << pl;
          }
          const unsigned ta = P.tab[ia], tb = P.tab[ib];
          pt[e] = uint2{(ta & 0xFFFFu) | (tb << 16), (ta >> 16) | (tb & 0xFFFF0000u)};
        }
      }
    }
  }

  // ---- score operand fragments of this (batch, KV head), from the prep kernel ----
  {
    const int nf = (prm.dk / 32) * 2 * 64;
    const u32x4* src = prm.qfrag + (int64_t)bgi * nf;
    for (int f = tid; f < nf; f += kSmThreads) frag[f] = src[f];
    if (tid < 2 * kSplitMaxGroup) sexp[tid / kSplitMaxGroup][tid % kSplitMaxGroup] = prm.qexp[bgi * 2 * kSplitMaxGroup + tid];
  }
  __syncthreads();

  // ---- one context split per wave; no workgroup barriers from here on ----
  const int split = blockIdx.x * kSmWaves + wave;
  if (split >= prm.n_splits) return;
  const int64_t len = min(max((int64_t)prm.lens[b], (int64_t)0), prm.T);  // lengths beyond the cache attend all of it
  const int64_t t0 = (int64_t)split * prm.split_tokens;
  const int64_t t1 = min(len, t0 + prm.split_tokens);
  uint8_t* wbase = lds + prm.wave_off + wave * prm.wave_bytes;
  // in their own LDS arrays, apart from the staging buffers the direct loads write
  float* wts = wts_s[wave];  // [8 heads][32 tokens] probabilities
  int* evs = evs_s[wave];    // per value part: weight exponent
  float* fix = fix_s[wave];  // per value part: accumulator rescale
  if (lane < kSplitMaxParts) evs[lane] = kSmEvUnset;
  int evr[C::fixed ? C::nv : 1];  // fixed parts: weight exponents and rescales in registers
  float fxr[C::fixed ? C::nv : 1];
#pragma unroll
  for (int p = 0; p < (C::fixed ? C::nv : 1); ++p) {
    evr[p] = kSmEvUnset;
    fxr[p] = 1.f;
  }
  const int hA = 2 * g4, hB = 2 * g4 + 1;  // this lane's heads in every C tile
  const float imA = hA < G ? ldexpf(1.f, -sexp[0][hA]) : 0.f, imB = hB < G ? ldexpf(1.f, -sexp[0][hB]) : 0.f;
  const float iqA = hA < G ? ldexpf(1.f, -sexp[1][hA]) : 0.f, iqB = hB < G ? ldexpf(1.f, -sexp[1][hB]) : 0.f;
  const uint2* ztab = (const uint2*)tabs;
  const unsigned offv[4] = {8u * g4, 8u * g4 + 2, 8u * g4 + 4, 8u * g4 + 6};  // bit offsets of this lane's coordinate pairs

  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  f32x4 acc[2 * NW];
#pragma unroll
  for (int t = 0; t < 2 * NW; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // fixed parts: a chunk's staging buffer is copied by dma_rounds 16-byte DMA
  // copies per lane; lane l of copy k fills staging bytes [1024 k + 16 l, + 16),
  // which lie in one segment: its source pointer (advanced one chunk per copy,
  // the chunks being copied in order from t0) and step are set up once here
  const uint8_t* dsrc[C::fixed ? C::dma_rounds : 1];
  unsigned dstep[C::fixed ? C::dma_rounds : 1];
  if constexpr (C::fixed) {
#pragma unroll
    for (int k = 0; k < C::dma_rounds; ++k) {
      const int pos = 1024 * k + 16 * lane;
      dsrc[k] = nullptr;
      dstep[k] = 0;
      static_for<0, C::nseg>([&](auto SI) {
        constexpr int si = decltype(SI)::value, elem = C::seg_elem(si), at = C::seg_lds(si);
        if (pos >= at && pos < at + kSmChunk * elem) {
          dsrc[k] = prm.seg[si].base + ((int64_t)bgi * prm.T + t0) * elem + (pos - at);
          dstep[k] = kSmChunk * elem;
        }
      });
    }
  }
  // copy the records of tokens [c0, c0 + 32) into a staging buffer; tokens at or
  // beyond t1 read copies of the last valid dword (finite, masked later)
  auto issue = [&](int64_t c0, uint8_t* dst) {
    const int nvalid = (int)min((int64_t)kSmChunk, t1 - c0);
    if constexpr (C::fixed) {
      // whole chunks: records of tokens at or beyond t1 (inside max_ctx) are
      // copied too; the tail chunk's value norms are zeroed before use
#pragma unroll
      for (int k = 0; k < C::dma_rounds; ++k) {
        if (dstep[k]) __builtin_amdgcn_global_load_lds((void*)dsrc[k], (lds_ptr)(dst + 1024 * k), 16, 0, 0);
        dsrc[k] += dstep[k];
      }
      (void)nvalid;
      return;
    }
    for (int si = 0; si < prm.n_seg; ++si) {
      const SmSeg S = prm.seg[si];
      const int wpt = S.elem >> 2;
      // per-token arrays: tokens at or beyond t1 read copies of the last valid
      // dword; a BLOCK32 chunk is read whole (its block lies inside max_ctx)
      const int nd = kSmChunk * wpt, nvd = S.blocked ? nd : nvalid * wpt;
      const unsigned* src = (const unsigned*)(S.base + ((int64_t)bgi * prm.T + c0) * S.elem);
      for (int e0 = 0; e0 < nd; e0 += 64) {
        const int e = e0 + lane;
        if (e < nd)
          __builtin_amdgcn_global_load_lds((void*)(src + min(e, nvd - 1)), (lds_ptr)(dst + S.lds + 4 * e0), 4, 0, 0);
      }
    }
  };

  if (t0 < t1) issue(t0, wbase);
  int it = 0;
  for (int64_t c0 = t0; c0 < t1; c0 += kSmChunk, ++it) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this chunk's records are in LDS
    asm volatile("" ::: "memory");
    const uint8_t* sb = wbase + (it & 1) * prm.stage_bytes;
    if (c0 + kSmChunk < t1) issue(c0 + kSmChunk, wbase + ((it + 1) & 1) * prm.stage_bytes);
    const int nvalid = (int)min((int64_t)kSmChunk, t1 - c0);
    if constexpr (C::fixed) {
      if (nvalid < kSmChunk) {  // tail chunk: tokens past the context weigh nothing
#pragma unroll
        for (int p = 0; p < C::nv; ++p)
          if (lane >= nvalid && lane < kSmChunk) ((float*)(sb + C::seg_lds(C::vnorm_seg[p])))[lane] = 0.f;
        __builtin_amdgcn_wave_barrier();
      }
    }

    // ---------------- scores: 2 tiles of 16 tokens x this lane's 2 heads ----------------
    float sv[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
    // one key part with PL planes (QJ: QJL signs); am / aq: <q', c~> and <q'', z> per tile
    // (DC, OC: the part's dimension and channel offset when fixed at compile time, else 0)
    auto key_part = [&](auto PLc, auto QJc, const SmPart& P, auto DC, auto OC) {
      constexpr int PL = decltype(PLc)::value;
      constexpr bool QJ = decltype(QJc)::value;
      constexpr int DF = decltype(DC)::value, OF = decltype(OC)::value;
      const int d = DF ? DF : P.d;
      const int dq = d >> 3, rec = PL * dq, kg0 = (DF ? OF : P.off) >> 5, nks = d >> 5;
      const uint8_t* kc = sb + P.st_codes;
      const uint8_t* ksg = sb + P.st_signs;
      const uint2* tk = (const uint2*)(lds + prm.tab_off + P.ptab);
      f32x4 am[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      f32x4 aq[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      auto step = [&](int ks) {
        const u32x4 fm = frag[(2 * (kg0 + ks)) * 64 + lane];
        const u32x4 fq = frag[(2 * (kg0 + ks) + 1) * 64 + lane];
#pragma unroll
        for (int tile = 0; tile < 2; ++tile) {
          const int tok = 16 * tile + r16;
          if constexpr (PL > 0) {
            unsigned w[PL];
#pragma unroll
            for (int pl = 0; pl < PL; ++pl) w[pl] = lds_u32(kc + tok * rec + pl * dq + 4 * ks);
            u32x4 bh, bl;
            if constexpr (quad_table(PL)) {
#pragma unroll
              for (int h = 0; h < 2; ++h) {  // coordinates 8 g4 + 4h .. + 3 of this step
                unsigned qi = bfe<4>(w[0], offv[2 * h]);
                if constexpr (PL == 2) qi |= bfe<4>(w[1], offv[2 * h]) << 4;
                const u32x4 en = ((const u32x4*)tk)[qi];
                bh[2 * h] = en.x;
                bh[2 * h + 1] = en.y;
                bl[2 * h] = en.z;
                bl[2 * h + 1] = en.w;
              }
            } else {
#pragma unroll
              for (int v = 0; v < 4; ++v) {  // coordinates 8 g4 + 2v, + 1 of this step
                unsigned pi = bfe<2>(w[0], offv[v]);
#pragma unroll
                for (int pl = 1; pl < PL; ++pl) pi |= bfe<2>(w[pl], offv[v]) << (2 * pl);
                const uint2 en = tk[pi];
                bh[v] = en.x;
                bl[v] = en.y;
              }
            }
            am[tile] = mfma16(fm, bh, am[tile]);
            am[tile] = mfma16(fm, bl, am[tile]);
          }
          if constexpr (QJ) {
            const unsigned z = lds_u32(ksg + tok * dq + 4 * ks);
            u32x4 bz;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const uint2 en = ztab[bfe<4>(z, offv[2 * h])];
              bz[2 * h] = en.x;
              bz[2 * h + 1] = en.y;
            }
            aq[tile] = mfma16(fq, bz, aq[tile]);
          }
        }
      };
      if constexpr (DF != 0) {
#pragma unroll
        for (int ks = 0; ks < DF / 32; ++ks) step(ks);
      } else {
        for (int ks = 0; ks < nks; ++ks) step(ks);
      }
      const float* kn = (const float*)(sb + P.st_norms);
      const float* kr = (const float*)(sb + P.st_rnorms);
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) {
        const int tok = 16 * tile + r16;
        const float nu = kn[tok], ga = QJ ? kr[tok] : 0.f;
        // |k| (<q', c~> + gamma <q'', z>): the residual norm gamma is relative to the unit vector
        sv[tile][0] += nu * fmaf(ga * iqA, aq[tile][0] + aq[tile][1], imA * (am[tile][0] + am[tile][1]));
        sv[tile][1] += nu * fmaf(ga * iqB, aq[tile][2] + aq[tile][3], imB * (am[tile][2] + am[tile][3]));
      }
    };
    using I0 = std::integral_constant<int, 0>;
    if constexpr (C::fixed) {
      static_for<0, C::nk>([&](auto PI) {
        constexpr int p = decltype(PI)::value;
        key_part(std::integral_constant<int, C::kpl[p]>{}, std::true_type{}, prm.kp[p],
                 std::integral_constant<int, C::kd[p]>{}, std::integral_constant<int, C::koff(p)>{});
      });
    } else {
      for (int p = 0; p < prm.nk; ++p) {
        const SmPart& P = prm.kp[p];
        using I1 = std::integral_constant<int, 1>;
        using I2 = std::integral_constant<int, 2>;
        using I3 = std::integral_constant<int, 3>;
        using I4 = std::integral_constant<int, 4>;
        using T_ = std::true_type;
        using F_ = std::false_type;
        switch (P.planes * 2 + (P.qjl ? 1 : 0)) {
          case 1: key_part(I0{}, T_{}, P, I0{}, I0{}); break;
          case 2: key_part(I1{}, F_{}, P, I0{}, I0{}); break;
          case 3: key_part(I1{}, T_{}, P, I0{}, I0{}); break;
          case 4: key_part(I2{}, F_{}, P, I0{}, I0{}); break;
          case 5: key_part(I2{}, T_{}, P, I0{}, I0{}); break;
          case 6: key_part(I3{}, F_{}, P, I0{}, I0{}); break;
          case 7: key_part(I3{}, T_{}, P, I0{}, I0{}); break;
          case 8: key_part(I4{}, F_{}, P, I0{}, I0{}); break;
          default: break;
        }
      }
    }

    // ---------------- online softmax per head over the chunk ----------------
    float alpha[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const float s0 = r16 < nvalid ? sv[0][hh] : -INFINITY;
      const float s1 = 16 + r16 < nvalid ? sv[1][hh] : -INFINITY;
      const float mn = fmaxf(m_run[hh], group16_max(fmaxf(s0, s1)));  // finite: the chunk has a valid token
      alpha[hh] = __expf(m_run[hh] - mn);
      const float p0 = __expf(s0 - mn), p1 = __expf(s1 - mn);
      l_run[hh] = l_run[hh] * alpha[hh] + p0 + p1;
      m_run[hh] = mn;
      wts[(2 * g4 + hh) * kSmChunk + r16] = p0;
      wts[(2 * g4 + hh) * kSmChunk + 16 + r16] = p1;
    }
    // value weight exponents: weights p |v| 2^-ev stay below 2^14
    bool refit = false;
    // (wave-uniform: fixed parts keep them in registers, others in LDS)
    auto exponent = [&](const SmPart& P, int ev, int* ev_out, float* fix_out) {
      const float nmx = wave_max(lane < kSmChunk ? ((const float*)(sb + P.st_norms))[lane] : 0.f);
      int e = 0;
      frexpf(nmx, &e);
      const int need = nmx > 0.f ? max(e - 14, -100) : kSmEvUnset;
      *fix_out = 1.f;
      *ev_out = ev;
      if (need > ev) {
        if (ev != kSmEvUnset) *fix_out = ldexpf(1.f, ev - need);
        refit = true;
        *ev_out = need;
      }
    };
    if constexpr (C::fixed) {
      static_for<0, C::nv>([&](auto PI) {
        constexpr int p = decltype(PI)::value;
        exponent(prm.vp[p], evr[p], &evr[p], &fxr[p]);
      });
    } else {
      for (int p = 0; p < prm.nv; ++p) {
        int ev_new;
        float f;
        exponent(prm.vp[p], evs[p], &ev_new, &f);
        __builtin_amdgcn_wave_barrier();
        if (lane == 0) {
          evs[p] = ev_new;
          fix[p] = f;
        }
      }
      __builtin_amdgcn_wave_barrier();
      asm volatile("" ::: "memory");
    }
    if (refit || __ballot(alpha[0] != 1.f || alpha[1] != 1.f)) {
#pragma unroll
      for (int np = 0; np < NW; ++np) {
        if (32 * np < (C::fixed ? C::dv : prm.dv)) {
          float f;
          if constexpr (C::fixed)
            f = fxr[C::vpart(np)];
          else
            f = fix[prm.vword_part[np]];
          const float fa = alpha[0] * f, fb = alpha[1] * f;
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            acc[2 * np + hf][0] *= fa;
            acc[2 * np + hf][1] *= fa;
            acc[2 * np + hf][2] *= fb;
            acc[2 * np + hf][3] *= fb;
          }
        }
      }
    }

    // ---------------- values: 16 coordinates x 8 heads per instruction ----------------
    u32x4 aw = {0u, 0u, 0u, 0u};
    // word np of the value vector: word wd of value part p (PLc planes; DC its
    // dimension when fixed at compile time, else 0)
    auto value_np = [&](const int np, const int p, const int wd, const SmPart& P, auto PLc, auto DC) {
        if (wd == 0) {  // first word of this part: its weight operand
          int ev;
          if constexpr (C::fixed)
            ev = evr[p];
          else
            ev = evs[p];
          const float wsc = ev == kSmEvUnset ? 0.f : ldexpf(1.f, -ev);
          // K slots 0-3 of lane group g4 are tokens 4 g4 + k, slots 4-7 tokens
          // 16 + 4 g4 + k: the token order of a BLOCK32 word's two halves
          const float* wr = wts + (r16 >> 1) * kSmChunk + 4 * g4;
          const float* nr = (const float*)(sb + P.st_norms) + 4 * g4;
          const float4 wa = *(const float4*)wr, wb = *(const float4*)(wr + 16);
          const float4 na = *(const float4*)nr, nb = *(const float4*)(nr + 16);
          const float x[8] = {wa.x * na.x * wsc, wa.y * na.y * wsc, wa.z * na.z * wsc, wa.w * na.w * wsc,
                              wb.x * nb.x * wsc, wb.y * nb.y * wsc, wb.z * nb.z * wsc, wb.w * nb.w * wsc};
          const bool lo = r16 & 1;
#pragma unroll
          for (int v = 0; v < 4; ++v) aw[v] = f16_part(x[2 * v], lo) | (f16_part(x[2 * v + 1], lo) << 16);
        }
        // one 32-coordinate word of a value part with PL planes: two tiles of 16
        // coordinates. BLOCK32 codes: block word (pl, g4, c / 4) holds plane pl of
        // coordinate c for this lane's eight tokens, nibble c % 4 of each half.
        {
          constexpr int PL = decltype(PLc)::value;
          constexpr int DF = decltype(DC)::value;
          const int d4 = (DF ? DF : P.d) >> 2;
          const uint8_t* vc = sb + P.st_codes;
          const uint2* tv = (const uint2*)(lds + prm.tab_off + P.ptab);
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const int c = 32 * wd + 16 * hf + r16;  // coordinate within the part
            const unsigned nib = 4u * (unsigned)(c & 3);
            unsigned w[PL];
#pragma unroll
            for (int pl = 0; pl < PL; ++pl) w[pl] = lds_u32(vc + 4 * ((pl * 4 + g4) * d4 + (c >> 2)));
            u32x4 bh, bl;
            if constexpr (quad_table(PL)) {
#pragma unroll
              for (int h = 0; h < 2; ++h) {  // K slots 4h .. 4h + 3: the four tokens of one half
                const unsigned at = nib + 16u * (unsigned)h;
                unsigned qi = bfe<4>(w[0], at);
                if constexpr (PL == 2) qi |= bfe<4>(w[1], at) << 4;
                const u32x4 en = ((const u32x4*)tv)[qi];
                bh[2 * h] = en.x;
                bh[2 * h + 1] = en.y;
                bl[2 * h] = en.z;
                bl[2 * h + 1] = en.w;
              }
            } else {
#pragma unroll
              for (int v = 0; v < 4; ++v) {  // K slots 2v, 2v + 1: two tokens of one half
                const unsigned at = nib + 16u * (unsigned)(v >> 1) + 2u * (unsigned)(v & 1);
                unsigned pi = bfe<2>(w[0], at);
#pragma unroll
                for (int pl = 1; pl < PL; ++pl) pi |= bfe<2>(w[pl], at) << (2 * pl);
                const uint2 en = tv[pi];
                bh[v] = en.x;
                bl[v] = en.y;
              }
            }
            acc[2 * np + hf] = mfma16(aw, bh, acc[2 * np + hf]);
            acc[2 * np + hf] = mfma16(aw, bl, acc[2 * np + hf]);
          }
        }
    };
    if constexpr (C::fixed) {
      static_for<0, C::dv / 32>([&](auto NP) {
        constexpr int np = decltype(NP)::value, p = C::vpart(np);
        value_np(np, p, np - C::voff(p) / 32, prm.vp[p], std::integral_constant<int, C::vpl[p]>{},
                 std::integral_constant<int, C::vd[p]>{});
      });
    } else {
#pragma unroll
      for (int np = 0; np < NW; ++np) {
        if (32 * np < prm.dv) {
          const int p = prm.vword_part[np];
          const SmPart& P = prm.vp[p];
          const int wd = np - (P.off >> 5);
          switch (P.planes) {
            case 1: value_np(np, p, wd, P, std::integral_constant<int, 1>{}, I0{}); break;
            case 2: value_np(np, p, wd, P, std::integral_constant<int, 2>{}, I0{}); break;
            case 3: value_np(np, p, wd, P, std::integral_constant<int, 3>{}, I0{}); break;
            case 4: value_np(np, p, wd, P, std::integral_constant<int, 4>{}, I0{}); break;
            default: break;
          }
        }
      }
    }
  }

  // ---- partials: acc[dv], m, l per head ----
  const float lA = group16_sum(l_run[0]), lB = group16_sum(l_run[1]);
  const int64_t rowA = (((int64_t)b * prm.Hq + g * G + hA) * prm.n_splits + split) * (prm.dv + 2);
  const int64_t rowB = (((int64_t)b * prm.Hq + g * G + hB) * prm.n_splits + split) * (prm.dv + 2);
#pragma unroll
  for (int np = 0; np < NW; ++np) {
    if (32 * np < prm.dv) {
      int ev;
      if constexpr (C::fixed)
        ev = evr[C::vpart(np)];
      else
        ev = evs[prm.vword_part[np]];
      const float sc = ev == kSmEvUnset ? 0.f : ldexpf(1.f, ev);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int j = 32 * np + 16 * hf + r16;
        if (hA < G) prm.part[rowA + j] = (acc[2 * np + hf][0] + acc[2 * np + hf][1]) * sc;
        if (hB < G) prm.part[rowB + j] = (acc[2 * np + hf][2] + acc[2 * np + hf][3]) * sc;
      }
    }
  }
  if (r16 == 0) {
    if (hA < G) {
      prm.part[rowA + prm.dv] = m_run[0];
      prm.part[rowA + prm.dv + 1] = lA;
    }
    if (hB < G) {
      prm.part[rowB + prm.dv] = m_run[1];
      prm.part[rowB + prm.dv + 1] = lB;
    }
  }
}

// one workgroup per (batch, query head): log-sum-exp merge of the splits, then
// each value part rotated back (Pi_p^T) and written to its channels
__global__ __launch_bounds__(kSmThreads) void split_combine_kernel(SmParams prm) {
  __shared__ float a[kSplitMaxDecodeDim];
  __shared__ float ml[2];
  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.x;
  const int hq = (int)(bh % prm.Hq);
  const int g = hq / prm.G;
  const float* src = prm.part + bh * prm.n_splits * (prm.dv + 2);
  __shared__ float red[kSmWaves];
  auto block_reduce = [&](float v, bool is_max) -> float {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float u = __shfl_xor(v, o);
      v = is_max ? fmaxf(v, u) : v + u;
    }
    __syncthreads();
    if ((tid & 63) == 0) red[tid >> 6] = v;
    __syncthreads();
    float r = red[0];
    for (int w = 1; w < kSmWaves; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
    return r;
  };
  float mloc = -INFINITY;
  for (int s = tid; s < prm.n_splits; s += kSmThreads) mloc = fmaxf(mloc, src[s * (prm.dv + 2) + prm.dv]);
  const float Mx = block_reduce(mloc, true);
  float lloc = 0.f;
  if (Mx > -INFINITY)
    for (int s = tid; s < prm.n_splits; s += kSmThreads) {
      const float ms = src[s * (prm.dv + 2) + prm.dv];
      if (ms > -INFINITY) lloc += src[s * (prm.dv + 2) + prm.dv + 1] * __expf(ms - Mx);
    }
  const float Lx = block_reduce(lloc, false);
  if (tid == 0) {
    ml[0] = Mx;
    ml[1] = Lx;
  }
  __syncthreads();
  const float L = ml[1];
  // weight of each split, exp(m_s - M) / L (0 for empty splits), then the merged sum
  __shared__ float sw[kSmSplitsCached];
  const int nsc = prm.n_splits < kSmSplitsCached ? prm.n_splits : kSmSplitsCached;
  for (int s = tid; s < nsc; s += kSmThreads) {
    const float ms = src[s * (prm.dv + 2) + prm.dv];
    sw[s] = (L > 0.f && ms > -INFINITY) ? __expf(ms - Mx) / L : 0.f;
  }
  __syncthreads();
  for (int j = tid; j < prm.dv; j += kSmThreads) {
    float v = 0.f;
#pragma unroll 8
    for (int s = 0; s < nsc; ++s) v = fmaf(src[s * (prm.dv + 2) + j], sw[s], v);
    for (int s = nsc; s < prm.n_splits; ++s) {
      const float ms = src[s * (prm.dv + 2) + prm.dv];
      if (L > 0.f && ms > -INFINITY) v = fmaf(src[s * (prm.dv + 2) + j], __expf(ms - Mx) / L, v);
    }
    a[j] = v;
  }
  __syncthreads();
  float* o = prm.out + bh * prm.dim;
  for (int j = tid; j < prm.dim; j += kSmThreads) o[j] = 0.f;  // channels no value part keeps
  __syncthreads();
  for (int p = 0; p < prm.nv; ++p) {
    const SmPart& P = prm.vp[p];
    for (int j = tid; j < P.d; j += kSmThreads) {
      float v = 0.f;
      const float* pc = P.pi[g] + j;
#pragma unroll 8
      for (int i = 0; i < P.d; ++i) v = fmaf(pc[(int64_t)i * P.d], a[P.off + i], v);
      o[prm.vchan[g][P.off + j]] = v;
    }
  }
}

size_t split_part_bytes(int B, int Hq, int n_splits, int dv) {
  return ((size_t)B * Hq * n_splits * (dv + 2) * sizeof(float) + 255) / 256 * 256;
}

// kernel arguments and dynamic LDS bytes of a split decode (lds = 0 when the
// parts need more LDS than a workgroup has)
static void build_split_params(const SplitDecodeLaunch& L, SmParams& prm, size_t* lds_out) {
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
  // staging buffer of one wave: every part's per-token arrays for 32 tokens, 16-byte aligned
  int st = 0;
  auto add_seg = [&](const void* base, int elem, bool blocked = false) -> int {
    const int at = st;
    prm.seg[prm.n_seg++] = SmSeg{(const uint8_t*)base, elem, at, blocked ? 1 : 0};
    st += (kSmChunk * elem + 15) / 16 * 16;
    return at;
  };
  for (int side = 0; side < 2; ++side) {
    const SplitSide& S = side == 0 ? L.k : L.v;
    SmPart* dst = side == 0 ? prm.kp : prm.vp;
    uint8_t (*chan)[kSplitMaxDecodeDim] = side == 0 ? prm.kchan : prm.vchan;
    int off = 0;
    for (int p = 0; p < S.n_parts; ++p) {
      const tq_quantizer* q0 = S.qz[p * L.Hkv];
      SmPart& P = dst[p];
      P.d = q0->d;
      P.planes = q0->planes;
      P.off = off;
      P.qjl = side == 0 && q0->variant == TQ_PROD;
      P.rec = P.planes * P.d / 8;
      // value codes in BLOCK32: a 32-token block is 32 rec bytes, like 32 records
      if (P.planes > 0) P.st_codes = add_seg(S.codes[p], P.rec, side == 1);
      if (P.qjl) P.st_signs = add_seg(S.signs[p], P.d / 8);
      P.st_norms = add_seg(S.norms[p], 4);
      if (P.qjl) P.st_rnorms = add_seg(S.rnorms[p], 4);
      for (int i = 0; i < (1 << q0->planes) && i < 16; ++i) {
        const float c = q0->cb.centroids[i];
        const _Float16 hi = (_Float16)c;
        const _Float16 lo = (_Float16)(c - (float)hi);
        P.tab[i] = (unsigned)__builtin_bit_cast(unsigned short, hi) |
                   ((unsigned)__builtin_bit_cast(unsigned short, lo) << 16);
      }
      P.kappa = (float)(std::sqrt(M_PI / 2.0) / q0->d);
      for (int g = 0; g < L.Hkv; ++g) {
        P.pi[g] = S.qz[p * L.Hkv + g]->pi32;
        P.s[g] = S.qz[p * L.Hkv + g]->s32;
      }
      // channels [n_parts][n_kv_heads][d_p]: part p of head g starts at Hkv off + g d_p
      for (int g = 0; g < L.Hkv; ++g)
        for (int j = 0; j < P.d; ++j) chan[g][off + j] = (uint8_t)S.channels[(int64_t)L.Hkv * off + g * P.d + j];
      if (side == 1)
        for (int w = off / 32; w < (off + P.d) / 32; ++w) prm.vword_part[w] = (uint8_t)p;
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
  prm.stage_bytes = st;
  prm.tab_off = (prm.dk / 32) * 2 * 64 * 16;
  int tb = kSignTableBytes;  // QJL sign nibbles first
  for (int p = 0; p < prm.nk; ++p) {
    prm.kp[p].ptab = tb;
    tb += table_bytes(prm.kp[p].planes);
  }
  for (int p = 0; p < prm.nv; ++p) {
    prm.vp[p].ptab = tb;
    tb += table_bytes(prm.vp[p].planes);
  }
  prm.wave_off = prm.tab_off + (tb + 15) / 16 * 16;
  prm.wave_bytes = 2 * st;  // per wave: two staging buffers
  const size_t lds = prm.wave_off + (size_t)kSmWaves * prm.wave_bytes;
  *lds_out = lds > 160 * 1024 ? 0 : lds;
  // workspace: partials, then the score fragments and their scales per (batch, KV head)
  const size_t part_bytes = split_part_bytes(L.B, L.Hq, L.n_splits, prm.dv);
  uint8_t* ws = (uint8_t*)L.workspace;
  prm.qfrag = ws ? (u32x4*)(ws + part_bytes) : nullptr;
  prm.qexp = ws ? (int*)(ws + part_bytes + (size_t)L.B * L.Hkv * (prm.dk / 32) * 2 * 64 * 16) : nullptr;
}

// the main kernel for these parts: the compile-time pages' split where the
// parts and their staging segments match it exactly, else the run-time one
template <class C>
static bool matches(const SmParams& prm) {
  if (prm.nk != C::nk || prm.nv != C::nv || prm.n_seg != C::nseg) return false;
  for (int p = 0; p < C::nk; ++p)
    if (prm.kp[p].d != C::kd[p] || prm.kp[p].planes != C::kpl[p] || !prm.kp[p].qjl || prm.kp[p].off != C::koff(p))
      return false;
  for (int p = 0; p < C::nv; ++p)
    if (prm.vp[p].d != C::vd[p] || prm.vp[p].planes != C::vpl[p] || prm.vp[p].off != C::voff(p)) return false;
  for (int si = 0; si < C::nseg; ++si)
    if (prm.seg[si].elem != C::seg_elem(si) || (prm.seg[si].blocked != 0) != C::seg_blocked(si) ||
        prm.seg[si].lds != C::seg_lds(si) || ((uintptr_t)prm.seg[si].base & 15))  // 16-byte copies
      return false;
  for (int p = 0; p < C::nv; ++p)
    if (prm.vp[p].st_norms != C::seg_lds(C::vnorm_seg[p])) return false;
  return prm.stage_bytes == C::stage_bytes;
}
static void (*split_kernel(const SmParams& prm))(SmParams) {
  // 32 channels at 3 bits and 96 at 2 (prod keys: 2 and 1 MSE-stage planes), and 4 + 3 bits
  if (matches<SmPages<2, 1, 3, 2>>(prm)) return split_main_kernel<4, SmPages<2, 1, 3, 2>>;
  if (matches<SmPages<3, 2, 4, 3>>(prm)) return split_main_kernel<4, SmPages<3, 2, 4, 3>>;
  return prm.dv <= 128 ? split_main_kernel<4, SmDyn> : split_main_kernel<8, SmDyn>;
}

}  // namespace

size_t split_decode_workspace_bytes(const SplitDecodeLaunch& L, int dk, int dv) {
  return split_part_bytes(L.B, L.Hq, L.n_splits, dv) + (size_t)L.B * L.Hkv * ((dk / 32) * 2 * 64 * 16 + 2 * kSplitMaxGroup * 4);
}

int split_decode_resident_waves(const SplitDecodeLaunch& L) {
  static thread_local SmParams prm;  // large; host only
  prm = SmParams{};
  size_t lds = 0;
  build_split_params(L, prm, &lds);
  int fallback = 3 * 4 * 256;  // 3 waves per SIMD on 256 CUs
  if (lds == 0) return fallback;
  auto kern = split_kernel(prm);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return fallback;
  }
  // the answer depends on (device, kernel, LDS bytes) only: remember it
  struct Entry {
    int dev;
    void (*kern)(SmParams);
    size_t lds;
    int waves;
  };
  static std::mutex mu;
  static std::vector<Entry> seen;
  {
    std::lock_guard<std::mutex> lock(mu);
    for (const Entry& e : seen)
      if (e.dev == dev && e.kern == kern && e.lds == lds) return e.waves;
  }
  int blocks = 0, cus = 0;
  if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, kern, kSmThreads, lds) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || blocks < 1 || cus < 1) {
    (void)hipGetLastError();
    return fallback;
  }
  const int waves = blocks * kSmWaves * cus;
  std::lock_guard<std::mutex> lock(mu);
  if (seen.size() < 64) seen.push_back(Entry{dev, kern, lds, waves});
  return waves;
}

tq_status launch_split_decode(const SplitDecodeLaunch& L, hipStream_t stream) {
  static thread_local SmParams prm;
  prm = SmParams{};
  size_t lds = 0;
  build_split_params(L, prm, &lds);
  if (lds == 0) return set_error(TQ_ERR_UNSUPPORTED, "split decode: parts need more LDS than a workgroup has");
  const dim3 grid((unsigned)((L.n_splits + kSmWaves - 1) / kSmWaves), (unsigned)(L.B * L.Hkv));
  auto kern = split_kernel(prm);
  int dmax = 0;
  for (int p = 0; p < prm.nk; ++p) dmax = prm.kp[p].d > dmax ? prm.kp[p].d : dmax;
  // prep LDS: q, q', q'' [G][dk] each, then as many rows of Pi and S as fit (at most 128)
  const int fit = (int)((160 * 1024 / 4 - (size_t)prm.G * 3 * prm.dk) / (2 * (dmax + 1)));
  prm.prep_rows = fit < 128 ? fit : 128;
  const size_t plds = ((size_t)prm.G * 3 * prm.dk + 2 * (size_t)prm.prep_rows * (dmax + 1)) * sizeof(float);
  hipError_t e = hipFuncSetAttribute((const void*)split_prep_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)plds);
  if (e != hipSuccess) return check_hip(e, "split decode: set prep LDS size");
  hipLaunchKernelGGL(split_prep_kernel, dim3((unsigned)(L.B * L.Hkv)), dim3(kSmThreads), plds, stream, prm);
  tq_status st0 = launch_check("split decode: prep launch");
  if (st0 != TQ_OK) return st0;
  e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return check_hip(e, "split decode: set LDS size");
  hipLaunchKernelGGL(kern, grid, dim3(kSmThreads), lds, stream, prm);
  tq_status st2 = launch_check("split decode: main launch");
  if (st2 != TQ_OK) return st2;
  hipLaunchKernelGGL(split_combine_kernel, dim3((unsigned)(L.B * L.Hq)), dim3(kSmThreads), 0, stream, prm);
  return launch_check("split decode: combine launch");
}

}  // namespace tq
