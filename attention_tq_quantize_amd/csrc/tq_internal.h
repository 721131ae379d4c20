// Internal declarations shared by the C ABI (tq_capi.cpp) and the kernels
// (tq_kernels.hip). Not installed; the public surface is include/tq.h.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "../../include/tq.h"

namespace tq {

constexpr int kMaxBits = 4;       // GPU path: b in [1, 4]
constexpr int kMaxWalsh = 8;      // odd-size subsets of up to 4 bit planes
constexpr int kMaxKvHeads = 64;   // per-head pointers travel as kernel arguments
constexpr int kBlock = 32;        // vectors per BLOCK32 block


// A codebook for one (d, planes) pair plus its odd Walsh expansion:
//   c[idx] = sum_s walsh_coef[s] * prod_{i in walsh_mask[s]} (2 bit_i(idx) - 1)
struct Codebook {
  int d = 0, planes = 0;
  float centroids[256] = {0};   // 2^planes used; planes <= 8 on the host
  float thresholds[255] = {0};
  double cost = 0.0;
  int n_walsh = 0;
  int walsh_mask[kMaxWalsh] = {0};
  float walsh_coef[kMaxWalsh] = {0};
};

}  // namespace tq

struct tq_quantizer {
  int d = 0;
  int bits = 0;
  int planes = 0;           // MSE-stage planes: bits (mse) or bits - 1 (prod)
  tq_variant variant = TQ_MSE;
  int device = 0;
  tq::Codebook cb;          // codebook of the MSE stage (planes bits)
  // Device tables, one allocation:
  //   pi_frag / sp_frag: bf16 hi/lo MFMA fragments of Pi and S' = S Pi^T,
  //                      ordered [hilo][mtile][kstep][lane][8]
  //   pi32 / s32 / sp32: float32 row-major copies of Pi, S and S' = S Pi^T
  //                      (sp32: prod with d <= 256, else NULL); pi32 is followed
  //                      by Pi^T 1 (d floats), s32 by S^T 1 (d floats) and an
  //                      upper bound of S's row norms (then 3 zero floats)
  void* dev_block = nullptr;
  const uint16_t* pi_frag = nullptr;
  const uint16_t* sp_frag = nullptr;
  const float* pi32 = nullptr;
  const float* s32 = nullptr;
  const float* sp32 = nullptr;
  // d a multiple of 128 above 256: fragment-ordered bf16 hi/lo Pi and S' = S Pi^T
  // for the GEMM quantize kernels (own allocation)
  void* lq_block = nullptr;
  const void* lq_pi = nullptr;
  const void* lq_sp = nullptr;
};

namespace tq {

tq_status set_error(tq_status s, const std::string& msg);
tq_status check_hip(hipError_t e, const char* what);

// Host-side codebook (cached per (d, planes); thread-safe).
tq_status get_codebook(int d, int planes, const Codebook** out);

// ---- launchers (tq_kernels.hip); arguments already validated ----
struct QuantizeLaunch {
  const tq_quantizer* const* qz;
  int n_groups;
  int64_t n_per_group;
  const void* x;
  int64_t x_stride;  // elements from one input vector to the next (>= d)
  tq_dtype x_dtype;
  tq_layout layout;
  uint8_t* codes;
  uint8_t* signs;
  float* norms;
  float* rnorms;
  float* rot_dbg;
  float* proj_dbg;
};
tq_status launch_quantize(const QuantizeLaunch& a, hipStream_t stream);
// keys (VECTOR) and values (BLOCK32) of one layer in one launch, when both are
// mse with the same (d <= 256, bits), dtype and groups, packed rows, no debug outputs
bool quantize_kv_fusable(const QuantizeLaunch& k, const QuantizeLaunch& v);
tq_status launch_quantize_kv(const QuantizeLaunch& k, const QuantizeLaunch& v, hipStream_t stream);
// d > 256 (tq_large.hip): vector layout only
tq_status launch_quantize_large(const QuantizeLaunch& a, hipStream_t stream);
// fp32 kernels for any d (multiple of 32): optional channel map (quantized
// coordinate j reads input channel chan[j] of a row of x_stride elements)
tq_status launch_quantize_fp32(const QuantizeLaunch& a, const uint16_t* chan, int64_t x_stride, hipStream_t stream);
// One part of a channel split over n_groups groups of d = 128 rows on the
// matrix cores (tq_quantize.hip); chan: [n_groups][d_p] channel lists.
bool quantize_split_fast(int dim, const tq_quantizer* q);
// in-place VECTOR -> BLOCK32 repack of n_blocks blocks of 32 records (d a
// multiple of 32, 4 planes d <= 8 KiB)
tq_status launch_repack_block32(uint8_t* codes, int64_t n_blocks, int planes, int d, hipStream_t stream);
// blk: codes in the BLOCK32 layout (mse parts, n_per_group % 32 == 0).
// qz1 / chan1 / out1 non-NULL: the fused two-part split (both parts in one pass;
// quantize_split_fusable says when).
bool quantize_split_fusable(int dim, const tq_quantizer* q0, const tq_quantizer* q1);
tq_status launch_quantize_split(const tq_quantizer* const* qz, const tq_quantizer* const* qz1, int n_groups,
                                int64_t n_per_group, const uint16_t* chan, const uint16_t* chan1, const void* x,
                                tq_dtype x_dtype, bool blk, const tq_records& out, const tq_records* out1,
                                hipStream_t stream);
tq_status launch_inner_products_fp32(const tq_quantizer* q, const float* y, int64_t y_stride, const uint16_t* chan,
                                     bool accumulate, int64_t m, const uint8_t* codes, const uint8_t* signs,
                                     const float* norms, const float* rnorms, int64_t n, float* out,
                                     hipStream_t stream);
constexpr int kSplitMaxDim = 512;  // widest input row of a channel split
// decode attention over split caches (tq_split_decode.hip)
constexpr int kSplitMaxParts = 4;
constexpr int kSplitMaxKv = 8;
constexpr int kSplitMaxGroup = 8;
constexpr int kSplitMaxDecodeDim = 256;
struct SplitSide {
  int n_parts;
  const tq_quantizer* const* qz;  // [n_parts][Hkv]
  const int32_t* channels;        // host, concatenated part lists
  const uint8_t* codes[kSplitMaxParts];
  const uint8_t* signs[kSplitMaxParts];
  const float* norms[kSplitMaxParts];
  const float* rnorms[kSplitMaxParts];
};
struct SplitDecodeLaunch {
  int B, Hq, Hkv, dim;
  int64_t max_ctx;
  const void* q;
  const int32_t* lens;
  float scale;
  float* out;
  void* workspace;
  int n_splits;
  int64_t split_tokens;
  SplitSide k, v;
};
tq_status launch_split_decode(const SplitDecodeLaunch& L, hipStream_t stream);
// waves of the split decode kernel resident on the current device at once (one
// context split per wave; a fixed estimate when the device cannot be queried)
int split_decode_resident_waves(const SplitDecodeLaunch& L);
// workspace bytes: softmax partials [B][Hq][n_splits][dv + 2], then the score
// operand fragments and their scales per (batch, KV head)
size_t split_decode_workspace_bytes(const SplitDecodeLaunch& L, int dk, int dv);
// d a multiple of 128 in (256, 4096]: the GEMM quantize tables, built at creation
bool lq_supported(int d);
tq_status build_large_tables(tq_quantizer* q);
// MFMA scoring of a packed database (tq_large.hip). Workspace: fragments
// [groups][nf][64] u32x4, constants [groups][48] f32, Pi y and S y [groups*8][d] f32.
struct SearchPlan {
  int nf = 0;  // fragments per query group
  size_t frag_off = 0, const_off = 0, qp_off = 0, qq_off = 0, total = 0;
};
tq_status search_plan(const tq_quantizer* q, int64_t m, SearchPlan* plan);
tq_status launch_search(const tq_quantizer* q, const float* y, int64_t m, const uint8_t* codes,
                        const uint8_t* signs, const float* norms, const float* rnorms, int64_t n, float* out,
                        void* workspace, hipStream_t stream);
tq_status launch_inner_products_large(const tq_quantizer* q, const float* y, int64_t m,
                                      const uint8_t* codes, const uint8_t* signs, const float* norms,
                                      const float* rnorms, int64_t n, float* out, hipStream_t stream);

tq_status launch_dequantize(const tq_quantizer* q, tq_layout layout, const uint8_t* codes,
                            const uint8_t* signs, const float* norms, const float* rnorms,
                            int64_t n, float* x_out, hipStream_t stream);

tq_status launch_inner_products(const tq_quantizer* q, const float* y, int64_t m,
                                const uint8_t* codes, const uint8_t* signs, const float* norms,
                                const float* rnorms, int64_t n, float* out, hipStream_t stream);

struct DecodePlan {
  int batch, n_q_heads, n_kv_heads, d, group, chunk_heads, n_chunks;
  int64_t max_ctx;
  int n_splits;             // waves per (batch, kv head, head chunk)
  int64_t split_tokens;     // tokens per split (multiple of 32)
  size_t frag_bytes, const_bytes, partial_bytes, total_bytes;
  int k_planes, k_walsh, k_words, v_bits, v_walsh;
  bool k_qjl;
};
tq_status plan_decode(const tq_attn_shape* s, const tq_quantizer* k0, const tq_quantizer* v0,
                      DecodePlan* plan);
// Decode step with append: the new key and value of every (batch, kv head) are
// quantized into the caches at ctx_lens[b] by the launch that precedes the main
// loop, which then attends ctx_lens[b] + 1 tokens (at most max_ctx).
struct AppendLaunch {
  const void* k_new;
  const void* v_new;
  tq_dtype x_dtype;
  float* rot_dbg;   // optional [B][Hkv][2][d]
  float* proj_dbg;  // optional [B][Hkv][d]
};
tq_status launch_decode(const DecodePlan& p, const void* q, const tq_packed_kv* k,
                        const tq_packed_kv* v, const int32_t* ctx_lens, float scale, float* out,
                        float* scores_dbg, void* workspace, hipStream_t stream,
                        const AppendLaunch* app = nullptr);

// Device address of the no-alloc decode scratch on the current device
// (kNoAllocScratchBytes bytes; looked up once per device).
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
tq_status noalloc_scratch(void** ptr);

}  // namespace tq
