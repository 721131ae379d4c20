// Device helpers shared by the kernel translation units (header-only, internal).
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "tq_internal.h"

namespace tq {
namespace {


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kMaxGroupsPerLaunch = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// lazy online-softmax rescale: keep the running max until a chunk exceeds it by this much
constexpr float kRescaleSlack = 8.0f;

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ unsigned bf16_bits(float v) {
  return (unsigned)__builtin_bit_cast(unsigned short, (__bf16)v);
}
__device__ __forceinline__ float bf16_val(unsigned h) { return __uint_as_float(h << 16); }

// hi (lo = false) or lo (lo = true) bf16 part of v; hi + lo carries 16 significant bits
__device__ __forceinline__ unsigned bf16_part(float v, bool lo) {
  const unsigned hi = bf16_bits(v);
  return lo ? bf16_bits(v - bf16_val(hi)) : hi;
}
__device__ __forceinline__ unsigned pack2(unsigned lo_half, unsigned hi_half) {
  return (lo_half & 0xFFFFu) | (hi_half << 16);
}

// Operand bits. Bit 4r+k of a word (and bit 16+4r+k) becomes an fp16 element of
// an MFMA operand: the word is shifted so that nibble r sits on bits 8-11 of each
// half (nibble 2 already does), and masked. An fp16 half whose only set bit is
// bit 8+k has the value 2^(k - 16) (bits 8 and 9 are subnormals, 10 and 11 the
// two lowest exponent values), so the element is the bit times 2^(k - 16). The
// matrix cores keep full product precision for these positions; bits further
// down (deeper subnormals) lose low product bits in the sum. The other operand
// carries the compensating powers of two.
__host__ __device__ constexpr int operand_pos(int k) { return 8 + k; }
__device__ __forceinline__ unsigned pos_mask(int p) { return (1u << p) | (1u << (16 + p)); }
__device__ __forceinline__ u32x4 bit_operand(unsigned w, int r) {
  const unsigned x = r == 0 ? (w << 8) : r == 1 ? (w << 4) : r == 2 ? w : (w >> 4);
  return u32x4{x & pos_mask(8), x & pos_mask(9), x & pos_mask(10), x & pos_mask(11)};
}

// odd-size subsets of P bit planes, in increasing mask order (matches the host's Walsh list)
__host__ __device__ constexpr int n_walsh(int P) { return P <= 0 ? 0 : (1 << (P - 1)); }
__host__ __device__ constexpr int walsh_mask(int P, int s) {
  int seen = 0;
  for (int m = 1; m < (1 << P); ++m) {
    int pc = 0;
    for (int b = 0; b < P; ++b) pc += (m >> b) & 1;
    if (pc & 1) {
      if (seen == s) return m;
      ++seen;
    }
  }
  return 0;
}

// Plane bits of the nearest-centroid index of y, by binary search over the
// float32 thresholds (t_i = largest float32 not above the midpoint of centroids
// i and i+1; y > t_i <=> strictly nearer centroid i+1; ties go low).
template <int P>
__device__ __forceinline__ void search_bits(float y, const float* T, bool* bit) {
  if constexpr (P == 1) {
    bit[0] = y > T[0];
  } else if constexpr (P == 2) {
    bit[1] = y > T[1];
    bit[0] = y > (bit[1] ? T[2] : T[0]);
  } else if constexpr (P == 3) {
    bit[2] = y > T[3];
    bit[1] = y > (bit[2] ? T[5] : T[1]);
    const float a = bit[2] ? T[4] : T[0];
    const float b = bit[2] ? T[6] : T[2];
    bit[0] = y > (bit[1] ? b : a);
  } else if constexpr (P == 4) {
    bit[3] = y > T[7];
    bit[2] = y > (bit[3] ? T[11] : T[3]);
    const float a1 = bit[3] ? T[9] : T[1];
    const float b1 = bit[3] ? T[13] : T[5];
    bit[1] = y > (bit[2] ? b1 : a1);
    const float c0 = bit[3] ? T[8] : T[0];
    const float c1 = bit[3] ? T[10] : T[2];
    const float c2 = bit[3] ? T[12] : T[4];
    const float c3 = bit[3] ? T[14] : T[6];
    const float lo = bit[1] ? c1 : c0;
    const float hi = bit[1] ? c3 : c2;
    bit[0] = y > (bit[2] ? hi : lo);
  }
}

template <int P>
__device__ __forceinline__ float centroid_of(const bool* bit, const float* C) {
  if constexpr (P == 0) {
    return 0.0f;
  } else if constexpr (P == 1) {
    return bit[0] ? C[1] : C[0];
  } else if constexpr (P == 2) {
    const float a = bit[0] ? C[1] : C[0];
    const float b = bit[0] ? C[3] : C[2];
    return bit[1] ? b : a;
  } else {
    int idx = 0;
#pragma unroll
    for (int p = 0; p < P; ++p) idx |= (bit[p] ? 1 : 0) << p;
    float v = C[0];
#pragma unroll
    for (int i = 1; i < (1 << P); ++i) v = idx == i ? C[i] : v;
    return v;
  }
}


// ---- fp16 matrix-core helpers shared by the decode and vector-search kernels ----
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

// exponent E such that |w| <= wmax keeps |w| 2^(E + 14) < 2^14 (the largest
// compensation is 2^14), so every scaled weight and its lo part stay normal fp16
// down to about 2^-10 of the largest weight
__device__ __forceinline__ int range_exp(float wmax) {
  if (!(wmax > 0.f)) return 0;
  int e;
  frexpf(wmax, &e);  // wmax < 2^e
  return -e;
}

// lanes l and l ^ 1 exchange a value (DPP quad permutation [1, 0, 3, 2])
__device__ __forceinline__ float swap_pair(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true));
}

// s_waitcnt immediate (gfx9 encoding) that waits for lgkmcnt(0) only
constexpr int kWaitLgkm0 = 0xC07F;

// an LDS address as the buffer/global-to-LDS load builtins take it
typedef __attribute__((address_space(3))) void* lds_ptr;

// A raw buffer resource as four SGPRs (48-bit base, 32-bit byte range, no
// stride) for the LDS loads below, which are written in assembly.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 make_rsrc4(const void* base, unsigned bytes) {
  const unsigned long long a = (unsigned long long)base;
  return i32x4{(int)(unsigned)a, (int)((a >> 32) & 0xFFFFu), (int)bytes, 0x00020000};
}
// 16 bytes per lane from byte voff of r straight into LDS at lds + 16 lane
// (lanes past the range load zeros), with the non-temporal hint: the bytes are
// streamed once. Written in assembly so that the compiler
// does not make every later LDS read wait for it: the caller waits with
// wait_vmcnt before it reads the bytes, and must not overwrite the
// destination's earlier reads before they have returned. m0 is restored.
__device__ __forceinline__ void lds_load16(i32x4 r, unsigned voff, unsigned lds) {
  unsigned save;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %2, %3, 0 offen nt lds\n\ts_mov_b32 m0, %0"
      : "=&s"(save)
      : "s"(lds), "v"(voff), "s"(r)
      : "memory");
}
// wait until at most N vector memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Buffer resources: a wave-uniform base in SGPRs plus a 32-bit lane offset keeps
// the hot loop free of 64-bit VGPR address arithmetic (raw buffer, 32-bit data).
typedef __amdgpu_buffer_rsrc_t buf_t;
__device__ __forceinline__ buf_t make_buf(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ unsigned ld32(buf_t r, unsigned voff, unsigned soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
__device__ __forceinline__ uint2 ld64(buf_t r, unsigned voff, unsigned soff) {
  typedef unsigned u2 __attribute__((ext_vector_type(2)));
  const u2 v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
  return uint2{v.x, v.y};
}
__device__ __forceinline__ void st32(buf_t r, unsigned v, unsigned voff, unsigned soff) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, voff, soff, 0);
}
__device__ __forceinline__ uint4 ld128(buf_t r, unsigned voff, unsigned soff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return uint4{v.x, v.y, v.z, v.w};
}

// ------------------------------- dispatch helpers -------------------------------
template <typename F>
tq_status dispatch_dim(int d, F&& f) {
  switch (d) {
    case 64: return f(std::integral_constant<int, 64>{});
    case 128: return f(std::integral_constant<int, 128>{});
    case 256: return f(std::integral_constant<int, 256>{});
  }
  return set_error(TQ_ERR_UNSUPPORTED, "unsupported head dimension");
}
template <typename F>
tq_status dispatch_planes(int p, F&& f) {
  switch (p) {
    case 0: return f(std::integral_constant<int, 0>{});
    case 1: return f(std::integral_constant<int, 1>{});
    case 2: return f(std::integral_constant<int, 2>{});
    case 3: return f(std::integral_constant<int, 3>{});
    case 4: return f(std::integral_constant<int, 4>{});
  }
  return set_error(TQ_ERR_UNSUPPORTED, "unsupported plane count");
}
template <typename F>
tq_status dispatch_bool(bool v, F&& f) {
  return v ? f(std::true_type{}) : f(std::false_type{});
}

tq_status launch_check(const char* what) { return check_hip(hipGetLastError(), what); }

// compute units of the current device, queried once (thread-safe static init;
// a process here drives one GPU model)
int device_cus() {
  static const int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    return n;
  }();
  return cus;
}

}  // namespace
}  // namespace tq
