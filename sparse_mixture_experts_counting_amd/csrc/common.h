// Shared device helpers for the libmoe kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#define MOE_WAVE 64

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round-to-nearest-even float -> bf16 (the hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  bf2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Unpack 8 bf16 held in a 16-byte word into floats.
__device__ __forceinline__ void unpack8(const u32x4 w, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(w[i]);
    f[2 * i + 1] = bf16_hi(w[i]);
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, MOE_WAVE);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, MOE_WAVE));
  return v;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint64_t w = __shfl_xor(v, o, MOE_WAVE);
    v = w > v ? w : v;
  }
  return v;
}

// The same reductions on the vector unit's lane exchanges (DPP) instead of the LDS crossbar, for
// the chains of reductions on one row (the gating's k arg-max rounds): exchanges with lane ^ 1 and
// lane ^ 2, then with the mirrored lane of each 8 and of each 16 leave every lane of a 16-lane row
// with that row's result; the four row results are read as uniform values and combined in a fixed
// order.  Each exchange pairs two lanes that combine the same two operands, so every lane ends with
// the same bits.  The whole wave must be active.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const uint32_t hi =
      (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ float readlane_f32(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_f32<0xB1>(v);    // lane ^ 1
  v += dpp_f32<0x4E>(v);    // lane ^ 2
  v += dpp_f32<0x141>(v);   // mirrored within 8
  v += dpp_f32<0x140>(v);   // mirrored within 16
  return (readlane_f32(v, 0) + readlane_f32(v, 16)) + (readlane_f32(v, 32) + readlane_f32(v, 48));
}
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x141>(v));
  v = fmaxf(v, dpp_f32<0x140>(v));
  return fmaxf(fmaxf(readlane_f32(v, 0), readlane_f32(v, 16)),
               fmaxf(readlane_f32(v, 32), readlane_f32(v, 48)));
}
__device__ __forceinline__ uint32_t wave_max_u32_dpp(uint32_t v) {
  auto ex = [](uint32_t x, auto ctrl) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, decltype(ctrl)::value, 0xF, 0xF, false);
  };
  v = max(v, ex(v, std::integral_constant<int, 0xB1>()));
  v = max(v, ex(v, std::integral_constant<int, 0x4E>()));
  v = max(v, ex(v, std::integral_constant<int, 0x141>()));
  v = max(v, ex(v, std::integral_constant<int, 0x140>()));
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(a, b), max(c, d));
}
__device__ __forceinline__ uint64_t wave_max_u64_dpp(uint64_t v) {
  uint64_t w;
  w = dpp_u64<0xB1>(v);
  v = w > v ? w : v;
  w = dpp_u64<0x4E>(v);
  v = w > v ? w : v;
  w = dpp_u64<0x141>(v);
  v = w > v ? w : v;
  w = dpp_u64<0x140>(v);
  v = w > v ? w : v;
  const uint64_t a = readlane_u64(v, 0), b = readlane_u64(v, 16);
  const uint64_t c = readlane_u64(v, 32), d = readlane_u64(v, 48);
  const uint64_t ab = a > b ? a : b, cd = c > d ? c : d;
  return ab > cd ? ab : cd;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Bits below this lane in a 64-bit ballot.
__device__ __forceinline__ uint64_t lanemask_lt() {
  int l = __lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + __expf(-z)); }

// log(sigmoid(v)) = min(v, 0) - log1p(exp(-|v|)), finite for every finite v.
__device__ __forceinline__ float log_sigmoid(float v) {
  return fminf(v, 0.f) - log1pf(expf(-fabsf(v)));
}
