// common.h - shared device helpers and host plumbing for libcsk (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "../../include/csk.h"

namespace csk {

// ------------------------------------------------------------- host side

// Thread-local error message; every ABI function returns through fail().
void set_error(const std::string& msg);
int fail(int code, const std::string& msg);
void clear_error();

// Measurement hook: brackets the armed kernel's launches with events.
void timer_before(const char* kernel, hipStream_t s);
void timer_after(const char* kernel, hipStream_t s);

// Launch helper: records timer events around the launch and turns a launch
// error into CSK_EHIP.
template <typename Kernel, typename... Args>
int launch(const char* name, Kernel k, dim3 grid, dim3 block, size_t lds, hipStream_t s,
           Args... args) {
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return CSK_OK;
  timer_before(name, s);
  hipLaunchKernelGGL(k, grid, block, lds, s, args...);
  hipError_t e = hipGetLastError();
  timer_after(name, s);
  if (e != hipSuccess) return fail(CSK_EHIP, std::string(name) + ": " + hipGetErrorString(e));
  return CSK_OK;
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ----------------------------------------------------------- device side

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// float -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// E2M1 code (0..7) of a scaled magnitude y = |x| / 2^s in [0, 8): nearest
// grid value of {0, .5, 1, 1.5, 2, 3, 4, 6}, halfway cases to the code with
// an even mantissa bit, everything past 5 to 6.
__device__ __forceinline__ uint32_t e2m1_code(float y) {
  uint32_t c = 7;
  c = (y <= 5.0f) ? 6u : c;
  c = (y < 3.5f) ? 5u : c;
  c = (y <= 2.5f) ? 4u : c;
  c = (y < 1.75f) ? 3u : c;
  c = (y <= 1.25f) ? 2u : c;
  c = (y < 0.75f) ? 1u : c;
  c = (y <= 0.25f) ? 0u : c;
  return c;
}

// E8M0 scale exponent of a 1x32 tile with absolute maximum amax > 0:
// floor(log2 amax) - 2 clamped to [-127, 127].
__device__ __forceinline__ int mx_scale_exp(float amax) {
  int e = ilogbf(amax);
  int s = e - 2;
  s = s < -127 ? -127 : s;
  s = s > 127 ? 127 : s;
  return s;
}

// Signed 4-bit code of x under the tile exponent s.
__device__ __forceinline__ uint32_t e2m1_encode(float x, int s) {
  float y = ldexpf(fabsf(x), -s);
  uint32_t c = e2m1_code(y);
  return (c != 0u && x < 0.0f) ? (c | 8u) : c;
}

// Partial RoPE frequencies theta_j = base^(-2j/d_rope), formed once per call
// on the host in fp64 and passed by value with the kernel arguments.
constexpr int MAX_ROPE_PAIRS = 64;
struct RopeTable {
  double theta[MAX_ROPE_PAIRS];
};
void fill_rope_table(RopeTable* t, int d_rope, double base);

// cos/sin of the angle pos * theta, formed in fp64, returned in fp32.
__device__ __forceinline__ void rope_cs(double pos, double theta, float* c, float* s) {
  double sd, cd;
  sincos(pos * theta, &sd, &cd);
  *c = (float)cd;
  *s = (float)sd;
}

template <typename T>
struct io;

template <>
struct io<float> {
  // two consecutive values
  __device__ static __forceinline__ float2 load2(const float* p) {
    return *reinterpret_cast<const float2*>(p);
  }
};

template <>
struct io<uint16_t> {
  __device__ static __forceinline__ float2 load2(const uint16_t* p) {
    uint32_t v = *reinterpret_cast<const uint32_t*>(p);
    return make_float2(bf16_bits_to_f32(v & 0xffffu), bf16_bits_to_f32(v >> 16));
  }
};

}  // namespace csk
