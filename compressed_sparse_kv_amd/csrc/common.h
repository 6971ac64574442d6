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

// CSK_OK when the calling thread's current HIP device is a gfx950 (the
// answer is kept per device after the first query); CSK_EUNSUPPORTED with a
// message naming fn otherwise, or when no device is visible.
int check_device(const std::string& fn);

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

// Entries pooled elsewhere (fp32 rows b*N + i of D values, with ncb partial
// sums of squares per entry): RMSNorm when gamma is given, RoPE of the last
// d_rope dims at entry_pos[b*N + i] (NULL: m*(entry0 + i)), then the
// output dtype (CSK_F32, CSK_BF16, CSK_MXFP4 with out_scale, CSK_FP8KV),
// written to row b*dst_bstride + i (0: N). Defined in compress.hip; the
// caller has checked the arguments.
int finalize_entries(const char* name, int B, int N, int D, int m, int entry0, int d_rope, float rope_base,
                     const int32_t* entry_pos, int out_dtype, void* out, uint8_t* out_scale, int64_t dst_bstride,
                     const float* pooled, const float* ss, int ncb, const float* gamma, float eps, hipStream_t s);

// ----------------------------------------------------------- device side

// 16-byte unit of (row, k chunk kc) in a K slab of 8 chunks per row staged
// for MFMA fragment reads (32 rows of one chunk per read): the chunk is
// XOR-swizzled by the row's low three bits and its eighth-row parity, so
// that any 8 and any 16 consecutive rows of one chunk fall on distinct
// 16-byte bank groups (128- and 256-byte bank rows alike).
__host__ __device__ __forceinline__ int slab_unit(int row, int kc) {
  return row * 8 + (kc ^ (row & 7) ^ ((row >> 3) & 1));
}

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

// OCP E4M3 code (sign bit 7, exponent bits 6..3 with bias 7, mantissa bits
// 2..0; exponent 0 is subnormal, m * 2^-9) of x under the block exponent s,
// for |x| / 2^s < 256 (the caller's scale choice): the nearest value, ties
// to the even mantissa (rintf), zero as +0. Scaling by a power of two is
// exact, so the code is decided on the exact quotient.
__device__ __forceinline__ uint32_t e4m3_encode(float x, int s) {
  const float y = ldexpf(fabsf(x), -s);
  const int e = ilogbf(y);
  uint32_t c;
  if (y == 0.0f) c = 0u;
  else if (e < -6) c = (uint32_t)rintf(ldexpf(y, 9));                          // 0..8 (8: 2^-6)
  else c = ((uint32_t)(e + 7) << 3) + (uint32_t)rintf(ldexpf(y, 3 - e)) - 8u;  // carries into e+1
  return (c != 0u && x < 0.0f) ? (c | 0x80u) : c;
}

// Block exponent of an FP8 KV block with absolute maximum amax > 0: the
// maximum lands in [128, 256); clamped to [-126, 127] so that 2^s is a
// normal fp32.
__device__ __forceinline__ int fp8kv_scale_exp(float amax) {
  int s = ilogbf(amax) - 7;
  s = s < -126 ? -126 : s;
  s = s > 127 ? 127 : s;
  return s;
}

// Bytes of one FP8 KV entry: [D - d_rope codes][d_rope bf16][scales],
// padded to a multiple of 16.
__host__ __device__ __forceinline__ int fp8kv_entry_bytes(int D, int d_rope) {
  const int dn = D - d_rope;
  return (dn + 2 * d_rope + dn / 32 + 15) / 16 * 16;
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

// cos/sin of the angle pos * theta, returned in fp32. The angle is formed
// in fp64 and reduced to r in [-pi/4, pi/4] plus a quadrant q (angle =
// q*pi/2 + r; pi/2 as a two-part constant, products folded with fma, so r
// keeps about 1e-10 absolute accuracy for angles up to 2^31 rad). sin r and
// cos r are Taylor polynomials in fp64 through the r^9 and r^10 terms
// (truncation below 2e-9 on |r| <= pi/4); the quadrant swaps and negates
// them. The fp32 results are within one ulp of the correctly rounded ones.
__device__ __forceinline__ void rope_cs(double pos, double theta, float* c, float* s) {
  constexpr double PI_2_HI = 1.5707963267948965580;     // nearest double to pi/2
  constexpr double PI_2_LO = 6.123233995736766036e-17;  // pi/2 - PI_2_HI
  constexpr double TWO_OVER_PI = 0.63661977236758134308;
  const double ang = pos * theta;
  const double q = rint(ang * TWO_OVER_PI);
  double r = fma(-q, PI_2_HI, ang);
  r = fma(-q, PI_2_LO, r);
  const double r2 = r * r;
  const double sp =
      r * (1.0 + r2 * (-1.0 / 6.0 + r2 * (1.0 / 120.0 + r2 * (-1.0 / 5040.0 + r2 * (1.0 / 362880.0)))));
  const double cp =
      1.0 + r2 * (-0.5 + r2 * (1.0 / 24.0 + r2 * (-1.0 / 720.0 + r2 * (1.0 / 40320.0 + r2 * (-1.0 / 3628800.0)))));
  const int iq = (int)((long long)q & 3);
  const double sv = iq == 0 ? sp : iq == 1 ? cp : iq == 2 ? -sp : -cp;
  const double cv = iq == 0 ? cp : iq == 1 ? -sp : iq == 2 ? -cp : sp;
  *s = (float)sv;
  *c = (float)cv;
}

// ------------------------------------------------------------ cross-lane
// Cross-lane steps built from DPP and permlane swaps (VALU operations).
// __shfl* compiles to ds_bpermute, an LDS round trip whose result must be
// waited for; chains of those dominate short reductions and scans.

// Inclusive prefix sum over a wave of 64 lanes: shifts within rows of 16
// lanes, then the row totals are carried by row broadcasts.
__device__ __forceinline__ int wave_incl_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return x;
}

// Lane l and lane l^32, then l and l^16: with both operands equal, the
// permlane swaps return the two halves that each lane combines.
__device__ __forceinline__ float group4_max(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group4_sum(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Lane l and lane l^32 (the two row halves of a 32x32 MFMA output column).
__device__ __forceinline__ float pair32_max(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
__device__ __forceinline__ float pair32_sum(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

// Reductions over all 64 lanes: within quads (quad_perm), across the quads
// of a row (row rotations), then across the four rows (group4_*).
#define CSK_DPP_F(x, ctrl) \
  __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), ctrl, 0xf, 0xf, false))
// Maximum over each row of 16 lanes (quads, then rotations within the row).
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, CSK_DPP_F(x, 0xB1));   // quad_perm [1,0,3,2]
  x = fmaxf(x, CSK_DPP_F(x, 0x4E));   // quad_perm [2,3,0,1]
  x = fmaxf(x, CSK_DPP_F(x, 0x124));  // row_ror:4
  x = fmaxf(x, CSK_DPP_F(x, 0x128));  // row_ror:8
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, CSK_DPP_F(x, 0xB1));   // quad_perm [1,0,3,2]
  x = fmaxf(x, CSK_DPP_F(x, 0x4E));   // quad_perm [2,3,0,1]
  x = fmaxf(x, CSK_DPP_F(x, 0x124));  // row_ror:4
  x = fmaxf(x, CSK_DPP_F(x, 0x128));  // row_ror:8
  return group4_max(x);
}
__device__ __forceinline__ float wave_sum(float x) {
  x += CSK_DPP_F(x, 0xB1);
  x += CSK_DPP_F(x, 0x4E);
  x += CSK_DPP_F(x, 0x124);
  x += CSK_DPP_F(x, 0x128);
  return group4_sum(x);
}

template <typename T>
struct io;

template <>
struct io<float> {
  // two consecutive values
  __device__ static __forceinline__ float2 load2(const float* p) {
    return *reinterpret_cast<const float2*>(p);
  }
  __device__ static __forceinline__ float load1(const float* p) { return *p; }
  __device__ static __forceinline__ void store1(float* p, float v) { *p = v; }
};

template <>
struct io<uint16_t> {
  __device__ static __forceinline__ float2 load2(const uint16_t* p) {
    uint32_t v = *reinterpret_cast<const uint32_t*>(p);
    return make_float2(bf16_bits_to_f32(v & 0xffffu), bf16_bits_to_f32(v >> 16));
  }
  __device__ static __forceinline__ float load1(const uint16_t* p) { return bf16_bits_to_f32(*p); }
  // round to nearest even
  __device__ static __forceinline__ void store1(uint16_t* p, float v) { *p = (uint16_t)f32_to_bf16_bits(v); }
};

}  // namespace csk
