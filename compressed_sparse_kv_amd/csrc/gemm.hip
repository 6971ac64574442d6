// gemm.hip - bf16 matrix products on the matrix cores (gfx950), and the
// grouped output projection built from them.
//
// The grouped output projection follows the DeepSeek-V4 technical report
// page («Техотчёт DeepSeek-V4 (2026): миллион токенов контекста»), section
// «CSA: сжать в 4 раза и выбрать top-k», step 4: the heads' outputs are
// split into g groups, each group is projected to an intermediate width,
// and the groups' intermediates together are projected to the hidden size.
//
// Both products are C[M,N] = A[M,K] B[N,K]^T with bf16 operands (K
// contiguous in both, i.e. weights stored [out, in]) and fp32 accumulation
// on v_mfma_f32_32x32x16_bf16. Two kernels:
//   - many rows: 256x256 output tiles, 64-deep K slabs staged by LDS DMA
//     into two buffers (the next slab loads while the current one is
//     multiplied), four waves of 128x128 each; tiles are handed out
//     XCD-contiguously so that tiles sharing operand rows run in one L2;
//   - at most 32 rows (decode): the product streams the weights, so each
//     workgroup owns 32 output columns (16 on 16x16x32 products when there
//     are at most 16 rows), its four waves split K four ways
//     and load their fragments straight from memory (many 16-byte loads in
//     flight per lane), and the four partial tiles are summed in a fixed
//     order through LDS.
#include "common.h"

namespace csk {
namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// s_waitcnt immediate: vmcnt(n), lgkmcnt(0), expcnt unchanged
#define CSK_G_VMCNT(n) ((((n) & 0xF) | ((((n) >> 4) & 0x3) << 14)) | (0x7 << 4))

struct GemmArgs {
  const uint16_t* A;   // A[m][k] at A + batch*a_bs + m*lda + k
  const uint16_t* B;   // B[n][k] at B + batch*b_bs + n*ldb + k
  void* C;             // C[m][n] at C + batch*c_bs + m*ldc + n
  int64_t lda, ldb, ldc, a_bs, b_bs, c_bs;
  int M, N, K;
  int c_f32;           // 1: C is fp32, 0: bf16 (round to nearest even)
};

__device__ __forceinline__ void store_c(const GemmArgs& g, int64_t off, float v) {
  if (g.c_f32) reinterpret_cast<float*>(g.C)[off] = v;
  else reinterpret_cast<uint16_t*>(g.C)[off] = (uint16_t)f32_to_bf16_bits(v);
}

// ------------------------------------------------------- many rows
constexpr int TM = 256, TN = 256, TK = 64;
constexpr int TU = TM * TK / 8;  // 16-byte units of one operand slab (2048)

// Slab layout: unit (row, kc) of a 256 x 64 slab (kc = k/8) sits at
// slab_unit(row, kc); a DMA instruction fills 64 consecutive units, i.e.
// eight rows of 128 contiguous bytes each, and a fragment read (32 rows,
// one kc) finds its units on distinct bank groups.
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_tile_kernel(GemmArgs g) {
  __shared__ __align__(16) uint4 lds[2][2][TU];  // [buffer][A, B][unit], 128 KB
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // eight waves, two per SIMD: wave (wr, wc) owns rows 128*wr.. and
  // columns 64*wc.. of the tile (4 x 2 accumulators of 32 x 32)
  const int wr = wave & 1, wc = wave >> 1;
  // XCD-contiguous tile order: workgroup w runs on XCD w % 8; XCD x takes
  // a contiguous run of the row-major tile list
  const int tn = (g.N + TN - 1) / TN, tm = (g.M + TM - 1) / TM;
  const int total = tn * tm;
  const int w = blockIdx.x, xcd = w & 7, per = total >> 3, rem = total & 7;
  const int L = xcd * per + min(xcd, rem) + (w >> 3);
  const int m0 = (L / tn) * TM, n0 = (L % tn) * TN;
  const int64_t bt = blockIdx.y;
  const uint16_t* A = g.A + bt * g.a_bs;
  const uint16_t* B = g.B + bt * g.b_bs;

  // ordinary stores into the slabs first (the DMA builtin is not seen as
  // a writer of them, and without one their reads could be folded away)
  for (int u = tid; u < 2 * 2 * TU; u += 512) (&lds[0][0][0])[u] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();

  // this lane's DMA sources: instruction i (0..3) of operand X covers
  // units 64*(4*wave + i) + lane: row 32*wave + 8*i + lane/8, slot lane%8,
  // the k chunk that slab_unit puts in that slot; rows past the matrix
  // read its last row (their products land in output rows or columns that
  // are not stored)
  const int r_base = 32 * wave + (lane >> 3);
  auto src = [&](const uint16_t* X, int64_t ld, int x0, int xmax, int i) {
    const int row = r_base + 8 * i;
    const int kc = (lane & 7) ^ (row & 7) ^ ((row >> 3) & 1);  // slab_unit's inverse
    return X + (int64_t)min(x0 + row, xmax - 1) * ld + 8 * kc;
  };
  const uint16_t* pa[4];
  const uint16_t* pb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pa[i] = src(A, g.lda, m0, g.M, i);
    pb[i] = src(B, g.ldb, n0, g.N, i);
  }
  auto issue = [&](int kt, int buf) {
    const int k0 = kt * TK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_global_load_lds(pa[i] + k0, &lds[buf][0][64 * (4 * wave + i)], 16, 0, 0);
      __builtin_amdgcn_global_load_lds(pb[i] + k0, &lds[buf][1][64 * (4 * wave + i)], 16, 0, 0);
    }
  };

  v16f acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int nk = g.K / TK;
  issue(0, 0);
  // fragment read position: row (lane%32) of a 32-row tile, k chunk
  // 2*ks + lane/32
  const int fr = lane & 31, fh = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) {
      issue(kt + 1, buf ^ 1);
      __builtin_amdgcn_s_waitcnt(CSK_G_VMCNT(8));  // slab kt landed (kt+1's 8 in flight)
    } else {
      __builtin_amdgcn_s_waitcnt(CSK_G_VMCNT(0));
    }
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const uint4* sa = lds[buf][0];
    const uint4* sb = lds[buf][1];
    // the fragments of K-step ks+1 are read while ks's 8 products run
    v8bf af[2][4], bfr[2][2];
    auto read_frags = [&](int ks, v8bf* fa, v8bf* fb) {
      const int kc = 2 * ks + fh;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ra = 128 * wr + 32 * i + fr;
        fa[i] = __builtin_bit_cast(v8bf, sa[slab_unit(ra, kc)]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int rb = 64 * wc + 32 * j + fr;
        fb[j] = __builtin_bit_cast(v8bf, sb[slab_unit(rb, kc)]);
      }
    };
    read_frags(0, af[0], bfr[0]);
#pragma unroll
    for (int ks = 0; ks < TK / 16; ++ks) {
      // two products, then the next step's reads (hidden by the other six)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[0][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][0], bfr[ks & 1][j], acc[0][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (ks + 1 < TK / 16) read_frags(ks + 1, af[(ks + 1) & 1], bfr[(ks + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 1; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][i], bfr[ks & 1][j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // every wave is done with this buffer before the next DMA into it
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(CSK_G_VMCNT(63));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }

  // lane holds, per (i, j): column n0 + 64*wc + 32*j + lane%32, rows
  // m0 + 128*wr + 32*i + 8*q + 4*(lane/32) + e for element 4q + e
  char* C = reinterpret_cast<char*>(g.C) + bt * g.c_bs * (g.c_f32 ? 4 : 2);
  GemmArgs gc = g;
  gc.C = C;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int col = n0 + 64 * wc + 32 * j + fr;
    if (col >= g.N) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = m0 + 128 * wr + 32 * i + 8 * q + 4 * fh + e;
          if (row < g.M) store_c(gc, (int64_t)row * g.ldc + col, acc[i][j][4 * q + e]);
        }
  }
}

// ------------------------------------------------------ at most 32 rows
constexpr int SK_UNROLL = 8;  // K-steps whose loads are issued together

__global__ __launch_bounds__(256) void gemm_skinny_kernel(GemmArgs g) {
  __shared__ float red[3][16][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * 32;
  const int64_t bt = blockIdx.y;
  const int kq = g.K / 4;  // this wave's K range: [wave*kq, (wave+1)*kq), a multiple of 16
  // fragment rows: A row lane%32 (rows past M read row M-1; their outputs
  // are not stored), B row (output column) n0 + lane%32
  const int fr = lane & 31, fh = lane >> 5;
  const uint16_t* pa = g.A + bt * g.a_bs + (int64_t)min(fr, g.M - 1) * g.lda + wave * kq + 8 * fh;
  const uint16_t* pb = g.B + bt * g.b_bs + (int64_t)min(n0 + fr, g.N - 1) * g.ldb + wave * kq + 8 * fh;
  v16f acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  int k = 0;
  for (; k + 16 * SK_UNROLL <= kq; k += 16 * SK_UNROLL) {
    v8bf af[SK_UNROLL], bfr[SK_UNROLL];
#pragma unroll
    for (int u = 0; u < SK_UNROLL; ++u) {
      bfr[u] = *reinterpret_cast<const v8bf*>(pb + k + 16 * u);
      af[u] = *reinterpret_cast<const v8bf*>(pa + k + 16 * u);
    }
#pragma unroll
    for (int u = 0; u < SK_UNROLL; ++u) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[u], bfr[u], acc, 0, 0, 0);
  }
  for (; k < kq; k += 16) {
    const v8bf bf1 = *reinterpret_cast<const v8bf*>(pb + k);
    const v8bf af1 = *reinterpret_cast<const v8bf*>(pa + k);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af1, bf1, acc, 0, 0, 0);
  }
  // partial tiles of waves 1..3 through LDS; wave 0 adds them in order
  if (wave > 0)
#pragma unroll
    for (int e = 0; e < 16; ++e) red[wave - 1][e][lane] = acc[e];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = ((acc[e] + red[0][e][lane]) + red[1][e][lane]) + red[2][e][lane];
  const int col = n0 + fr;
  if (col >= g.N) return;
  char* C = reinterpret_cast<char*>(g.C) + bt * g.c_bs * (g.c_f32 ? 4 : 2);
  GemmArgs gc = g;
  gc.C = C;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 8 * q + 4 * fh + e;
      if (row < g.M) store_c(gc, (int64_t)row * g.ldc + col, acc[4 * q + e]);
    }
}

// At most 16 rows: 16 output columns per workgroup on 16x16x32 products
// (twice the workgroups of the 32-column form, for the same weight bytes),
// four lanes reading 64 contiguous bytes of a weight row per K-step.
constexpr int SK16_UNROLL = 16;

typedef float v4f __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void gemm_skinny16_kernel(GemmArgs g) {
  __shared__ float red[3][4][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * 16;
  const int64_t bt = blockIdx.y;
  const int kq = g.K / 4;  // this wave's K range, a multiple of 16
  // fragment rows: A row lane%16 (rows past M read row M-1; not stored),
  // B row n0 + lane%16; k chunk lane/16 of each 32-deep step
  const int fr = lane & 15, fq = lane >> 4;
  const uint16_t* pa = g.A + bt * g.a_bs + (int64_t)min(fr, g.M - 1) * g.lda + wave * kq + 8 * fq;
  const uint16_t* pb = g.B + bt * g.b_bs + (int64_t)min(n0 + fr, g.N - 1) * g.ldb + wave * kq + 8 * fq;
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  int k = 0;
  for (; k + 32 * SK16_UNROLL <= kq; k += 32 * SK16_UNROLL) {
    v8bf af[SK16_UNROLL], bfr[SK16_UNROLL];
#pragma unroll
    for (int u = 0; u < SK16_UNROLL; ++u) {
      bfr[u] = *reinterpret_cast<const v8bf*>(pb + k + 32 * u);
      af[u] = *reinterpret_cast<const v8bf*>(pa + k + 32 * u);
    }
#pragma unroll
    for (int u = 0; u < SK16_UNROLL; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[u], bfr[u], acc, 0, 0, 0);
  }
  for (; k < kq; k += 32) {
    const v8bf bf1 = *reinterpret_cast<const v8bf*>(pb + k);
    const v8bf af1 = *reinterpret_cast<const v8bf*>(pa + k);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af1, bf1, acc, 0, 0, 0);
  }
  if (wave > 0)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wave - 1][e][lane] = acc[e];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int e = 0; e < 4; ++e) acc[e] = ((acc[e] + red[0][e][lane]) + red[1][e][lane]) + red[2][e][lane];
  // lane holds column n0 + lane%16, rows 4*(lane/16) + e
  const int col = n0 + fr;
  if (col >= g.N) return;
  char* C = reinterpret_cast<char*>(g.C) + bt * g.c_bs * (g.c_f32 ? 4 : 2);
  GemmArgs gc = g;
  gc.C = C;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int row = 4 * fq + e;
    if (row < g.M) store_c(gc, (int64_t)row * g.ldc + col, acc[e]);
  }
}

// Launches C = A B^T for `batches` products. Caller checks: K % 64 == 0,
// leading dimensions and batch strides multiples of 8 elements, operands
// 16-byte aligned, M, N >= 1.
int launch_gemm(const char* name, const GemmArgs& g, int batches, hipStream_t s) {
  if (g.M <= 16 && (g.K / 4) % 32 == 0)
    return launch(name, gemm_skinny16_kernel, dim3((unsigned)ceil_div(g.N, 16), (unsigned)batches), dim3(256), 0,
                  s, g);
  if (g.M <= 32)
    return launch(name, gemm_skinny_kernel, dim3((unsigned)ceil_div(g.N, 32), (unsigned)batches), dim3(256), 0, s,
                  g);
  const int64_t tiles = ceil_div(g.M, TM) * ceil_div(g.N, TN);
  return launch(name, gemm_tile_kernel, dim3((unsigned)tiles, (unsigned)batches), dim3(512), 0, s, g);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace
}  // namespace csk

using namespace csk;

extern "C" size_t grouped_out_proj_workspace_size(int R, int g, int dg) {
  if (R <= 0 || g <= 0 || dg <= 0) return 0;
  return (size_t)R * g * dg * 2;
}

extern "C" int grouped_out_proj(const void* o, const void* w1, const void* w2, int R, int H, int dv, int g,
                                int dg, int d, int y_dtype, void* y, void* workspace, size_t ws_bytes,
                                void* stream) {
  clear_error();
  const std::string f = "grouped_out_proj";
  if (R < 0 || H <= 0 || dv <= 0 || g <= 0 || dg <= 0 || d <= 0 || H % g)
    return fail(CSK_EINVAL, f + ": need R >= 0, H, dv, g, dg, d > 0 and g dividing H");
  if (y_dtype != CSK_BF16 && y_dtype != CSK_F32)
    return fail(CSK_EUNSUPPORTED, f + ": y_dtype must be CSK_BF16 or CSK_F32");
  const int64_t K1 = (int64_t)(H / g) * dv, K2 = (int64_t)g * dg;
  if (K1 % 64 || K2 % 64 || d % 8)
    return fail(CSK_EUNSUPPORTED, f + ": built for (H/g)*dv and g*dg multiples of 64 and d a multiple of 8");
  if (R == 0) return CSK_OK;
  if (!o || !w1 || !w2 || !y || !workspace) return fail(CSK_EINVAL, f + ": null pointer");
  if (!aligned16(o) || !aligned16(w1) || !aligned16(w2) || !aligned16(workspace) || !aligned16(y))
    return fail(CSK_EINVAL, f + ": o, w1, w2, y and workspace must be 16-byte aligned");
  if (ws_bytes < grouped_out_proj_workspace_size(R, g, dg))
    return fail(CSK_EWORKSPACE, f + ": workspace smaller than grouped_out_proj_workspace_size()");
  if (const int dc = check_device(f); dc != CSK_OK) return dc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint16_t* u = reinterpret_cast<uint16_t*>(workspace);
  // u[:, i*dg:(i+1)*dg] = o[:, i*K1:(i+1)*K1] w1[i]^T, one product per group
  GemmArgs g1{};
  g1.A = reinterpret_cast<const uint16_t*>(o);
  g1.B = reinterpret_cast<const uint16_t*>(w1);
  g1.C = u;
  g1.lda = (int64_t)H * dv; g1.ldb = K1; g1.ldc = K2;
  g1.a_bs = K1; g1.b_bs = (int64_t)dg * K1; g1.c_bs = dg;
  g1.M = R; g1.N = dg; g1.K = (int)K1; g1.c_f32 = 0;
  if (const int rc = launch_gemm("out_proj_groups", g1, g, s); rc != CSK_OK) return rc;
  // y = u w2^T
  GemmArgs g2{};
  g2.A = u;
  g2.B = reinterpret_cast<const uint16_t*>(w2);
  g2.C = y;
  g2.lda = K2; g2.ldb = K2; g2.ldc = d;
  g2.M = R; g2.N = d; g2.K = (int)K2; g2.c_f32 = y_dtype == CSK_F32;
  return launch_gemm("out_proj_hidden", g2, 1, s);
}
