// indexer.hip - lightning indexer scores and top-k selection on gfx950.
//
// Scores ([P1] «CSA: сжать в 4 раза и выбрать top-k», step 2; [P3] FP4
// lightning indexer with a ReLU-scored multi-head dot product):
//   I[t,s] = sum_h w[t,h] * ReLU(q[t,h] . k[s]).
//
// MXFP4 path: q.k for 16 heads x 16 keys is one scaled FP4 MFMA
// (v_mfma_scale_f32_16x16x128_f8f6f4, E2M1 operands with per-32 E8M0
// scales). Lane l of an operand holds row l%16 and the 32 consecutive
// elements 32*(l/16).. of the 128-wide K slice, with that tile's scale byte;
// the result lane l holds column l%16, rows 4*(l/16)..+3. Each tile sum is
// an integer times a power of two, so the MFMA result is the exact dot
// product whenever the four tile exponents of a (q, k) pair lie within the
// fp32 significand (inputs from the MXFP4 quantiser of Gaussian data do).
//
// The head sum must be a fp32 fma chain over h ascending, which a lane can
// only run if it holds all heads of one key. Query heads are permuted into
// the MFMA rows so that lane group g holds heads 4*HT*g .. 4*HT*g+4*HT-1 of
// its key column; four key tiles (64 keys) are then transposed across lane
// groups with v_permlane32_swap / v_permlane16_swap, after which lane l
// holds every head of key 64*iter + l and runs the chain in registers.
//
// Top-k: the k highest scores (ties to the lower index) in ascending index
// order. Rows with at most TOPK_CAP candidates are selected in LDS on an
// order-preserving 32-bit key, by histograms over the keys' own range that
// narrow it to the k-th largest key, followed by an index-ordered
// compaction. Longer rows (decode over 32K-1M entries) are
// first filtered with a threshold L that provably keeps at least k keys:
// the scoring kernel writes the maximum of every group of GS consecutive
// keys, and L is at most the k-th largest of those group maxima (each is a
// distinct element, so at least k elements are >= L). Filtering writes
// per-slice candidate lists in index order, and the same range select
// finishes.
#include <algorithm>
#include <type_traits>
#include <atomic>
#include <mutex>

#include "common.h"

namespace csk {

constexpr int TOPK_CAP = 16384;   // elements a row select keeps in LDS
constexpr int TOPK_THREADS = 1024;
constexpr int SLICE = 2048;       // keys per filter workgroup
constexpr int IDX_MIN_ITERS = 4;      // 64-key groups per wave, at least
constexpr int IDX_TARGET_WGS = 512;   // two resident 4-wave workgroups per CU

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

struct IdxArgs {
  const uint8_t* qc;   // MXFP4 q codes   [R, HI, dI/2]
  const uint8_t* qs;   // MXFP4 q scales  [R, HI, dI/32]
  const float* qf;     // fp32 q          [R, HI, dI]
  const float* w;      // [R, HI]
  const uint8_t* kc;   // [B, Nmax, dI/2]
  const uint8_t* ks;   // [B, Nmax, dI/32]
  const float* kf;     // [B, Nmax, dI]
  const int32_t* q_pos;
  const int32_t* n_entries;
  int B, T, HI, dI, Nmax, m;
  float* scores;       // [R, Nmax]
  float* samples;      // [R, NG] or null
  int gs_log2, ng;
  int iters;           // 64-key groups per wave (MFMA path; also a template value)
  bool bf16_scores;    // scores rounded once to bf16 before they are stored
};

// A score as the top-k sees it: the fp32 value, or its nearest bf16 (ties
// to even) when the call asks for BF16 scores.
__device__ __forceinline__ float topk_score(const IdxArgs& a, float x) {
  return a.bf16_scores ? __uint_as_float(f32_to_bf16_bits(x) << 16) : x;
}

// (r is the workgroup's row: uniform.) Both loads are issued before either
// value is used (the empty asm takes them as scalar operands), so they
// cost one memory round trip; the arithmetic is branch-free 32-bit.
__device__ __forceinline__ int visible_count_of(const IdxArgs& a, int p, int ne) {
  unsigned nv = p < 0 ? 0u : ((unsigned)p + 1u) / (unsigned)a.m;  // p + 1 <= 2^31 fits
  nv = min(nv, ne < 0 ? 0u : (unsigned)ne);
  nv = min(nv, (unsigned)a.Nmax);
  return (int)nv;
}
__device__ __forceinline__ int visible_count(const IdxArgs& a, int r) {
  const unsigned b = (unsigned)r / (unsigned)a.T;
  const int p = a.q_pos[r];
  const int ne = a.n_entries[b];
  asm volatile("" ::"s"(p), "s"(ne));
  return visible_count_of(a, p, ne);
}

// order-preserving key: larger score -> larger key; -0 is folded onto +0
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

__device__ __forceinline__ void swap32(float& x, float& y) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  x = __uint_as_float(r[0]);
  y = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap16(float& x, float& y) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  x = __uint_as_float(r[0]);
  y = __uint_as_float(r[1]);
}

// Group maxima of the scores held by a wave (one per lane, key = base+lane),
// written for groups of 2^gs_log2 keys (gs <= 64): maxima within aligned
// lane groups of 2, 4 (quad permutes), 8 (half-row mirror), 16 (row
// mirror), then across rows (permlane swaps), all VALU steps.
__device__ __forceinline__ float group_max(const IdxArgs& a, float v) {
  const int g = a.gs_log2;
  float mx = v;
  if (g >= 1) mx = fmaxf(mx, CSK_DPP_F(mx, 0xB1));   // quad_perm [1,0,3,2]
  if (g >= 2) mx = fmaxf(mx, CSK_DPP_F(mx, 0x4E));   // quad_perm [2,3,0,1]
  if (g >= 3) mx = fmaxf(mx, CSK_DPP_F(mx, 0x141));  // row_half_mirror
  if (g >= 4) mx = fmaxf(mx, CSK_DPP_F(mx, 0x140));  // row_mirror
  if (g >= 5) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mx = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  }
  if (g >= 6) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mx = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  }
  return mx;
}
__device__ __forceinline__ void store_sample(const IdxArgs& a, int r, int base, float mx) {
  const int lane = threadIdx.x & 63;
  const int key = base + lane;
  if ((lane & ((1 << a.gs_log2) - 1)) == 0 && key < a.Nmax)
    a.samples[(int64_t)r * a.ng + (key >> a.gs_log2)] = mx;
}
__device__ __forceinline__ void write_samples(const IdxArgs& a, int r, int base, float v) {
  store_sample(a, r, base, group_max(a, v));
}

// ---------------------------------------------------------------- MFMA path
// HT = HI/16 head tiles, KS = dI/128 MFMA K-steps. One workgroup = 4 waves
// and one query row. Wave w handles the 64-key groups
// base = blockIdx.y*256*ITERS + 256*it + 64*w, it < ITERS, so the four waves
// of a workgroup stream 256 consecutive keys per iteration. Key fragments
// rotate through three register buffers: the two groups after the current
// one are in flight while its MFMAs, transpose and head chain run. ITERS is
// chosen on the host so that short grids (decode: a few rows over a long
// cache) come out at about two resident workgroups per CU.
typedef unsigned v4u __attribute__((ext_vector_type(4)));

template <int HT, int KS, int ITERS>
__global__ __launch_bounds__(256) void idx_fp4_kernel(IdxArgs a) {
  const int r = blockIdx.x;
  const int b = __builtin_amdgcn_readfirstlane(r / a.T);  // (uniform: scalar address bases)
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wg_base = blockIdx.y * (256 * ITERS) + wave * 64;
  const int nv = visible_count(a, r);
  if (wg_base >= nv) return;
  const int HI = HT * 16;
  const int rho = lane & 15, kb = lane >> 4;

  // A operands: q rows permuted so lane group g ends up with heads 4*HT*g..
  v8i qa[HT][KS];
  int qsc[HT][KS];
#pragma unroll
  for (int t = 0; t < HT; ++t) {
    const int h = 4 * HT * (rho >> 2) + 4 * t + (rho & 3);
    const int64_t qrow = (int64_t)r * HI + h;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint4 v = *reinterpret_cast<const uint4*>(a.qc + qrow * (a.dI / 2) + s * 64 + kb * 16);
      qa[t][s] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      qsc[t][s] = a.qs[qrow * (a.dI / 32) + s * 4 + kb];
    }
  }
  // the row's head weights: one LDS copy per wave, then made wave-uniform
  // (readfirstlane) so that they sit in scalar registers for the whole
  // kernel and the head chain's fma reads them directly (a global load in
  // the loop would be counted with the in-flight key loads, and an LDS read
  // per four heads would stall the chain on its latency)
  __shared__ __align__(16) float wsh[4][64];
  if (lane < HI) wsh[wave][lane] = a.w[(int64_t)r * HI + lane];
  float wsc[4 * HT * 4];
#pragma unroll
  for (int i = 0; i < HT * 4; ++i) {
    const float4 w4 = *reinterpret_cast<const float4*>(&wsh[wave][4 * i]);
    wsc[4 * i] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(w4.x)));
    wsc[4 * i + 1] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(w4.y)));
    wsc[4 * i + 2] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(w4.z)));
    wsc[4 * i + 3] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(w4.w)));
  }

  // key fragments of one 64-key group: lane (rho, kb) holds bytes 16*kb..
  // of key 16*kt + rho in each of the four key tiles kt. The loads are
  // unconditional (keys past the cache are clamped to its last row and their
  // scores dropped), so no load sits under a branch.
  struct Group {
    v4u v[4][KS];
    int sc[4][KS];
  };
  // (the row's code and scale bases are uniform, and every key's bytes are
  // a 32-bit offset from them with compile-time strides (dI = 128*KS), so
  // each load takes a scalar base and one vector offset: no 64-bit address
  // or integer multiply per key)
  const uint8_t* kc_row = a.kc + (int64_t)b * a.Nmax * (64 * KS);
  // (a key's KS*4 scales are KS whole dwords: each lane loads the dword of
  // its K-step and takes byte kb, so a load instruction reads dwords, not
  // single bytes)
  const uint32_t* ks_row = reinterpret_cast<const uint32_t*>(a.ks + (int64_t)b * a.Nmax * (4 * KS));
  auto load_keys = [&](Group& gr, int base) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      int key = base + 16 * kt + rho;
      key = key < a.Nmax ? key : a.Nmax - 1;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const uint32_t off = (uint32_t)key * (uint32_t)(64 * KS) + (uint32_t)(s * 64 + kb * 16);
        gr.v[kt][s] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(kc_row + off));
        const uint32_t so = (uint32_t)key * (uint32_t)(4 * KS) + (uint32_t)(4 * s);
        gr.sc[kt][s] = (int)((*reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(ks_row) + so) >>
                              (8 * kb)) & 0xffu);
      }
    }
  };

  float* const score_row = a.scores + (int64_t)r * a.Nmax;
  auto process = [&](const Group& gr, int base) {
    v4f acc[4][HT];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int t = 0; t < HT; ++t) acc[kt][t] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const v8i kbv = v8i{(int)gr.v[kt][s].x, (int)gr.v[kt][s].y, (int)gr.v[kt][s].z,
                            (int)gr.v[kt][s].w, 0, 0, 0, 0};
#pragma unroll
        for (int t = 0; t < HT; ++t)
          acc[kt][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              qa[t][s], kbv, acc[kt][t], 4, 4, 0, qsc[t][s], 0, gr.sc[kt][s]);
      }
    }

    // transpose (key tile, lane group): lane group G of register set g then
    // holds heads 4*HT*g + 4t + j of key 16*G + (lane % 16)
    float d[4][HT][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int t = 0; t < HT; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) d[kt][t][j] = acc[kt][t][j];
#pragma unroll
    for (int t = 0; t < HT; ++t) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        swap32(d[0][t][j], d[2][t][j]);
        swap32(d[1][t][j], d[3][t][j]);
        swap16(d[0][t][j], d[1][t][j]);
        swap16(d[2][t][j], d[3][t][j]);
      }
    }

    // ascending head chain, weights from scalar registers. ReLU as an
    // integer max on the bits: +0 for every negative value and for -0, the
    // value itself otherwise (a float max would also canonicalise each
    // value coming out of the lane swaps)
    float score = 0.0f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
      for (int t = 0; t < HT; ++t) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float v = __int_as_float(max(__float_as_int(d[g][t][j]), 0));
          score = __builtin_fmaf(wsc[4 * HT * g + 4 * t + j], v, score);
        }
      }
    }

    score = topk_score(a, score);
    const int key = base + lane;
    if (key < nv) *reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(score_row) + (uint32_t)key * 4u) = score;
    if (a.samples) write_samples(a, r, base, key < nv ? score : -INFINITY);
  };

  // fully unrolled: group it is computed while groups it+1 and it+2 are in
  // flight; all counts are compile-time, so every wait the compiler inserts
  // is exact
  Group buf[3];
#pragma unroll
  for (int j = 0; j < 3 && j < ITERS; ++j) load_keys(buf[j], wg_base + 256 * j);
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int base = wg_base + 256 * it;
    if (base >= nv) break;
    process(buf[it % 3], base);
    if (it + 3 < ITERS) load_keys(buf[it % 3], base + 3 * 256);
  }
}

// ------------------------------------------------------ MFMA path, 32 heads
// The same scores for HI a multiple of 32, on the 32x32 scaled FP4 MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4): operand lane l holds row l%32 and the
// 32 elements of K block l/32 of the 64-wide K-step (16 bytes), with that
// block's scale byte; result lane l holds column l%32 (the key) and rows
// 8i + 4*(l/32) + j in element 4i+j. A wave's 64 keys are two key tiles, so
// one v_permlane32_swap per register pair (half the exchanges of the 16x16
// form) leaves lane l with every head of key base + l, and half as many
// MFMA instructions cover the same products. With the four tile exponents
// of a pair within the fp32 significand every partial sum is exact, so
// splitting K into 64-wide steps gives the same bits as one 128-wide step.
//
// Keys reach LDS by DMA: each wave streams its 64-key groups through NB
// stages, so that NB groups are in flight and no key occupies a register
// before its products. The waits are explicit: the stage's DMA count, then
// the fragment reads in one asm block that waits for them itself (the
// compiler's own tracking would wait for every DMA in flight). The queries
// come by DMA as well, and the scores and group maxima stay in registers
// until the end, so no plain load or store is counted between a stage's DMA
// and its wait. Used for prefill rows, where the head chain's VALU work
// bounds the indexer.
// HT2 = HI/32 head tiles, KB = dI/32 16-byte chunks (and scale bytes) per key.
typedef __attribute__((address_space(3))) uint32_t lds_u32;

__device__ __forceinline__ void idx_dma16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds(src, lds_base, 16, 0, 0);
}
__device__ __forceinline__ void idx_dma4(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds(src, lds_base, 4, 0, 0);
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((const lds_u32*)(const uint32_t*)p);
}
// Four 16-byte and two 4-byte LDS reads (byte addresses), waited for inside
// the same asm block, so no output register is live while a read is in
// flight.
__device__ __forceinline__ void lds_read_4x16_2x4(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3,
                                                   uint32_t b0, uint32_t b1, v4u& f0, v4u& f1, v4u& f2,
                                                   v4u& f3, uint32_t& w0, uint32_t& w1) {
  asm volatile(
      "ds_read_b128 %0, %6\n\t"
      "ds_read_b128 %1, %7\n\t"
      "ds_read_b128 %2, %8\n\t"
      "ds_read_b128 %3, %9\n\t"
      "ds_read_b32 %4, %10\n\t"
      "ds_read_b32 %5, %11\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(f0), "=&v"(f1), "=&v"(f2), "=&v"(f3), "=&v"(w0), "=&v"(w1)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "v"(b0), "v"(b1)
      : "memory");
}
// Two 16-byte and one 4-byte LDS reads, waited for inside the asm block.
__device__ __forceinline__ void lds_read_2x16_1x4(uint32_t a0, uint32_t a1, uint32_t b0, v4u& f0, v4u& f1,
                                                   uint32_t& w0) {
  asm volatile(
      "ds_read_b128 %0, %3\n\t"
      "ds_read_b128 %1, %4\n\t"
      "ds_read_b32 %2, %5\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(f0), "=&v"(f1), "=&v"(w0)
      : "v"(a0), "v"(a1), "v"(b0)
      : "memory");
}
// s_waitcnt immediate: vmcnt(n) only
#define CSK_IDX_VMCNT(n) ((((n) & 0xF) | ((((n) >> 4) & 0x3) << 14)) | (0x7 << 4) | (0xF << 8))

template <int KB>
struct IdxStage {
  uint4 code[4][64 * KB];              // [wave][unit]: 64 keys x KB chunks, swizzled
  uint32_t scale[4][(KB + 3) / 4][64]; // [wave][dword][key]
};

// (dI = 128: four waves per SIMD, 39 KB of LDS per workgroup with two stages)
template <int HT2, int KB, int ITERS, int NB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(KB == 4 ? 4 : 2, KB == 4 ? 4 : 2)))
void idx_fp4_w32_kernel(IdxArgs a) {
  static_assert(NB >= 2 && NB <= 4, "two to four stages");
  static_assert(KB == 4 || KB == 8, "dI of 128 or 256");
  constexpr int KS2 = KB / 2;       // 64-deep K-steps
  constexpr int SD = (KB + 3) / 4;  // scale dwords per key
  constexpr int HI = HT2 * 32;
  constexpr int SWS = KB == 4 ? 2 : 1;  // chunk swizzle: unit KB*k + (c ^ ((k >> SWS) % KB))
  constexpr int PER = KB + SD;          // DMA instructions per group
  __shared__ IdxStage<KB> st0, st1, st2, st3;
  const int r = blockIdx.x;
  const int b = r / a.T;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // (uniform: scalar branches)
  const int wg_base = blockIdx.y * (256 * ITERS) + wave * 64;
  const int rho = lane & 31, hb = lane >> 5;
  auto stage = [&](int j) -> IdxStage<KB>& {
    return (j % NB) == 0 ? st0 : ((j % NB) == 1 ? st1 : ((j % NB) == 2 ? st2 : st3));
  };

  // scalar loads first, before any DMA (once a DMA precedes them in the
  // program they can no longer be proven unclobbered and become vector
  // loads, whose wait would cover every DMA issued ahead of them): the
  // row's position and cache length, and its head weights (scalar
  // registers for the whole kernel: the head chain's fma takes them as
  // scalar operands)
  const int q_pos = a.q_pos[r];
  const int n_ent = a.n_entries[b];
  const float* w_row = a.w + (int64_t)r * HI;
  float wsc[HI];
#pragma unroll
  for (int i = 0; i < HI; ++i) wsc[i] = w_row[i];

  // DMA of group j (keys base..base+63, clamped to the cache): instruction
  // i, lane l fills unit 64i + l = KB*k + p with chunk p ^ swizzle(k) of key
  // k; the scale dwords go one instruction per dword
  const uint8_t* kc_b = a.kc + (int64_t)b * a.Nmax * (KB * 16);
  const uint8_t* ks_b = a.ks + (int64_t)b * a.Nmax * KB;
  auto issue = [&](int j) {
    IdxStage<KB>& S = stage(j);
    const int base = wg_base + 256 * j;
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      const int u = 64 * i + lane, k = u / KB, pp = u % KB;
      const int c = pp ^ ((k >> SWS) % KB);
      const int key = min(base + k, a.Nmax - 1);
      idx_dma16(kc_b + (uint32_t)key * (uint32_t)(KB * 16) + 16 * c, &S.code[wave][64 * i]);
    }
    const int key = min(base + lane, a.Nmax - 1);
#pragma unroll
    for (int d = 0; d < SD; ++d)
      idx_dma4(ks_b + (uint32_t)key * (uint32_t)KB + 4 * d, &S.scale[wave][d][0]);
  };

  // The row's queries reach LDS by DMA as well (a plain vector load pending
  // beside DMA makes every compiler wait a full drain), one copy per
  // workgroup in the keys' swizzled chunk layout; the waves split the
  // instructions, wait for their own, and meet at one barrier before any
  // wave may leave.
  __shared__ __align__(16) uint4 qlds[HI * KB];
  __shared__ uint32_t qsl[HI * SD < 64 ? 64 : HI * SD];
  constexpr int QI = HI * KB / 64;         // 16-byte DMA instructions
  constexpr int QSI = (HI * SD + 63) / 64; // scale-dword DMA instructions (wave 0)
  {
    const uint8_t* q_row = a.qc + (int64_t)r * HI * (KB * 16);
#pragma unroll
    for (int i = 0; i < QI; ++i) {
      if (i % 4 != wave) continue;
      const int u = 64 * i + lane, h = u / KB, pp = u % KB;
      const int c = pp ^ ((h >> SWS) % KB);
      idx_dma16(q_row + h * (KB * 16) + 16 * c, &qlds[64 * i]);
    }
    if (wave == 0) {
      const uint8_t* qs_row = a.qs + (int64_t)r * HI * KB;
#pragma unroll
      for (int i = 0; i < QSI; ++i) {
        const int dw = min(64 * i + lane, HI * SD - 1);
        idx_dma4(qs_row + 4 * dw, &qsl[64 * i]);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(CSK_IDX_VMCNT(0));
  // (a bare barrier: the wait above already covers the query DMA)
  __builtin_amdgcn_s_barrier();
  // A operands: head 32t + rho in row rho of head tile t (no permutation:
  // after the swap, register x, tile t, element 4i+j holds head
  // 32t + 8i + 4x + j, so the chain below visits heads in ascending order)
  v8i qa[HT2][KS2];
  int qsc[HT2][KS2];
#pragma unroll
  for (int t = 0; t < HT2; ++t) {
    const int h = 32 * t + rho;
#pragma unroll
    for (int s = 0; s < KS2; s += 2) {
      const int c0 = 2 * s + hb, c1 = 2 * (s + 1) + hb;
      v4u f0, f1;
      uint32_t dw;
      lds_read_2x16_1x4(lds_addr(&qlds[KB * h + (c0 ^ ((h >> SWS) % KB))]),
                        lds_addr(&qlds[KB * h + (c1 ^ ((h >> SWS) % KB))]), lds_addr(&qsl[h * SD + (c0 >> 2)]),
                        f0, f1, dw);
      qa[t][s] = v8i{(int)f0.x, (int)f0.y, (int)f0.z, (int)f0.w, 0, 0, 0, 0};
      qa[t][s + 1] = v8i{(int)f1.x, (int)f1.y, (int)f1.z, (int)f1.w, 0, 0, 0, 0};
      qsc[t][s] = (int)((dw >> (8 * (c0 & 3))) & 0xffu);
      qsc[t][s + 1] = (int)((dw >> (8 * (c1 & 3))) & 0xffu);
    }
  }

  const int nv = visible_count_of(a, q_pos, n_ent);
  if (wg_base >= nv) {
    __builtin_amdgcn_s_waitcnt(0);  // no DMA outlives the wave
    return;
  }
#pragma unroll
  for (int j = 0; j < NB && j < ITERS; ++j) issue(j);
  // (nothing that uses the queries moves above the DMA issue: its wait
  // would cover the DMA too)
  __builtin_amdgcn_sched_barrier(0);

  float score[ITERS], gmax[ITERS];
  int done = ITERS;
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int base = wg_base + 256 * it;
    if (base >= nv) {
      done = it;
      break;
    }
    // this stage's DMA done: the groups after it stay in flight
    {
      const int ahead = NB - 1 < ITERS - 1 - it ? NB - 1 : ITERS - 1 - it;  // groups issued after it
      if (ahead >= 3) __builtin_amdgcn_s_waitcnt(CSK_IDX_VMCNT(3 * PER));
      else if (ahead == 2) __builtin_amdgcn_s_waitcnt(CSK_IDX_VMCNT(2 * PER));
      else if (ahead == 1) __builtin_amdgcn_s_waitcnt(CSK_IDX_VMCNT(PER));
      else __builtin_amdgcn_s_waitcnt(CSK_IDX_VMCNT(0));
    }
    IdxStage<KB>& S = stage(it);
    // fragments: key tile kt, K-step s -> chunk c = 2s + hb of key 32kt + rho
    v4u fr[2][KS2];
    uint32_t scw[2][SD];
    {
      auto code_at = [&](int kt, int s) {
        const int k = 32 * kt + rho, c = 2 * s + hb;
        return lds_addr(&S.code[wave][KB * k + (c ^ ((k >> SWS) % KB))]);
      };
      if constexpr (KB == 4) {
        lds_read_4x16_2x4(code_at(0, 0), code_at(0, 1), code_at(1, 0), code_at(1, 1),
                          lds_addr(&S.scale[wave][0][rho]), lds_addr(&S.scale[wave][0][32 + rho]),
                          fr[0][0], fr[0][1], fr[1][0], fr[1][1], scw[0][0], scw[1][0]);
      } else {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
          lds_read_4x16_2x4(code_at(kt, 0), code_at(kt, 1), code_at(kt, 2), code_at(kt, 3),
                            lds_addr(&S.scale[wave][0][32 * kt + rho]),
                            lds_addr(&S.scale[wave][SD - 1][32 * kt + rho]),
                            fr[kt][0], fr[kt][1], fr[kt][2], fr[kt][3], scw[kt][0], scw[kt][SD - 1]);
      }
    }
    // the stage is free again (the reads above have completed): refill it
    if (it + NB < ITERS) issue(it + NB);

    v16f acc[2][HT2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int t = 0; t < HT2; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[kt][t][e] = 0.f;
#pragma unroll
      for (int s = 0; s < KS2; ++s) {
        const int c = 2 * s + hb;
        const v8i kbv = v8i{(int)fr[kt][s].x, (int)fr[kt][s].y, (int)fr[kt][s].z, (int)fr[kt][s].w, 0, 0, 0, 0};
        const int ksc = (int)((scw[kt][s >> 1] >> (8 * (c & 3))) & 0xffu);
#pragma unroll
        for (int t = 0; t < HT2; ++t)
          acc[kt][t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              qa[t][s], kbv, acc[kt][t], 4, 4, 0, qsc[t][s], 0, ksc);
      }
    }

    // one exchange per register pair: lanes 32-63 of key tile 0 with lanes
    // 0-31 of key tile 1. Register x then holds the rows 8i + 4x + j of key
    // base + lane.
    float d[2][HT2][16];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int t = 0; t < HT2; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) d[kt][t][e] = acc[kt][t][e];
#pragma unroll
    for (int t = 0; t < HT2; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) swap32(d[0][t][e], d[1][t][e]);

    // ascending head chain (ReLU as an integer max on the bits)
    float sum = 0.0f;
#pragma unroll
    for (int t = 0; t < HT2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float v = __int_as_float(max(__float_as_int(d[x][t][4 * i + j]), 0));
            sum = __builtin_fmaf(wsc[32 * t + 8 * i + 4 * x + j], v, sum);
          }
    score[it] = topk_score(a, sum);
    if (a.samples) gmax[it] = group_max(a, base + lane < nv ? score[it] : -INFINITY);
  }
  // a wave that left early (groups past the visible count) may still have
  // key DMA in flight: none outlives the wave
  if (done < ITERS) __builtin_amdgcn_s_waitcnt(CSK_IDX_VMCNT(0));

#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    if (it >= done) break;
    const int base = wg_base + 256 * it;
    if (base + lane < nv) a.scores[(int64_t)r * a.Nmax + base + lane] = score[it];
    if (a.samples) store_sample(a, r, base, gmax[it]);
  }
}

// -------------------------------------------------------------- VALU path
// One thread per (row, key). fp32: per-head dot is an fma chain over the
// channels. MXFP4: per-tile integer dot products combined in fp64 (exact for
// any tile exponents within 2^38 of each other) and rounded once to fp32.
__device__ __forceinline__ float e2m1_twice(uint32_t c) {
  const float tbl[8] = {0.f, 1.f, 2.f, 3.f, 4.f, 6.f, 8.f, 12.f};
  float v = tbl[c & 7u];
  return (c & 8u) ? -v : v;
}

template <bool MX>
__global__ __launch_bounds__(256) void idx_valu_kernel(IdxArgs a) {
  const int r = blockIdx.x;
  const int b = r / a.T;
  const int s = blockIdx.y * 256 + threadIdx.x;
  const int nv = visible_count(a, r);
  if (s >= nv) return;
  const int64_t krow = (int64_t)b * a.Nmax + s;
  float score = 0.0f;
  for (int h = 0; h < a.HI; ++h) {
    const int64_t qrow = (int64_t)r * a.HI + h;
    float d;
    if (!MX) {
      d = 0.0f;
      const float* q = a.qf + qrow * a.dI;
      const float* k = a.kf + krow * a.dI;
      for (int i = 0; i < a.dI; ++i) d = __builtin_fmaf(q[i], k[i], d);
    } else {
      double tot = 0.0;
      for (int g = 0; g < a.dI / 32; ++g) {
        float pg = 0.0f;  // integer-valued, |pg| <= 4608: exact in fp32
        for (int i = 0; i < 16; ++i) {
          const uint32_t qb = a.qc[qrow * (a.dI / 2) + g * 16 + i];
          const uint32_t kbyte = a.kc[krow * (a.dI / 2) + g * 16 + i];
          pg += e2m1_twice(qb & 15u) * e2m1_twice(kbyte & 15u);
          pg += e2m1_twice(qb >> 4) * e2m1_twice(kbyte >> 4);
        }
        const int e = (int)a.qs[qrow * (a.dI / 32) + g] + (int)a.ks[krow * (a.dI / 32) + g] - 256;
        tot += ldexp((double)pg, e);
      }
      d = (float)tot;
    }
    score = __builtin_fmaf(a.w[qrow], d > 0.0f ? d : 0.0f, score);
  }
  a.scores[(int64_t)r * a.Nmax + s] = topk_score(a, score);
}

// Group maxima for the VALU path (the MFMA path writes them itself).
__global__ __launch_bounds__(256) void idx_samples_kernel(IdxArgs a) {
  const int r = blockIdx.x;
  const int g = blockIdx.y * 256 + threadIdx.x;
  if (g >= a.ng) return;
  const int nv = visible_count(a, r);
  const int gs = 1 << a.gs_log2;
  float mx = -INFINITY;
  for (int i = 0; i < gs; ++i) {
    const int s = g * gs + i;
    if (s < nv) mx = fmaxf(mx, a.scores[(int64_t)r * a.Nmax + s]);
  }
  a.samples[(int64_t)r * a.ng + g] = mx;
}

// ------------------------------------------------------------ block scans
// Exclusive prefix sums of two ints over a workgroup of NT threads (NT/64
// waves <= 16): wave scans, then every wave scans the wave totals itself
// (one barrier between, one before the totals can be reused).
struct ScanShared {
  int2 wtot[16];
};

template <int NT>
__device__ __forceinline__ int2 block_scan2(int a, int b, ScanShared& sh, int2* total) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int x = wave_incl_sum(a), y = wave_incl_sum(b);
  if (lane == 63) sh.wtot[wave] = make_int2(x, y);
  __syncthreads();
  const int2 w = lane < NT / 64 ? sh.wtot[lane] : make_int2(0, 0);
  const int wx = wave_incl_sum(w.x), wy = wave_incl_sum(w.y);
  const int offx = __builtin_amdgcn_readlane(wx - w.x, wave);
  const int offy = __builtin_amdgcn_readlane(wy - w.y, wave);
  *total = make_int2(__builtin_amdgcn_readlane(wx, NT / 64 - 1), __builtin_amdgcn_readlane(wy, NT / 64 - 1));
  __syncthreads();  // the wave totals may be reused by the next scan
  return make_int2(offx + x - a, offy + y - b);
}

// ------------------------------------------------------------ range select
// Block-wide (NT threads) selection of the k largest of n keys get(e), as a
// SelectState: every element whose masked key is > prefix, plus the first
// `take` elements (in element order) whose masked key == prefix. The keys
// in [kmin, kmax] are binned linearly over the range (bin = (key - lo) >>
// sb, at most SEL_BINS bins); the bin that holds the k-th largest key is
// found and becomes the next, narrower range. With 32-bit keys three levels
// reach single key values (sb <= 20, then <= 8, then 0); a level ends early
// when the whole bin is taken. Binning over the keys' own range keeps the
// LDS atomics spread even when the keys share their leading bits (near a
// top-k threshold they do).
constexpr int SEL_BINS = 4096;

struct SelectState {
  uint32_t mask, prefix;
  int take;
};

constexpr int SEL_SMALL = 64;  // a bin this small is finished by one wave's rank count

template <int BINS>
struct SelectSharedT {
  int hist[BINS];
  int digit, above, binc, nsmall, take;
  uint32_t thr;
  uint32_t kmin[16], kmax[16];
  uint32_t small[SEL_SMALL];
  ScanShared scan;
};
using SelectShared = SelectSharedT<SEL_BINS>;

// Index-ordered compaction of the selected elements. Each thread owns a
// contiguous run of elements; counts of strictly-greater and tied elements
// are scanned across the block.
template <int NT, typename Get, typename Emit, typename SS>
__device__ void compact_selected(Get get, Emit emit, int n, const SelectState& st, SS& sh) {
  const int tid = threadIdx.x;
  const int per = (n + NT - 1) / NT;
  const int e0 = tid * per;
  const int e1 = min(n, e0 + per);
  int gt = 0, eq = 0;
  for (int e = e0; e < e1; ++e) {
    const uint32_t u = get(e) & st.mask;
    gt += u > st.prefix;
    eq += u == st.prefix;
  }
  int2 tot;
  const int2 before = block_scan2<NT>(gt, eq, sh.scan, &tot);
  int gt_before = before.x, eq_before = before.y;
  for (int e = e0; e < e1; ++e) {
    const uint32_t u = get(e) & st.mask;
    if (u > st.prefix) {
      emit(gt_before + min(eq_before, st.take), e);
      ++gt_before;
    } else if (u == st.prefix) {
      if (eq_before < st.take) emit(gt_before + eq_before, e);
      ++eq_before;
    }
  }
}

struct TopkArgs {
  IdxArgs ia;
  int k;
  int n_slices;
  int* cand_cnt;            // [R, n_slices]
  float* cand_score;        // [R, Nmax]: slice f at [f*SLICE, f*SLICE+cnt)
  int* cand_idx;            // [R, Nmax]
  uint32_t* flat_key;       // [R, Nmax] spill when a row exceeds TOPK_CAP
  int* flat_idx;            // [R, Nmax]
  int32_t* idx;             // [R, k]
  float* out_score;         // [R, k] or null
};

struct TopkShared {
  SelectShared sel;
  uint32_t key[TOPK_CAP];
  int eidx[TOPK_CAP];
  int slice_off[1024 + 1];
};
// Unfiltered rows (at most TOPK_CAP entries, element index = key index):
// keys only, and 2048 histogram bins, so that two workgroups fit a CU.
struct TopkSharedU {
  SelectSharedT<2048> sel;
  uint32_t key[TOPK_CAP];
};

// Threshold from the group maxima: the samples' order-preserving keys are
// binned linearly over their own range [kmin, kmax] (bin = (key - kmin) >>
// sb, at most 4096 bins), the bin d holding the k-th largest sample is
// found, and the threshold is its lower edge kmin + (d << sb), so at least k
// samples (hence at least k elements of the row) are >= it. (Binning by the
// leading key bits would put nearly all maxima, which share sign and
// exponent, into a handful of bins, and the histogram's LDS atomics would
// then serialise.) 0 keeps everything when the row has at most k entries or
// too few samples. Every workgroup of the row forms it (the samples are a
// few KB, read from L2), which saves a launch.
constexpr int THR_BINS = 4096;
constexpr int THR_BATCH = 16;       // samples per thread per load batch
constexpr int FUSED_THREADS = 256;

struct FusedShared {
  int hist[THR_BINS];
  ScanShared scan;
  uint32_t thr;
  uint32_t kmin[FUSED_THREADS / 64], kmax[FUSED_THREADS / 64];
};

// Wave-wide minimum / maximum of an unsigned value (DPP within rows, then
// the row swaps).
template <bool MAX>
__device__ __forceinline__ uint32_t wave_ext_u32(uint32_t x) {
  auto op = [](uint32_t u, uint32_t v) { return MAX ? (u > v ? u : v) : (u < v ? u : v); };
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xf, 0xf, false));   // quad_perm [1,0,3,2]
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xf, 0xf, false));   // quad_perm [2,3,0,1]
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x124, 0xf, 0xf, false));  // row_ror:4
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x128, 0xf, 0xf, false));  // row_ror:8
  const auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  x = op(p[0], p[1]);
  const auto q = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return op(q[0], q[1]);
}

// Suffix search over PER * FUSED_THREADS bins: the bin d holding the
// element of rank `want` (1-based, from the top) and the count of elements
// in bins above it. Exactly one thread returns true (none when fewer than
// `want` elements exist).
template <int NT, int PER>
__device__ bool find_rank_bin(const int* hist, int want, ScanShared& scan, int* out_d, int* out_above) {
  const int tid = threadIdx.x;
  const int G = NT - 1 - tid;  // thread t owns bins PER*G .. PER*G+PER-1
  int sg = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) sg += hist[PER * G + i];
  int2 tot;
  const int ex = block_scan2<NT>(sg, 0, scan, &tot).x;  // bins above this group
  if (ex < want && ex + sg >= want) {
    int above = ex;
    int d = PER * G + PER - 1;
    for (; d > PER * G; --d) {
      if (above + hist[d] >= want) break;
      above += hist[d];
    }
    *out_d = d;
    *out_above = above;
    return true;
  }
  return false;
}

// (cleared: the caller has zeroed sh.hist and sh.nsmall, and passed a
// barrier since, so level 0 skips its own clear.)
template <int NT, int BINS, typename Get>
__device__ SelectState range_select(Get get, int n, int k, uint32_t kmin, uint32_t kmax, SelectSharedT<BINS>& sh,
                                    bool cleared) {
  static_assert(BINS == 2048 || BINS == 4096, "three levels reach single key values");
  constexpr int LB = BINS == 4096 ? 12 : 11;  // bits per level
  const int tid = threadIdx.x;
  uint32_t lo = kmin, span = kmax - kmin;  // the current range [lo, lo + span]
  int want = k;                            // rank of the target inside it
  for (int level = 0; level < 3; ++level) {
    const int sb = span < (uint32_t)BINS ? 0 : (32 - LB) - __clz(span);  // span >> sb < BINS
    if (level > 0 || !cleared) {
      for (int i = tid; i < BINS; i += NT) sh.hist[i] = 0;
      if (tid == 0) sh.nsmall = 0;
      __syncthreads();
    }
    for (int e = tid; e < n; e += NT) {
      const uint32_t u = get(e) - lo;  // wraps for keys below the range
      if (u <= span) atomicAdd(&sh.hist[u >> sb], 1);
    }
    __syncthreads();
    int d = 0, above = 0;
    if (find_rank_bin<NT, BINS / NT>(sh.hist, want, sh.scan, &d, &above)) {
      sh.digit = d;
      sh.above = above;
      sh.binc = sh.hist[d];
    }
    __syncthreads();
    d = sh.digit;
    want -= sh.above;
    const int binc = sh.binc;
    const uint32_t edge = lo + ((uint32_t)d << sb);
    __syncthreads();  // the shared results and bins are reused
    if (sb == 0) return SelectState{0xffffffffu, edge, want};  // one key value: ties by element order
    if (binc == want && edge > 0u) return SelectState{0xffffffffu, edge - 1u, 0};  // every key >= edge
    if (binc <= SEL_SMALL) {
      // the few keys of the bin: wave 0 ranks them (lane j counts the keys
      // above and equal to its own) and publishes the want-th largest
      // (nsmall was zeroed with this level's histogram)
      for (int e = tid; e < n; e += NT) {
        const uint32_t u = get(e);
        if (u - edge < (1u << sb)) sh.small[atomicAdd(&sh.nsmall, 1)] = u;
      }
      __syncthreads();
      if (tid < 64) {
        const uint32_t kj = tid < binc ? sh.small[tid] : 0u;
        int gt = 0, eq = 0;
        for (int i = 0; i < binc; ++i) {
          const uint32_t ki = (uint32_t)__builtin_amdgcn_readlane((int)kj, i);
          gt += ki > kj;
          eq += ki == kj;
        }
        if (tid < binc && gt < want && want <= gt + eq) {  // every lane holding the target agrees
          sh.thr = kj;
          sh.take = want - gt;
        }
      }
      __syncthreads();
      // (thr and take are not written again: no barrier after the reads)
      return SelectState{0xffffffffu, sh.thr, sh.take};
    }
    lo = edge;
    span = (1u << sb) - 1u;
  }
  return SelectState{0xffffffffu, lo, want};  // not reached: the third level has sb == 0
}

// Candidate filter for long rows: workgroup (r, f) forms the row's
// threshold and writes the candidates of slice f (keys >= threshold, in
// index order) and their count. (A last-arriving-workgroup select in the
// same kernel was measured slower: each workgroup's device-scope release
// writes back its L2, while a kernel boundary does that once.)
__global__ __launch_bounds__(FUSED_THREADS) void topk_filter_kernel(TopkArgs a) {
  __shared__ FusedShared sh;
  const int r = blockIdx.x, f = blockIdx.y;
  const int tid = threadIdx.x;
  const int s0 = f * SLICE;
  const int k = a.k;

  // The slice's scores and (when they fit one batch) the row's samples are
  // loaded before the row's visible count is known, their addresses clamped
  // to the allocated row, so that the count and all of them arrive in one
  // memory round trip; the count then decides which of them are valid. (A
  // barrier waits for every load in flight, so each barrier comes after
  // loads that are needed anyway.)
  const float* sc = a.ia.scores + (int64_t)r * a.ia.Nmax + s0;
  const int slim = min(SLICE, a.ia.Nmax - s0);
  const int j0 = tid * (SLICE / FUSED_THREADS);
  float v[SLICE / FUSED_THREADS];
#pragma unroll
  for (int i = 0; i < SLICE / FUSED_THREADS; ++i) v[i] = sc[min(j0 + i, slim - 1)];  // unconditional
  const float* smp = a.ia.samples + (int64_t)r * a.ia.ng;
  const bool one_batch = a.ia.ng <= FUSED_THREADS * THR_BATCH;
  float sraw[THR_BATCH];  // raw values: converted only once the count is in
#pragma unroll
  for (int i = 0; i < THR_BATCH; ++i) sraw[i] = smp[min(FUSED_THREADS * i + tid, a.ia.ng - 1)];
  const int nv = visible_count(a.ia, r);

  // ---- filter
  if (s0 < nv) {
    const int gs = 1 << a.ia.gs_log2;
    const int ng = (nv + gs - 1) / gs;
    const bool thresholded = nv > k && ng >= k;
    if (thresholded) {
      for (int i = tid; i < THR_BINS; i += FUSED_THREADS) sh.hist[i] = 0;
      if (tid == 0) sh.thr = 0u;
      __syncthreads();
    }
    const int lim = min(SLICE, nv - s0);
    uint32_t thr = 0u;
    if (thresholded) {
      // the samples' key range (a single batch stays in registers for the
      // histogram; longer rows load theirs in batches, twice)
      uint32_t kx[THR_BATCH];
      uint32_t kmin = 0xffffffffu, kmax = 0u;
      if (one_batch) {
#pragma unroll
        for (int i = 0; i < THR_BATCH; ++i) {
          kx[i] = order_key(sraw[i]);
          const bool ok = FUSED_THREADS * i + tid < ng;
          kmin = min(kmin, ok ? kx[i] : 0xffffffffu);
          kmax = max(kmax, ok ? kx[i] : 0u);
        }
      } else {
        for (int e0 = 0; e0 < ng; e0 += FUSED_THREADS * THR_BATCH) {
#pragma unroll
          for (int i = 0; i < THR_BATCH; ++i) kx[i] = order_key(smp[min(e0 + FUSED_THREADS * i + tid, ng - 1)]);
#pragma unroll
          for (int i = 0; i < THR_BATCH; ++i) {
            kmin = min(kmin, kx[i]);
            kmax = max(kmax, kx[i]);
          }
        }
      }
      kmin = wave_ext_u32<false>(kmin);
      kmax = wave_ext_u32<true>(kmax);
      if ((tid & 63) == 0) {
        sh.kmin[tid >> 6] = kmin;
        sh.kmax[tid >> 6] = kmax;
      }
      __syncthreads();
#pragma unroll
      for (int w = 0; w < FUSED_THREADS / 64; ++w) {
        kmin = min(kmin, sh.kmin[w]);
        kmax = max(kmax, sh.kmax[w]);
      }
      const uint32_t span = kmax - kmin;
      const int sb = span < (uint32_t)THR_BINS ? 0 : 20 - __clz(span);  // span >> sb < 4096
      for (int e0 = 0; e0 < ng; e0 += FUSED_THREADS * THR_BATCH) {
        if (!one_batch) {
#pragma unroll
          for (int i = 0; i < THR_BATCH; ++i) kx[i] = order_key(smp[min(e0 + FUSED_THREADS * i + tid, ng - 1)]);
        }
#pragma unroll
        for (int i = 0; i < THR_BATCH; ++i)
          if (e0 + FUSED_THREADS * i + tid < ng) atomicAdd(&sh.hist[(kx[i] - kmin) >> sb], 1);
      }
      __syncthreads();
      int d = 0, above = 0;
      // the owner of the bin publishes its lower edge
      if (find_rank_bin<FUSED_THREADS, THR_BINS / FUSED_THREADS>(sh.hist, k, sh.scan, &d, &above))
        sh.thr = kmin + ((uint32_t)d << sb);
      __syncthreads();
      thr = sh.thr;
    }
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < SLICE / FUSED_THREADS; ++i) cnt += (j0 + i < lim && order_key(v[i]) >= thr) ? 1 : 0;
    int2 tot;
    int pos = block_scan2<FUSED_THREADS>(cnt, 0, sh.scan, &tot).x;
    float* cs = a.cand_score + (int64_t)r * a.ia.Nmax + s0;
    int* ci = a.cand_idx + (int64_t)r * a.ia.Nmax + s0;
#pragma unroll
    for (int i = 0; i < SLICE / FUSED_THREADS; ++i) {
      const int j = j0 + i;
      if (j < lim && order_key(v[i]) >= thr) {
        cs[pos] = v[i];
        ci[pos] = s0 + j;
        ++pos;
      }
    }
    if (tid == 0) a.cand_cnt[(int64_t)r * a.n_slices + f] = tot.x;
  } else if (tid == 0) {
    a.cand_cnt[(int64_t)r * a.n_slices + f] = 0;
  }

}

// Final selection for one row. FILTERED = false: the row's scores
// themselves (index = position); FILTERED = true: the slice candidates.
template <bool FILTERED>
__global__ __launch_bounds__(TOPK_THREADS) void topk_select_kernel(TopkArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  using SH = std::conditional_t<FILTERED, TopkShared, TopkSharedU>;
  constexpr int BINS = FILTERED ? SEL_BINS : 2048;
  SH& sh = *reinterpret_cast<SH*>(smem);
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int k = a.k;
  int32_t* oidx = a.idx + (int64_t)r * k;
  float* osc = a.out_score ? a.out_score + (int64_t)r * k : nullptr;

  // the first 64 candidates of each of a wave's first PRE slices, and the
  // slice counts, are loaded before the visible count is known (addresses
  // clamped to the allocated row); validity is decided once it is
  constexpr int NW = TOPK_THREADS / 64, PRE = 8;
  const int lane = tid & 63, wv = tid >> 6;
  const int64_t rbase = (int64_t)r * a.ia.Nmax;
  float psv[PRE];
  int piv[PRE];
  int craw = 0;
  if (FILTERED) {
#pragma unroll
    for (int u = 0; u < PRE; ++u) {
      const int fc = min(wv + u * NW, a.n_slices - 1);
      const int64_t off = rbase + min((int64_t)fc * SLICE + lane, (int64_t)a.ia.Nmax - 1);
      psv[u] = a.cand_score[off];
      piv[u] = a.cand_idx[off];
    }
    craw = a.cand_cnt[(int64_t)r * a.n_slices + min(tid, a.n_slices - 1)];
  }
  const int nv = visible_count(a.ia, r);
  int n;
  const int ns = (nv + SLICE - 1) / SLICE;
  if constexpr (!FILTERED) {
    n = nv;
  } else {
    // slice offsets: exclusive scan of the per-slice counts (ns <= 1024)
    const int cnt = tid < ns ? craw : 0;
    int2 tot;
    const int off = block_scan2<TOPK_THREADS>(cnt, 0, sh.sel.scan, &tot).x;
    if (tid < ns) sh.slice_off[tid] = off;
    if (tid == 0) sh.slice_off[ns] = tot.x;
    __syncthreads();
    n = tot.x;
  }
  const bool in_lds = n <= TOPK_CAP;
  uint32_t* gkey = a.flat_key + (int64_t)r * a.ia.Nmax;
  int* gidx = a.flat_idx + (int64_t)r * a.ia.Nmax;
  const float* srow = a.ia.scores + (int64_t)r * a.ia.Nmax;

  // gather elements (in index order) into LDS, or into the spill buffer,
  // with the range of their keys
  uint32_t umin = 0xffffffffu, umax = 0u;
  if constexpr (!FILTERED) {
    // (unfiltered rows have at most TOPK_CAP entries: always in LDS)
    for (int e = tid; e < n; e += TOPK_THREADS) {
      const uint32_t u = order_key(srow[e]);
      sh.key[e] = u;
      umin = min(umin, u);
      umax = max(umax, u);
    }
  } else {
    // each wave copies whole slices (wave w: slices w, w + NW, ...): the
    // preloaded first 64 candidates of its first PRE slices, then the rest
    auto put = [&](int e, float sv, int iv) {
      const uint32_t u = order_key(sv);
      umin = min(umin, u);
      umax = max(umax, u);
      if (in_lds) {
        sh.key[e] = u;
        sh.eidx[e] = iv;
      } else {
        gkey[e] = u;
        gidx[e] = iv;
      }
    };
#pragma unroll
    for (int u = 0; u < PRE; ++u) {
      const int f = wv + u * NW;
      if (f < ns) {
        const int dst = sh.slice_off[f], cnt = sh.slice_off[f + 1] - dst;
        if (lane < cnt) put(dst + lane, psv[u], piv[u]);
        const int64_t src = rbase + (int64_t)f * SLICE;
        for (int j = 64 + lane; j < cnt; j += 64) put(dst + j, a.cand_score[src + j], a.cand_idx[src + j]);
      }
    }
    for (int f = wv + PRE * NW; f < ns; f += NW) {
      const int dst = sh.slice_off[f], cnt = sh.slice_off[f + 1] - dst;
      const int64_t src = rbase + (int64_t)f * SLICE;
      for (int j = lane; j < cnt; j += 64) put(dst + j, a.cand_score[src + j], a.cand_idx[src + j]);
    }
  }
  umin = wave_ext_u32<false>(umin);
  umax = wave_ext_u32<true>(umax);
  if ((tid & 63) == 0) {
    sh.sel.kmin[tid >> 6] = umin;
    sh.sel.kmax[tid >> 6] = umax;
  }
  // the first level's histogram is cleared here, before the barrier the
  // key range needs anyway
  for (int i = tid; i < BINS; i += TOPK_THREADS) sh.sel.hist[i] = 0;
  if (tid == 0) sh.sel.nsmall = 0;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < TOPK_THREADS / 64; ++w) {
    umin = min(umin, sh.sel.kmin[w]);
    umax = max(umax, sh.sel.kmax[w]);
  }

  auto get = [&](int e) -> uint32_t {
    if (in_lds) return sh.key[e];
    if (!FILTERED) return order_key(srow[e]);
    return gkey[e];
  };
  auto index_of = [&](int e) -> int {
    if constexpr (!FILTERED) return e;
    else return in_lds ? sh.eidx[e] : gidx[e];
  };
  auto emit = [&](int pos, int e) {
    oidx[pos] = index_of(e);
    if (osc) osc[pos] = key_to_float(get(e));
  };

  int nsel;
  if (n <= k) {
    for (int e = tid; e < n; e += TOPK_THREADS) emit(e, e);
    nsel = n;
  } else {
    SelectState st = range_select<TOPK_THREADS>(get, n, k, umin, umax, sh.sel, true);
    compact_selected<TOPK_THREADS>(get, emit, n, st, sh.sel);
    nsel = k;
  }
  for (int j = nsel + tid; j < k; j += TOPK_THREADS) {
    oidx[j] = -1;
    if (osc) osc[j] = -INFINITY;
  }
}

// ------------------------------------------------------------ host layout
struct IdxPlan {
  bool filtered;
  int gs_log2, ng, n_slices;
  size_t off_scores, off_samples, off_cnt, off_cscore, off_cidx, off_fkey, off_fidx,
      total;
};

static size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

static IdxPlan plan_indexer(int B, int T, int Nmax, int k) {
  IdxPlan p{};
  const size_t R = (size_t)B * T;
  p.filtered = Nmax > TOPK_CAP;
  int gs = 1;
  if (p.filtered) {
    while (gs < 64 && (int64_t)Nmax / (2 * gs) >= 2 * (int64_t)k) gs *= 2;
  }
  p.gs_log2 = 0;
  while ((1 << p.gs_log2) < gs) ++p.gs_log2;
  p.ng = (int)ceil_div(Nmax, gs);
  p.n_slices = (int)ceil_div(Nmax, SLICE);
  size_t o = 0;
  p.off_scores = o; o = align_up(o + R * Nmax * 4);
  if (p.filtered) {
    p.off_samples = o; o = align_up(o + R * p.ng * 4);
    p.off_cnt = o; o = align_up(o + R * p.n_slices * 4);
    p.off_cscore = o; o = align_up(o + R * Nmax * 4);
    p.off_cidx = o; o = align_up(o + R * Nmax * 4);
    p.off_fkey = o; o = align_up(o + R * Nmax * 4);
    p.off_fidx = o; o = align_up(o + R * Nmax * 4);
  }
  p.total = o;
  return p;
}

// Scratch of indexer_topk_noalloc: one copy per device, in the code object's
// zero-initialised data (no allocation at call time). Host code never passes
// this name to a kernel: it stands for a host-side shadow, not the device
// address. The device address comes from hipGetSymbolAddress, once per
// device, and is kept in g_scratch_ptr.
static __device__ __align__(256) unsigned char scratch[CSK_NOALLOC_SCRATCH_BYTES];

constexpr int SCRATCH_DEVICES = 64;
static std::mutex g_scratch_mu;
static std::atomic<void*> g_scratch_ptr[SCRATCH_DEVICES];

// The calling thread's current device's scratch address (looked up on the
// first call on that device).
static int scratch_on_device(const char* fn, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(CSK_EUNSUPPORTED, std::string(fn) + ": no HIP device is visible");
  }
  if (dev >= SCRATCH_DEVICES)
    return fail(CSK_EUNSUPPORTED, std::string(fn) + ": device index " + std::to_string(dev) + " past 63");
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p) {
        (void)hipGetLastError();
        return fail(CSK_EHIP, std::string(fn) + ": hipGetSymbolAddress(scratch) failed: " + hipGetErrorString(e));
      }
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return CSK_OK;
}

static int indexer_topk_impl(const char* fn, bool noalloc, const void* q, const uint8_t* q_scale,
                             const float* w, const void* kk, const uint8_t* k_scale,
                             const int32_t* q_pos, const int32_t* n_entries, int B, int T, int HI,
                             int dI, int Nmax, int m, int k, int dtype, int score_dtype,
                             int32_t* idx, float* score, void* workspace, size_t ws_bytes,
                             void* stream) {
  clear_error();
  const std::string f(fn);
  if (!q || !w || !kk || !q_pos || !n_entries || !idx)
    return fail(CSK_EINVAL, f + ": null pointer");
  if (B <= 0 || T <= 0 || HI <= 0 || dI <= 0 || Nmax <= 0 || m <= 0 || k <= 0)
    return fail(CSK_EINVAL, f + ": sizes must be positive");
  if (dtype != CSK_MXFP4 && dtype != CSK_F32)
    return fail(CSK_EUNSUPPORTED, f + ": dtype must be CSK_MXFP4 or CSK_F32");
  if (dtype == CSK_MXFP4 && (dI % 32 || !q_scale || !k_scale))
    return fail(CSK_EINVAL, f + ": MXFP4 needs dI % 32 == 0 and both scale arrays");
  if (score_dtype != CSK_F32 && score_dtype != CSK_BF16)
    return fail(CSK_EUNSUPPORTED, f + ": score_dtype must be CSK_F32 or CSK_BF16");
  if (dtype == CSK_MXFP4 && ((reinterpret_cast<uintptr_t>(k_scale) | reinterpret_cast<uintptr_t>(q_scale)) & 3))
    return fail(CSK_EINVAL, f + ": k_scale and q_scale must be 4-byte aligned (read as dwords)");
  if ((int64_t)B * T > (1LL << 30) || ceil_div(Nmax, 256 * IDX_MIN_ITERS) > 65535)
    return fail(CSK_EUNSUPPORTED, f + ": B*T or Nmax too large");
  IdxPlan p = plan_indexer(B, T, Nmax, k);
  if (p.n_slices > 1024) return fail(CSK_EUNSUPPORTED, f + ": Nmax too large");
  if (noalloc) {
    if (p.total > (size_t)CSK_NOALLOC_SCRATCH_BYTES)
      return fail(CSK_EWORKSPACE, f + ": needs " + std::to_string(p.total) +
                                      " bytes of scratch; the static scratch holds " +
                                      std::to_string((size_t)CSK_NOALLOC_SCRATCH_BYTES));
  } else if (!workspace || ws_bytes < p.total) {
    return fail(CSK_EWORKSPACE, f + ": workspace smaller than indexer_topk_workspace_size()");
  }
  if (const int dc = check_device(f); dc != CSK_OK) return dc;
  if (noalloc) {
    if (const int sc = scratch_on_device(fn, &workspace); sc != CSK_OK) return sc;
  }
  char* ws = reinterpret_cast<char*>(workspace);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int R = B * T;

  IdxArgs ia{};
  ia.qc = dtype == CSK_MXFP4 ? reinterpret_cast<const uint8_t*>(q) : nullptr;
  ia.qs = q_scale;
  ia.qf = dtype == CSK_F32 ? reinterpret_cast<const float*>(q) : nullptr;
  ia.w = w;
  ia.kc = dtype == CSK_MXFP4 ? reinterpret_cast<const uint8_t*>(kk) : nullptr;
  ia.ks = k_scale;
  ia.kf = dtype == CSK_F32 ? reinterpret_cast<const float*>(kk) : nullptr;
  ia.q_pos = q_pos;
  ia.n_entries = n_entries;
  ia.B = B; ia.T = T; ia.HI = HI; ia.dI = dI; ia.Nmax = Nmax; ia.m = m;
  ia.scores = reinterpret_cast<float*>(ws + p.off_scores);
  ia.samples = p.filtered ? reinterpret_cast<float*>(ws + p.off_samples) : nullptr;
  ia.gs_log2 = p.gs_log2;
  ia.ng = p.ng;
  ia.bf16_scores = score_dtype == CSK_BF16;

  int rc = CSK_OK;
  // (the MFMA paths read the codes in 16-byte chunks: other alignments take
  // the VALU path)
  const bool mfma = dtype == CSK_MXFP4 && HI % 16 == 0 && HI <= 64 && dI % 128 == 0 && dI <= 256 &&
                    ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(kk)) & 15) == 0;
  if (mfma) {
    // 64-key groups per wave: 8 when the grid is short (a few rows over a
    // long cache: it then still has about two workgroups per CU), else 4
    const int64_t groups = (int64_t)R * ceil_div(Nmax, 256);
    const int iters = groups >= 8 * IDX_TARGET_WGS ? 8 : 4;
    ia.iters = iters;
    dim3 grid((unsigned)R, (unsigned)ceil_div(Nmax, 256 * iters)), block(256);
    const int HT = HI / 16, KS = dI / 128;
    // Prefill rows (several queries per sequence) with 32 or 64 heads: the
    // 32x32 DMA form (VALU-bound there; it issues fewer VALU instructions
    // per key). Decode rows, and 16 or 48 heads: the 16x16 form (measured
    // faster where the key stream dominates).
    const bool w32 = HI % 32 == 0 && T > 1;
#define CSK_IDX_CASE(ht, ks)                                                                     \
  if (!w32 && HT == ht && KS == ks)                                                              \
    rc = iters == 8 ? launch("indexer_scores_fp4", idx_fp4_kernel<ht, ks, 8>, grid, block, 0, s, ia) \
                    : launch("indexer_scores_fp4", idx_fp4_kernel<ht, ks, 4>, grid, block, 0, s, ia);
    CSK_IDX_CASE(1, 1) CSK_IDX_CASE(2, 1) CSK_IDX_CASE(3, 1) CSK_IDX_CASE(4, 1)
    CSK_IDX_CASE(1, 2) CSK_IDX_CASE(2, 2) CSK_IDX_CASE(3, 2) CSK_IDX_CASE(4, 2)
#undef CSK_IDX_CASE
#define CSK_IDX_W32_CASE(ht2, kb)                                                                  \
  if (w32 && HI == 32 * ht2 && dI == 32 * kb) {                                                    \
    constexpr int nb = 2;  /* two stages: 39 KB of LDS, four workgroups per CU */                  \
    rc = iters == 8 ? launch("indexer_scores_fp4", idx_fp4_w32_kernel<ht2, kb, 8, nb>, grid, block, 0, s, ia) \
                    : launch("indexer_scores_fp4", idx_fp4_w32_kernel<ht2, kb, 4, nb>, grid, block, 0, s, ia); \
  }
    CSK_IDX_W32_CASE(1, 4) CSK_IDX_W32_CASE(2, 4) CSK_IDX_W32_CASE(1, 8) CSK_IDX_W32_CASE(2, 8)
#undef CSK_IDX_W32_CASE
  } else {
    dim3 grid((unsigned)R, (unsigned)ceil_div(Nmax, 256)), block(256);
    rc = dtype == CSK_MXFP4 ? launch("indexer_scores_valu", idx_valu_kernel<true>, grid, block, 0, s, ia)
                            : launch("indexer_scores_valu", idx_valu_kernel<false>, grid, block, 0, s, ia);
    if (rc == CSK_OK && p.filtered) {
      dim3 g2((unsigned)R, (unsigned)ceil_div(p.ng, 256));
      rc = launch("indexer_samples", idx_samples_kernel, g2, block, 0, s, ia);
    }
  }
  if (rc != CSK_OK) return rc;

  TopkArgs ta{};
  ta.ia = ia;
  ta.k = k;
  ta.n_slices = p.n_slices;
  ta.idx = idx;
  ta.out_score = score;
  const size_t lds = sizeof(TopkShared), lds_u = sizeof(TopkSharedU);
  static std::once_flag attr_once;
  std::call_once(attr_once, [&] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(topk_select_kernel<true>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(topk_select_kernel<false>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_u);
  });
  if (p.filtered) {
    ta.cand_cnt = reinterpret_cast<int*>(ws + p.off_cnt);
    ta.cand_score = reinterpret_cast<float*>(ws + p.off_cscore);
    ta.cand_idx = reinterpret_cast<int*>(ws + p.off_cidx);
    ta.flat_key = reinterpret_cast<uint32_t*>(ws + p.off_fkey);
    ta.flat_idx = reinterpret_cast<int*>(ws + p.off_fidx);
    rc = launch("topk_filter", topk_filter_kernel, dim3(R, p.n_slices), dim3(FUSED_THREADS), 0, s, ta);
    if (rc == CSK_OK)
      rc = launch("topk_select", topk_select_kernel<true>, dim3(R), dim3(TOPK_THREADS), lds, s, ta);
  } else {
    rc = launch("topk_select", topk_select_kernel<false>, dim3(R), dim3(TOPK_THREADS), lds_u, s, ta);
  }
  return rc;
}

}  // namespace csk

extern "C" {

size_t indexer_topk_workspace_size(int B, int T, int HI, int dI, int Nmax, int k, int dtype) {
  (void)HI; (void)dI; (void)dtype;
  if (B <= 0 || T <= 0 || Nmax <= 0 || k <= 0) return 0;
  return csk::plan_indexer(B, T, Nmax, k).total;
}

int indexer_topk(const void* q, const uint8_t* q_scale, const float* w, const void* kk,
                 const uint8_t* k_scale, const int32_t* q_pos, const int32_t* n_entries, int B,
                 int T, int HI, int dI, int Nmax, int m, int k, int dtype, int score_dtype,
                 int32_t* idx, float* score, void* workspace, size_t ws_bytes, void* stream) {
  return csk::indexer_topk_impl("indexer_topk", false, q, q_scale, w, kk, k_scale, q_pos, n_entries, B, T, HI,
                                dI, Nmax, m, k, dtype, score_dtype, idx, score, workspace, ws_bytes, stream);
}

int indexer_topk_noalloc(const void* q, const uint8_t* q_scale, const float* w, const void* kk,
                         const uint8_t* k_scale, const int32_t* q_pos, const int32_t* n_entries, int B,
                         int T, int HI, int dI, int Nmax, int m, int k, int dtype, int score_dtype,
                         int32_t* idx, float* score, void* stream) {
  return csk::indexer_topk_impl("indexer_topk_noalloc", true, q, q_scale, w, kk, k_scale, q_pos, n_entries, B,
                                T, HI, dI, Nmax, m, k, dtype, score_dtype, idx, score, nullptr, 0, stream);
}

}  // extern "C"
