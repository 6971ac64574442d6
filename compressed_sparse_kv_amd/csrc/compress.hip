// compress.hip - CSA / HCA softmax-gated pooling with partial-RoPE and
// MXFP4 epilogues, and the standalone MXFP4 quantiser.
//
// Pooling ([P1] «CSA: сжать в 4 раза и выбрать top-k», step 1; «HCA: сжать
// в 128 раз…»): per channel, a softmax over the gate logits Z + bias of the
// entry's source slots weights the matching C values. The work is a pure
// stream (each source byte read once, each output written once), so it is
// HBM-bound: one thread owns two adjacent channels of one entry, so a wave
// reads 64 consecutive channel pairs of a source row (coalesced), loops over
// the entry's slots with an online softmax in fp32, and finishes with the
// RoPE rotation and the output rounding or MXFP4 encoding in registers. For
// MXFP4, 16 consecutive lanes own one 1x32 tile; the tile maximum is a
// 16-lane shuffle reduction.
#include <cstring>

#include "common.h"

namespace csk {

enum { OUT_F32 = 0, OUT_BF16 = 1, OUT_MXFP4 = 2, OUT_FP8KV = 3 };

struct CompressArgs {
  const void* ca;
  const void* za;
  const void* cb;
  const void* zb;
  const float* bias_a;
  const float* bias_b;
  int B, N, D, m, entry0, d_rope;
  int64_t src_bstride, dst_bstride;
  RopeTable rope;
  const int32_t* entry_pos;
  void* out;
  uint8_t* out_scale;
};

// Gate logit Z + bias and value C of one source slot for a channel pair;
// an absent slot (ok false) has logit -inf and contributes nothing. The loads
// are unconditional (an absent slot reads the valid row `safe_row` instead)
// so that a batch of them stays in flight together: a load under a branch
// would have to complete before the branch's other side could write the
// same registers.
template <typename IN>
__device__ __forceinline__ void load_slot(const IN* c, const IN* z, const float* bias, int64_t row,
                                          int brow, int D, int ch, bool ok, int64_t safe_row,
                                          float2& l, float2& v) {
  const int64_t off = (ok ? row : safe_row) * (int64_t)D + ch;
  const float2 zz = io<IN>::load2(z + off);
  const float2 cc = io<IN>::load2(c + off);
  const float2 bb = *reinterpret_cast<const float2*>(bias + (int64_t)(ok ? brow : 0) * D + ch);
  // the masks are applied arithmetically: a select whose operand is a load
  // would let the compiler sink that load back under a branch
  const float pen = ok ? 0.f : -INFINITY, keep = ok ? 1.f : 0.f;
  l = make_float2(zz.x + bb.x + pen, zz.y + bb.y + pen);
  v = make_float2(cc.x * keep, cc.y * keep);
}

// Folds a batch of NB slots into the running softmax state (max,
// denominator, numerator) of a channel pair, rescaling once per batch.
template <int NB>
__device__ __forceinline__ void fold(const float2* l, const float2* v, float2& mx, float2& den,
                                     float2& num) {
  float2 bm = mx;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    bm.x = fmaxf(bm.x, l[j].x);
    bm.y = fmaxf(bm.y, l[j].y);
  }
  const float f0 = mx.x == -INFINITY ? 0.f : expf(mx.x - bm.x);
  const float f1 = mx.y == -INFINITY ? 0.f : expf(mx.y - bm.y);
  den.x *= f0;
  num.x *= f0;
  den.y *= f1;
  num.y *= f1;
  mx = bm;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const float e0 = l[j].x == -INFINITY ? 0.f : expf(l[j].x - bm.x);
    const float e1 = l[j].y == -INFINITY ? 0.f : expf(l[j].y - bm.y);
    den.x += e0;
    den.y += e1;
    num.x = fmaf(e0, v[j].x, num.x);
    num.y = fmaf(e1, v[j].y, num.y);
  }
}

// Softmax over `m` slots starting at row r0 (relative to src), in batches of
// NB slots: all loads of a batch are issued before any arithmetic depends on
// them (no branch between them, so they are in flight together).
template <int NB, typename IN>
__device__ __forceinline__ void pool_slots(const IN* c, const IN* z, const float* bias, int64_t r0,
                                           int m, int D, int ch, float2& mx, float2& den,
                                           float2& num) {
  for (int rb = 0; rb < m; rb += NB) {
    float2 l[NB], v[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j)
      load_slot(c, z, bias, r0 + rb + j, rb + j, D, ch, rb + j < m, r0, l[j], v[j]);
    fold<NB>(l, v, mx, den, num);
  }
}

// Exactly N slots starting at row r0, all loads issued before the fold.
template <int N, typename IN>
__device__ __forceinline__ void pool_fixed(const IN* c, const IN* z, const float* bias, int64_t r0, int D,
                                           int ch, float2& mx, float2& den, float2& num) {
  float2 l[N], v[N];
#pragma unroll
  for (int j = 0; j < N; ++j) load_slot(c, z, bias, r0 + j, j, D, ch, true, r0, l[j], v[j]);
  fold<N>(l, v, mx, den, num);
}

template <int OUT>
__device__ __forceinline__ void store_pair(const CompressArgs& a, int64_t orow, int p, float v0,
                                           float v1) {
  if (OUT == OUT_F32) {
    float* o = reinterpret_cast<float*>(a.out) + orow * a.D + 2 * p;
    *reinterpret_cast<float2*>(o) = make_float2(v0, v1);
  } else if (OUT == OUT_BF16) {
    uint32_t* o = reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(a.out) + orow * a.D + 2 * p);
    *o = f32_to_bf16_bits(v0) | (f32_to_bf16_bits(v1) << 16);
  } else if (OUT == OUT_FP8KV) {
    // FP8 KV entry: 16 consecutive lanes hold one block of 32 non-RoPE
    // channels (E4M3 codes under the block's scale); RoPE channels stay bf16.
    // Every lane forms the block maximum (the DPP steps need the whole row
    // of 16 lanes; RoPE lanes ignore it). D - d_rope is a multiple of 32, so
    // a row of 16 lanes is all codes or all RoPE.
    const int dn = a.D - a.d_rope;
    const int es = fp8kv_entry_bytes(a.D, a.d_rope);
    uint8_t* e = reinterpret_cast<uint8_t*>(a.out) + orow * es;
    const float amax = row16_max(fmaxf(fabsf(v0), fabsf(v1)));
    const int ch = 2 * p;
    if (ch < dn) {
      uint32_t codes = 0u, sc = 127u;
      if (amax != 0.0f) {
        const int s = fp8kv_scale_exp(amax);
        codes = e4m3_encode(v0, s) | (e4m3_encode(v1, s) << 8);
        sc = (uint32_t)(s + 127);
      }
      *reinterpret_cast<uint16_t*>(e + ch) = (uint16_t)codes;
      if ((p & 15) == 0) e[dn + 2 * a.d_rope + ch / 32] = (uint8_t)sc;
    } else {
      *reinterpret_cast<uint32_t*>(e + dn + 2 * (ch - dn)) = f32_to_bf16_bits(v0) | (f32_to_bf16_bits(v1) << 16);
    }
    if (p == 0)  // the padding past the scales
      for (int z = dn + 2 * a.d_rope + dn / 32; z < es; ++z) e[z] = 0;
  } else {
    // 16 consecutive lanes hold one tile of 32 channels
    float amax = fmaxf(fabsf(v0), fabsf(v1));
    amax = row16_max(amax);
    uint32_t byte, sc;
    if (amax == 0.0f) {
      byte = 0;
      sc = 127;
    } else {
      int s = mx_scale_exp(amax);
      byte = e2m1_encode(v0, s) | (e2m1_encode(v1, s) << 4);
      sc = (uint32_t)(s + 127);
    }
    reinterpret_cast<uint8_t*>(a.out)[orow * (a.D / 2) + p] = (uint8_t)byte;
    if ((p & 15) == 0) a.out_scale[orow * (a.D / 32) + p / 16] = (uint8_t)sc;
  }
}

// Channel pair p of entry `row` (batch-major) of a one-wave-per-row
// compression: pool the entry's slots, rotate, round or encode, store.
template <typename IN, int OUT, bool CSA>
__device__ __forceinline__ void compress_pair(const CompressArgs& a, int p, int64_t row) {
  const int b = (int)(row / a.N);
  const int i = (int)(row - (int64_t)b * a.N);
  const int ch = 2 * p;

  float2 mx = make_float2(-INFINITY, -INFINITY);
  float2 den = make_float2(0.f, 0.f), num = make_float2(0.f, 0.f);
  const int64_t src0 = (int64_t)b * a.src_bstride;
  const IN* ca = reinterpret_cast<const IN*>(a.ca) + src0 * a.D;
  const IN* za = reinterpret_cast<const IN*>(a.za) + src0 * a.D;
  const bool has_b = CSA && (a.entry0 + i) > 0;
  if (CSA && a.m == 4) {
    // 4x compression (the CSA ratio): both series, 8 slots, one batch
    const IN* cb = reinterpret_cast<const IN*>(a.cb) + src0 * a.D;
    const IN* zb = reinterpret_cast<const IN*>(a.zb) + src0 * a.D;
    float2 l[8], v[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      load_slot(ca, za, a.bias_a, 4 * (int64_t)i + j, j, a.D, ch, true, 4 * (int64_t)i, l[j], v[j]);
      load_slot(cb, zb, a.bias_b, 4 * ((int64_t)i - 1) + j, j, a.D, ch, has_b, 4 * (int64_t)i, l[4 + j],
                v[4 + j]);
    }
    fold<8>(l, v, mx, den, num);
  } else if (CSA && a.m <= 8) {
    // both series of the entry in one batch: 2m loads in flight together
    const IN* cb = reinterpret_cast<const IN*>(a.cb) + src0 * a.D;
    const IN* zb = reinterpret_cast<const IN*>(a.zb) + src0 * a.D;
    float2 l[16], v[16];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      load_slot(ca, za, a.bias_a, (int64_t)a.m * i + j, j, a.D, ch, j < a.m, (int64_t)a.m * i, l[j],
                v[j]);
      load_slot(cb, zb, a.bias_b, (int64_t)a.m * (i - 1) + j, j, a.D, ch, has_b && j < a.m,
                (int64_t)a.m * i, l[8 + j], v[8 + j]);
    }
    fold<16>(l, v, mx, den, num);
  } else {
    pool_slots<8, IN>(ca, za, a.bias_a, (int64_t)a.m * i, a.m, a.D, ch, mx, den, num);
    if (has_b)
      pool_slots<8, IN>(reinterpret_cast<const IN*>(a.cb) + src0 * a.D,
                        reinterpret_cast<const IN*>(a.zb) + src0 * a.D, a.bias_b, (int64_t)a.m * (i - 1),
                        a.m, a.D, ch, mx, den, num);
  }
  float v0 = num.x / den.x, v1 = num.y / den.y;

  const int rope0 = a.D - a.d_rope;
  if (ch >= rope0) {
    const double pos = a.entry_pos ? (double)a.entry_pos[(int64_t)b * a.N + i]
                                   : (double)a.m * (double)(a.entry0 + i);
    float c, s;
    rope_cs(pos, a.rope.theta[(ch - rope0) / 2], &c, &s);
    float r0 = v0 * c - v1 * s;
    float r1 = v0 * s + v1 * c;
    v0 = r0;
    v1 = r1;
  }
  store_pair<OUT>(a, (int64_t)b * a.dst_bstride + i, p, v0, v1);
}

template <typename IN, int OUT, bool CSA>
__global__ __launch_bounds__(64) void compress_kernel(CompressArgs a) {
  const int half = a.D / 2;
  // grid: x = channel-pair blocks of one row, y = rows (b, i) in two levels
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= half) return;
  const int64_t row = (int64_t)blockIdx.z * gridDim.y + blockIdx.y;
  if (row >= (int64_t)a.B * a.N) return;
  compress_pair<IN, OUT, CSA>(a, p, row);
}

// Wide blocks (HCA, m >= 32): the m slots of a channel pair are split over
// 8 slot groups so that a wave keeps many independent loads in flight; the
// 8 partial softmax states (max, denominator, numerator) are merged in LDS.
// Block = 32 channel pairs x 8 slot groups; grid = (pair blocks, entries).
template <typename IN, int OUT, bool CSA>
__global__ __launch_bounds__(256) void compress_wide_kernel(CompressArgs a) {
  __shared__ float part[8][32][6];
  const int half = a.D / 2;
  const int cpl = threadIdx.x & 31, sg = threadIdx.x >> 5;
  const int p = blockIdx.x * 32 + cpl;
  const int64_t row = blockIdx.y;
  const int b = (int)(row / a.N);
  const int i = (int)(row % a.N);
  float2 mx = make_float2(-INFINITY, -INFINITY);
  float2 den = make_float2(0.f, 0.f), num = make_float2(0.f, 0.f);
  if (p < half) {
    const int per = a.m / 8;
    const int64_t src0 = (int64_t)b * a.src_bstride;
    const IN* cs = reinterpret_cast<const IN*>(a.ca) + src0 * a.D + (int64_t)sg * per * a.D;
    const IN* zs = reinterpret_cast<const IN*>(a.za) + src0 * a.D + (int64_t)sg * per * a.D;
    const float* bs = a.bias_a + (int64_t)sg * per * a.D;
    // m' = 128 (16 slots per group): a compile-time count, so that all 16
    // slot loads are in flight together
    if (per == 16) pool_fixed<16, IN>(cs, zs, bs, (int64_t)a.m * i, a.D, 2 * p, mx, den, num);
    else pool_slots<16, IN>(cs, zs, bs, (int64_t)a.m * i, per, a.D, 2 * p, mx, den, num);
  }
  part[sg][cpl][0] = mx.x; part[sg][cpl][1] = mx.y;
  part[sg][cpl][2] = den.x; part[sg][cpl][3] = den.y;
  part[sg][cpl][4] = num.x; part[sg][cpl][5] = num.y;
  __syncthreads();
  if (sg != 0 || p >= half) return;
  float M0 = -INFINITY, M1 = -INFINITY;
  for (int q = 0; q < 8; ++q) {
    M0 = fmaxf(M0, part[q][cpl][0]);
    M1 = fmaxf(M1, part[q][cpl][1]);
  }
  float d0 = 0.f, d1 = 0.f, n0 = 0.f, n1 = 0.f;
  for (int q = 0; q < 8; ++q) {
    const float f0 = expf(part[q][cpl][0] - M0), f1 = expf(part[q][cpl][1] - M1);
    d0 += part[q][cpl][2] * f0;
    d1 += part[q][cpl][3] * f1;
    n0 += part[q][cpl][4] * f0;
    n1 += part[q][cpl][5] * f1;
  }
  float v0 = n0 / d0, v1 = n1 / d1;
  const int ch = 2 * p;
  const int rope0 = a.D - a.d_rope;
  if (ch >= rope0) {
    const double pos = a.entry_pos ? (double)a.entry_pos[(int64_t)b * a.N + i]
                                   : (double)a.m * (double)(a.entry0 + i);
    float c, sn;
    rope_cs(pos, a.rope.theta[(ch - rope0) / 2], &c, &sn);
    const float r0 = v0 * c - v1 * sn, r1 = v0 * sn + v1 * c;
    v0 = r0;
    v1 = r1;
  }
  store_pair<OUT>(a, (int64_t)b * a.dst_bstride + i, p, v0, v1);
}

// MXFP4 encode of channel pair p of row r; 16 consecutive lanes hold one
// 1x32 tile, so a tile's lanes must be converged here.
template <typename IN>
__device__ __forceinline__ void quant_pair(const IN* x, int64_t r, int cols, int p, uint8_t* codes,
                                           uint8_t* scales) {
  const int half = cols / 2;
  float2 v = io<IN>::load2(x + r * cols + 2 * p);
  float amax = fmaxf(fabsf(v.x), fabsf(v.y));
  amax = row16_max(amax);
  uint32_t byte, sc;
  if (amax == 0.0f) {
    byte = 0;
    sc = 127;
  } else {
    int s = mx_scale_exp(amax);
    byte = e2m1_encode(v.x, s) | (e2m1_encode(v.y, s) << 4);
    sc = (uint32_t)(s + 127);
  }
  codes[r * half + p] = (uint8_t)byte;
  if ((p & 15) == 0) scales[r * (cols / 32) + p / 16] = (uint8_t)sc;
}

template <typename IN>
__global__ __launch_bounds__(256) void mxfp4_quant_kernel(const IN* x, int64_t rows, int cols,
                                                           uint8_t* codes, uint8_t* scales) {
  const int half = cols / 2;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= rows * half) return;
  quant_pair<IN>(x, gid / half, cols, (int)(gid % half), codes, scales);
}

// Streaming form for whole tensors: sixteen consecutive values per lane (one
// 64-byte fp32 or 32-byte bf16 load, one 8-byte code store); the two lanes
// of a 32-value tile (lanes 2i and 2i+1: the element count is a multiple of
// 32) share the tile maximum through one DPP swap. The encoding is the
// per-pair one's, value for value. Lanes past the end work on a copy of the
// last values (their pair partner is past the end too) and store nothing.
template <typename IN>
__global__ __launch_bounds__(256) void mxfp4_quant16_kernel(const IN* x, int64_t n16, uint8_t* codes,
                                                             uint8_t* scales) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t tc = t < n16 ? t : n16 - 1;
  float v[16];
  if constexpr (sizeof(IN) == 4) {
    typedef float f4 __attribute__((ext_vector_type(4)));
    const f4* src = reinterpret_cast<const f4*>(x) + 4 * tc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f4 f = __builtin_nontemporal_load(src + i);
      v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
    }
  } else {
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    const u4* src = reinterpret_cast<const u4*>(x) + 2 * tc;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const u4 u = __builtin_nontemporal_load(src + i);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[8 * i + 2 * k] = bf16_bits_to_f32(w[k] & 0xffffu);
        v[8 * i + 2 * k + 1] = bf16_bits_to_f32(w[k] >> 16);
      }
    }
  }
  float amax = fabsf(v[0]);
#pragma unroll
  for (int i = 1; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, CSK_DPP_F(amax, 0xB1));  // quad_perm [1,0,3,2]: the tile's other lane
  uint32_t lo = 0u, hi = 0u, sc = 127u;
  if (amax != 0.0f) {
    const int s = mx_scale_exp(amax);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      lo |= (e2m1_encode(v[2 * k], s) | (e2m1_encode(v[2 * k + 1], s) << 4)) << (8 * k);
      hi |= (e2m1_encode(v[8 + 2 * k], s) | (e2m1_encode(v[8 + 2 * k + 1], s) << 4)) << (8 * k);
    }
    sc = (uint32_t)(s + 127);
  }
  if (t < n16) {
    *reinterpret_cast<uint2*>(codes + 8 * t) = make_uint2(lo, hi);
    if ((t & 1) == 0) scales[t >> 1] = (uint8_t)sc;
  }
}

// Several independent small compressions and MXFP4 encodes in one launch
// (a decode step issues a few, each too small to fill the chip, and each
// launch boundary costs more than its work). The grid is one dimension:
// job z owns blocks [first[z], first[z+1]), one block per 64 channel pairs
// of one of its rows (entry rows of a compression, rows of an encode), so
// no block is idle. Every job runs the same per-pair code as its own
// kernel, so results are identical.
struct BatchJob {
  CompressArgs a;  // compression job; an encode job uses out, out_scale, D
  const void* x;   // encode job input
  int64_t rows;    // rows of the job (compression: B * N)
  int kind, in_bf16, out_kind, xblocks;
};
struct BatchArgs {
  BatchJob j[CSK_MAX_JOBS];
  int first[CSK_MAX_JOBS + 1];
  int n;
};

__global__ __launch_bounds__(64) void compress_batch_kernel(BatchArgs args) {
  const int blk = blockIdx.x;
  // the workgroup's job: first[] is increasing, so z counts the job starts
  // at or below blk (all of them read at once, not one per step)
  int z = 0;
#pragma unroll
  for (int q = 1; q < CSK_MAX_JOBS; ++q) z += (q < args.n && blk >= args.first[q]) ? 1 : 0;
  const BatchJob& j = args.j[z];
  // (the job's fields read together, before any branch on them: the empty
  // asm takes them all, so their loads share one wait instead of each
  // waiting in turn at its first use; the reads below and inside the
  // pooling find the same values)
  const int first = args.first[z], xblocks = j.xblocks, D = j.a.D;
  const int kind = j.kind, in_bf16 = j.in_bf16, out_kind = j.out_kind;
  asm volatile("" ::"s"(first), "s"(xblocks), "s"(D), "s"(kind), "s"(in_bf16), "s"(out_kind), "s"(j.a.ca),
               "s"(j.a.za), "s"(j.a.cb), "s"(j.a.zb), "s"(j.a.bias_a), "s"(j.a.bias_b), "s"(j.a.out),
               "s"(j.a.out_scale), "s"(j.x));
  asm volatile("" ::"s"(j.a.B), "s"(j.a.N), "s"(j.a.m), "s"(j.a.entry0), "s"(j.a.d_rope), "s"(j.a.src_bstride),
               "s"(j.a.dst_bstride), "s"(j.a.entry_pos));
  const int local = blk - first;
  const int row = local / xblocks;
  const int p = (local - row * xblocks) * 64 + threadIdx.x;
  if (p >= D / 2) return;
  if (kind == CSK_JOB_MXFP4) {
    uint8_t* codes = reinterpret_cast<uint8_t*>(j.a.out);
    if (in_bf16) quant_pair<uint16_t>(reinterpret_cast<const uint16_t*>(j.x), row, D, p, codes, j.a.out_scale);
    else quant_pair<float>(reinterpret_cast<const float*>(j.x), row, D, p, codes, j.a.out_scale);
  } else if (in_bf16) {
    if (out_kind == OUT_BF16) compress_pair<uint16_t, OUT_BF16, true>(j.a, p, row);
    else if (out_kind == OUT_MXFP4) compress_pair<uint16_t, OUT_MXFP4, true>(j.a, p, row);
    else if (out_kind == OUT_FP8KV) compress_pair<uint16_t, OUT_FP8KV, true>(j.a, p, row);
    else compress_pair<uint16_t, OUT_F32, true>(j.a, p, row);
  } else {
    if (out_kind == OUT_BF16) compress_pair<float, OUT_BF16, true>(j.a, p, row);
    else if (out_kind == OUT_MXFP4) compress_pair<float, OUT_MXFP4, true>(j.a, p, row);
    else if (out_kind == OUT_FP8KV) compress_pair<float, OUT_FP8KV, true>(j.a, p, row);
    else compress_pair<float, OUT_F32, true>(j.a, p, row);
  }
}

// Entries pooled by another kernel (fp32, row b*N + i, D values) with
// per-block partial sums of squares (ncb per entry): RMSNorm when gamma is
// given (the partials summed in ascending block order), then RoPE at the
// entry's position, then the output rounding or encoding. Same lane layout
// as compress_kernel: one lane per channel pair, 64 pairs per workgroup.
struct FinalizeArgs {
  CompressArgs a;
  const float* pooled;
  const float* ss;
  const float* gamma;
  int ncb;
  float eps;
};

template <int OUT>
__global__ __launch_bounds__(64) void finalize_kernel(FinalizeArgs f) {
  const CompressArgs& a = f.a;
  const int half = a.D / 2;
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= half) return;
  const int64_t row = (int64_t)blockIdx.z * gridDim.y + blockIdx.y;
  if (row >= (int64_t)a.B * a.N) return;
  const int b = (int)(row / a.N);
  const int i = (int)(row - (int64_t)b * a.N);
  const int ch = 2 * p;
  const float2 v = *reinterpret_cast<const float2*>(f.pooled + row * a.D + ch);
  float v0 = v.x, v1 = v.y;
  if (f.gamma) {
    float ss = 0.f;
    for (int cb = 0; cb < f.ncb; ++cb) ss += f.ss[row * f.ncb + cb];
    const float inv = 1.0f / sqrtf(ss / (float)a.D + f.eps);
    v0 = v0 * inv * f.gamma[ch];
    v1 = v1 * inv * f.gamma[ch + 1];
  }
  const int rope0 = a.D - a.d_rope;
  if (ch >= rope0) {
    const double pos = a.entry_pos ? (double)a.entry_pos[(int64_t)b * a.N + i]
                                   : (double)a.m * (double)(a.entry0 + i);
    float c, sn;
    rope_cs(pos, a.rope.theta[(ch - rope0) / 2], &c, &sn);
    const float r0 = v0 * c - v1 * sn, r1 = v0 * sn + v1 * c;
    v0 = r0;
    v1 = r1;
  }
  store_pair<OUT>(a, (int64_t)b * a.dst_bstride + i, p, v0, v1);
}

int finalize_entries(const char* name, int B, int N, int D, int m, int entry0, int d_rope, float rope_base,
                     const int32_t* entry_pos, int out_dtype, void* out, uint8_t* out_scale, int64_t dst_bstride,
                     const float* pooled, const float* ss, int ncb, const float* gamma, float eps, hipStream_t s) {
  const int64_t rows = (int64_t)B * N;
  if (rows <= 0) return CSK_OK;
  CompressArgs a{};
  a.B = B; a.N = N; a.D = D; a.m = m; a.entry0 = entry0; a.d_rope = d_rope;
  a.dst_bstride = dst_bstride ? dst_bstride : N;
  fill_rope_table(&a.rope, d_rope, (double)rope_base);
  a.entry_pos = entry_pos;
  a.out = out; a.out_scale = out_scale;
  FinalizeArgs f{a, pooled, ss, gamma, ncb, eps};
  const unsigned gy = (unsigned)(rows < 65535 ? rows : 65535);
  dim3 grid((unsigned)ceil_div(a.D / 2, 64), gy, (unsigned)ceil_div(rows, gy)), block(64);
  switch (out_dtype) {
    case CSK_F32: return launch(name, finalize_kernel<OUT_F32>, grid, block, 0, s, f);
    case CSK_BF16: return launch(name, finalize_kernel<OUT_BF16>, grid, block, 0, s, f);
    case CSK_FP8KV: return launch(name, finalize_kernel<OUT_FP8KV>, grid, block, 0, s, f);
    default: return launch(name, finalize_kernel<OUT_MXFP4>, grid, block, 0, s, f);
  }
}

template <typename IN, bool CSA>
static int launch_compress_out(const char* name, const CompressArgs& a, int out_dtype,
                               hipStream_t s) {
  if (!CSA && a.m >= 32 && a.m % 8 == 0 && (int64_t)a.B * a.N <= 65535) {
    dim3 grid((unsigned)ceil_div(a.D / 2, 32), (unsigned)((int64_t)a.B * a.N)), block(256);
    switch (out_dtype) {
      case CSK_F32: return launch(name, compress_wide_kernel<IN, OUT_F32, CSA>, grid, block, 0, s, a);
      case CSK_BF16: return launch(name, compress_wide_kernel<IN, OUT_BF16, CSA>, grid, block, 0, s, a);
      case CSK_FP8KV: return launch(name, compress_wide_kernel<IN, OUT_FP8KV, CSA>, grid, block, 0, s, a);
      default: return launch(name, compress_wide_kernel<IN, OUT_MXFP4, CSA>, grid, block, 0, s, a);
    }
  }
  // one wave per 64 channel pairs of a row; rows over grid.y (and grid.z
  // past 65535 rows)
  const int64_t rows = (int64_t)a.B * a.N;
  if (rows <= 0) return CSK_OK;
  const unsigned gy = (unsigned)(rows < 65535 ? rows : 65535);
  dim3 grid((unsigned)ceil_div(a.D / 2, 64), gy, (unsigned)ceil_div(rows, gy)), block(64);
  switch (out_dtype) {
    case CSK_F32: return launch(name, compress_kernel<IN, OUT_F32, CSA>, grid, block, 0, s, a);
    case CSK_BF16: return launch(name, compress_kernel<IN, OUT_BF16, CSA>, grid, block, 0, s, a);
    case CSK_FP8KV: return launch(name, compress_kernel<IN, OUT_FP8KV, CSA>, grid, block, 0, s, a);
    default: return launch(name, compress_kernel<IN, OUT_MXFP4, CSA>, grid, block, 0, s, a);
  }
}

// Checks the arguments of one compression call and fills its kernel
// arguments; *empty is set when the call reads and writes nothing.
static int prepare_compress(const std::string& f, bool csa, const void* ca, const void* za,
                            const void* cb, const void* zb, const float* bias_a,
                            const float* bias_b, int B, int S, int D, int m, int entry0,
                            int64_t src_bstride, int d_rope, float rope_base,
                            const int32_t* entry_pos, int in_dtype, int out_dtype, void* out,
                            uint8_t* out_scale, int64_t dst_bstride, CompressArgs* ap,
                            bool* empty_p) {
  if (B < 0 || S < 0 || D <= 0 || (D & 1) || m <= 0 || entry0 < 0)
    return fail(CSK_EINVAL, f + ": need B >= 0, S >= 0, even D > 0, m > 0, entry0 >= 0");
  const bool empty = B == 0 || S / m == 0;  // nothing is read or written
  if (!empty && (!ca || !za || !bias_a || !out || (csa && (!cb || !zb || !bias_b))))
    return fail(CSK_EINVAL, f + ": null pointer");
  if (d_rope < 0 || d_rope > D || (d_rope & 1))
    return fail(CSK_EINVAL, f + ": d_rope must be even and in [0, D]");
  if (d_rope > 2 * MAX_ROPE_PAIRS)
    return fail(CSK_EUNSUPPORTED, f + ": at most 128 rotated channels are built");
  if (in_dtype != CSK_F32 && in_dtype != CSK_BF16)
    return fail(CSK_EUNSUPPORTED, f + ": in_dtype must be CSK_F32 or CSK_BF16");
  if (out_dtype != CSK_F32 && out_dtype != CSK_BF16 && out_dtype != CSK_MXFP4 && out_dtype != CSK_FP8KV)
    return fail(CSK_EUNSUPPORTED, f + ": out_dtype must be CSK_F32, CSK_BF16, CSK_MXFP4 or CSK_FP8KV");
  if (out_dtype == CSK_MXFP4 && (D % 32 || (!out_scale && !empty)))
    return fail(CSK_EINVAL, f + ": MXFP4 output needs D % 32 == 0 and out_scale");
  if (out_dtype == CSK_FP8KV && (D - d_rope) % 32)
    return fail(CSK_EINVAL, f + ": FP8KV output needs (D - d_rope) % 32 == 0");
  const int N = S / m;
  if (src_bstride < 0 || (src_bstride != 0 && src_bstride < S))
    return fail(CSK_EINVAL, f + ": src_bstride must be 0 or >= S");
  if (dst_bstride < 0 || (dst_bstride != 0 && dst_bstride < N))
    return fail(CSK_EINVAL, f + ": dst_bstride must be 0 or >= S/m");
  *empty_p = B == 0 || N == 0;
  if (*empty_p) return CSK_OK;
  CompressArgs& a = *ap;
  a.ca = ca; a.za = za; a.cb = cb; a.zb = zb;
  a.bias_a = bias_a; a.bias_b = bias_b;
  a.B = B; a.N = N; a.D = D; a.m = m; a.entry0 = entry0; a.d_rope = d_rope;
  a.src_bstride = src_bstride ? src_bstride : S;
  a.dst_bstride = dst_bstride ? dst_bstride : N;
  fill_rope_table(&a.rope, d_rope, (double)rope_base);
  a.entry_pos = entry_pos;
  a.out = out; a.out_scale = out_scale;
  return CSK_OK;
}

static int compress_common(const char* fn, bool csa, const void* ca, const void* za,
                           const void* cb, const void* zb, const float* bias_a,
                           const float* bias_b, int B, int S, int D, int m, int entry0,
                           int64_t src_bstride, int d_rope, float rope_base,
                           const int32_t* entry_pos, int in_dtype, int out_dtype, void* out,
                           uint8_t* out_scale, int64_t dst_bstride, void* stream) {
  clear_error();
  CompressArgs a;
  bool empty = false;
  const int rc = prepare_compress(fn, csa, ca, za, cb, zb, bias_a, bias_b, B, S, D, m, entry0,
                                  src_bstride, d_rope, rope_base, entry_pos, in_dtype, out_dtype,
                                  out, out_scale, dst_bstride, &a, &empty);
  if (rc != CSK_OK || empty) return rc;
  if (const int dc = check_device(fn); dc != CSK_OK) return dc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // (a launch with MXFP4 output - an indexer-key series - is timed apart
  // from the KV series' launch)
  const char* name = csa ? (out_dtype == CSK_MXFP4 ? "csa_compress_mxfp4" : "csa_compress")
                         : (out_dtype == CSK_MXFP4 ? "hca_compress_mxfp4" : "hca_compress");
  if (in_dtype == CSK_F32)
    return csa ? launch_compress_out<float, true>(name, a, out_dtype, s)
               : launch_compress_out<float, false>(name, a, out_dtype, s);
  return csa ? launch_compress_out<uint16_t, true>(name, a, out_dtype, s)
             : launch_compress_out<uint16_t, false>(name, a, out_dtype, s);
}

static int check_quantize(const std::string& f, const void* x, int in_dtype, int64_t rows,
                          int cols, const uint8_t* codes, const uint8_t* scales) {
  if (!x || !codes || !scales) return fail(CSK_EINVAL, f + ": null pointer");
  if (rows < 0 || cols <= 0 || cols % 32)
    return fail(CSK_EINVAL, f + ": need rows >= 0 and cols % 32 == 0");
  if (in_dtype != CSK_F32 && in_dtype != CSK_BF16)
    return fail(CSK_EUNSUPPORTED, f + ": in_dtype must be CSK_F32 or CSK_BF16");
  return CSK_OK;
}

static int compress_batch(const csk_compress_job* jobs, int n_jobs, void* stream) {
  clear_error();
  if (!jobs || n_jobs < 1 || n_jobs > CSK_MAX_JOBS)
    return fail(CSK_EINVAL, "csk_compress_batch: need 1 <= n_jobs <= CSK_MAX_JOBS and a job array");
  BatchArgs args;
  memset(&args, 0, sizeof(args));
  int nz = 0;
  int64_t total = 0;
  for (int q = 0; q < n_jobs; ++q) {
    const csk_compress_job& j = jobs[q];
    const std::string f = "csk_compress_batch: job " + std::to_string(q);
    BatchJob& bj = args.j[nz];
    int64_t rows;
    if (j.kind == CSK_JOB_CSA) {
      bool empty = false;
      const int rc = prepare_compress(f + " (csa_compress)", true, j.ca, j.za, j.cb, j.zb, j.bias_a,
                                      j.bias_b, j.B, j.S, j.D, j.m, j.entry0, j.src_bstride,
                                      j.d_rope, j.rope_base, j.entry_pos, j.in_dtype, j.out_dtype,
                                      j.out, j.out_scale, j.dst_bstride, &bj.a, &empty);
      if (rc != CSK_OK) return rc;
      if (j.m > 8) return fail(CSK_EUNSUPPORTED, f + ": batched compression needs m <= 8");
      if (empty) continue;
      rows = (int64_t)bj.a.B * bj.a.N;
      bj.in_bf16 = j.in_dtype == CSK_BF16;
      bj.out_kind = j.out_dtype == CSK_F32 ? OUT_F32 : j.out_dtype == CSK_BF16 ? OUT_BF16
                    : j.out_dtype == CSK_FP8KV ? OUT_FP8KV : OUT_MXFP4;
    } else if (j.kind == CSK_JOB_MXFP4) {
      const int rc = check_quantize(f + " (mxfp4_quantize)", j.x, j.in_dtype, j.rows, j.cols,
                                    reinterpret_cast<const uint8_t*>(j.out), j.out_scale);
      if (rc != CSK_OK) return rc;
      if (j.rows == 0) continue;
      rows = j.rows;
      bj.x = j.x;
      bj.a.out = j.out;
      bj.a.out_scale = j.out_scale;
      bj.a.D = j.cols;
      bj.in_bf16 = j.in_dtype == CSK_BF16;
    } else {
      return fail(CSK_EINVAL, f + ": kind must be CSK_JOB_CSA or CSK_JOB_MXFP4");
    }
    if (rows > 65535) return fail(CSK_EUNSUPPORTED, f + ": at most 65535 rows per batched job");
    bj.kind = j.kind;
    bj.rows = rows;
    bj.xblocks = (int)ceil_div(bj.a.D / 2, 64);
    args.first[nz] = (int)total;
    total += rows * bj.xblocks;
    if (total * 64 > (int64_t)UINT32_MAX)
      return fail(CSK_EUNSUPPORTED, "csk_compress_batch: too many channel pairs in one batch");
    ++nz;
  }
  if (nz == 0) return CSK_OK;
  if (const int dc = check_device("csk_compress_batch"); dc != CSK_OK) return dc;
  args.first[nz] = (int)total;
  args.n = nz;
  dim3 grid((unsigned)total), block(64);
  return launch("csk_compress_batch", compress_batch_kernel, grid, block, 0,
                reinterpret_cast<hipStream_t>(stream), args);
}

}  // namespace csk

extern "C" {

int csa_compress(const void* ca, const void* za, const void* cb, const void* zb,
                 const float* bias_a, const float* bias_b, int B, int S, int D, int m,
                 int entry0, int64_t src_bstride, int d_rope, float rope_base,
                 const int32_t* entry_pos, int in_dtype, int out_dtype, void* out,
                 uint8_t* out_scale, int64_t dst_bstride, void* stream) {
  return csk::compress_common("csa_compress", true, ca, za, cb, zb, bias_a, bias_b, B, S, D, m,
                              entry0, src_bstride, d_rope, rope_base, entry_pos, in_dtype,
                              out_dtype, out, out_scale, dst_bstride, stream);
}

int hca_compress(const void* c, const void* z, const float* bias, int B, int S, int D, int m,
                 int entry0, int64_t src_bstride, int d_rope, float rope_base,
                 const int32_t* entry_pos, int in_dtype, int out_dtype, void* out,
                 uint8_t* out_scale, int64_t dst_bstride, void* stream) {
  return csk::compress_common("hca_compress", false, c, z, nullptr, nullptr, bias, nullptr, B, S,
                              D, m, entry0, src_bstride, d_rope, rope_base, entry_pos, in_dtype,
                              out_dtype, out, out_scale, dst_bstride, stream);
}

int mxfp4_quantize(const void* x, int in_dtype, int64_t rows, int cols, uint8_t* codes,
                   uint8_t* scales, void* stream) {
  csk::clear_error();
  const int rc = csk::check_quantize("mxfp4_quantize", x, in_dtype, rows, cols, codes, scales);
  if (rc != CSK_OK) return rc;
  if (rows == 0) return CSK_OK;
  if (const int dc = csk::check_device("mxfp4_quantize"); dc != CSK_OK) return dc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // aligned tensors: sixteen values per lane
  if ((reinterpret_cast<uintptr_t>(x) & 15) == 0 && (reinterpret_cast<uintptr_t>(codes) & 7) == 0) {
    const int64_t n16 = rows * (cols / 16);
    dim3 grid((unsigned)csk::ceil_div(n16, 256)), block(256);
    if (in_dtype == CSK_F32)
      return csk::launch("mxfp4_quantize", csk::mxfp4_quant16_kernel<float>, grid, block, 0, s,
                         reinterpret_cast<const float*>(x), n16, codes, scales);
    return csk::launch("mxfp4_quantize", csk::mxfp4_quant16_kernel<uint16_t>, grid, block, 0, s,
                       reinterpret_cast<const uint16_t*>(x), n16, codes, scales);
  }
  const int64_t total = rows * (cols / 2);
  dim3 grid((unsigned)csk::ceil_div(total, 256)), block(256);
  if (in_dtype == CSK_F32)
    return csk::launch("mxfp4_quantize", csk::mxfp4_quant_kernel<float>, grid, block, 0, s,
                       reinterpret_cast<const float*>(x), rows, cols, codes, scales);
  return csk::launch("mxfp4_quantize", csk::mxfp4_quant_kernel<uint16_t>, grid, block, 0, s,
                     reinterpret_cast<const uint16_t*>(x), rows, cols, codes, scales);
}

int csk_compress_batch(const csk_compress_job* jobs, int n_jobs, void* stream) {
  return csk::compress_batch(jobs, n_jobs, stream);
}

}  // extern "C"
