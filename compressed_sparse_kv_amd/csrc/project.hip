// project.hip - the KV series projected from hidden states and pooled into
// compressed entries in one matrix-core kernel, then RMS-normalised,
// rotated and encoded; and the standalone RMSNorm for queries.
//
// Page passages (DeepSeek-V4 technical report page, «Техотчёт DeepSeek-V4
// (2026): миллион токенов контекста»):
//   - «CSA: сжать в 4 раза и выбрать top-k», step 1: the two KV series C^a,
//     C^b and the two weight series Z^a, Z^b come from the hidden states;
//     every m = 4 tokens fold into one entry by a softmax over the weights
//     plus learned positional biases, the a and b windows overlapping (2m
//     sources per entry);
//   - «HCA: сжать в 128 раз…»: the same pooling over non-overlapping blocks
//     of m' = 128 tokens;
//   - «Muon и борьба с нестабильностью»: queries and KV entries normalised
//     directly by RMSNorm.
//
// Fused kernel: one workgroup (waves of 32 token rows, two per SIMD)
// computes a token x 64-channel tile of every series with bf16
// MFMAs (X W^T, fp32 accumulation), staged by LDS DMA in 64-deep K slabs
// like the plain matrix product, and pools it in its epilogue, so the
// series never reach memory:
//   - CSA (m = 4): 256 tokens (eight waves) x 64 channels x 4 series. The b
//     series is computed on the token rows shifted back by 4 (four extra
//     rows staged per slab), so the a slots (tokens 4j..4j+3) and b slots
//     (4j-4..4j-1) of entry j land in the same four accumulator rows of the
//     same lane: the 8-slot softmax runs in registers.
//   - HCA (m = 128): 128 tokens (one entry, four waves) x 64 channels x 2
//     series, so that 16K tokens make 256 workgroups; each lane folds its
//     16 rows, the two half-waves and then the four waves merge their (max,
//     sum, weighted sum) in a fixed order.
// The epilogue writes the pooled fp32 entry values and, per entry, the sum
// of squares of the block's channels; finalize_entries (compress.hip) then
// applies the RMSNorm (partials summed in ascending block order), RoPE and
// the output encoding.
#include "common.h"

namespace csk {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

#define CSK_P_VMCNT(n) ((((n) & 0xF) | ((((n) >> 4) & 0x3) << 14)) | (0x7 << 4))

struct ProjArgs {
  const uint16_t* x;   // token t of batch b at x + (b*src_bstride + t)*hidden
  const uint16_t* w;   // [NS, D, hidden]
  const float* bias_a;
  const float* bias_b;
  float* pooled;       // [B*N, D]
  float* ss;           // [B*N, ncb]
  int64_t src_bstride;
  int S, N, hidden, D, entry0, ncb;
};

constexpr int PK = 64;            // K slab depth
constexpr int PX = 64;            // CSA: eight more token rows (T0-8 .. T0-1)

namespace {

// 16 bytes per lane by LDS DMA into lds_base + 16*lane (a plain function:
// the builtin written inside a kernel template leaves the template without
// its host launch stub)
__device__ __forceinline__ void dma16(const void* src, uint4* lds_base) {
  __builtin_amdgcn_global_load_lds(src, lds_base, 16, 0, 0);
}

__device__ __forceinline__ float shfl_xor(float v, int mask) {
  const int l = (int)(threadIdx.x & 63);
  return __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (l ^ mask), __float_as_int(v)));
}

// Online-softmax state of one channel: running max, denominator, numerator.
struct Fold {
  float mx, den, num;
};

__device__ __forceinline__ Fold merge(Fold a, Fold b) {
  const float m = fmaxf(a.mx, b.mx);
  if (m == -INFINITY) return a;
  const float fa = a.mx == -INFINITY ? 0.f : expf(a.mx - m);
  const float fb = b.mx == -INFINITY ? 0.f : expf(b.mx - m);
  return Fold{m, a.den * fa + b.den * fb, a.num * fa + b.num * fb};
}

}  // namespace

template <bool CSA>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void project_compress_kernel(ProjArgs p) {
  constexpr int CH = 64;                // channels of a tile
  constexpr int NWV = CSA ? 8 : 4;      // waves
  constexpr int TT = 32 * NWV;          // token rows of a tile
  constexpr int NCT = CSA ? 8 : 4;      // 32-column tiles: CSA 4 series, HCA 2, of 64 channels
  constexpr int AU = TT * PK / 8;       // 16-byte units of the A (token) slab
  constexpr int BU = 32 * NCT * PK / 8; // of the B (weight) slab
  constexpr int XU = CSA ? PX : 0;
  static_assert(AU / 64 / NWV == 4 && BU / 64 / NWV == 4, "four DMA instructions per slab and wave");
  __shared__ __align__(16) uint4 lds[2][AU + BU + (CSA ? PX : 1)];  // [stage][A | B | A extra]
  const int tid = threadIdx.x, lane = tid & 63;
  // two waves per SIMD; wave w owns token rows 32w .. 32w+31 of the tile
  // and every column tile
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ntc = (p.D + CH - 1) / CH;
  const int total = ((p.S + TT - 1) / TT) * ntc;
  const int wg = blockIdx.x, xcd = wg & 7, per = total >> 3, rem = total & 7;
  const int L = xcd * per + min(xcd, rem) + (wg >> 3);
  const int tm = L / ntc, tc = L % ntc;
  const int T0 = TT * tm, c0 = CH * tc;
  const int b = blockIdx.y;
  const uint16_t* X = p.x + (int64_t)b * p.src_bstride * p.hidden;
  // lowest readable token row: the previous block (b series of the first
  // entry) exists in memory only when the call continues a sequence
  const int lo = (CSA && p.entry0 > 0) ? -4 : 0;

  for (int u = tid; u < 2 * (AU + BU + XU); u += 64 * NWV) {
    const int st = u / (AU + BU + XU), o = u % (AU + BU + XU);
    lds[st][o] = make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();

  // DMA sources. Slab unit (row, kc) at slab_unit(row, kc); lane l of
  // instruction i (0..3) fills unit 64*(4*wave + i) + l: row 32*wave + 8*i
  // + l/8, k chunk (l%8) ^ (row%8) ^ (row/8 % 2) = (l%8) ^ ((l/8)%8) ^ (i%2).
  const int kc_l = (lane & 7) ^ ((lane >> 3) & 7);
  const int r_base = 32 * wave + (lane >> 3);
  const uint16_t* pa[4];
  const uint16_t* pb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = r_base + 8 * i;
    const int kc = kc_l ^ (i & 1);
    pa[i] = X + (int64_t)min(max(T0 + r, lo), p.S - 1) * p.hidden + 8 * kc;
    const int s = r >> 6, c = r & 63;  // series, channel of weight row r
    pb[i] = p.w + ((int64_t)s * p.D + min(c0 + c, p.D - 1)) * p.hidden + 8 * kc;
  }
  const uint16_t* px = X + (int64_t)min(max(T0 - 8 + (lane >> 3), lo), p.S - 1) * p.hidden + 8 * kc_l;
  auto issue = [&](int kt, int st) {
    const int k0 = kt * PK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dma16(pa[i] + k0, &lds[st][64 * (4 * wave + i)]);
      dma16(pb[i] + k0, &lds[st][AU + 64 * (4 * wave + i)]);
    }
    if (CSA && wave == 0) dma16(px + k0, &lds[st][AU + BU]);
  };

  v16f acc[NCT];
#pragma unroll
  for (int j = 0; j < NCT; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;

  const int fr = lane & 31, fh = lane >> 5;
  constexpr int NA = CSA ? 2 : 1;  // A fragments per K-step (CSA: a rows, then b rows)
  const int nk = p.hidden / PK;
  issue(0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) {
      issue(kt + 1, st ^ 1);
      if (CSA && wave == 0) __builtin_amdgcn_s_waitcnt(CSK_P_VMCNT(9));
      else __builtin_amdgcn_s_waitcnt(CSK_P_VMCNT(8));
    } else {
      __builtin_amdgcn_s_waitcnt(CSK_P_VMCNT(0));
    }
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const uint4* sl = lds[st];
    v8bf af[2][NA], bfr[2][NCT];
    auto read_frags = [&](int ks, v8bf* fa, v8bf* fb) {
      const int kc = 2 * ks + fh;
      const int ra = 32 * wave + fr;
      fa[0] = __builtin_bit_cast(v8bf, sl[slab_unit(ra, kc)]);
      if (CSA) {
        // token T0 - 4 + ra: slab row ra - 4, or extra row ra + 4
        const int rb = ra - 4;
        const int u = rb >= 0 ? slab_unit(rb, kc) : AU + BU + slab_unit(rb + 8, kc);
        fa[1] = __builtin_bit_cast(v8bf, sl[u]);
      }
#pragma unroll
      for (int j = 0; j < NCT; ++j) {
        const int rw = 32 * j + fr;
        fb[j] = __builtin_bit_cast(v8bf, sl[AU + slab_unit(rw, kc)]);
      }
    };
    read_frags(0, af[0], bfr[0]);
#pragma unroll
    for (int ks = 0; ks < PK / 16; ++ks) {
      // CSA: column tiles 0-3 (C^a, Z^a) take the a rows, 4-7 (C^b, Z^b)
      // the shifted b rows; HCA: every tile (C 0-1, Z 2-3) takes the
      // block's rows. Half the products, then the next step's reads
      // (hidden by the other half).
#pragma unroll
      for (int j = 0; j < NCT / 2; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][0], bfr[ks & 1][j], acc[j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (ks + 1 < PK / 16) read_frags(ks + 1, af[(ks + 1) & 1], bfr[(ks + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = NCT / 2; j < NCT; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][CSA ? 1 : 0], bfr[ks & 1][j], acc[j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(CSK_P_VMCNT(63));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }

  // lane holds, per column tile j: column lane%32; rows 32*wave + 8*q +
  // 4*fh + e for element 4q + e
  const int64_t row0 = (int64_t)b * p.N;
  if (CSA) {
    // entry j = 8*wave + 2*q + fh of the tile: a slots at rows 4j..4j+3 of
    // tiles 0-3, b slots at the same rows of tiles 4-7
    float ba[2][4], bb[2][4];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int ch = min(c0 + 32 * ct + fr, p.D - 1);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ba[ct][e] = p.bias_a[e * p.D + ch];
        bb[ct][e] = p.bias_b[e * p.D + ch];
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int E = T0 / 4 + 8 * wave + 2 * q + fh;
      const bool has_b = (p.entry0 + E) > 0;
      float sq = 0.f;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const int ch = c0 + 32 * ct + fr;
        float l[8], v[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          l[e] = acc[2 + ct][4 * q + e] + ba[ct][e];
          v[e] = acc[ct][4 * q + e];
          l[4 + e] = has_b ? acc[6 + ct][4 * q + e] + bb[ct][e] : -INFINITY;
          v[4 + e] = acc[4 + ct][4 * q + e];
        }
        float mx = l[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mx = fmaxf(mx, l[e]);
        float den = 0.f, num = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = l[e] == -INFINITY ? 0.f : expf(l[e] - mx);
          den += x;
          num = fmaf(x, v[e], num);
        }
        const float pv = num / den;
        if (ch < p.D) {
          sq = fmaf(pv, pv, sq);
          if (E < p.N) p.pooled[(row0 + E) * p.D + ch] = pv;
        }
      }
      // the entry's sum over this block's 64 channels: the 32 lanes of
      // this half-wave, in a fixed butterfly order
#pragma unroll
      for (int mk = 1; mk < 32; mk <<= 1) sq += shfl_xor(sq, mk);
      if (fr == 0 && E < p.N) p.ss[(row0 + E) * p.ncb + tc] = sq;
    }
  } else {
    // the tile is one entry (128 rows: the four waves); this lane's 16 rows
    // of it: 32*wave + 8*q + 4*fh + e. Column tiles: C^a 0..CTN-1, Z^a
    // CTN..2*CTN-1.
    constexpr int CTN = NCT / 2;  // 32-channel tiles
    const int k = 0, wq = wave;
    const int E = T0 / 128;
    Fold fo[CTN];
#pragma unroll
    for (int ct = 0; ct < CTN; ++ct) {
      const int ch = min(c0 + 32 * ct + fr, p.D - 1);
      float mx = -INFINITY;
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int rr = 32 * wq + 8 * q + 4 * fh + e;
          mx = fmaxf(mx, acc[CTN + ct][4 * q + e] + p.bias_a[rr * p.D + ch]);
        }
      float den = 0.f, num = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int rr = 32 * wq + 8 * q + 4 * fh + e;
          const float x = expf(acc[CTN + ct][4 * q + e] + p.bias_a[rr * p.D + ch] - mx);
          den += x;
          num = fmaf(x, acc[ct][4 * q + e], num);
        }
      // the two half-waves (rows 4*fh + ...), merged low half first
      const Fold mine{mx, den, num};
      const Fold other{shfl_xor(mx, 32), shfl_xor(den, 32), shfl_xor(num, 32)};
      fo[ct] = fh == 0 ? merge(mine, other) : merge(other, mine);
    }
    // the four waves of the entry through LDS (the slabs are free), merged
    // in wave order
    float* xf = reinterpret_cast<float*>(&lds[0][0]);
    if (wq != 0 && fh == 0)
#pragma unroll
      for (int ct = 0; ct < CTN; ++ct) {
        const int o = (((k * 3 + wq - 1) * CTN + ct) * 32 + fr) * 3;
        xf[o] = fo[ct].mx;
        xf[o + 1] = fo[ct].den;
        xf[o + 2] = fo[ct].num;
      }
    __syncthreads();
    if (wq == 0) {
      float sq = 0.f;
#pragma unroll
      for (int ct = 0; ct < CTN; ++ct) {
        Fold f = fo[ct];
#pragma unroll
        for (int w2 = 1; w2 < 4; ++w2) {
          const int o = (((k * 3 + w2 - 1) * CTN + ct) * 32 + fr) * 3;
          f = merge(f, Fold{xf[o], xf[o + 1], xf[o + 2]});
        }
        const float pv = f.num / f.den;
        const int ch = c0 + 32 * ct + fr;
        if (ch < p.D) {
          sq = fmaf(pv, pv, sq);
          if (fh == 0 && E < p.N) p.pooled[(row0 + E) * p.D + ch] = pv;
        }
      }
#pragma unroll
      for (int mk = 1; mk < 32; mk <<= 1) sq += shfl_xor(sq, mk);
      if (lane == 0 && E < p.N) p.ss[(row0 + E) * p.ncb + tc] = sq;
    }
  }
}

// RMSNorm of rows of D values: one wave per row, lane c takes channels
// c, c+64, ...; the sum of squares in fp32 (each lane in ascending channel
// order, then a fixed butterfly), y = x * gamma / sqrt(mean(x^2) + eps).
template <typename IN, typename OUT>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const IN* x, const float* gamma, int64_t rows, int D,
                                                      float eps, OUT* y) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;
  const IN* xr = x + r * D;
  float ss = 0.f;
  for (int c = lane; c < D; c += 64) {
    const float v = io<IN>::load1(xr + c);
    ss = fmaf(v, v, ss);
  }
#pragma unroll
  for (int mk = 1; mk < 64; mk <<= 1) ss += shfl_xor(ss, mk);
  const float inv = 1.0f / sqrtf(ss / (float)D + eps);
  OUT* yr = y + r * D;
  for (int c = lane; c < D; c += 64) io<OUT>::store1(yr + c, io<IN>::load1(xr + c) * inv * gamma[c]);
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace csk

using namespace csk;

extern "C" size_t project_compress_workspace_size(int csa, int B, int S, int D, int m) {
  if (B <= 0 || S <= 0 || D <= 0 || m <= 0 || S / m == 0) return 0;
  const int64_t n = (int64_t)B * (S / m);
  const int ncb = (int)ceil_div(D, 64);
  return (size_t)(ceil_div(n * D * 4, 256) * 256 + n * ncb * 4);
}

extern "C" int project_compress(int csa, const void* x, const void* w, const float* bias_a, const float* bias_b,
                                const float* gamma, float eps, int B, int S, int hidden, int D, int m, int entry0,
                                int64_t src_bstride, int d_rope, float rope_base, const int32_t* entry_pos,
                                int out_dtype, void* out, uint8_t* out_scale, int64_t dst_bstride, void* workspace,
                                size_t ws_bytes, void* stream) {
  clear_error();
  const std::string f = "project_compress";
  if (B < 0 || S < 0 || hidden <= 0 || D <= 0 || entry0 < 0 || !(eps >= 0.f))
    return fail(CSK_EINVAL, f + ": need B, S >= 0, hidden, D > 0, entry0 >= 0, eps >= 0");
  if ((csa && m != 4) || (!csa && m != 128))
    return fail(CSK_EUNSUPPORTED, f + ": built for CSA with m = 4 and HCA with m = 128");
  if (hidden % 64 || D % 32)
    return fail(CSK_EUNSUPPORTED, f + ": built for hidden a multiple of 64 and D a multiple of 32");
  if (d_rope < 0 || d_rope > D || (d_rope & 1) || d_rope > 2 * MAX_ROPE_PAIRS)
    return fail(CSK_EINVAL, f + ": d_rope must be even, <= D and <= 128");
  if (out_dtype != CSK_F32 && out_dtype != CSK_BF16 && out_dtype != CSK_MXFP4 && out_dtype != CSK_FP8KV)
    return fail(CSK_EUNSUPPORTED, f + ": out_dtype must be CSK_F32, CSK_BF16, CSK_MXFP4 or CSK_FP8KV");
  if (out_dtype == CSK_FP8KV && (D - d_rope) % 32)
    return fail(CSK_EINVAL, f + ": FP8KV output needs (D - d_rope) % 32 == 0");
  const int N = S / m;
  if (src_bstride < 0 || (src_bstride != 0 && src_bstride < S))
    return fail(CSK_EINVAL, f + ": src_bstride must be 0 or >= S");
  if (dst_bstride < 0 || (dst_bstride != 0 && dst_bstride < N))
    return fail(CSK_EINVAL, f + ": dst_bstride must be 0 or >= S/m");
  if (B == 0 || N == 0) return CSK_OK;
  if (!x || !w || !bias_a || (csa && !bias_b) || !out || !workspace || (out_dtype == CSK_MXFP4 && !out_scale))
    return fail(CSK_EINVAL, f + ": null pointer");
  if (!aligned16(x) || !aligned16(w) || !aligned16(workspace))
    return fail(CSK_EINVAL, f + ": x, w and workspace must be 16-byte aligned");
  if (ws_bytes < project_compress_workspace_size(csa, B, S, D, m))
    return fail(CSK_EWORKSPACE, f + ": workspace smaller than project_compress_workspace_size()");
  if (const int dc = check_device(f); dc != CSK_OK) return dc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int CH = 64;  // channels of a tile (both forms)
  ProjArgs a{};
  a.x = reinterpret_cast<const uint16_t*>(x);
  a.w = reinterpret_cast<const uint16_t*>(w);
  a.bias_a = bias_a;
  a.bias_b = bias_b;
  a.pooled = reinterpret_cast<float*>(workspace);
  a.ncb = (int)ceil_div(D, CH);
  a.ss = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) +
                                  ceil_div((int64_t)B * N * D * 4, 256) * 256);
  a.src_bstride = src_bstride ? src_bstride : S;
  a.S = S; a.N = N; a.hidden = hidden; a.D = D; a.entry0 = entry0;
  // CSA: 256-token tiles, eight waves; HCA: 128-token tiles (one entry),
  // four waves
  const dim3 grid((unsigned)(ceil_div(S, csa ? 256 : 128) * a.ncb), (unsigned)B);
  const int rc = csa ? launch("csa_project_pool", project_compress_kernel<true>, grid, dim3(512), 0, s, a)
                     : launch("hca_project_pool", project_compress_kernel<false>, grid, dim3(256), 0, s, a);
  if (rc != CSK_OK) return rc;
  return finalize_entries(csa ? "csa_project_finalize" : "hca_project_finalize", B, N, D, m, entry0, d_rope,
                          rope_base, entry_pos, out_dtype, out, out_scale, dst_bstride, a.pooled, a.ss, a.ncb,
                          gamma, eps, s);
}

extern "C" int rmsnorm(const void* x, const float* gamma, int64_t rows, int D, float eps, int in_dtype,
                       int out_dtype, void* y, void* stream) {
  clear_error();
  const std::string f = "rmsnorm";
  if (rows < 0 || D <= 0 || !(eps >= 0.f)) return fail(CSK_EINVAL, f + ": need rows >= 0, D > 0, eps >= 0");
  if ((in_dtype != CSK_F32 && in_dtype != CSK_BF16) || (out_dtype != CSK_F32 && out_dtype != CSK_BF16))
    return fail(CSK_EUNSUPPORTED, f + ": dtypes must be CSK_F32 or CSK_BF16");
  if (rows == 0) return CSK_OK;
  if (!x || !gamma || !y) return fail(CSK_EINVAL, f + ": null pointer");
  if (const int dc = check_device(f); dc != CSK_OK) return dc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)ceil_div(rows, 4)), block(256);
  if (in_dtype == CSK_BF16) {
    const uint16_t* xi = reinterpret_cast<const uint16_t*>(x);
    return out_dtype == CSK_BF16
               ? launch("rmsnorm", rmsnorm_kernel<uint16_t, uint16_t>, grid, block, 0, s, xi, gamma, rows, D, eps,
                        reinterpret_cast<uint16_t*>(y))
               : launch("rmsnorm", rmsnorm_kernel<uint16_t, float>, grid, block, 0, s, xi, gamma, rows, D, eps,
                        reinterpret_cast<float*>(y));
  }
  const float* xi = reinterpret_cast<const float*>(x);
  return out_dtype == CSK_BF16
             ? launch("rmsnorm", rmsnorm_kernel<float, uint16_t>, grid, block, 0, s, xi, gamma, rows, D, eps,
                      reinterpret_cast<uint16_t*>(y))
             : launch("rmsnorm", rmsnorm_kernel<float, float>, grid, block, 0, s, xi, gamma, rows, D, eps,
                      reinterpret_cast<float*>(y));
}
