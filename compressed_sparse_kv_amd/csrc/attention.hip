// attention.hip - CSA sparse and HCA dense MQA attention over compressed KV
// entries plus a sliding window and an attention sink, on gfx950.
//
// [P1] «CSA: сжать в 4 раза и выбрать top-k», step 3: every compressed
// entry is both key and value for all query heads (MQA). «HCA: сжать в 128
// раз…»: dense attention over the compressed entries and a 128-token window
// of uncompressed tokens. [P4]: SWA branch, attention sink, partial RoPE on
// the last dims. One softmax runs over the union of candidates and the sink.
//
// Candidate index space of a query row: [0, Lc) compressed slots (sparse:
// the k selected indices; dense: entries 0..Nmax-1, masked past the visible
// count) followed by [0, W) window slots (window rows wr0.. of that row).
// Invalid slots are masked. The space is split into chunks; each chunk of
// each row is one workgroup, and chunks are merged by log-sum-exp.
//
// bf16 path: one wave per 16 heads of one query token (all heads of a
// token in one workgroup, so a gathered KV tile in LDS serves every head).
// Per tile of 32 candidates:
//   S^T[cand, head] = K[cand, :] . q~[head, :]  (16x16x32 bf16 MFMA; the K
//     fragment is a 16-byte LDS read of one candidate row, the rotated query
//     fragments stay in registers for the whole chunk),
//   online softmax in the log2 domain per head (one head per lane column),
//   O^T[dv, head] += V^T[dv, cand] . P^T[cand, head]  (the P^T fragment is
//     the lane's own 8 probabilities: candidate order inside the MFMA's K
//     slot is chosen to match the S^T output layout, so no shuffle is
//     needed; the V^T fragment is gathered from the row-major LDS tile).
#include <math.h>

#include "common.h"

namespace csk {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

struct AttnArgs {
  const void* q;          // [R, H, D]
  const int32_t* q_pos;   // [R]
  const void* kv_c;       // [B, Nmax, D]
  const int32_t* idx;     // sparse: [R, k]
  const int32_t* n_entries;  // dense: [B]
  const void* kv_w;       // [B, S_w, D]
  const int32_t* w_pos0;  // [B]
  const float* sink;      // [H] or null
  int B, T, H, D, dv, d_rope, Nmax, k, m, S_w, W;
  int Lc;                 // compressed slots per row
  int chunk, nch;         // candidates per chunk, chunks per row
  float scale;
  double base;
  bool dense;
  void* out;              // [R, H, dv]
  float* lse;             // [R, H] or null
  float* part_o;          // [R, nch, H, dv]
  float* part_ml;         // [R, nch, H, 2]
};

struct RowInfo {
  int b;
  int64_t p;
  int nvis;      // dense: visible compressed entries
  int wr0, wr1;  // window rows [wr0, wr1)
};

__device__ __forceinline__ RowInfo row_info(const AttnArgs& a, int r) {
  RowInfo ri;
  ri.b = r / a.T;
  ri.p = a.q_pos[r];
  ri.nvis = 0;
  if (a.dense && ri.p >= 0) {
    int64_t nv = (ri.p + 1) / a.m;
    nv = nv < a.n_entries[ri.b] ? nv : a.n_entries[ri.b];
    nv = nv < a.Nmax ? nv : a.Nmax;
    ri.nvis = (int)(nv < 0 ? 0 : nv);
  }
  ri.wr0 = ri.wr1 = 0;
  if (a.W > 0 && a.S_w > 0) {
    int64_t lo = ri.p - a.W + 1;
    lo = lo < 0 ? 0 : lo;
    const int64_t w0 = a.w_pos0[ri.b];
    int64_t r0 = lo - w0, r1 = ri.p - w0 + 1;
    r0 = r0 < 0 ? 0 : r0;
    r1 = r1 > a.S_w ? a.S_w : r1;
    if (r1 > r0) {
      ri.wr0 = (int)r0;
      ri.wr1 = (int)r1;
    }
  }
  return ri;
}

// Element offset of candidate slot j's KV row, or -1 when the slot is empty.
// Window rows are returned as offsets into kv_w tagged by *is_win.
__device__ __forceinline__ int64_t slot_row(const AttnArgs& a, const RowInfo& ri, int r, int j,
                                            bool* is_win) {
  *is_win = false;
  if (j < a.Lc) {
    int e;
    if (a.dense) {
      if (j >= ri.nvis) return -1;
      e = j;
    } else {
      e = a.idx[(int64_t)r * a.k + j];
      if (e < 0 || e >= a.Nmax) return -1;
    }
    return ((int64_t)ri.b * a.Nmax + e) * a.D;
  }
  const int wrow = ri.wr0 + (j - a.Lc);
  if (wrow >= ri.wr1) return -1;
  *is_win = true;
  return ((int64_t)ri.b * a.S_w + wrow) * a.D;
}

// Final normalisation with the sink: (m, l) in log2 units.
__device__ __forceinline__ void finish_row(float m, float l, const float* sink, int h, float* M,
                                           float* inv_z, float* lse) {
  float s2 = sink ? sink[h] * LOG2E : -INFINITY;
  float mm = fmaxf(m, s2);
  if (mm == -INFINITY) {
    *M = 0.f;
    *inv_z = 0.f;
    *lse = -INFINITY;
    return;
  }
  float z = (m == -INFINITY ? 0.f : l * exp2f(m - mm)) + (sink ? exp2f(s2 - mm) : 0.f);
  *M = mm;
  *inv_z = 1.0f / z;
  *lse = (mm + log2f(z)) * LN2;
}

// ------------------------------------------------------------- bf16 MFMA
template <int D, int DV>
__global__ __launch_bounds__(256) void attn_bf16_kernel(AttnArgs a) {
  constexpr int KS = D / 32;        // MFMA K-steps over the key dim
  constexpr int DT = DV / 16;       // 16-row tiles of the value dim
  constexpr int LD = D + 8;         // LDS row stride in bf16 (16 bytes of padding)
  __shared__ __align__(16) uint16_t tile[32 * LD];

  const int r = blockIdx.x;
  const int chunk_id = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nthr = blockDim.x;
  const int col = lane & 15, g = lane >> 4;
  const int h = wave * 16 + col;
  const RowInfo ri = row_info(a, r);

  // rotated query fragments (B operand of S^T): dims 32*ks + 8*g .. +7
  v8bf qf[KS];
  {
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)r * a.H + h) * D;
    const int rope0 = D - a.d_rope;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int d0 = 32 * ks + 8 * g;
      const uint4 raw = *reinterpret_cast<const uint4*>(qrow + d0);
      float x[8];
      const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = bf16_bits_to_f32(wv[i] & 0xffffu);
        x[2 * i + 1] = bf16_bits_to_f32(wv[i] >> 16);
      }
      if (d0 + 8 > rope0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = d0 + 2 * i;
          if (c >= rope0) {
            float cs, sn;
            rope_cs((double)ri.p, (c - rope0) / 2, a.d_rope, a.base, &cs, &sn);
            const float x0 = x[2 * i], x1 = x[2 * i + 1];
            x[2 * i] = x0 * cs - x1 * sn;
            x[2 * i + 1] = x0 * sn + x1 * cs;
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) qf[ks][i] = __builtin_bit_cast(__bf16, (uint16_t)f32_to_bf16_bits(x[i]));
    }
  }

  v4f acc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_part = 0.f;
  const float sl2 = a.scale * LOG2E;

  const int c0 = chunk_id * a.chunk;
  int c1 = c0 + a.chunk;
  const int total = a.Lc + a.W;
  c1 = c1 < total ? c1 : total;

  for (int t0 = c0; t0 < c1; t0 += 32) {
    // gather 32 candidate rows into LDS (invalid rows are zero)
    __syncthreads();
    constexpr int CPR = D / 8;  // 16-byte chunks per row
    for (int id = threadIdx.x; id < 32 * CPR; id += nthr) {
      const int row = id / CPR, cc = id % CPR;
      const int j = t0 + row;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (j < c1) {
        bool win;
        const int64_t off = slot_row(a, ri, r, j, &win);
        if (off >= 0) {
          const uint16_t* src = reinterpret_cast<const uint16_t*>(win ? a.kv_w : a.kv_c) + off;
          v = *reinterpret_cast<const uint4*>(src + 8 * cc);
        }
      }
      *reinterpret_cast<uint4*>(&tile[row * LD + 8 * cc]) = v;
    }
    __syncthreads();

    // S^T for two 16-candidate tiles
    v4f s[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      s[ct] = v4f{0.f, 0.f, 0.f, 0.f};
      const uint16_t* krow = &tile[(ct * 16 + col) * LD + 8 * g];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const v8bf kfrag = *reinterpret_cast<const v8bf*>(krow + 32 * ks);
        s[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfrag, qf[ks], s[ct], 0, 0, 0);
      }
    }
    // mask + scale: lane holds candidates 4g+i (tile 0) and 16+4g+i (tile 1)
    float p[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = t0 + ct * 16 + 4 * g + i;
        bool win;
        const bool ok = j < c1 && slot_row(a, ri, r, j, &win) >= 0;
        const float v = ok ? s[ct][i] * sl2 : -INFINITY;
        p[ct * 4 + i] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = (m_new == -INFINITY) ? 0.f : exp2f(p[i] - m_new);
      psum += p[i];
    }
    l_part = l_part * alpha + psum;
    m_run = m_new;
    v8bf pf;
#pragma unroll
    for (int i = 0; i < 8; ++i) pf[i] = __builtin_bit_cast(__bf16, (uint16_t)f32_to_bf16_bits(p[i]));

    // O^T += V^T P^T; V^T fragment: dv row 16*dt+col, candidates of slot j
    const int cand0 = 4 * g, cand1 = 16 + 4 * g;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int dvr = 16 * dt + col;
      v8bf vf;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vf[i] = __builtin_bit_cast(__bf16, tile[(cand0 + i) * LD + dvr]);
        vf[4 + i] = __builtin_bit_cast(__bf16, tile[(cand1 + i) * LD + dvr]);
      }
      acc[dt] *= alpha;
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, acc[dt], 0, 0, 0);
    }
  }

  // per-head totals across the four lane groups
  float l_tot = l_part;
  l_tot += __shfl_xor(l_tot, 16);
  l_tot += __shfl_xor(l_tot, 32);

  if (a.nch == 1) {
    float M, inv_z, lse;
    finish_row(m_run, l_tot, a.sink, h, &M, &inv_z, &lse);
    const float f = (m_run == -INFINITY) ? 0.f : exp2f(m_run - M) * inv_z;
    uint16_t* ob = reinterpret_cast<uint16_t*>(a.out) + ((int64_t)r * a.H + h) * DV;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d0 = 16 * dt + 4 * g;
      const uint32_t lo = f32_to_bf16_bits(acc[dt][0] * f) | (f32_to_bf16_bits(acc[dt][1] * f) << 16);
      const uint32_t hi = f32_to_bf16_bits(acc[dt][2] * f) | (f32_to_bf16_bits(acc[dt][3] * f) << 16);
      *reinterpret_cast<uint2*>(ob + d0) = make_uint2(lo, hi);
    }
    if (a.lse && g == 0) a.lse[(int64_t)r * a.H + h] = lse;
  } else {
    float* po = a.part_o + (((int64_t)r * a.nch + chunk_id) * a.H + h) * DV;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<float4*>(po + 16 * dt + 4 * g) =
          make_float4(acc[dt][0], acc[dt][1], acc[dt][2], acc[dt][3]);
    if (g == 0) {
      float* pm = a.part_ml + (((int64_t)r * a.nch + chunk_id) * a.H + h) * 2;
      pm[0] = m_run;
      pm[1] = l_tot;
    }
  }
}

// ------------------------------------------------------------ VALU path
// One wave per (row, head): 64 candidates at a time, each lane one
// candidate; online softmax in fp32; lane c accumulates value channels
// c, c+64, ... Handles fp32 and bf16 data of any shape.
template <typename T>
__device__ __forceinline__ float ld(const T* p, int64_t i);
template <>
__device__ __forceinline__ float ld<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_bits_to_f32(p[i]);
}

template <typename T>
__global__ __launch_bounds__(64) void attn_valu_kernel(AttnArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* qr = reinterpret_cast<float*>(smem);        // [D]
  float* pr = qr + a.D;                              // [64]
  int64_t* rows = reinterpret_cast<int64_t*>(pr + 64);  // [64]
  const int r = blockIdx.x;
  const int h = blockIdx.y % a.H;
  const int chunk_id = blockIdx.y / a.H;
  const int lane = threadIdx.x;
  const RowInfo ri = row_info(a, r);
  const T* q = reinterpret_cast<const T*>(a.q) + ((int64_t)r * a.H + h) * a.D;
  const int rope0 = a.D - a.d_rope;
  for (int c = 2 * lane; c < a.D; c += 128) {
    float x0 = ld(q, c), x1 = ld(q, c + 1);
    if (c >= rope0) {
      float cs, sn;
      rope_cs((double)ri.p, (c - rope0) / 2, a.d_rope, a.base, &cs, &sn);
      const float y0 = x0 * cs - x1 * sn, y1 = x0 * sn + x1 * cs;
      x0 = y0;
      x1 = y1;
    }
    qr[c] = x0;
    qr[c + 1] = x1;
  }
  __syncthreads();
  const int nacc = (a.dv + 63) / 64;
  float accv[9];  // dv <= 576
  for (int i = 0; i < 9; ++i) accv[i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const int c0 = chunk_id * a.chunk;
  int c1 = c0 + a.chunk;
  c1 = c1 < a.Lc + a.W ? c1 : a.Lc + a.W;
  const float sl2 = a.scale * LOG2E;
  for (int t0 = c0; t0 < c1; t0 += 64) {
    const int j = t0 + lane;
    float logit = -INFINITY;
    int64_t off = -1;
    bool win = false;
    if (j < c1) off = slot_row(a, ri, r, j, &win);
    rows[lane] = off < 0 ? -1 : (win ? -(off + 2) : off);
    if (off >= 0) {
      const T* kr = reinterpret_cast<const T*>(win ? a.kv_w : a.kv_c) + off;
      float dot = 0.f;
      for (int c = 0; c < a.D; ++c) dot = fmaf(qr[c], ld(kr, c), dot);
      logit = dot * sl2;
    }
    float tmax = logit;
    for (int o = 32; o >= 1; o >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, o));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_run - m_new);
    const float pj = m_new == -INFINITY ? 0.f : exp2f(logit - m_new);
    float ps = pj;
    for (int o = 32; o >= 1; o >>= 1) ps += __shfl_xor(ps, o);
    l_run = l_run * alpha + ps;
    m_run = m_new;
    pr[lane] = pj;
    __syncthreads();
    for (int i = 0; i < nacc; ++i) accv[i] *= alpha;
    const int nj = min(64, c1 - t0);
    for (int jj = 0; jj < nj; ++jj) {
      const int64_t code = rows[jj];
      if (code == -1) continue;
      const bool w2 = code < -1;
      const int64_t o2 = w2 ? -(code + 2) : code;
      const T* vr = reinterpret_cast<const T*>(w2 ? a.kv_w : a.kv_c) + o2;
      const float pp = pr[jj];
      for (int i = 0; i < nacc; ++i) {
        const int c = lane + 64 * i;
        if (c < a.dv) accv[i] = fmaf(pp, ld(vr, c), accv[i]);
      }
    }
    __syncthreads();
  }
  if (a.nch == 1) {
    float M, inv_z, lse;
    finish_row(m_run, l_run, a.sink, h, &M, &inv_z, &lse);
    const float f = (m_run == -INFINITY) ? 0.f : exp2f(m_run - M) * inv_z;
    for (int i = 0; i < nacc; ++i) {
      const int c = lane + 64 * i;
      if (c >= a.dv) continue;
      const int64_t o = ((int64_t)r * a.H + h) * a.dv + c;
      if (sizeof(T) == 4) reinterpret_cast<float*>(a.out)[o] = accv[i] * f;
      else reinterpret_cast<uint16_t*>(a.out)[o] = (uint16_t)f32_to_bf16_bits(accv[i] * f);
    }
    if (a.lse && lane == 0) a.lse[(int64_t)r * a.H + h] = lse;
  } else {
    float* po = a.part_o + (((int64_t)r * a.nch + chunk_id) * a.H + h) * a.dv;
    for (int i = 0; i < nacc; ++i) {
      const int c = lane + 64 * i;
      if (c < a.dv) po[c] = accv[i];
    }
    if (lane == 0) {
      float* pm = a.part_ml + (((int64_t)r * a.nch + chunk_id) * a.H + h) * 2;
      pm[0] = m_run;
      pm[1] = l_run;
    }
  }
}

// ---------------------------------------------------------------- merge
// One workgroup per (row, head): log-sum-exp combination of the chunks'
// partial (m, l, o) with the sink.
template <typename T>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
  const int r = blockIdx.x, h = blockIdx.y;
  float m = -INFINITY;
  for (int c = 0; c < a.nch; ++c)
    m = fmaxf(m, a.part_ml[(((int64_t)r * a.nch + c) * a.H + h) * 2]);
  float l = 0.f;
  for (int c = 0; c < a.nch; ++c) {
    const float* pm = a.part_ml + (((int64_t)r * a.nch + c) * a.H + h) * 2;
    if (pm[0] != -INFINITY) l += pm[1] * exp2f(pm[0] - m);
  }
  float M, inv_z, lse;
  finish_row(m, l, a.sink, h, &M, &inv_z, &lse);
  for (int d = threadIdx.x; d < a.dv; d += blockDim.x) {
    float o = 0.f;
    for (int c = 0; c < a.nch; ++c) {
      const float mc = a.part_ml[(((int64_t)r * a.nch + c) * a.H + h) * 2];
      if (mc == -INFINITY) continue;
      o += a.part_o[(((int64_t)r * a.nch + c) * a.H + h) * a.dv + d] * exp2f(mc - M);
    }
    o *= inv_z;
    const int64_t oi = ((int64_t)r * a.H + h) * a.dv + d;
    if (sizeof(T) == 4) reinterpret_cast<float*>(a.out)[oi] = o;
    else reinterpret_cast<uint16_t*>(a.out)[oi] = (uint16_t)f32_to_bf16_bits(o);
  }
  if (a.lse && threadIdx.x == 0) a.lse[(int64_t)r * a.H + h] = lse;
}

// ------------------------------------------------------------ host side
struct AttnPlan {
  int chunk, nch;
  bool mfma;
  size_t off_o, off_ml, total;
};

static bool mfma_shape(int H, int D, int dv, int dtype) {
  if (dtype != CSK_BF16 || H % 16 || H > 64) return false;
  return (D == 576 && (dv == 512 || dv == 576)) || (D == 128 && dv == 128) ||
         (D == 64 && dv == 64) || (D == 256 && dv == 256);
}

static AttnPlan plan_attn(int B, int T, int H, int D, int dv, int Lc, int W, int dtype) {
  AttnPlan p{};
  const int64_t R = (int64_t)B * T;
  const int total = Lc + W;
  p.mfma = mfma_shape(H, D, dv, dtype);
  const int gran = p.mfma ? 32 : 64;
  int64_t want = ceil_div(R * (int64_t)total, 256);  // aim at ~256 workgroups
  int64_t ch = ceil_div(want < 128 ? 128 : want, gran) * gran;
  if (ch >= total) ch = ceil_div(total > 0 ? total : 1, gran) * gran;
  p.chunk = (int)ch;
  p.nch = (int)ceil_div(total > 0 ? total : 1, ch);
  size_t o = 0;
  if (p.nch > 1) {
    p.off_o = o;
    o += (size_t)R * p.nch * H * dv * 4;
    o = (o + 255) & ~(size_t)255;
    p.off_ml = o;
    o += (size_t)R * p.nch * H * 2 * 4;
    o = (o + 255) & ~(size_t)255;
  }
  p.total = o;
  return p;
}

static int attn_common(const char* fn, bool dense, const void* q, const int32_t* q_pos,
                       const void* kv_c, int Nmax, const int32_t* idx, int k,
                       const int32_t* n_entries, int m, const void* kv_w,
                       const int32_t* w_pos0, int S_w, int W, const float* sink, int B, int T,
                       int H, int D, int dv, int d_rope, float rope_base, float scale, int dtype,
                       void* out, float* lse, void* workspace, size_t ws_bytes, void* stream) {
  clear_error();
  std::string f(fn);
  if (!q || !q_pos || !kv_c || !out) return fail(CSK_EINVAL, f + ": null pointer");
  if (!dense && !idx) return fail(CSK_EINVAL, f + ": null idx");
  if (dense && !n_entries) return fail(CSK_EINVAL, f + ": null n_entries");
  if (B <= 0 || T <= 0 || H <= 0 || D <= 0 || (D & 1) || dv <= 0 || dv > D || Nmax <= 0)
    return fail(CSK_EINVAL, f + ": need positive B, T, H, Nmax, even D and 0 < dv <= D");
  if (d_rope < 0 || d_rope > D || (d_rope & 1)) return fail(CSK_EINVAL, f + ": bad d_rope");
  if (W < 0 || S_w < 0 || (S_w > 0 && (!kv_w || !w_pos0)))
    return fail(CSK_EINVAL, f + ": bad window arguments");
  if (!dense && k < 0) return fail(CSK_EINVAL, f + ": k must be >= 0");
  if (dense && m <= 0) return fail(CSK_EINVAL, f + ": m must be > 0");
  if (dtype != CSK_BF16 && dtype != CSK_F32)
    return fail(CSK_EUNSUPPORTED, f + ": dtype must be CSK_BF16 or CSK_F32");
  if (dv > 576) return fail(CSK_EUNSUPPORTED, f + ": dv > 576 not built");
  const int Wslots = S_w > 0 ? W : 0;
  const int Lc = dense ? Nmax : k;
  AttnPlan p = plan_attn(B, T, H, D, dv, Lc, Wslots, dtype);
  if (p.nch > 65535 || (int64_t)p.nch * H > 65535 || (int64_t)B * T > (1LL << 30))
    return fail(CSK_EUNSUPPORTED, f + ": problem too large");
  if (p.total > 0 && (!workspace || ws_bytes < p.total))
    return fail(CSK_EWORKSPACE, f + ": workspace smaller than the *_workspace_size() value");
  AttnArgs a{};
  a.q = q; a.q_pos = q_pos; a.kv_c = kv_c; a.idx = idx; a.n_entries = n_entries;
  a.kv_w = kv_w; a.w_pos0 = w_pos0; a.sink = sink;
  a.B = B; a.T = T; a.H = H; a.D = D; a.dv = dv; a.d_rope = d_rope; a.Nmax = Nmax; a.k = k;
  a.m = m; a.S_w = S_w; a.W = Wslots; a.Lc = Lc; a.chunk = p.chunk; a.nch = p.nch;
  a.scale = scale; a.base = (double)rope_base; a.dense = dense;
  a.out = out; a.lse = lse;
  char* ws = reinterpret_cast<char*>(workspace);
  a.part_o = p.nch > 1 ? reinterpret_cast<float*>(ws + p.off_o) : nullptr;
  a.part_ml = p.nch > 1 ? reinterpret_cast<float*>(ws + p.off_ml) : nullptr;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const unsigned R = (unsigned)(B * T);
  int rc;
  if (p.mfma) {
    dim3 grid(R, p.nch), block(64 * (H / 16));
#define CSK_ATT_CASE(d, v) \
  if (D == d && dv == v)     \
    rc = launch(dense ? "attn_bf16_dense" : "attn_bf16_sparse", attn_bf16_kernel<d, v>, grid, block, 0, s, a);
    rc = CSK_EUNSUPPORTED;
    CSK_ATT_CASE(576, 512) CSK_ATT_CASE(576, 576) CSK_ATT_CASE(128, 128) CSK_ATT_CASE(64, 64)
    CSK_ATT_CASE(256, 256)
#undef CSK_ATT_CASE
  } else {
    dim3 grid(R, p.nch * H), block(64);
    const size_t lds = (size_t)D * 4 + 64 * 4 + 64 * 8;
    rc = dtype == CSK_F32 ? launch("attn_valu", attn_valu_kernel<float>, grid, block, lds, s, a)
                          : launch("attn_valu", attn_valu_kernel<uint16_t>, grid, block, lds, s, a);
  }
  if (rc != CSK_OK || p.nch == 1) return rc;
  dim3 mg(R, H), mb(256);
  return dtype == CSK_F32 ? launch("attn_merge", attn_merge_kernel<float>, mg, mb, 0, s, a)
                          : launch("attn_merge", attn_merge_kernel<uint16_t>, mg, mb, 0, s, a);
}

}  // namespace csk

extern "C" {

size_t sparse_attn_workspace_size(int B, int T, int H, int D, int dv, int k, int W, int dtype) {
  if (B <= 0 || T <= 0 || H <= 0 || D <= 0 || dv <= 0 || k < 0 || W < 0) return 0;
  return csk::plan_attn(B, T, H, D, dv, k, W, dtype).total;
}

size_t dense_compressed_attn_workspace_size(int B, int T, int H, int D, int dv, int Nmax, int m,
                                            int W, int dtype) {
  (void)m;
  if (B <= 0 || T <= 0 || H <= 0 || D <= 0 || dv <= 0 || Nmax <= 0 || W < 0) return 0;
  return csk::plan_attn(B, T, H, D, dv, Nmax, W, dtype).total;
}

int sparse_attn(const void* q, const int32_t* q_pos, const void* kv_c, int Nmax,
                const int32_t* idx, int k, const void* kv_w, const int32_t* w_pos0, int S_w,
                int W, const float* sink, int B, int T, int H, int D, int dv, int d_rope,
                float rope_base, float scale, int dtype, void* out, float* lse, void* workspace,
                size_t ws_bytes, void* stream) {
  return csk::attn_common("sparse_attn", false, q, q_pos, kv_c, Nmax, idx, k, nullptr, 1, kv_w,
                          w_pos0, S_w, W, sink, B, T, H, D, dv, d_rope, rope_base, scale, dtype,
                          out, lse, workspace, ws_bytes, stream);
}

int dense_compressed_attn(const void* q, const int32_t* q_pos, const void* kv_c, int Nmax,
                          const int32_t* n_entries, int m, const void* kv_w,
                          const int32_t* w_pos0, int S_w, int W, const float* sink, int B, int T,
                          int H, int D, int dv, int d_rope, float rope_base, float scale,
                          int dtype, void* out, float* lse, void* workspace, size_t ws_bytes,
                          void* stream) {
  return csk::attn_common("dense_compressed_attn", true, q, q_pos, kv_c, Nmax, nullptr, 0,
                          n_entries, m, kv_w, w_pos0, S_w, W, sink, B, T, H, D, dv, d_rope,
                          rope_base, scale, dtype, out, lse, workspace, ws_bytes, stream);
}

}  // extern "C"
