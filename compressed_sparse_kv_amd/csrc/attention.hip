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
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

// LDS transpose read (ds_read_b64_tr_b16). Within each group of 16 lanes,
// source lane s supplies an 8-byte address (4 consecutive bf16 e[s][0..3]);
// lane i receives e[4k + i/4][i%4] for k = 0..3.
__device__ __forceinline__ v4s lds_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(lds_u16*)(uint16_t*)p);
}

// V^T fragment of the O^T MFMA for value rows 16*dt + col: the lane's 8
// candidates {4g..4g+3, 16+4g..16+4g+3}, fetched with two transpose reads.
// p0 must point at dims 16*dt + 4*(col%4) .. +3 of candidate 4*g + col/4 and
// p1 at the same dims of candidate 16 + 4*g + col/4.
__device__ __forceinline__ v8bf vt_fragment(const uint16_t* p0, const uint16_t* p1) {
  // whole-vector bit casts only: element-wise short -> bf16 inserts of the
  // transpose-read result are lowered wrongly (only the low half of each
  // dword survives)
  const v4s r0 = lds_tr16(p0), r1 = lds_tr16(p1);
  const v8s both = __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(v8bf, both);
}

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
  int extra;              // whole-chunk kernel: rows past the MFMA tiles (VALU), <= MAX_EXTRA
  float scale;
  RopeTable rope;
  bool dense;
  void* out;              // [R, H, dv]
  float* lse;             // [R, H] or null
  float* part_o;          // [R, nch, H, dv], fp32 (bf16 when part_bf16)
  float* part_ml;         // [R, nch, H, 2]
  bool part_bf16;         // partial O stored as bf16 (the streamed-row kernel)
};

struct RowInfo {
  int b;
  int64_t p;
  int nvis;      // dense: visible compressed entries
  int wr0, wr1;  // window rows [wr0, wr1)
};

__device__ __forceinline__ RowInfo row_info(const AttnArgs& a, int r) {
  RowInfo ri;
  ri.b = (int)((unsigned)r / (unsigned)a.T);
  // the row's three loads first and unconditionally (an array the row does
  // not use is replaced by q_pos, which has at least B entries), so that
  // they are in flight together
  const bool win = a.W > 0 && a.S_w > 0;
  const int32_t* ne_src = a.dense ? a.n_entries : a.q_pos;
  const int32_t* w0_src = win ? a.w_pos0 : a.q_pos;
  const int p = a.q_pos[r];
  const int ne_raw = ne_src[ri.b];
  const int w0_raw = w0_src[ri.b];
  // (an empty asm that takes all three keeps the compiler from sinking each
  // load into the branch that uses it, which would serialise them)
  asm volatile("" ::"s"(p), "s"(ne_raw), "s"(w0_raw));
  const int ne = a.dense ? ne_raw : 0;
  const int w0 = win ? w0_raw : 0;
  ri.p = p;
  ri.nvis = 0;
  if (a.dense && p >= 0) {
    // p + 1 <= 2^31 fits an unsigned 32-bit division
    int nv = (int)(((unsigned)p + 1u) / (unsigned)a.m);
    nv = nv < ne ? nv : ne;
    nv = nv < a.Nmax ? nv : a.Nmax;
    ri.nvis = nv < 0 ? 0 : nv;
  }
  ri.wr0 = ri.wr1 = 0;
  if (win) {
    int64_t lo = (int64_t)p - a.W + 1;
    lo = lo < 0 ? 0 : lo;
    int64_t r0 = lo - w0, r1 = (int64_t)p - w0 + 1;
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
constexpr int MAX_CHUNK = 4096;   // candidates per workgroup (row codes kept in LDS)

// Row code of candidate slot j: >= 0 compressed entry, <= -2 window row
// (-2 - row), -1 empty.
__device__ __forceinline__ int slot_code(const AttnArgs& a, const RowInfo& ri, int r, int j) {
  if (j < a.Lc) {
    if (a.dense) return j < ri.nvis ? j : -1;
    const int e = a.idx[(int64_t)r * a.k + j];
    return (e < 0 || e >= a.Nmax) ? -1 : e;
  }
  const int wrow = ri.wr0 + (j - a.Lc);
  return wrow < ri.wr1 ? -2 - wrow : -1;
}

template <int D, int DV, int NW>
__global__ __launch_bounds__(64 * NW) void attn_bf16_kernel(AttnArgs a) {
  constexpr int KS = D / 32;        // MFMA K-steps over the key dim
  constexpr int DT = DV / 16;       // 16-row tiles of the value dim
  constexpr int LD = D + 8;         // LDS row stride in bf16 (16 bytes of padding)
  constexpr int CPR = D / 8;        // 16-byte chunks per KV row
  constexpr int NT = 64 * NW;
  constexpr int PT = (32 * CPR + NT - 1) / NT;  // chunks per thread per tile
  __shared__ __align__(16) uint16_t tile[32 * LD];
  __shared__ int codes[MAX_CHUNK];

  const int r = blockIdx.x;
  const int chunk_id = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int h = wave * 16 + col;
  const RowInfo ri = row_info(a, r);
  const uint16_t* kvc = reinterpret_cast<const uint16_t*>(a.kv_c) + (int64_t)ri.b * a.Nmax * D;
  const uint16_t* kvw = reinterpret_cast<const uint16_t*>(a.kv_w) + (int64_t)ri.b * a.S_w * D;

  const int total = a.Lc + a.W;
  const int c0 = chunk_id * a.chunk;
  const int nc = min(a.chunk, total - c0);
  for (int j = tid; j < nc; j += NT) codes[j] = slot_code(a, ri, r, c0 + j);
  // cos/sin of the query position, one rotated pair per thread
  __shared__ float2 rtab[MAX_ROPE_PAIRS];
  if (tid < a.d_rope / 2) {
    float cs, sn;
    rope_cs((double)ri.p, a.rope.theta[tid], &cs, &sn);
    rtab[tid] = make_float2(cs, sn);
  }
  __syncthreads();

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
            const float2 csn = rtab[(c - rope0) / 2];
            const float cs = csn.x, sn = csn.y;
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
  __syncthreads();  // codes visible

  // register prefetch of one tile: each thread owns fixed 16-byte chunks
  // (row id/CPR, column id%CPR) of every tile
  uint4 pref[PT];
  auto load_tile = [&](int t0) {
#pragma unroll
    for (int q = 0; q < PT; ++q) {
      const int id = tid + q * NT;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (id < 32 * CPR) {
        const int j = t0 + id / CPR;
        if (j < nc) {
          const int code = codes[j];
          if (code != -1) {
            const uint16_t* src = code >= 0 ? kvc + (int64_t)code * D : kvw + (int64_t)(-2 - code) * D;
            v = *reinterpret_cast<const uint4*>(src + 8 * (id % CPR));
          }
        }
      }
      pref[q] = v;
    }
  };

  v4f acc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_part = 0.f;
  const float sl2 = a.scale * LOG2E;

  if (nc > 0) load_tile(0);
  for (int t0 = 0; t0 < nc; t0 += 32) {
    __syncthreads();  // every wave is done with the previous tile
#pragma unroll
    for (int q = 0; q < PT; ++q) {
      const int id = tid + q * NT;
      if (id < 32 * CPR)
        *reinterpret_cast<uint4*>(&tile[(id / CPR) * LD + 8 * (id % CPR)]) = pref[q];
    }
    if (t0 + 32 < nc) load_tile(t0 + 32);  // next tile's loads overlap this tile's math
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
        const bool ok = j < nc && codes[j] != -1;
        const float v = ok ? s[ct][i] * sl2 : -INFINITY;
        p[ct * 4 + i] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = group4_max(tmax);
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

    // O^T += V^T P^T (rescale only when some head's running max moved)
    if (__ballot(alpha != 1.0f) != 0ull) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
    }
    const uint16_t* vbase = &tile[(4 * g + (col >> 2)) * LD + 4 * (col & 3)];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const v8bf vf = vt_fragment(vbase + 16 * dt, vbase + 16 * LD + 16 * dt);
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, acc[dt], 0, 0, 0);
    }
  }

  // per-head totals across the four lane groups
  float l_tot = l_part;
  l_tot = group4_sum(l_tot);

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

// 16-byte LDS DMA of one lane: src -> lds_base + 16 * lane. (Kept in a
// device function: a kernel body that names this builtin directly is
// dropped from the host compilation pass, and its launch stub with it.)
__device__ __forceinline__ void lds_dma16(const void* src, uint4* lds_base) {
  __builtin_amdgcn_global_load_lds(src, lds_base, 16, 0, 0);
}

// s_waitcnt immediate: vmcnt(n), lgkmcnt(0), expcnt unchanged
#define CSK_VMCNT_LGKM0(n) ((((n) & 0xF) | ((((n) >> 4) & 0x3) << 14)) | (0x7 << 4))

// ------------------------------------------------- bf16 MFMA, whole chunk
// One workgroup = one query row and a chunk of CHUNK_TILES*32 candidates
// (2 or 4 tiles), all of which are resident in LDS at once (4 x 32 x 576
// bf16 = 144 KB; with 2 tiles two workgroups share a CU).
//   1. q fragments are loaded first, the row codes and the RoPE cos/sin
//      table next (one barrier for all of them);
//   2. every KV row of the chunk is requested with LDS DMA in one burst, so
//      all of the chunk's memory traffic is in flight together;
//   3. S = q.k of each tile as soon as that tile has landed; the scores of
//      all candidates stay in registers, and the softmax of each head is
//      exact over the chunk (one maximum, no rescaling of the accumulators);
//   4. O^T += V^T P^T over the chunk, V^T fragments from transpose reads.
// Each tile is 32 rows in column-major 16-byte units (unit = chunk*32 +
// row); one wave-level DMA instruction fills a 1 KB block of a tile (chunks
// 2b and 2b+1 of its 32 rows). Waves own 16 heads each (MFMA columns).
constexpr int MAX_EXTRA = 4;  // rows a whole-chunk workgroup takes past its tiles
constexpr int QTILE_ROPE_PAIRS = 32;  // query-tile kernel: rotated pairs per row (d_rope <= 64)

template <int D, int DV, int NW, bool DENSE, int CHUNK_TILES>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_bf16_chunk_kernel(AttnArgs a) {
  constexpr int TILE_CANDS = 32 * CHUNK_TILES;
  constexpr int KS = D / 32;            // MFMA K-steps over the key dims
  constexpr int DT = DV / 16;           // 16-row tiles of the value dims
  constexpr int TU = 32 * D / 8;        // 16-byte units per tile
  constexpr int BLK = D / 16;           // 1 KB DMA blocks per tile
  constexpr int NB = CHUNK_TILES * BLK;
  static_assert(NB % NW == 0, "DMA blocks must split evenly over the waves");
  // one array per tile (not one indexed array): the compiler then tells a
  // tile being read from the tiles whose DMAs are still in flight, and the
  // first tiles are computed while the later ones load
  __shared__ __align__(16) uint4 kv0[TU];
  __shared__ __align__(16) uint4 kv1[TU];
  __shared__ __align__(16) uint4 kv2[CHUNK_TILES > 2 ? TU : 1];
  __shared__ __align__(16) uint4 kv3[CHUNK_TILES > 2 ? TU : 1];
  auto tile = [&](int t) -> uint4* { return t == 0 ? kv0 : t == 1 ? kv1 : t == 2 ? kv2 : kv3; };
  __shared__ __align__(16) int codes[TILE_CANDS + MAX_EXTRA];
  // up to MAX_EXTRA rows past the tiles, row-major (unit = row * D/8 + chunk),
  // padded to whole 64-unit DMA blocks
  constexpr int XU = (MAX_EXTRA * (D / 8) + 63) / 64 * 64;
  __shared__ __align__(16) uint4 kvx[XU];
  __shared__ float2 rtab[MAX_ROPE_PAIRS];

  const int r = blockIdx.x;
  const int chunk_id = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int h = wave * 16 + col;
  const RowInfo ri = row_info(a, r);
  const uint16_t* kvc = reinterpret_cast<const uint16_t*>(a.kv_c) + (int64_t)ri.b * a.Nmax * D;
  const uint16_t* kvw = reinterpret_cast<const uint16_t*>(a.kv_w) + (int64_t)ri.b * a.S_w * D;
  const int total = a.Lc + a.W;
  const int cands = TILE_CANDS + a.extra;
  const int c0 = chunk_id * cands;
  const int nall = min(cands, total - c0);      // candidates of this chunk
  const int nc = min(nall, TILE_CANDS);          // of them in the MFMA tiles
  const int nx = nall - nc;                      // extra rows (VALU)

  // 1. q fragments (dims 32*ks + 8*g .. +7 of head h), codes, RoPE table
  uint4 qraw[KS];
  {
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)r * a.H + h) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qraw[ks] = *reinterpret_cast<const uint4*>(qrow + 32 * ks + 8 * g);
  }
  for (int j = tid; j < TILE_CANDS + MAX_EXTRA; j += 64 * NW) codes[j] = j < nall ? slot_code(a, ri, r, c0 + j) : -1;
  if (tid < a.d_rope / 2) {
    float cs, sn;
    rope_cs((double)ri.p, a.rope.theta[tid], &cs, &sn);
    rtab[tid] = make_float2(cs, sn);
  }
  // an ordinary store into the KV buffer: the DMA intrinsic is not seen as
  // a writer of it, and without one the reads below could be folded away
#pragma unroll
  for (int t = 0; t < CHUNK_TILES; ++t) tile(t)[tid] = make_uint4(0u, 0u, 0u, 0u);
  if (tid < XU) kvx[tid] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();

  // rotated query fragments as bf16, formed before the DMA burst: the q
  // loads completed at the barrier, and a use of their registers after the
  // burst would make the compiler wait for every DMA first
  v8bf qf[KS];
  {
    const int rope0 = D - a.d_rope;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int d0 = 32 * ks + 8 * g;
      float x[8];
      const uint32_t wv[4] = {qraw[ks].x, qraw[ks].y, qraw[ks].z, qraw[ks].w};
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
            const float2 csn = rtab[(c - rope0) / 2];
            const float x0 = x[2 * i], x1 = x[2 * i + 1];
            x[2 * i] = x0 * csn.x - x1 * csn.y;
            x[2 * i + 1] = x0 * csn.y + x1 * csn.x;
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) qf[ks][i] = __builtin_bit_cast(__bf16, (uint16_t)f32_to_bf16_bits(x[i]));
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // 2. one burst of DMA for the whole chunk; empty slots read row 0 of the
  // cache (finite data, weight 0)
  {
    // the lane's row in each tile, read once
    const int row = lane & 31;
    const uint16_t* src[CHUNK_TILES];
#pragma unroll
    for (int t = 0; t < CHUNK_TILES; ++t) {
      const int code = codes[t * 32 + row];
      src[t] = code >= 0 ? kvc + (int64_t)code * D : (code <= -2 ? kvw + (int64_t)(-2 - code) * D : kvc);
    }
    // the extra rows first (wave 0; older than every tile's DMAs, so the
    // tile waits below still count right), row-major 16-byte units
    if (wave == 0 && nx > 0) {
      const int nu = nx * (D / 8);
      for (int u0 = 0; u0 < nu; u0 += 64) {
        const int u = min(u0 + lane, nu - 1);  // the tail lanes repeat the last unit
        const int xr = u / (D / 8), xc = u - xr * (D / 8);
        const int code = codes[TILE_CANDS + xr];
        const uint16_t* xs = code >= 0 ? kvc + (int64_t)code * D : (code <= -2 ? kvw + (int64_t)(-2 - code) * D : kvc);
        lds_dma16(xs + 8 * xc, kvx + u0);
      }
    }
    // tile by tile, so that a tile's DMAs are older than the next tile's
#pragma unroll
    for (int t = 0; t < CHUNK_TILES; ++t)
#pragma unroll
      for (int q = 0; q < BLK / NW; ++q) {
        const int b = wave + NW * q;
        lds_dma16(src[t] + 8 * (2 * b + (lane >> 5)), tile(t) + b * 64);
      }
  }

  const int ntiles = (nc + 31) / 32;
  const float sl2 = a.scale * LOG2E;

  // 3. scores of all candidates (lane holds candidates 32t + 16ct + 4g + i)
  v4f sc[CHUNK_TILES][2];
#pragma unroll
  for (int t = 0; t < CHUNK_TILES; ++t) {
    // tile t has landed once this wave's DMAs for it are done (the later
    // tiles' BLK/NW each may remain) and every wave has passed the barrier;
    // the fences keep the compiler from moving memory accesses across it
    asm volatile("" ::: "memory");
    {
      // (vmcnt holds at most 63: a larger count clamps, which only waits longer)
      constexpr int PER = BLK / NW;
      const int rem = CHUNK_TILES - 1 - t;
      if (rem <= 0) __builtin_amdgcn_s_waitcnt(CSK_VMCNT_LGKM0(0));
      else if (rem == 1) __builtin_amdgcn_s_waitcnt(CSK_VMCNT_LGKM0(PER < 63 ? PER : 63));
      else if (rem == 2) __builtin_amdgcn_s_waitcnt(CSK_VMCNT_LGKM0(2 * PER < 63 ? 2 * PER : 63));
      else __builtin_amdgcn_s_waitcnt(CSK_VMCNT_LGKM0(3 * PER < 63 ? 3 * PER : 63));
    }
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    sc[t][0] = sc[t][1] = v4f{0.f, 0.f, 0.f, 0.f};
    if (t < ntiles) {
      // fragments in blocks of QB K-steps, the next block's reads issued
      // before the current block's MFMAs (the scheduling barriers keep that
      // order; left alone, the scheduler keeps one read in flight)
      const uint4* sb = tile(t);
      constexpr int QB = 3, NQB = (KS + QB - 1) / QB;
      v8bf kf[2][QB][2];
      auto load_q = [&](int blk, v8bf (&dst)[QB][2]) {
#pragma unroll
        for (int u = 0; u < QB; ++u) {
          const int ks = blk * QB + u;
          if (ks < KS)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
              dst[u][ct] = *reinterpret_cast<const v8bf*>(&sb[(4 * ks + g) * 32 + ct * 16 + col]);
        }
      };
      load_q(0, kf[0]);
#pragma unroll
      for (int blk = 0; blk < NQB; ++blk) {
        if (blk + 1 < NQB) load_q(blk + 1, kf[(blk + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < QB; ++u) {
          const int ks = blk * QB + u;
          if (ks < KS)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
              sc[t][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[blk & 1][u][ct], qf[ks], sc[t][ct], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  // scores of the extra rows (VALU): the lane's partial dot over its dims,
  // summed over the four lane groups of its head
  float sx[MAX_EXTRA];
#pragma unroll
  for (int x = 0; x < MAX_EXTRA; ++x) {
    sx[x] = -INFINITY;
    if (x < nx) {
      const uint4* xr = kvx + x * (D / 8);
      float dot = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 kk = xr[4 * ks + g];
        const uint32_t kw[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          dot = __builtin_fmaf((float)qf[ks][2 * i], bf16_bits_to_f32(kw[i] & 0xffffu), dot);
          dot = __builtin_fmaf((float)qf[ks][2 * i + 1], bf16_bits_to_f32(kw[i] >> 16), dot);
        }
      }
      dot = group4_sum(dot);
      if (codes[TILE_CANDS + x] != -1) sx[x] = dot * sl2;
    }
  }
  // the lane's 32 candidates are 4 consecutive codes per (tile, half):
  // eight vector reads, then the mask is register arithmetic
  int4 cd[CHUNK_TILES][2];
#pragma unroll
  for (int t = 0; t < CHUNK_TILES; ++t)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) cd[t][ct] = *reinterpret_cast<const int4*>(&codes[32 * t + 16 * ct + 4 * g]);
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < CHUNK_TILES; ++t)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int c4[4] = {cd[t][ct].x, cd[t][ct].y, cd[t][ct].z, cd[t][ct].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // codes of slots past nc are -1 (set in the prologue)
        const float v = c4[i] != -1 ? sc[t][ct][i] * sl2 : -INFINITY;
        sc[t][ct][i] = v;
        mx = fmaxf(mx, v);
      }
    }
  mx = group4_max(mx);
#pragma unroll
  for (int x = 0; x < MAX_EXTRA; ++x) mx = fmaxf(mx, sx[x]);  // equal in all lane groups
  float l_part = 0.f;
  float px[MAX_EXTRA];
#pragma unroll
  for (int x = 0; x < MAX_EXTRA; ++x) {
    px[x] = (mx == -INFINITY || sx[x] == -INFINITY) ? 0.f : exp2f(sx[x] - mx);
    if (g == 0) l_part += px[x];  // counted once per head
  }
  v8bf pf[CHUNK_TILES];
#pragma unroll
  for (int t = 0; t < CHUNK_TILES; ++t)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = mx == -INFINITY ? 0.f : exp2f(sc[t][ct][i] - mx);
        l_part += pv;
        pf[t][4 * ct + i] = __builtin_bit_cast(__bf16, (uint16_t)f32_to_bf16_bits(pv));
      }
  const float l_tot = group4_sum(l_part);

  // 4. O^T += V^T P^T over the chunk
  v4f acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < CHUNK_TILES; ++t) {
    if (t < ntiles) {
      // V^T fragments in blocks of VB value tiles, pipelined like the QK
      // fragments
      const uint16_t* sb16 = reinterpret_cast<const uint16_t*>(tile(t));
      constexpr int VB = 4, NVB = (DT + VB - 1) / VB;
      v8bf vf[2][VB];
      auto load_v = [&](int blk, v8bf (&dst)[VB]) {
#pragma unroll
        for (int u = 0; u < VB; ++u) {
          const int dt = blk * VB + u;
          if (dt < DT) {
            const int dvb = 16 * dt + 4 * (col & 3);
            const uint16_t* p0 = sb16 + ((dvb >> 3) * 32 + 4 * g + (col >> 2)) * 8 + (dvb & 7);
            dst[u] = vt_fragment(p0, p0 + 16 * 8);
          }
        }
      };
      load_v(0, vf[0]);
#pragma unroll
      for (int blk = 0; blk < NVB; ++blk) {
        if (blk + 1 < NVB) load_v(blk + 1, vf[(blk + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < VB; ++u) {
          const int dt = blk * VB + u;
          if (dt < DT) acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[blk & 1][u], pf[t], acc[dt], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // the extra rows' values (VALU): lane (head col, group g) holds value dims
  // 16*dt + 4*g .. +3
#pragma unroll
  for (int x = 0; x < MAX_EXTRA; ++x) {
    if (x < nx && px[x] != 0.f) {
      const uint16_t* xr = reinterpret_cast<const uint16_t*>(kvx + x * (D / 8));
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint2 vv = *reinterpret_cast<const uint2*>(xr + 16 * dt + 4 * g);
        acc[dt][0] = __builtin_fmaf(px[x], bf16_bits_to_f32(vv.x & 0xffffu), acc[dt][0]);
        acc[dt][1] = __builtin_fmaf(px[x], bf16_bits_to_f32(vv.x >> 16), acc[dt][1]);
        acc[dt][2] = __builtin_fmaf(px[x], bf16_bits_to_f32(vv.y & 0xffffu), acc[dt][2]);
        acc[dt][3] = __builtin_fmaf(px[x], bf16_bits_to_f32(vv.y >> 16), acc[dt][3]);
      }
    }
  }

  if (a.nch == 1) {
    float M, inv_z, lse;
    finish_row(mx, l_tot, a.sink, h, &M, &inv_z, &lse);
    const float f = (mx == -INFINITY) ? 0.f : exp2f(mx - M) * inv_z;
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
      pm[0] = mx;
      pm[1] = l_tot;
    }
  }
}

// ------------------------------------------- bf16 MFMA, query-row tiles
// Dense attention over consecutive query rows of one sequence (prefill).
// Rows that sit next to each other see the same compressed entries (each up
// to its own visibility bound) and overlapping windows, so one workgroup
// stages the union of its rows' candidates in LDS once, and every K or V
// fragment read from LDS feeds the MFMAs of CT column tiles (16 heads of one
// row each). Candidate j of the union: j < nvmax is compressed entry j,
// otherwise window row w0 + j - nvmax; row i keeps j < nvis_i and the window
// span of its own rows. Online softmax per head, with the running maximum
// moved only when a tile's maximum passes it by more than 8 (log2 units), so
// the accumulators are rarely rescaled (probabilities stay below 2^8).
template <int D, int DV, int HG, int CT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3)))
void attn_bf16_qtile_kernel(AttnArgs a) {
  constexpr int NW = 4;
  constexpr int TQ = NW * CT / HG;           // query rows per workgroup
  constexpr int KS = D / 32;                 // MFMA K-steps over the key dims
  constexpr int DT = DV / 16;                // 16-row tiles of the value dims
  constexpr int TU = 32 * D / 8;             // 16-byte units per 32-row tile
  constexpr int BLK = D / 16;                // 1 KB DMA blocks per tile
  constexpr int PER = BLK / NW;              // of them per wave
  constexpr int TILES = 49152 / (64 * D);    // tiles staged at once (48 KB: three workgroups per CU)
  constexpr int RP = QTILE_ROPE_PAIRS;
  static_assert(BLK % NW == 0 && TQ * HG == NW * CT && TILES >= 1, "unsupported shape");
  __shared__ __align__(16) uint4 kv[TILES * TU];
  __shared__ float2 rtab[TQ][RP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int tpb = (a.T + TQ - 1) / TQ;
  const int b = blockIdx.x / tpb;
  const int t0 = (blockIdx.x - b * tpb) * TQ;
  const uint16_t* kvc = reinterpret_cast<const uint16_t*>(a.kv_c) + (int64_t)b * a.Nmax * D;
  const uint16_t* kvw = reinterpret_cast<const uint16_t*>(a.kv_w) + (int64_t)b * a.S_w * D;

  // 1. lane i < TQ reads row t0+i's position and derives its candidate
  // spans (one vector load, issued before the q loads so that waiting for
  // it leaves those in flight); readlane then makes them uniform
  // (w_pos0 may be null without a window: the load then re-reads n_entries,
  // unconditionally, so that both loads go out together)
  const int ne_raw = a.n_entries[b];
  const int wp_raw = (a.S_w > 0 ? a.w_pos0 : a.n_entries)[b];
  const int ne = min(ne_raw, a.Nmax);
  const int wpos0 = a.S_w > 0 ? wp_raw : 0;
  const int mdiv = a.m;
  const int li = min(lane, TQ - 1);
  const int qpl = a.q_pos[(int64_t)b * a.T + min(t0 + li, a.T - 1)];
  // q fragments of the wave's column tiles (rows past T load row T-1)
  int qrow_i[CT], qh[CT];
  uint4 qraw[CT][KS];
#pragma unroll
  for (int i = 0; i < CT; ++i) {
    const int c = wave * CT + i;
    qrow_i[i] = c / HG;
    qh[i] = 16 * (c % HG) + col;
    const int t = min(t0 + qrow_i[i], a.T - 1);
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + (((int64_t)b * a.T + t) * a.H + qh[i]) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qraw[i][ks] = *reinterpret_cast<const uint4*>(qrow + 32 * ks + 8 * g);
  }
  int pl, nvl, w0l, w1l;
  {
    const bool valid = t0 + li < a.T;
    const int64_t p = valid ? qpl : -1;
    pl = (int)p;
    const int nvv = p >= 0 ? (int)((uint32_t)(p + 1) / (uint32_t)mdiv) : 0;
    nvl = nvv < ne ? nvv : ne;
    int64_t lo = p - a.W + 1;
    lo = lo < 0 ? 0 : lo;
    int64_t r0 = lo - wpos0, r1 = p - wpos0 + 1;
    r0 = r0 < 0 ? 0 : r0;
    r1 = r1 > a.S_w ? a.S_w : r1;
    const bool win = valid && a.W > 0 && a.S_w > 0 && r1 > r0;
    w0l = win ? (int)r0 : 0;
    w1l = win ? (int)r1 : 0;
  }
  int rpos[TQ], rnv[TQ], rw0[TQ], rw1[TQ];
  int nvmax = 0, w0 = 0x7fffffff, w1 = 0;
#pragma unroll
  for (int i = 0; i < TQ; ++i) {
    rpos[i] = __builtin_amdgcn_readlane(pl, i);
    rnv[i] = __builtin_amdgcn_readlane(nvl, i);
    rw0[i] = __builtin_amdgcn_readlane(w0l, i);
    rw1[i] = __builtin_amdgcn_readlane(w1l, i);
    nvmax = max(nvmax, rnv[i]);
    if (rw1[i] > rw0[i]) {
      w0 = min(w0, rw0[i]);
      w1 = max(w1, rw1[i]);
    }
  }
  if (w1 == 0) w0 = 0;
  const int Lt = nvmax + (w1 - w0);
  // the column tiles' candidate spans: compressed [0, nv), window [wlo, whi)
  int nv[CT], wlo[CT], whi[CT];
#pragma unroll
  for (int i = 0; i < CT; ++i) {
    const int ri = qrow_i[i];
    nv[i] = rnv[ri];
    const bool win = rw1[ri] > rw0[ri];
    wlo[i] = win ? nvmax + rw0[ri] - w0 : 0;
    whi[i] = win ? nvmax + rw1[ri] - w0 : 0;
  }
  // an ordinary store into the KV buffer (the DMA intrinsic is not seen as
  // a writer of it, and without one the reads below could be folded away),
  // finished by every wave before any DMA is issued
  kv[tid] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();

  const int row = lane & 31;
  auto stage = [&](int s0, int nt) {
    // every KV row of a stage by LDS DMA; slots past Lt read row 0 of the
    // cache (finite data, masked)
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      if (t < nt) {
        const int j = s0 + 32 * t + row;
        const uint16_t* src = j < nvmax ? kvc + (int64_t)j * D : (j < Lt ? kvw + (int64_t)(w0 + j - nvmax) * D : kvc);
#pragma unroll
        for (int q = 0; q < PER; ++q) {
          const int bb = wave + NW * q;
          lds_dma16(src + 8 * (2 * bb + (lane >> 5)), kv + t * TU + bb * 64);
        }
      }
    }
  };
  int nt = min(TILES, (Lt + 31) / 32);
  if (Lt > 0) stage(0, nt);

  // 2. cos/sin of every row's position while the first stage lands
  const int npairs = a.d_rope / 2;
  for (int e = tid; e < TQ * RP; e += 64 * NW) {
    const int i = e / RP, pr = e - i * RP;
    if (pr < npairs) {
      float cs, sn;
      rope_cs((double)rpos[i], a.rope.theta[pr], &cs, &sn);
      rtab[i][pr] = make_float2(cs, sn);
    }
  }
  __syncthreads();

  v8bf qf[CT][KS];
  {
    const int rope0 = D - a.d_rope;
#pragma unroll
    for (int i = 0; i < CT; ++i)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int d0 = 32 * ks + 8 * g;
        float x[8];
        const uint32_t wv[4] = {qraw[i][ks].x, qraw[i][ks].y, qraw[i][ks].z, qraw[i][ks].w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          x[2 * u] = bf16_bits_to_f32(wv[u] & 0xffffu);
          x[2 * u + 1] = bf16_bits_to_f32(wv[u] >> 16);
        }
        if (d0 + 8 > rope0) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int c = d0 + 2 * u;
            if (c >= rope0) {
              const float2 csn = rtab[qrow_i[i]][(c - rope0) / 2];
              const float x0 = x[2 * u], x1 = x[2 * u + 1];
              x[2 * u] = x0 * csn.x - x1 * csn.y;
              x[2 * u + 1] = x0 * csn.y + x1 * csn.x;
            }
          }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) qf[i][ks][u] = __builtin_bit_cast(__bf16, (uint16_t)f32_to_bf16_bits(x[u]));
      }
  }

  float m[CT], l[CT];
  v4f acc[CT][DT];
#pragma unroll
  for (int i = 0; i < CT; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[i][dt] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  const float sl2 = a.scale * LOG2E;

  for (int s0 = 0; s0 < Lt; s0 += 32 * TILES) {
    if (s0 > 0) {
      __syncthreads();  // every wave is done with the previous stage
      nt = min(TILES, (Lt - s0 + 31) / 32);
      stage(s0, nt);
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(CSK_VMCNT_LGKM0(0));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    for (int t = 0; t < nt; ++t) {
      const uint4* sb = kv + t * TU;
      const int c0 = s0 + 32 * t;
      // 3. S^T = K q~ for the tile's two 16-candidate halves, each K
      // fragment shared by the wave's CT column tiles
      v4f s[CT][2];
#pragma unroll
      for (int i = 0; i < CT; ++i) s[i][0] = s[i][1] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const v8bf kf = *reinterpret_cast<const v8bf*>(&sb[(4 * ks + g) * 32 + h2 * 16 + col]);
#pragma unroll
          for (int i = 0; i < CT; ++i)
            s[i][h2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[i][ks], s[i][h2], 0, 0, 0);
        }
      // 4. online softmax; lane holds candidates c0 + 16*h2 + 4g + e. The
      // spans are uniform per column tile, so only tiles that straddle a
      // span edge are masked element by element.
      v8bf pf[CT];
      float alpha[CT];
      bool moved = false;
#pragma unroll
      for (int i = 0; i < CT; ++i) {
        const bool full = c0 + 32 <= nv[i] || (c0 >= wlo[i] && c0 + 32 <= whi[i]);
        float v[8];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int e = 0; e < 4; ++e) v[4 * h2 + e] = s[i][h2][e];
        if (!full) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int j = c0 + 16 * (e >> 2) + 4 * g + (e & 3);
            const int ok = (j < nv[i]) | ((unsigned)(j - wlo[i]) < (unsigned)(whi[i] - wlo[i]));
            v[e] = ok ? v[e] : -INFINITY;
          }
        }
        float tm = fmaxf(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])), fmaxf(fmaxf(v[4], v[5]), fmaxf(v[6], v[7])));
        tm = group4_max(tm) * sl2;  // scale > 0: the maximum of the scaled logits
        const float mn = tm > m[i] + 8.f ? tm : m[i];
        alpha[i] = mn == m[i] ? 1.f : __builtin_amdgcn_exp2f(m[i] - mn);
        moved |= mn != m[i];
        m[i] = mn;
        // v_exp_f32 directly: arguments are <= 8, masked logits give 0, and
        // a weight that underflows is negligible next to the row's largest
        const float nm = mn == -INFINITY ? 0.f : -mn;
        float ps = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(v[e], sl2, nm));
          ps += p;
          pf[i][e] = (__bf16)p;
        }
        l[i] = l[i] * alpha[i] + ps;
      }
      if (__ballot(moved) != 0ull) {
#pragma unroll
        for (int i = 0; i < CT; ++i)
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) acc[i][dt] *= alpha[i];
      }
      // 5. O^T += V^T P^T, each V^T fragment shared by the CT column tiles
      const uint16_t* sb16 = reinterpret_cast<const uint16_t*>(sb);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int dvb = 16 * dt + 4 * (col & 3);
        const uint16_t* p0 = sb16 + ((dvb >> 3) * 32 + 4 * g + (col >> 2)) * 8 + (dvb & 7);
        const v8bf vf = vt_fragment(p0, p0 + 16 * 8);
#pragma unroll
        for (int i = 0; i < CT; ++i) acc[i][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[i], acc[i][dt], 0, 0, 0);
      }
    }
  }

  // 6. normalise with the sink and write
#pragma unroll
  for (int i = 0; i < CT; ++i) {
    const float lt = group4_sum(l[i]);
    const int t = t0 + qrow_i[i];
    if (t >= a.T) continue;
    const int64_t r = (int64_t)b * a.T + t;
    float M, inv_z, lse;
    finish_row(m[i], lt, a.sink, qh[i], &M, &inv_z, &lse);
    const float f = (m[i] == -INFINITY) ? 0.f : exp2f(m[i] - M) * inv_z;
    uint16_t* ob = reinterpret_cast<uint16_t*>(a.out) + (r * a.H + qh[i]) * DV;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d0 = 16 * dt + 4 * g;
      const v2bf lo = {(__bf16)(acc[i][dt][0] * f), (__bf16)(acc[i][dt][1] * f)};
      const v2bf hi = {(__bf16)(acc[i][dt][2] * f), (__bf16)(acc[i][dt][3] * f)};
      *reinterpret_cast<uint2*>(ob + d0) = make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
    }
    if (a.lse && g == 0) a.lse[r * a.H + qh[i]] = lse;
  }
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// accesses, not for its global loads (__syncthreads would also wait for
// every LDS DMA in flight).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(CSK_VMCNT_LGKM0(63));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The lane's index, formed again at each use: the values derived from it
// are cheap to recompute, and holding them across a long loop takes
// registers that the loop's own values need (the compiler spills them, and a
// reload waits for every DMA in flight). Volatile, so that separate calls
// are not merged into one long-lived value.
__device__ __forceinline__ int fresh_lane() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// ------------------------------------------ bf16 32x32 MFMA, streamed rows
// Sparse or dense attention of one query row with 64 heads. The row's
// candidates stream through LDS in 64-row tiles, two buffers deep, each
// filled by LDS DMA. Rows with long candidate lists and few rows to spread
// (decode) are split into runs of tiles, one workgroup each, that write
// unnormalised partials (O in bf16, m and l in fp32) for the merge kernel; otherwise (prefill) a
// workgroup keeps its row whole and writes the output. Dense rows take
// compressed entries 0..nvis-1 in order, so they read no index list. Wave w = (head group hg = w&1,
// half ch = w>>1) scores 32 heads against tile rows [32ch, 32ch+32) with
// 32x32x16 MFMAs (S^T = K q~^T; the q~ fragments stay in registers). The
// two waves of a head group then agree on the running maximum (tile maxima
// through LDS) and swap their probabilities, and each accumulates
// O^T += V^T P^T over all 64 rows for its half of the value dims.
// LDS tile layout (16-byte units): rows in groups of eight, G = j/8; chunk
// c (dims 8c..8c+7) of row j sits at unit G*8*NCH + 8*(c ^ (G&1)) + j%8.
// One DMA instruction (64 consecutive units) then reads 8 chunks of each
// of eight rows, i.e. eight 128-byte runs (for rows gathered from a large
// cache this spreads better than longer runs from fewer rows), and both the
// K reads (32 rows of one chunk) and the transposed V^T reads (4 rows x 2
// chunks per 16 lanes) find their units on distinct bank groups. The DMA
// of the next tile is issued one instruction per K-step block of the
// current tile's QK.
constexpr int R32_QB = 2;  // K fragments per pipelined block (two blocks in flight)
constexpr int R32_VB = 2;  // V^T fragments per pipelined block

template <int D, int DV, bool DENSE, bool KV8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_bf16_row32_kernel(AttnArgs a) {
  constexpr int NCH = D / 8;             // 16-byte chunks per KV row
  constexpr int GU = 8 * NCH;            // units per group of eight rows
  constexpr int TU = 8 * GU;             // units per 64-row tile
  constexpr int IPG = NCH / 8;           // DMA instructions per row group
  constexpr int KS = D / 16;             // 32x32x16 K-steps over the key dims
  constexpr int HDT = DV / 64;           // 32-row value tiles per wave (half of DV)
  constexpr int CPW = NCH / 4;           // DMA instructions per wave per tile
  constexpr int QB = R32_QB, NQB = KS / QB;
  static_assert(NCH % 8 == 0 && DV % 64 == 0 && DV <= D && KS % QB == 0 && NQB == CPW &&
                    CPW - (CPW + 1) / 2 <= 4 * HDT / R32_VB,
                "unsupported shape");
  // FP8 KV entries (KV8; built for 512 + 64): entry = [512 E4M3 codes][64
  // bf16 RoPE dims][16 scale bytes] = 41 units. A tile of 64 entries is
  // staged by DMA as-is (code units, then the rows' 9-unit tails) and
  // converted in LDS into the bf16 tile layout below, on which the rest of
  // the kernel runs unchanged.
  constexpr int DN8 = D - 64;                       // code bytes per entry
  constexpr int ESU = (DN8 + 128 + DN8 / 32 + 15) / 16;  // 16-byte units per entry
  constexpr int ES8 = 16 * ESU;                     // entry bytes
  constexpr int CU8 = DN8 / 16;                     // code units per entry (32)
  constexpr int STU = 64 * ESU;                     // staged tile units
  constexpr int TAIL0 = 64 * CU8;                   // first tail unit of a staged tile
  static_assert(!KV8 || (D == 576 && DV == 512 && CU8 == 32 && ESU == 41), "FP8 KV tiles are built for 512 + 64");
  // bf16: two tile buffers; KV8: the converted tile (buf0) and the two
  // staged tiles (buf1). Separate objects: the compiler then knows that a
  // tile's DMA into one does not write what is read from the other, and
  // does not wait for the DMA in flight before each LDS read.
  __shared__ __align__(16) uint4 buf0[TU];
  __shared__ __align__(16) uint4 buf1[KV8 ? 2 * STU : TU];
  __shared__ __align__(16) uint4 pex_b[KV8 ? 1 : 4 * 2 * 64];  // probabilities, B-operand fragments
  __shared__ int rowtab[KV8 ? 2 * 64 : 1];                     // KV8: the row codes of tiles t, t+1
  __shared__ float mx[4][32];                      // tile maxima per head
  __shared__ float xl[4][32];                      // end-of-row sums per head
  __shared__ float2 rtab[MAX_ROPE_PAIRS];
  // staged tile T (KV8)
  auto stg = [&](int T) { return buf1 + STU * (T & 1); };

  const int r = blockIdx.x;
  const int split = blockIdx.y;
  const int tid = threadIdx.x;
  // wave-uniform (readfirstlane): everything derived from it stays scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hg = wave & 1, ch = wave >> 1, pw = wave ^ 2;
  // lane terms (prologue only; the loop and the epilogue form them again)
  const int lane = tid & 63;
  const int c32 = lane & 31, hi = lane >> 5;
  const RowInfo ri = row_info(a, r);
  const uint16_t* kvc = reinterpret_cast<const uint16_t*>(a.kv_c) + (int64_t)ri.b * a.Nmax * D;
  const uint16_t* kvw = reinterpret_cast<const uint16_t*>(a.kv_w) + (int64_t)ri.b * a.S_w * D;
  const char* kvc8 = reinterpret_cast<const char*>(a.kv_c) + (int64_t)ri.b * a.Nmax * ES8;
  const char* kvw8 = reinterpret_cast<const char*>(a.kv_w) + (int64_t)ri.b * a.S_w * ES8;
  const int total = a.Lc + a.W;
  // this workgroup's 64-row tiles [t0, t1) of the row's candidate slots
  // (a.nch workgroups share a row; the merge kernel combines them)
  const int nt_row = (total + 63) / 64;
  const int t0 = (int)((int64_t)split * nt_row / a.nch);
  const int ntiles = (int)((int64_t)(split + 1) * nt_row / a.nch) - t0;
  const int j0 = 64 * t0;
  const int32_t* idxr = DENSE ? nullptr : a.idx + (int64_t)r * a.k;

  // index read (clamped, issued unconditionally; dense rows read none),
  // code (>= 0 entry, <= -2 window row, -1 empty) of the workgroup's slot
  // j0 + j, KV row address (selects, no branches)
  auto idx_load = [&](int j) -> int { return DENSE ? 0 : idxr[min(j0 + j, a.k - 1)]; };
  auto code_of = [&](int j, int e) -> int {
    const int jj = j0 + j;
    if (jj < a.Lc) {
      if (DENSE) return jj < ri.nvis ? jj : -1;
      return (e < 0 || e >= a.Nmax) ? -1 : e;
    }
    const int wrow = ri.wr0 + (jj - a.Lc);
    return (jj < total && wrow < ri.wr1) ? -2 - wrow : -1;
  };
  auto row_addr = [&](int code) -> const uint16_t* {
    const bool win = code <= -2;
    const int rowi = code >= 0 ? code : (win ? -2 - code : 0);
    return (win ? kvw : kvc) + (int64_t)rowi * D;
  };
  // DMA instruction q of this wave: units 64i .. 64i+63, i = CPW*wave + q,
  // so the wave covers row groups 2w and 2w+1 and instruction q is block
  // q%IPG of group 2w + q/IPG (compile-time but for the wave term, and
  // G&1 = q/IPG&1); the lane loads row 16w + 8(q/IPG) + lane%8, whose
  // address it holds itself (two per tile), at chunk 8*block + lane/8,
  // swizzled
  auto dma_row_of = [&](int ln) { return 16 * wave + (ln & 7); };
  auto dma_one = [&](uint4* dst, const uint16_t* const (&rp)[2], int q, int ln) {
    const int gq = q / IPG, blk = q % IPG;
    const uint16_t* src = rp[gq] + 64 * blk + 8 * ((ln >> 3) ^ (gq & 1));
    lds_dma16(src, dst + 64 * (CPW * wave + q));
  };
  // tile T's index reads of this lane: row = lane (its mask bit) and the two
  // rows its DMAs load (KV8: the row = lane only; its code goes to the row
  // table from which every lane takes the rows it stages)
  struct TileIdx { int em, e0, e1; };
  auto tile_idx = [&](int T, int ln) -> TileIdx {
    if (KV8) return TileIdx{idx_load(64 * T + ln), 0, 0};
    const int dr = dma_row_of(ln);
    return TileIdx{idx_load(64 * T + ln), idx_load(64 * T + dr), idx_load(64 * T + dr + 8)};
  };
  // KV8 staging: this wave's DMA instruction q of tile T. q < 8: code units
  // of instruction i = 8*wave + q, rows 8(i%8) + lane%8, code units
  // 8(i/8) + lane/8 (eight 128-byte runs of eight rows), into staged units
  // 64i + lane; q >= 8: tail instruction i = wave + 4(q - 8) (< 9), unit
  // 64i + lane of the rows' tails (row t/9, unit t%9 for t = 64i + lane).
  // Wave 0 issues 11 instructions, the others 10.
  auto entry8 = [&](int code) -> const char* {
    const bool win = code <= -2;
    const int rowi = code >= 0 ? code : (win ? -2 - code : 0);
    return (win ? kvw8 : kvc8) + (int64_t)rowi * ES8;
  };
  const int nq8 = wave == 0 ? 11 : 10;
  auto dma8 = [&](int T, int q, int ln) {
    uint4* st = stg(T);
    const int* rt = rowtab + 64 * (T & 1);
    if (q < 8) {
      const int i = 8 * wave + q;
      const int j = 8 * (i & 7) + (ln & 7), cu = 8 * (i >> 3) + (ln >> 3);
      lds_dma16(entry8(rt[j]) + 16 * cu, st + 64 * i);
    } else {
      const int i = wave + 4 * (q - 8);
      const int t = 64 * i + ln, j = t / 9;
      lds_dma16(entry8(rt[j]) + DN8 + 16 * (t - 9 * j), st + TAIL0 + 64 * i);
    }
  };
  // KV8: staged tile T -> bf16 tile buf0. Staged code unit u = 64i + l holds
  // codes 16cu .. 16cu+15 of row j (as the DMA placed them); its two bf16
  // chunks go to units (j/8)*GU + 8*(c ^ (j/8 & 1)) + j%8 for c = 2cu, 2cu+1
  // (scaled by the row's scale byte of block cu/2, exact in bf16); the
  // RoPE units are copied. Eight consecutive lanes write eight consecutive
  // units.
  auto convert8 = [&](int T) {
    const uint4* st = stg(T);
    const uint8_t* st8 = reinterpret_cast<const uint8_t*>(st);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int u = tid + 256 * k;
      const int i = u >> 6, l = u & 63;
      const int j = 8 * (i & 7) + (l & 7), cu = 8 * (i >> 3) + (l >> 3);
      const uint4 c16 = st[u];
      const uint32_t sb = st8[16 * (TAIL0 + 9 * j + 8) + (cu >> 1)];
      const float scl = __uint_as_float(sb << 23);
      const v2bf b0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c16.x, scl, false);
      const v2bf b1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c16.x, scl, true);
      const v2bf b2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c16.y, scl, false);
      const v2bf b3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c16.y, scl, true);
      const v2bf b4 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c16.z, scl, false);
      const v2bf b5 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c16.z, scl, true);
      const v2bf b6 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c16.w, scl, false);
      const v2bf b7 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c16.w, scl, true);
      const int G = j >> 3, g1 = G & 1;
      buf0[G * GU + 8 * ((2 * cu) ^ g1) + (j & 7)] =
          make_uint4(__builtin_bit_cast(uint32_t, b0), __builtin_bit_cast(uint32_t, b1),
                     __builtin_bit_cast(uint32_t, b2), __builtin_bit_cast(uint32_t, b3));
      buf0[G * GU + 8 * ((2 * cu + 1) ^ g1) + (j & 7)] =
          make_uint4(__builtin_bit_cast(uint32_t, b4), __builtin_bit_cast(uint32_t, b5),
                     __builtin_bit_cast(uint32_t, b6), __builtin_bit_cast(uint32_t, b7));
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int v = tid + 256 * k;
      const int j = v & 63, ru = v >> 6;  // row, RoPE unit (bf16 chunk 64 + ru)
      const int G = j >> 3;
      buf0[G * GU + 8 * ((2 * CU8 + ru) ^ (G & 1)) + (j & 7)] = st[TAIL0 + 9 * j + ru];
    }
  };

  // 1. the lane's RoPE frequency and the index reads of tiles 0..2;
  // ordinary stores into the KV buffers (the DMA intrinsic is not seen as a
  // writer of them, and without one the reads below could be folded away),
  // complete in every wave before any DMA is issued
  const double theta = a.rope.theta[min(tid, MAX_ROPE_PAIRS - 1)];
  const TileIdx ix0 = tile_idx(0, lane), ix1 = tile_idx(1, lane);
  TileIdx ixp = tile_idx(2, lane);  // index reads of tile t+2 during tile t
  buf0[tid] = make_uint4(0u, 0u, 0u, 0u);
  buf1[tid] = make_uint4(0u, 0u, 0u, 0u);
  if (KV8) {
    stg(1)[tid] = make_uint4(0u, 0u, 0u, 0u);
    // the row codes of tiles 0 and 1 (wave w writes rows 16w .. 16w+15)
    if ((lane >> 4) == wave) {
      rowtab[lane] = code_of(lane, ix0.em);
      rowtab[64 + lane] = code_of(64 + lane, ix1.em);
    }
  }
  lds_barrier();

  // 2. tile 0 requested (tile t+1 goes out during tile t's QK); bit j of
  // the masks: tile row j holds a candidate (tiles t and t+1)
  uint64_t vm_cur = __ballot(code_of(lane, ix0.em) != -1);
  uint64_t vm_n1 = __ballot(code_of(64 + lane, ix1.em) != -1);
  const int dma_row = dma_row_of(lane);
  const uint16_t* rp0[2] = {row_addr(code_of(dma_row, ix0.e0)), row_addr(code_of(dma_row + 8, ix0.e1))};
  const uint16_t* rp1[2] = {row_addr(code_of(64 + dma_row, ix1.e0)), row_addr(code_of(64 + dma_row + 8, ix1.e1))};
  if (KV8) {
    for (int q = 0; q < nq8; ++q) dma8(0, q, lane);
  } else {
#pragma unroll
    for (int q = 0; q < CPW; ++q) dma_one(buf0, rp0, q, lane);
  }

  // 3. the row's q (64 heads, contiguous) into buf1 by DMA while tile 0
  // loads, 1 KB per instruction: 16-byte piece p = NCH*h + c (head h, chunk
  // c), instruction i = p/64; lane l of instruction i loads piece
  // 64i + (l ^ (i%16)) into unit 64i + l, so that the fragment reads below
  // (16 heads of one chunk per 16 lanes) spread over the bank groups
  {
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + (int64_t)r * a.H * D;
    // (KV8: into the bf16 tile buffer, free until tile 0 is converted)
    uint4* qdst = KV8 ? buf0 : buf1;
#pragma unroll
    for (int q = 0; q < CPW; ++q) {
      const int i = CPW * wave + q;
      lds_dma16(qrow + 8 * (64 * i + (lane ^ (i & 15))), qdst + 64 * i);
    }
  }
  if (tid < a.d_rope / 2) {
    float cs, sn;
    rope_cs((double)ri.p, theta, &cs, &sn);
    rtab[tid] = make_float2(cs, sn);
  }
  // every wave's DMAs (tile 0 and q) and RoPE table writes are in
  __syncthreads();

  // 4. rotated query fragments (B operand: head h = 32hg + c32, chunk
  // c = 2ks + hi: piece p = NCH*h + c); at most 128 dims rotate (checked on
  // the host), all within the last eight K-steps
  constexpr int KR = KS > 8 ? KS - 8 : 0;
  v8bf qf[KS];
  {
    const int pb = NCH * (32 * hg + c32) + hi;
    const int rope0 = D - a.d_rope;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int pc = pb + 2 * ks, ic = pc >> 6;
      qf[ks] = *reinterpret_cast<const v8bf*>((KV8 ? buf0 : buf1) + ((pc & ~63) | ((pc & 63) ^ (ic & 15))));
      if (ks >= KR) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int c = 16 * ks + 8 * hi + 2 * u;
          const float2 csn = c >= rope0 ? rtab[(c - rope0) >> 1] : make_float2(1.f, 0.f);
          const float x0 = (float)qf[ks][2 * u], x1 = (float)qf[ks][2 * u + 1];
          qf[ks][2 * u] = (__bf16)(x0 * csn.x - x1 * csn.y);
          qf[ks][2 * u + 1] = (__bf16)(x0 * csn.y + x1 * csn.x);
        }
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // row addresses of the tile that tile t's QK requests (t+1; set at the
  // end of tile t-1)
  const uint16_t* rp_nxt[2] = {rp1[0], rp1[1]};

  v16f acc[HDT];
#pragma unroll
  for (int u = 0; u < HDT; ++u)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[u][i] = 0.f;
  float m_run = -INFINITY, l_part = 0.f;
  const float sl2 = a.scale * LOG2E;

  // K fragment base: row 32ch + c32 (group G = 4ch + c32/8, G&1 = g1),
  // chunk 2ks + hi: unit G*GU + 8(2ks + (hi ^ g1)) + c32%8 = kb + 16ks
  auto k_base = [&](int ln) {
    const int c = ln & 31, h = ln >> 5;
    return (4 * ch + (c >> 3)) * GU + 8 * (h ^ ((c >> 3) & 1)) + (c & 7);
  };
  // V^T fragment bases: rows 16kc + 8s + 4hi + k4 (G = 2kc + s, G&1 = s),
  // dims 32(ch*HDT + dtl) + 16g16 + 4j4 (chunk 4(ch*HDT + dtl) + cl with
  // cl = 2g16 + j4/2): unit base_s + 2kc*GU + 32dtl (elements x8)
  auto v_bases = [&](int ln, int& vb0, int& vb1) {
    const int h = ln >> 5, k4 = (ln & 15) >> 2, j4 = ln & 3, g16 = (ln & 31) >> 4;
    const int cl = 2 * g16 + (j4 >> 1);
    vb0 = (8 * cl + 4 * h + k4 + 32 * ch * HDT) * 8 + 4 * (j4 & 1);
    vb1 = (GU + 8 * (cl ^ 1) + 4 * h + k4 + 32 * ch * HDT) * 8 + 4 * (j4 & 1);
  };

  auto tile_step = [&](const uint4* sb, uint4* other, int t) {
    // tile t has landed in every wave's view
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(CSK_VMCNT_LGKM0(0));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const bool issue = t + 1 < ntiles;  // tile t+1
    // KV8: the staged tile t becomes the bf16 tile (every wave is past tile
    // t-1 and the query reads); its staging area then holds the probability
    // exchange of this tile
    if (KV8) {
      convert8(t);
      lds_barrier();
    }
    uint4* const pex = KV8 ? stg(t) : pex_b;

    // S^T[row 32ch + (8(i/4) + 4hi + i%4), head c32]; one DMA instruction
    // of tile t+1 per K-step block
    v16f s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
    {
      const int lq = fresh_lane();
      const int kb = k_base(lq);
      v8bf kf[2][QB];
      auto load_k = [&](int blk, v8bf (&dst)[QB]) {
#pragma unroll
        for (int u = 0; u < QB; ++u) {
          const int ks = blk * QB + u;
          dst[u] = *reinterpret_cast<const v8bf*>(sb + kb + 16 * ks);
        }
      };
      load_k(0, kf[0]);
#pragma unroll
      for (int blk = 0; blk < NQB; ++blk) {
        if (blk + 1 < NQB) load_k(blk + 1, kf[(blk + 1) & 1]);
        if (KV8) {
          if (issue && (blk & 1) == 0) dma8(t + 1, blk >> 1, lq);
        } else {
          if (issue && (blk & 1) == 0) dma_one(other, rp_nxt, blk >> 1, lq);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < QB; ++u) {
          const int ks = blk * QB + u;
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[blk & 1][u], qf[ks], s, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // mask (only when the tile has empty rows); this half's maxima to LDS
    const int lm = fresh_lane();
    if (vm_cur != ~0ull) {
      // this half's rows of the tile, shifted down by the lane's 4hi
      const uint32_t vmh = (uint32_t)(vm_cur >> (32 * ch + 4 * (lm >> 5)));
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 8 * (i >> 2) + (i & 3);
        s[i] = ((vmh >> row) & 1u) ? s[i] : -INFINITY;
      }
    }
    float tm = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) tm = fmaxf(tm, s[i]);
    tm = pair32_max(tm);
    if (lm < 32) mx[wave][lm] = tm;
    lds_barrier();
    // one running maximum for the head group (both halves compute it alike)
    tm = fmaxf(tm, mx[pw][lm & 31]) * sl2;
    const float mn = tm > m_run + 8.f ? tm : m_run;
    const float alpha = mn == m_run ? 1.f : __builtin_amdgcn_exp2f(m_run - mn);
    const bool moved = mn != m_run;
    m_run = mn;
    const float nm = mn == -INFINITY ? 0.f : -mn;
    v8bf pf[2];
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      // v_exp_f32 directly: arguments are <= 8; masked rows give 0
      const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], sl2, nm));
      ps += pv;
      pf[i >> 3][i & 7] = (__bf16)pv;
    }
    l_part = l_part * alpha + ps;
    pex[(2 * wave) * 64 + lm] = __builtin_bit_cast(uint4, pf[0]);
    pex[(2 * wave + 1) * 64 + lm] = __builtin_bit_cast(uint4, pf[1]);
    if (__ballot(moved) != 0ull) {
#pragma unroll
      for (int u = 0; u < HDT; ++u) acc[u] *= alpha;
    }
    lds_barrier();
    v8bf pp[2];
    const int lp = fresh_lane();
    pp[0] = __builtin_bit_cast(v8bf, pex[(2 * pw) * 64 + lp]);
    pp[1] = __builtin_bit_cast(v8bf, pex[(2 * pw + 1) * 64 + lp]);
    // O^T[dv, head] += V^T P^T over the 64 rows: K-chunk kc holds rows
    // 32(kc/2) + 16(kc%2) + {4hi+k, 8+4hi+k}, k < 4, whose probabilities are
    // elements 8(kc%2) .. +7 of half kc/2's lanes
    {
      const uint16_t* sb16 = reinterpret_cast<const uint16_t*>(sb);
      int vbase0, vbase1;
      v_bases(lp, vbase0, vbase1);
      constexpr int VB = R32_VB;
      constexpr int NV = 4 * HDT, NVB = NV / VB;
      v8bf vf[2][VB];
      auto load_v = [&](int blk, v8bf (&dst)[VB]) {
#pragma unroll
        for (int u = 0; u < VB; ++u) {
          const int v = blk * VB + u;
          const int kc = v / HDT, dtl = v % HDT;
          const int off = (2 * kc * GU + 32 * dtl) * 8;
          dst[u] = vt_fragment(sb16 + vbase0 + off, sb16 + vbase1 + off);
        }
      };
      load_v(0, vf[0]);
#pragma unroll
      for (int blk = 0; blk < NVB; ++blk) {
        if (blk + 1 < NVB) load_v(blk + 1, vf[(blk + 1) & 1]);
        // the second half of tile t+1's DMA, spread over the PV blocks
        constexpr int QD = (CPW + 1) / 2;  // issued during QK
        if (KV8) {
          if (issue && 9 + blk < nq8) dma8(t + 1, 9 + blk, lp);  // (KV8: nine go out during QK)
        } else {
          if (issue && blk < CPW - QD) dma_one(other, rp_nxt, QD + blk, lp);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < VB; ++u) {
          const int v = blk * VB + u;
          const int kc = v / HDT, dtl = v % HDT;
          const v8bf pb = (kc >> 1) == ch ? pf[kc & 1] : pp[kc & 1];
          acc[dtl] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[blk & 1][u], pb, acc[dtl], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // tile t+2 (index reads made a tile ago): the row addresses tile t+1's
    // QK requests and its mask; then tile t+3's index reads
    const int le = fresh_lane();
    const int dre = dma_row_of(le);
    if (KV8) {
      // tile t+2's row codes (its DMA goes out during tile t+1; tile t's
      // table, the one overwritten, was read during tile t-1)
      if ((le >> 4) == wave) rowtab[64 * (t & 1) + le] = code_of(64 * (t + 2) + le, ixp.em);
    } else {
      rp_nxt[0] = row_addr(code_of(64 * (t + 2) + dre, ixp.e0));
      rp_nxt[1] = row_addr(code_of(64 * (t + 2) + dre + 8, ixp.e1));
    }
    vm_cur = vm_n1;
    vm_n1 = __ballot(code_of(64 * (t + 2) + le, ixp.em) != -1);
    ixp = tile_idx(t + 3, le);
  };

  // (KV8: every tile is converted into buf0; the staging areas alternate)
  for (int t = 0; t < ntiles; t += 2) {
    tile_step(buf0, buf1, t);
    if (t + 1 < ntiles) tile_step(KV8 ? buf0 : buf1, buf0, t + 1);
  }

  // 4. the head group's sum over both halves, the sink, the output
  const int lo_ = fresh_lane();
  const int c32o = lo_ & 31, hio = lo_ >> 5, heado = 32 * hg + c32o;
  const float l_half = pair32_sum(l_part);
  if (hio == 0) xl[wave][c32o] = l_half;
  __builtin_amdgcn_s_waitcnt(CSK_VMCNT_LGKM0(0));  // no DMA outlives the workgroup
  __syncthreads();
  const float l_tot = l_half + xl[pw][c32o];
  // the output scale: 1 for a partial of a split row (unnormalised O, merged
  // with the sink by the merge kernel), else the softmax normaliser with the
  // sink
  float f = 1.f, M = m_run, z = l_tot;
  if (a.nch == 1) {
    const float s2 = a.sink ? a.sink[heado] * LOG2E : -INFINITY;
    M = fmaxf(m_run, s2);
    f = 0.f;
    z = 0.f;
    if (M != -INFINITY) {
      const float fo = m_run == -INFINITY ? 0.f : exp2f(m_run - M);
      z = l_tot * fo + (a.sink ? exp2f(s2 - M) : 0.f);
      f = z > 0.f ? fo / z : 0.f;
    }
  }
  // 5. O through LDS as bf16 (every wave is past its last tile: both
  // buffers are free), so that each store instruction writes contiguous
  // memory. Head group hg uses buffer hg; the 8-byte unit du (value dims
  // 4du..4du+3) of head h's row sits at (h%32)*DU + 2*((du/2) ^ h%16) +
  // du%2 (h%8 when a row has 8 pairs), which keeps the scattered writes on distinct bank groups and
  // leaves each pair of units (16 bytes, one store) adjacent for the
  // row-wise reads. (Rounded once, as it is stored; the same bits as
  // rounding after the staging.)
  constexpr int DU = DV / 4;
  constexpr int SWM = DU / 2 >= 16 ? 15 : DU / 2 - 1;  // pair swizzle mask (within a row)
  static_assert((DU / 2) % (SWM + 1) == 0 && (64 * DU) % 512 == 0 && 32 * DV * 2 <= TU * 16 &&
                    32 * DV * 2 <= (KV8 ? 2 * STU : TU) * 16,
                "staging layout");
  {
    uint2* st = reinterpret_cast<uint2*>(hg ? buf1 : buf0);
#pragma unroll
    for (int u = 0; u < HDT; ++u)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int du = 8 * ch * HDT + 8 * u + 2 * q4 + hio;
        const v2bf p0 = {(__bf16)(acc[u][4 * q4] * f), (__bf16)(acc[u][4 * q4 + 1] * f)};
        const v2bf p1 = {(__bf16)(acc[u][4 * q4 + 2] * f), (__bf16)(acc[u][4 * q4 + 3] * f)};
        st[c32o * DU + 2 * ((du >> 1) ^ (c32o & SWM)) + (du & 1)] =
            make_uint2(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1));
      }
  }
  lds_barrier();
  {
    // eight value dims (one staged pair of units) per lane and store
    const int ls = fresh_lane() + 64 * wave;
    const int64_t row0 = a.nch > 1 ? ((int64_t)r * a.nch + split) * a.H : (int64_t)r * a.H;
    uint16_t* dst = reinterpret_cast<uint16_t*>(a.nch > 1 ? static_cast<void*>(a.part_o) : a.out);
#pragma unroll 4
    for (int k = 0; k < 64 * DU / 512; ++k) {
      const int idx = 256 * k + ls;
      const int h = idx / (DU / 2), pd = idx % (DU / 2);
      const uint2* st = reinterpret_cast<const uint2*>(h >= 32 ? buf1 : buf0);
      const uint4 v = *reinterpret_cast<const uint4*>(st + (h & 31) * DU + 2 * (pd ^ (h & SWM)));
      *reinterpret_cast<uint4*>(dst + (row0 + h) * DV + 8 * pd) = v;
    }
  }
  if (ch == 0 && hio == 0) {
    if (a.nch > 1) {
      float* pm = a.part_ml + (((int64_t)r * a.nch + split) * a.H + heado) * 2;
      pm[0] = m_run;
      pm[1] = l_tot;
    } else if (a.lse) {
      a.lse[(int64_t)r * a.H + heado] = M == -INFINITY ? -INFINITY : (M + log2f(z)) * LN2;
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
      rope_cs((double)ri.p, a.rope.theta[(c - rope0) / 2], &cs, &sn);
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
// One workgroup of two waves per (row, head): log-sum-exp combination of
// the chunks' partial (m, l, o) with the sink (o in fp32, or in bf16 from the
// streamed-row kernel, whose partials are as large as its KV reads and so
// are written and read at half the bytes). The chunks' (m, l) pairs are
// read once into LDS and turned into weights 2^(m_c - M); each thread then
// sums four value dims over the chunks with MB independent 16-byte loads in
// flight (the merge is a short, latency-bound pass over the partials).
constexpr int MERGE_MAX_CH = 2048;

template <typename T>
__global__ __launch_bounds__(128) void attn_merge_kernel(AttnArgs a) {
  __shared__ float wts[MERGE_MAX_CH];
  __shared__ float lsv[MERGE_MAX_CH];
  __shared__ float red[4];
  __shared__ float fin[2];
  const int r = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = a.nch;
  const float* ml = a.part_ml + ((int64_t)r * nch * a.H + h) * 2;
  const int64_t cstride = (int64_t)a.H * 2;
  float m = -INFINITY;
  for (int c = tid; c < nch; c += 128) {
    const float2 v = *reinterpret_cast<const float2*>(ml + c * cstride);
    wts[c] = v.x;
    lsv[c] = v.y;
    m = fmaxf(m, v.x);
  }
  m = wave_max(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  m = fmaxf(red[0], red[1]);
  float l = 0.f;
  for (int c = tid; c < nch; c += 128) {
    const float mc = wts[c];
    const float w = (mc == -INFINITY) ? 0.f : exp2f(mc - m);
    wts[c] = w;
    l += w * lsv[c];
  }
  l = wave_sum(l);
  if (lane == 0) red[2 + wave] = l;
  __syncthreads();
  if (tid == 0) {
    float M, inv_z, lse;
    finish_row(m, red[2] + red[3], a.sink, h, &M, &inv_z, &lse);
    fin[0] = (m == -INFINITY) ? 0.f : exp2f(m - M) * inv_z;
    fin[1] = lse;
  }
  __syncthreads();
  const float f = fin[0];
  const float* po = a.part_o + ((int64_t)r * nch * a.H + h) * a.dv;
  const int64_t ostride = (int64_t)a.H * a.dv;
  const int64_t orow = ((int64_t)r * a.H + h) * a.dv;
  auto store4 = [&](int d, float4 o) {
    if (sizeof(T) == 4) {
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + orow + d) =
          make_float4(o.x * f, o.y * f, o.z * f, o.w * f);
    } else {
      const uint32_t lo = f32_to_bf16_bits(o.x * f) | (f32_to_bf16_bits(o.y * f) << 16);
      const uint32_t hi = f32_to_bf16_bits(o.z * f) | (f32_to_bf16_bits(o.w * f) << 16);
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + orow + d) = make_uint2(lo, hi);
    }
  };
  if (a.part_bf16) {
    // bf16 partials (dv is a multiple of 64 on this path)
    const uint16_t* pb = reinterpret_cast<const uint16_t*>(a.part_o) + ((int64_t)r * nch * a.H + h) * a.dv;
    constexpr int MB = 16;
    for (int d = 4 * tid; d < a.dv; d += 4 * 128) {
      float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
      auto acc4 = [&](uint2 v, float w) {
        o.x += bf16_bits_to_f32(v.x & 0xffffu) * w;
        o.y += bf16_bits_to_f32(v.x >> 16) * w;
        o.z += bf16_bits_to_f32(v.y & 0xffffu) * w;
        o.w += bf16_bits_to_f32(v.y >> 16) * w;
      };
      int c = 0;
      for (; c + MB <= nch; c += MB) {
        uint2 v[MB];
#pragma unroll
        for (int u = 0; u < MB; ++u) v[u] = *reinterpret_cast<const uint2*>(pb + (c + u) * ostride + d);
#pragma unroll
        for (int u = 0; u < MB; ++u) acc4(v[u], wts[c + u]);
      }
      for (; c < nch; ++c) acc4(*reinterpret_cast<const uint2*>(pb + c * ostride + d), wts[c]);
      store4(d, o);
    }
  } else if ((a.dv & 3) == 0) {
    constexpr int MB = 16;
    for (int d = 4 * tid; d < a.dv; d += 4 * 128) {
      float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
      int c = 0;
      for (; c + MB <= nch; c += MB) {
        float4 v[MB];
#pragma unroll
        for (int u = 0; u < MB; ++u) v[u] = *reinterpret_cast<const float4*>(po + (c + u) * ostride + d);
#pragma unroll
        for (int u = 0; u < MB; ++u) {
          const float w = wts[c + u];
          o.x += v[u].x * w;
          o.y += v[u].y * w;
          o.z += v[u].z * w;
          o.w += v[u].w * w;
        }
      }
      for (; c < nch; ++c) {
        const float4 v = *reinterpret_cast<const float4*>(po + c * ostride + d);
        const float w = wts[c];
        o.x += v.x * w;
        o.y += v.y * w;
        o.z += v.z * w;
        o.w += v.w * w;
      }
      store4(d, o);
    }
  } else {
    for (int d = tid; d < a.dv; d += 128) {
      float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
      int c = 0;
      for (; c + 4 <= nch; c += 4) {
        o0 += po[(c + 0) * ostride + d] * wts[c + 0];
        o1 += po[(c + 1) * ostride + d] * wts[c + 1];
        o2 += po[(c + 2) * ostride + d] * wts[c + 2];
        o3 += po[(c + 3) * ostride + d] * wts[c + 3];
      }
      for (; c < nch; ++c) o0 += po[c * ostride + d] * wts[c];
      const float o = ((o0 + o1) + (o2 + o3)) * f;
      if (sizeof(T) == 4) reinterpret_cast<float*>(a.out)[orow + d] = o;
      else reinterpret_cast<uint16_t*>(a.out)[orow + d] = (uint16_t)f32_to_bf16_bits(o);
    }
  }
  if (a.lse && tid == 0) a.lse[(int64_t)r * a.H + h] = fin[1];
}

// Merge of bf16 partials from at most 64 chunks with dv <= 512, dv % 8 == 0
// (split rows of the streamed-row kernel at decode): one workgroup of eight
// waves per (row, head); wave g sums chunks g, g + 8, ... over eight value
// dims per lane. Every partial and (m, l) load is issued before any of them
// is needed, so the pass costs one memory round trip instead of one per
// dependent step; each wave forms all chunk weights itself (one chunk per
// lane, no barrier), and the eight waves' sums meet once in LDS.
constexpr int MERGE8_WAVES = 8;

template <typename T, int PER>
__global__ __launch_bounds__(64 * MERGE8_WAVES) void attn_merge8_kernel(AttnArgs a) {
  __shared__ float4 red[MERGE8_WAVES - 1][2][64];
  const int r = blockIdx.x, h = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nch = a.nch;
  const int64_t ostride = (int64_t)a.H * a.dv;
  const uint16_t* pb = reinterpret_cast<const uint16_t*>(a.part_o) + ((int64_t)r * nch * a.H + h) * a.dv;
  const int d = 8 * lane;
  const bool dok = d < a.dv;
  const int dd = dok ? d : 0;
  uint4 v[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int c = min(g + MERGE8_WAVES * u, nch - 1);  // unconditional: the loads issue together
    v[u] = *reinterpret_cast<const uint4*>(pb + c * ostride + dd);
  }
  const float* ml = a.part_ml + ((int64_t)r * nch * a.H + h) * 2;
  const float2 mlc = *reinterpret_cast<const float2*>(ml + (int64_t)min(lane, nch - 1) * a.H * 2);
  const float mc = lane < nch ? mlc.x : -INFINITY;
  const float m = wave_max(mc);
  const float w = mc == -INFINITY ? 0.f : exp2f(mc - m);
  const float l = wave_sum(lane < nch ? w * mlc.y : 0.f);
  float M, inv_z, lse;
  finish_row(m, l, a.sink, h, &M, &inv_z, &lse);
  const float f = (m == -INFINITY) ? 0.f : exp2f(m - M) * inv_z;
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = 0.f;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int c = g + MERGE8_WAVES * u;  // < 64
    const float wc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), c));
    if (c < nch) {
      const uint32_t q[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[2 * i] += bf16_bits_to_f32(q[i] & 0xffffu) * wc;
        o[2 * i + 1] += bf16_bits_to_f32(q[i] >> 16) * wc;
      }
    }
  }
  if (g > 0) {
    red[g - 1][0][lane] = make_float4(o[0], o[1], o[2], o[3]);
    red[g - 1][1][lane] = make_float4(o[4], o[5], o[6], o[7]);
  }
  __syncthreads();
  if (g != 0) return;
#pragma unroll
  for (int j = 0; j < MERGE8_WAVES - 1; ++j) {
    const float4 x = red[j][0][lane], y = red[j][1][lane];
    o[0] += x.x; o[1] += x.y; o[2] += x.z; o[3] += x.w;
    o[4] += y.x; o[5] += y.y; o[6] += y.z; o[7] += y.w;
  }
  if (dok) {
    const int64_t orow = ((int64_t)r * a.H + h) * a.dv + d;
    if (sizeof(T) == 4) {
      float4* op = reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + orow);
      op[0] = make_float4(o[0] * f, o[1] * f, o[2] * f, o[3] * f);
      op[1] = make_float4(o[4] * f, o[5] * f, o[6] * f, o[7] * f);
    } else {
      uint32_t q[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) q[i] = f32_to_bf16_bits(o[2 * i] * f) | (f32_to_bf16_bits(o[2 * i + 1] * f) << 16);
      *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.out) + orow) = make_uint4(q[0], q[1], q[2], q[3]);
    }
  }
  if (a.lse && lane == 0) a.lse[(int64_t)r * a.H + h] = lse;
}

// The same merge for at most NCHM partials and many (row, head) pairs
// (batched decode rows split over few workgroups): one wave per (row,
// head), four heads per workgroup. The
// wave issues every partial's load at once, forms the chunk weights itself
// and sums the chunks in ascending order; no LDS, no barrier.
template <typename T, int NCHM>
__global__ __launch_bounds__(256) void attn_merge_wave_kernel(AttnArgs a) {
  const int r = blockIdx.x;
  const int h = 4 * blockIdx.y + (int)(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int nch = a.nch;
  const int64_t ostride = (int64_t)a.H * a.dv;
  const uint16_t* pb = reinterpret_cast<const uint16_t*>(a.part_o) + ((int64_t)r * nch * a.H + h) * a.dv;
  const int d = 8 * lane;
  const bool dok = d < a.dv;
  const int dd = dok ? d : 0;
  uint4 v[NCHM];
#pragma unroll
  for (int u = 0; u < NCHM; ++u) {
    const int c = min(u, nch - 1);  // unconditional: the loads issue together
    v[u] = *reinterpret_cast<const uint4*>(pb + c * ostride + dd);
  }
  const float* ml = a.part_ml + ((int64_t)r * nch * a.H + h) * 2;
  const float2 mlc = *reinterpret_cast<const float2*>(ml + (int64_t)min(lane, nch - 1) * a.H * 2);
  const float mc = lane < nch ? mlc.x : -INFINITY;
  const float m = wave_max(mc);
  const float w = mc == -INFINITY ? 0.f : exp2f(mc - m);
  const float l = wave_sum(lane < nch ? w * mlc.y : 0.f);
  float M, inv_z, lse;
  finish_row(m, l, a.sink, h, &M, &inv_z, &lse);
  const float f = (m == -INFINITY) ? 0.f : exp2f(m - M) * inv_z;
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = 0.f;
#pragma unroll
  for (int u = 0; u < NCHM; ++u) {
    const float wc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), u));
    if (u < nch) {
      const uint32_t q[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[2 * i] += bf16_bits_to_f32(q[i] & 0xffffu) * wc;
        o[2 * i + 1] += bf16_bits_to_f32(q[i] >> 16) * wc;
      }
    }
  }
  if (dok) {
    const int64_t orow = ((int64_t)r * a.H + h) * a.dv + d;
    if (sizeof(T) == 4) {
      float4* op = reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + orow);
      op[0] = make_float4(o[0] * f, o[1] * f, o[2] * f, o[3] * f);
      op[1] = make_float4(o[4] * f, o[5] * f, o[6] * f, o[7] * f);
    } else {
      uint32_t q[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) q[i] = f32_to_bf16_bits(o[2 * i] * f) | (f32_to_bf16_bits(o[2 * i + 1] * f) << 16);
      *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.out) + orow) = make_uint4(q[0], q[1], q[2], q[3]);
    }
  }
  if (a.lse && lane == 0) a.lse[(int64_t)r * a.H + h] = lse;
}

template <typename T>
static int launch_merge8(const AttnArgs& a, unsigned R, int H, hipStream_t s) {
  // (a wave per pair: needs enough pairs to spread its loads; few rows keep
  // eight waves per pair)
  if (a.nch <= 16 && H % 4 == 0 && (int64_t)R * H >= 1024) {
    dim3 grid(R, H / 4), block(256);
    return a.nch <= 8 ? launch("attn_merge", attn_merge_wave_kernel<T, 8>, grid, block, 0, s, a)
                      : launch("attn_merge", attn_merge_wave_kernel<T, 16>, grid, block, 0, s, a);
  }
  dim3 grid(R, H), block(64 * MERGE8_WAVES);
  switch ((a.nch + MERGE8_WAVES - 1) / MERGE8_WAVES) {
    case 1: return launch("attn_merge", attn_merge8_kernel<T, 1>, grid, block, 0, s, a);
    case 2: return launch("attn_merge", attn_merge8_kernel<T, 2>, grid, block, 0, s, a);
    case 3: return launch("attn_merge", attn_merge8_kernel<T, 3>, grid, block, 0, s, a);
    case 4: return launch("attn_merge", attn_merge8_kernel<T, 4>, grid, block, 0, s, a);
    case 5: return launch("attn_merge", attn_merge8_kernel<T, 5>, grid, block, 0, s, a);
    case 6: return launch("attn_merge", attn_merge8_kernel<T, 6>, grid, block, 0, s, a);
    case 7: return launch("attn_merge", attn_merge8_kernel<T, 7>, grid, block, 0, s, a);
    default: return launch("attn_merge", attn_merge8_kernel<T, 8>, grid, block, 0, s, a);
  }
}

// ------------------------------------------------------------ host side
struct AttnPlan {
  int chunk, nch, tiles, extra;
  bool mfma, whole;
  bool row32;   // 64 heads: the streaming 32x32 kernel, rows split over nch workgroups
  bool qtile;   // dense prefill: query-row tiles
  int qt_ct;    // column tiles per wave of the query-tile kernel
  size_t off_o, off_ml, total;
};

static bool mfma_shape(int H, int D, int dv, int dtype) {
  if (dtype != CSK_BF16 || H % 16 || H > 64) return false;
  return (D == 576 && (dv == 512 || dv == 576)) || (D == 128 && dv == 128) ||
         (D == 64 && dv == 64) || (D == 256 && dv == 256);
}

// The whole-chunk kernel splits its DMA blocks (D/4 per chunk) over H/16
// waves.
static bool chunk_kernel_shape(int H, int D) { return (D / 4) % (H / 16) == 0; }

// The query-tile kernel keeps CT column tiles of 16 heads per wave (its q
// and accumulator registers grow with D), and a workgroup's four waves must
// cover whole rows.
static int qtile_ct(int H, int D) {
  const int ct = D <= 128 ? 2 : 1;
  return (D <= 256 && (4 * ct) % (H / 16) == 0) ? ct : 0;
}

// The 32x32 streamed-row kernel: 64 heads, value dims split into two halves
// of 32-row tiles, DMA chunks split over four waves.
static bool row32_shape(int D, int dv) {
  return (D == 576 && dv == 512) || (D == 256 && dv == 256) || (D == 128 && dv == 128) || (D == 64 && dv == 64);
}

// max_wg: workgroup cap of a split-row launch (0: about one per CU).
static AttnPlan plan_attn(bool dense, int B, int T, int H, int D, int dv, int Lc, int W, int dtype,
                          int max_wg) {
  AttnPlan p{};
  const int64_t R = (int64_t)B * T;
  const int total = Lc + W;
  p.mfma = mfma_shape(H, D, dv, dtype);
  // dense attention over many consecutive query rows: query-row tiles, rows
  // kept whole
  p.qt_ct = p.mfma ? qtile_ct(H, D) : 0;
  p.qtile = dense && p.qt_ct > 0 && T >= 16;
  if (p.qtile) {
    p.chunk = total;
    p.nch = 1;
    return p;
  }
  // 64 heads of a supported shape: the streaming 32x32 kernel; rows are
  // split into runs of 64-row tiles until about one workgroup per CU
  // (few rows with long candidate lists: decode)
  if (p.mfma && H == 64 && row32_shape(D, dv) && (dense || Lc >= 1)) {
    const int64_t nt = ceil_div(total, 64);
    // about one workgroup per CU, or at most the cap in all (at least one a row)
    int64_t nch = max_wg > 0 ? max_wg / (int64_t)R : ceil_div(256, R);
    nch = nch < 1 ? 1 : nch;
    nch = nch < nt ? nch : nt;
    // the fewest runs that keep the longest one: a row of 34 tiles over 8
    // workgroups has runs of 5 and 4 tiles, over 7 the same longest run of 5
    // with an eighth fewer partials to write and merge
    nch = ceil_div(nt, ceil_div(nt, nch));
    p.row32 = true;
    p.chunk = total;
    p.nch = (int)(nch < 1 ? 1 : nch);
  } else {
  const int gran = p.mfma ? 32 : 64;
  int64_t want = ceil_div(R * (int64_t)total, 256);  // aim at ~256 workgroups
  int64_t ch = ceil_div(want < 128 ? 128 : want, gran) * gran;
  if (ch >= total) ch = ceil_div(total > 0 ? total : 1, gran) * gran;
  if (p.mfma && ch > MAX_CHUNK) ch = MAX_CHUNK;
  // rows split into chunks (few rows, long candidate lists: decode) go to
  // the whole-chunk kernel; rows kept whole (prefill) to the streaming one
  p.whole = p.mfma && chunk_kernel_shape(H, D) && ch < total;
  if (p.whole) {
    // 2- or 4-tile chunks: a small cost model of one launch (workgroup
    // waves over the CUs x per-workgroup time, plus the partials each chunk
    // writes and the merge reads); the 4-tile workgroup holds a CU alone
    auto cost = [&](int tiles) {
      const int64_t wgs = R * ceil_div(total, 32 * tiles);
      const int64_t slots = 256 * (tiles == 2 ? 2 : 1);
      const double waves = (double)ceil_div(wgs, slots);
      const double partial_us = (double)wgs * H * dv * 8 / 4.0e6;  // write + read at ~4 TB/s
      return waves * (20.0 + 2.0 * tiles) + partial_us;
    };
    p.tiles = (D * 2 * 32 * 4 > 150 * 1024 || cost(2) < cost(4)) ? 2 : 4;
    ch = 32 * p.tiles;  // the chunk is resident in LDS as a whole
    // a few rows past the tiles (VALU) when that saves a wave of
    // workgroups: 1M-context HCA has 8320 candidates, 65 x 128, 64 x 130
    const int64_t slots = 256 * (p.tiles == 2 ? 2 : 1);
    if (R * ceil_div(total, ch) > slots)
      for (int e = 1; e <= MAX_EXTRA; ++e)
        if (ceil_div(R * ceil_div(total, ch + e), slots) < ceil_div(R * ceil_div(total, ch), slots)) {
          p.extra = e;
          ch += e;
          break;
        }
  }
  p.chunk = (int)ch;
  p.nch = (int)ceil_div(total > 0 ? total : 1, ch);
  }
  size_t o = 0;
  if (p.nch > 1) {
    p.off_o = o;
    o += (size_t)R * p.nch * H * dv * (p.row32 ? 2 : 4);  // the streamed-row kernel writes bf16
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
                       int kv_dtype, void* out, float* lse, int max_wg, void* workspace,
                       size_t ws_bytes, void* stream) {
  clear_error();
  std::string f(fn);
  if (!q || !q_pos || !kv_c || !out) return fail(CSK_EINVAL, f + ": null pointer");
  // the kernels move q, the caches, the output and the partials in 16-byte pieces
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(kv_c) | reinterpret_cast<uintptr_t>(kv_w) |
       reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(workspace)) & 15)
    return fail(CSK_EINVAL, f + ": q, kv_c, kv_w, out and workspace must be 16-byte aligned");
  if (!dense && !idx) return fail(CSK_EINVAL, f + ": null idx");
  if (dense && !n_entries) return fail(CSK_EINVAL, f + ": null n_entries");
  if (B <= 0 || T <= 0 || H <= 0 || D <= 0 || (D & 1) || dv <= 0 || dv > D || Nmax <= 0)
    return fail(CSK_EINVAL, f + ": need positive B, T, H, Nmax, even D and 0 < dv <= D");
  if (d_rope < 0 || d_rope > D || (d_rope & 1)) return fail(CSK_EINVAL, f + ": bad d_rope");
  if (d_rope > 2 * MAX_ROPE_PAIRS)
    return fail(CSK_EUNSUPPORTED, f + ": at most 128 rotated channels are built");
  if (W < 0 || S_w < 0 || (S_w > 0 && (!kv_w || !w_pos0)))
    return fail(CSK_EINVAL, f + ": bad window arguments");
  if (!dense && k < 0) return fail(CSK_EINVAL, f + ": k must be >= 0");
  if (dense && m <= 0) return fail(CSK_EINVAL, f + ": m must be > 0");
  if (dtype != CSK_BF16 && dtype != CSK_F32)
    return fail(CSK_EUNSUPPORTED, f + ": dtype must be CSK_BF16 or CSK_F32");
  if (dv > 576) return fail(CSK_EUNSUPPORTED, f + ": dv > 576 not built");
  if (max_wg < 0) return fail(CSK_EINVAL, f + ": max_workgroups must be >= 0");
  const bool kv8 = kv_dtype == CSK_FP8KV;
  if (kv_dtype != dtype && !kv8)
    return fail(CSK_EUNSUPPORTED, f + ": kv_dtype must equal dtype or be CSK_FP8KV");
  if (kv8 && (dtype != CSK_BF16 || H != 64 || D != 576 || dv != 512 || d_rope != 64))
    return fail(CSK_EUNSUPPORTED,
                f + ": FP8 KV entries are built for bf16 queries, 64 heads, D = 576 (512 + 64 RoPE), dv = 512");
  const int Wslots = S_w > 0 ? W : 0;
  const int Lc = dense ? Nmax : k;
  AttnPlan p = plan_attn(dense, B, T, H, D, dv, Lc, Wslots, dtype, max_wg);
  if (p.nch > MERGE_MAX_CH || (int64_t)p.nch * H > 65535 || (int64_t)B * T > (1LL << 30))
    return fail(CSK_EUNSUPPORTED, f + ": problem too large");
  if (p.total > 0 && (!workspace || ws_bytes < p.total))
    return fail(CSK_EWORKSPACE, f + ": workspace smaller than the *_workspace_size() value");
  if (const int dc = check_device(f); dc != CSK_OK) return dc;
  AttnArgs a{};
  a.q = q; a.q_pos = q_pos; a.kv_c = kv_c; a.idx = idx; a.n_entries = n_entries;
  a.kv_w = kv_w; a.w_pos0 = w_pos0; a.sink = sink;
  a.B = B; a.T = T; a.H = H; a.D = D; a.dv = dv; a.d_rope = d_rope; a.Nmax = Nmax; a.k = k;
  a.m = m; a.S_w = S_w; a.W = Wslots; a.Lc = Lc; a.chunk = p.chunk; a.nch = p.nch; a.extra = p.extra;
  a.scale = scale; a.dense = dense;
  fill_rope_table(&a.rope, d_rope, (double)rope_base);
  a.out = out; a.lse = lse;
  char* ws = reinterpret_cast<char*>(workspace);
  a.part_o = p.nch > 1 ? reinterpret_cast<float*>(ws + p.off_o) : nullptr;
  a.part_ml = p.nch > 1 ? reinterpret_cast<float*>(ws + p.off_ml) : nullptr;
  a.part_bf16 = p.row32;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const unsigned R = (unsigned)(B * T);
  int rc;
  if (p.qtile) {
    if (d_rope > 2 * QTILE_ROPE_PAIRS)
      return fail(CSK_EUNSUPPORTED, f + ": dense prefill with more than 64 rotated channels is not built");
    const int HG = H / 16, CT = p.qt_ct, TQ = 4 * CT / HG;
    dim3 grid((unsigned)(B * ceil_div(T, TQ))), block(256);
    rc = CSK_EUNSUPPORTED;
#define CSK_QT_CASE(d, v, hg, ct) \
  if (D == d && dv == v && HG == hg && CT == ct) rc = launch("attn_bf16_dense", attn_bf16_qtile_kernel<d, v, hg, ct>, grid, block, 0, s, a);
    CSK_QT_CASE(128, 128, 1, 2) CSK_QT_CASE(128, 128, 2, 2) CSK_QT_CASE(128, 128, 4, 2)
    CSK_QT_CASE(64, 64, 1, 2) CSK_QT_CASE(64, 64, 2, 2) CSK_QT_CASE(64, 64, 4, 2)
    CSK_QT_CASE(256, 256, 1, 1) CSK_QT_CASE(256, 256, 2, 1) CSK_QT_CASE(256, 256, 4, 1)
#undef CSK_QT_CASE
    return rc;
  }
  if (kv8 && !p.row32) return fail(CSK_EUNSUPPORTED, f + ": FP8 KV entries need the 64-head streamed-row kernel");
  if (p.row32) {
    rc = CSK_EUNSUPPORTED;
    const dim3 grid(R, p.nch);
#define CSK_R32_CASE(d, v)                                                                       \
  if (D == d && dv == v && !kv8)                                                                 \
    rc = dense ? launch("attn_bf16_dense", attn_bf16_row32_kernel<d, v, true, false>, grid, dim3(256), 0, s, a) \
               : launch("attn_bf16_sparse", attn_bf16_row32_kernel<d, v, false, false>, grid, dim3(256), 0, s, a);
    CSK_R32_CASE(576, 512) CSK_R32_CASE(256, 256) CSK_R32_CASE(128, 128) CSK_R32_CASE(64, 64)
#undef CSK_R32_CASE
    if (kv8)
      rc = dense ? launch("attn_bf16_dense", attn_bf16_row32_kernel<576, 512, true, true>, grid, dim3(256), 0, s, a)
                 : launch("attn_bf16_sparse", attn_bf16_row32_kernel<576, 512, false, true>, grid, dim3(256), 0,
                          s, a);
  } else if (p.mfma) {
    dim3 grid(R, p.nch), block(64 * (H / 16));
const int NW = H / 16;
    const char* kname = dense ? "attn_bf16_dense" : "attn_bf16_sparse";
#define CSK_ATT_CASE(d, v, nw)                                                         \
  if (D == d && dv == v && NW == nw) {                                                 \
    if (p.whole) {                                                                     \
      constexpr int nwc = (d / 4) % nw == 0 ? nw : 1;                                  \
      if (p.tiles == 2)                                                                \
        rc = dense ? launch(kname, attn_bf16_chunk_kernel<d, v, nwc, true, 2>, grid, block, 0, s, a) \
                   : launch(kname, attn_bf16_chunk_kernel<d, v, nwc, false, 2>, grid, block, 0, s, a); \
      else                                                                             \
        rc = dense ? launch(kname, attn_bf16_chunk_kernel<d, v, nwc, true, 4>, grid, block, 0, s, a) \
                   : launch(kname, attn_bf16_chunk_kernel<d, v, nwc, false, 4>, grid, block, 0, s, a); \
    } else                                                                             \
      rc = launch("attn_bf16_stream", attn_bf16_kernel<d, v, nw>, grid, block, 0, s, a); \
  }
#define CSK_ATT_NW(d, v) CSK_ATT_CASE(d, v, 1) CSK_ATT_CASE(d, v, 2) CSK_ATT_CASE(d, v, 3) CSK_ATT_CASE(d, v, 4)
    rc = CSK_EUNSUPPORTED;
    CSK_ATT_NW(576, 512) CSK_ATT_NW(576, 576) CSK_ATT_NW(128, 128) CSK_ATT_NW(64, 64) CSK_ATT_NW(256, 256)
#undef CSK_ATT_NW
#undef CSK_ATT_CASE
  } else {
    dim3 grid(R, p.nch * H), block(64);
    const size_t lds = (size_t)D * 4 + 64 * 4 + 64 * 8;
    rc = dtype == CSK_F32 ? launch("attn_valu", attn_valu_kernel<float>, grid, block, lds, s, a)
                          : launch("attn_valu", attn_valu_kernel<uint16_t>, grid, block, lds, s, a);
  }
  if (rc != CSK_OK || p.nch == 1) return rc;
  if (a.part_bf16 && p.nch <= 8 * MERGE8_WAVES && dv % 8 == 0 && dv <= 512)
    return dtype == CSK_F32 ? launch_merge8<float>(a, R, H, s) : launch_merge8<uint16_t>(a, R, H, s);
  dim3 mg(R, H), mb(128);
  return dtype == CSK_F32 ? launch("attn_merge", attn_merge_kernel<float>, mg, mb, 0, s, a)
                          : launch("attn_merge", attn_merge_kernel<uint16_t>, mg, mb, 0, s, a);
}

}  // namespace csk

extern "C" {

size_t sparse_attn_workspace_size(int B, int T, int H, int D, int dv, int k, int W, int dtype,
                                  int max_workgroups) {
  if (B <= 0 || T <= 0 || H <= 0 || D <= 0 || dv <= 0 || k < 0 || W < 0 || max_workgroups < 0) return 0;
  return csk::plan_attn(false, B, T, H, D, dv, k, W, dtype, max_workgroups).total;
}

size_t dense_compressed_attn_workspace_size(int B, int T, int H, int D, int dv, int Nmax, int m,
                                            int W, int dtype, int max_workgroups) {
  (void)m;
  if (B <= 0 || T <= 0 || H <= 0 || D <= 0 || dv <= 0 || Nmax <= 0 || W < 0 || max_workgroups < 0) return 0;
  return csk::plan_attn(true, B, T, H, D, dv, Nmax, W, dtype, max_workgroups).total;
}

int sparse_attn(const void* q, const int32_t* q_pos, const void* kv_c, int Nmax,
                const int32_t* idx, int k, const void* kv_w, const int32_t* w_pos0, int S_w,
                int W, const float* sink, int B, int T, int H, int D, int dv, int d_rope,
                float rope_base, float scale, int dtype, int kv_dtype, void* out, float* lse,
                int max_workgroups, void* workspace, size_t ws_bytes, void* stream) {
  return csk::attn_common("sparse_attn", false, q, q_pos, kv_c, Nmax, idx, k, nullptr, 1, kv_w,
                          w_pos0, S_w, W, sink, B, T, H, D, dv, d_rope, rope_base, scale, dtype,
                          kv_dtype, out, lse, max_workgroups, workspace, ws_bytes, stream);
}

int dense_compressed_attn(const void* q, const int32_t* q_pos, const void* kv_c, int Nmax,
                          const int32_t* n_entries, int m, const void* kv_w,
                          const int32_t* w_pos0, int S_w, int W, const float* sink, int B, int T,
                          int H, int D, int dv, int d_rope, float rope_base, float scale,
                          int dtype, int kv_dtype, void* out, float* lse, int max_workgroups,
                          void* workspace, size_t ws_bytes, void* stream) {
  return csk::attn_common("dense_compressed_attn", true, q, q_pos, kv_c, Nmax, nullptr, 0,
                          n_entries, m, kv_w, w_pos0, S_w, W, sink, B, T, H, D, dv, d_rope,
                          rope_base, scale, dtype, kv_dtype, out, lse, max_workgroups, workspace,
                          ws_bytes, stream);
}

}  // extern "C"
