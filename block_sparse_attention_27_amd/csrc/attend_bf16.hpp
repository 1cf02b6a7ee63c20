// Weighted block-sparse flash attention (and its dense special case) on bf16
// MFMA for gfx950.
//
// What is computed (AB-Attention, Abstract and transcript on the tiled kernel;
// InstaGen, Abstract): for the query rows of one query block and the list of
// (key unit j, weight w_j) chosen for that block, the online-softmax sums
//   num_r = sum_j w_j sum_t 2^(x_rt - m_r) v_t,  den_r = sum_j w_j sum_t 2^(x_rt - m_r),
// with x_rt = sm_scale * log2(e) * <q_r, k_t>, and out_r = num_r / den_r. The
// weight enters as an additive shift log2(w_j) of the exponent, folded into the
// per-row subtraction constant, so it costs nothing per element. Key units
// smaller than the 128-key tile (32 or 64 keys) are gathered into one tile.
//
// Work decomposition: one workgroup per (b, h, query block); each of its
// BQ/32 waves owns 32 query rows. Every 128-key tile of the list is staged in
// LDS (K row-major, V transposed), then per wave:
//   S^T[key][row] = K . Q^T   (A = K from LDS, B = Q^T held in registers)
//   O^T[d][row]  += V^T . P^T (A = V^T from LDS, B = P^T straight from the
//                              S^T accumulators after exp and bf16 packing)
// using v_mfma_f32_32x32x16_bf16. In the S^T orientation a lane holds one
// query row, so row max and row sum never leave the lane except for one
// exchange between the two 32-lane halves per tile.
#pragma once

#include "bsa_internal.hpp"

#include <math.h>

namespace bsa {
namespace attend_bf16_impl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int TILE = 128;           // keys per staged tile
constexpr float RESCALE_SLACK = 8;  // log2 units the running max may lag the true max

struct AttendArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* perm;
  const int32_t* idx;
  const float* w;
  void* out;
  float* lse;
  int H, N, N_pad, nQB, nKU, L, n_tiles, n_wg;
  float c;  // sm_scale * log2(e)
};

// XOR swizzle of the 16-byte chunk index within an LDS row: eight consecutive
// rows read at one column land on eight different bank groups.
__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// Position p in [0,16) of a 16-key group inside the transposed V tile holds
// key sigma(p) of that group. The permutation matches the key order in which
// the S^T accumulators hand P to the PV product (see the derivation in the
// kernel body).
__device__ __forceinline__ constexpr int sigma(int p) { return 8 * ((p % 8) / 4) + 4 * (p / 8) + p % 4; }

struct TileMeta {
  int base[4];   // first global (pre-permutation) key row of each unit in the tile
  int lim[4];    // valid keys of each unit (0 for an empty or rejected entry)
  float lw[4];   // log2 of the unit's weight
};

template <int BK, bool DENSE>
__device__ __forceinline__ TileMeta tile_meta(const AttendArgs& a, const int32_t* idx_row,
                                              const float* w_row, int t) {
  constexpr int U = TILE / BK;
  TileMeta m;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    m.base[u] = 0;
    m.lim[u] = 0;
    m.lw[u] = 0.f;
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if constexpr (DENSE) {
      const int b0 = t * TILE;
      m.base[u] = b0;
      m.lim[u] = min(TILE, a.N - b0);
    } else {
      const int e = t * U + u;
      int j = -1;
      float wv = 0.f;
      if (e < a.L) {
        j = idx_row[e];
        wv = w_row[e];
      }
      const bool ok = j >= 0 && j < a.nKU && wv > 0.f && wv < INFINITY;
      const int b0 = ok ? j * BK : 0;
      m.base[u] = b0;
      m.lim[u] = ok ? max(0, min(BK, a.N - b0)) : 0;
      m.lw[u] = ok ? __builtin_amdgcn_logf(wv) : 0.f;
    }
  }
  return m;
}

template <int BK>
__device__ __forceinline__ int pick(const int (&x)[4], int u) {
  if constexpr (BK == 128) {
    return x[0];
  } else if constexpr (BK == 64) {
    return u == 0 ? x[0] : x[1];
  } else {
    return u == 0 ? x[0] : u == 1 ? x[1] : u == 2 ? x[2] : x[3];
  }
}

template <bool PERM>
__device__ __forceinline__ int gather_row(const AttendArgs& a, int r, bool& ok) {
  if constexpr (PERM) {
    if (!ok) return 0;
    const int g = a.perm[r];
    ok = static_cast<unsigned>(g) < static_cast<unsigned>(a.N_pad);
    return ok ? g : 0;
  } else {
    return r;
  }
}

// Global -> LDS staging of one 128-key tile: K row-major [key][d], V transposed
// [d][key] with keys of each 16-key group in sigma order. Rows that are padding,
// belong to a rejected entry or fall outside the list are written as zeros.
template <int D, int NT, int BK, bool PERM>
__device__ __forceinline__ void stage_tile(const AttendArgs& a, const uint16_t* kb, const uint16_t* vb,
                                           char* ks, char* vts, const TileMeta& m, int tid) {
  constexpr int KCH = D / 8;          // 16-byte chunks per K row
  constexpr int KRPP = NT / KCH;      // K rows per pass
  constexpr int KP = TILE / KRPP;     // passes
  static_assert(BK % KRPP == 0, "a K pass must stay inside one unit");
  constexpr int VDG = D / 8;          // 8-column groups of V
  constexpr int VITEMS = 16 * VDG;    // (8-key group, 8-column group) items
  constexpr int VPT = (VITEMS + NT - 1) / NT;

  // ---- K ----
  {
    const int cc = tid % KCH, rb = tid / KCH;
    u32x4 r[KP];
    int gr[KP];
    bool ok[KP];
#pragma unroll
    for (int e = 0; e < KP; ++e) {
      const int row = rb + KRPP * e;
      const int u = (KRPP * e) / BK;  // compile-time: a pass never straddles units
      const int o = row - u * BK;
      ok[e] = o < m.lim[u];
      gr[e] = gather_row<PERM>(a, m.base[u] + o, ok[e]);
    }
#pragma unroll
    for (int e = 0; e < KP; ++e) {
      r[e] = ok[e] ? ldg16(kb + static_cast<size_t>(gr[e]) * D + cc * 8) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int e = 0; e < KP; ++e) {
      const int row = rb + KRPP * e;
      *reinterpret_cast<u32x4*>(ks + row * (D * 2) + ((cc ^ swz(row)) << 4)) = r[e];
    }
  }
  // ---- V (8 keys x 8 columns per item, transposed in registers) ----
#pragma unroll
  for (int x = 0; x < VPT; ++x) {
    const int it = tid + NT * x;
    if (VITEMS % NT != 0 && it >= VITEMS) break;
    const int dg = it % VDG, kg = it / VDG;
    const int g16 = kg >> 1, hh = kg & 1;
    const int u = (16 * g16) / BK;
    const int ubase = pick<BK>(m.base, u), ulim = pick<BK>(m.lim, u);
    u32x4 r[8];
    int gr[8];
    bool ok[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int key = 16 * g16 + sigma(8 * hh + e);
      const int o = key - u * BK;
      ok[e] = o < ulim;
      gr[e] = gather_row<PERM>(a, ubase + o, ok[e]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      r[e] = ok[e] ? ldg16(vb + static_cast<size_t>(gr[e]) * D + dg * 8) : u32x4{0u, 0u, 0u, 0u};
    }
    // column c of the 8x8 block: 8 keys (rows e = 0..7), two bf16 per dword
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      u32x4 col;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const uint32_t lo = r[2 * jj][c / 2], hi = r[2 * jj + 1][c / 2];
        col[jj] = (c & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
      }
      const int d = dg * 8 + c;
      const int chunk = 2 * g16 + hh;
      *reinterpret_cast<u32x4*>(vts + d * (TILE * 2) + ((chunk ^ swz(d)) << 4)) = col;
    }
  }
}

template <int D, int BQ, int BK, bool DENSE, bool PERM, bool OUT32>
__global__ __launch_bounds__(BQ * 2, 2) void attend_bf16_kernel(AttendArgs a) {
  constexpr int NW = BQ / 32;
  constexpr int NT = 64 * NW;
  constexpr int KBYTES = TILE * D * 2;
  __shared__ __attribute__((aligned(16))) char smem[KBYTES + D * TILE * 2];
  char* ks = smem;
  char* vts = smem + KBYTES;

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64;
  const int n = lane % 32, h = lane / 32;

  const int logical = xcd_remap(blockIdx.x, a.n_wg);
  const int bh = logical / a.nQB, qi = logical % a.nQB;
  const size_t bh_off = static_cast<size_t>(bh) * a.N_pad * D;
  const uint16_t* qb = a.q + bh_off;
  const uint16_t* kb = a.k + bh_off;
  const uint16_t* vb = a.v + bh_off;
  const int32_t* idx_row = DENSE ? nullptr : a.idx + static_cast<size_t>(logical) * a.L;
  const float* w_row = DENSE ? nullptr : a.w + static_cast<size_t>(logical) * a.L;

  // Q^T fragments (B operand): lane (row n, half h) holds d = 16 s + 8 h .. +7.
  const int qrow = qi * BQ + 32 * wave + n;
  bool qok = qrow < a.N;
  const int qg = gather_row<PERM>(a, qrow, qok);
  bf16x8 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    qf[s] = as_bf16x8(qok ? ldg16(qb + static_cast<size_t>(qg) * D + 16 * s + 8 * h)
                          : u32x4{0u, 0u, 0u, 0u});
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16{};
  float m_ref = -INFINITY;  // running max of x over this row (shared by both halves)
  float l_part = 0.f;       // this half's share of the weighted denominator

  for (int t = 0; t < a.n_tiles; ++t) {
    const TileMeta meta = tile_meta<BK, DENSE>(a, idx_row, w_row, t);
    if (t > 0) __syncthreads();  // every wave is done reading the previous tile
    stage_tile<D, NT, BK, PERM>(a, kb, vb, ks, vts, meta, tid);
    __syncthreads();

    // ---- S^T = K Q^T : 4 sub-tiles of 32 keys; acc register r of sub-tile kt
    // holds key 32 kt + 8 (r/4) + 4 h + r%4 for query row n.
    f32x16 sacc[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      sacc[kt] = f32x16{};
      const int key = 32 * kt + n;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        const int chunk = 2 * s + h;
        const u32x4 kv = *reinterpret_cast<const u32x4*>(ks + key * (D * 2) + ((chunk ^ swz(key)) << 4));
        sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kv), qf[s], sacc[kt], 0, 0, 0);
      }
    }

    // ---- mask keys past the valid range of their unit (uniform branch) ----
    bool full = true;
#pragma unroll
    for (int u = 0; u < TILE / BK; ++u) full = full && (meta.lim[u] == BK);
    if (!full) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const int u = (32 * kt) / BK;
        const int lim = meta.lim[u];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = (32 * kt) % BK + 8 * (r / 4) + 4 * h + (r % 4);
          if (off >= lim) sacc[kt][r] = -INFINITY;
        }
      }
    }

    // ---- tile max, lazily re-based running max ----
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kt][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    mx *= a.c;  // c > 0
    const bool need = mx > m_ref + RESCALE_SLACK;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float m_new = need ? mx : m_ref;
      const float alpha = (m_ref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new);
      l_part *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
      m_ref = m_new;
    }
    const float mb = (m_ref == -INFINITY) ? 0.f : m_ref;

    // ---- P = 2^(x - m + log2 w), row sums ----
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const float bias = meta.lw[(32 * kt) / BK] - mb;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kt][r], a.c, bias));
        sacc[kt][r] = p;
        l_part += p;
      }
    }

    // ---- O^T += V^T P^T over 8 steps of 16 keys. Step ks takes registers
    // 8 (ks%2) + e of sub-tile ks/2: lane half h then holds keys
    // 16 ks + sigma(8 h + e), the order in which V^T is staged.
#pragma unroll
    for (int ks_ = 0; ks_ < 8; ++ks_) {
      const int kt = ks_ / 2, s2 = ks_ % 2;
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = static_cast<__bf16>(sacc[kt][8 * s2 + e]);
      const int chunk = 2 * ks_ + h;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const int d = 32 * dt + n;
        const u32x4 vv = *reinterpret_cast<const u32x4*>(vts + d * (TILE * 2) + ((chunk ^ swz(d)) << 4));
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vv), pb, o[dt], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: O^T register r of d-tile dt holds d = 32 dt + 8 (r/4) + 4 h + r%4 ----
  const float l_tot = l_part + __shfl_xor(l_part, 32);
  bool ok = true;
  int orow = qrow;
  float inv = 0.f;
  if (qrow < a.N) {
    orow = gather_row<PERM>(a, qrow, ok);
    inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  }
  if (ok) {  // rows >= N (inv = 0) are written as zeros
    const size_t obase = bh_off + static_cast<size_t>(orow) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = 32 * dt + 8 * g + 4 * h;
        float x[4];
#pragma unroll
        for (int z = 0; z < 4; ++z) x[z] = o[dt][4 * g + z] * inv;
        if constexpr (OUT32) {
          float* op = static_cast<float*>(a.out) + obase + col;
          *reinterpret_cast<float4*>(op) = make_float4(x[0], x[1], x[2], x[3]);
        } else {
          uint32_t pk[2];
#pragma unroll
          for (int z = 0; z < 2; ++z) {
            const __bf16 lo = static_cast<__bf16>(x[2 * z]);
            const __bf16 hi = static_cast<__bf16>(x[2 * z + 1]);
            pk[z] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) |
                    (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) << 16);
          }
          uint16_t* op = static_cast<uint16_t*>(a.out) + obase + col;
          *reinterpret_cast<uint2*>(op) = make_uint2(pk[0], pk[1]);
        }
      }
    }
    if (a.lse != nullptr && h == 0) {
      a.lse[static_cast<size_t>(bh) * a.N_pad + orow] =
          (qrow < a.N && l_tot > 0.f) ? (m_ref + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f : -INFINITY;
    }
  }
}

template <int D, int BQ, int BK, bool DENSE, bool PERM, bool OUT32>
hipError_t launch_one(const AttendArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((attend_bf16_kernel<D, BQ, BK, DENSE, PERM, OUT32>), dim3(a.n_wg), dim3(BQ * 2), 0, s, a);
  return hipGetLastError();
}

template <int D, int BQ, bool DENSE, bool PERM, bool OUT32>
hipError_t dispatch_bk(const AttendArgs& a, int bk, hipStream_t s) {
  if constexpr (DENSE) {
    return launch_one<D, BQ, 128, true, PERM, OUT32>(a, s);
  } else {
    switch (bk) {
      case 32: return launch_one<D, BQ, 32, false, PERM, OUT32>(a, s);
      case 64: return launch_one<D, BQ, 64, false, PERM, OUT32>(a, s);
      default: return launch_one<D, BQ, 128, false, PERM, OUT32>(a, s);
    }
  }
}

template <int D, int BQ, bool OUT32>
hipError_t dispatch_mode(const AttendArgs& a, int bk, bool dense, bool perm, hipStream_t s) {
  if (dense) return perm ? dispatch_bk<D, BQ, true, true, OUT32>(a, bk, s) : dispatch_bk<D, BQ, true, false, OUT32>(a, bk, s);
  return perm ? dispatch_bk<D, BQ, false, true, OUT32>(a, bk, s) : dispatch_bk<D, BQ, false, false, OUT32>(a, bk, s);
}

// Launch for one head dimension D (one translation unit per D).
template <int D>
hipError_t launch_d(const Geometry& g, const void* q, const void* k, const void* v, const int32_t* perm,
                    const int32_t* idx, const float* w, void* out, float* lse, bool out_fp32, hipStream_t s) {
  const bool dense = idx == nullptr;
  AttendArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.perm = perm;
  a.idx = idx;
  a.w = w;
  a.out = out;
  a.lse = lse;
  a.H = g.H;
  a.N = g.N;
  a.N_pad = g.N_pad;
  a.nQB = g.nQB;
  a.nKU = g.nKU;
  a.L = dense ? 0 : g.L;
  a.n_tiles = dense ? (g.N + TILE - 1) / TILE : (g.L * g.block_k + TILE - 1) / TILE;
  a.n_wg = g.B * g.H * g.nQB;
  a.c = g.sm_scale * 1.4426950408889634f;
  const bool p = perm != nullptr;
  if (out_fp32) {
    return g.block_q == 128 ? dispatch_mode<D, 128, true>(a, g.block_k, dense, p, s)
                            : dispatch_mode<D, 64, true>(a, g.block_k, dense, p, s);
  }
  return g.block_q == 128 ? dispatch_mode<D, 128, false>(a, g.block_k, dense, p, s)
                          : dispatch_mode<D, 64, false>(a, g.block_k, dense, p, s);
}

}  // namespace attend_bf16_impl
}  // namespace bsa
