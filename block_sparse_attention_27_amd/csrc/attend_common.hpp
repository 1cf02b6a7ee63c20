// Helpers shared by the bf16 MFMA attention kernels for gfx950 (the
// 128-row-block kernel with two workgroups per CU in attend_bf16_t64.hpp and
// the 64-row-block kernel in attend_bf16_w32.hpp): tile staging from global
// memory into LDS, list sorting and tile descriptions, LDS read addressing,
// masking and row reductions.
//
// What the kernels compute (AB-Attention, Abstract and transcript on the
// tiled kernel; InstaGen, Abstract): for the query rows of one query block and
// the list of (key unit j, weight w_j) chosen for that block, the
// online-softmax sums
//   num_r = sum_j w_j sum_t 2^(x_rt - m_r) v_t,  den_r = sum_j w_j sum_t 2^(x_rt - m_r),
// with x_rt = sm_scale * log2(e) * <q_r, k_t>, and out_r = num_r / den_r. The
// weight enters as an additive shift log2(w_j) of the exponent, folded into the
// per-row subtraction constant, so it costs nothing per element. Key units
// smaller than a tile are gathered into one tile.
//
// Data movement. K and V tiles go from global memory straight into LDS
// (global_load_lds_dwordx4, no registers), double-buffered so the next tile
// streams in while the current one is computed; both are stored row-major
// with the 16-byte chunks of each row XOR-permuted so that the K reads and
// the transposed V reads are free of bank conflicts. Each lane's share of a
// staged tile sits at a fixed offset from the unit's first row, so a full
// tile costs one address add per load. The list of a query block is first
// rank-sorted by unit index so that concurrent workgroups sweep the keys of a
// head in the same order, and workgroups are mapped so that all 8 XCDs work
// on the same head at once, each on a contiguous run of query blocks.
#pragma once

#include "bsa_internal.hpp"

#include <math.h>

#include <type_traits>

namespace bsa {
namespace attend_bf16_impl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define BSA_LDS __attribute__((address_space(3)))

constexpr int TILE = 128;           // keys per staged tile of attend_w32_kernel
constexpr int LMAX = 1024;          // list entries sorted and held in LDS at a time
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
  int H, N, N_pad, nQB, nKU, L, n_wg, qchunk;
  float c;  // sm_scale * log2(e)
};

// LDS tiles are row-major [128 keys][D] bf16 with the 16-byte chunks of each
// row permuted by an XOR with a function of the row. gfx950 serves 64 banks
// (256 bytes) per LDS cycle, so
//   K: the 16 lanes of one cycle read 16 consecutive rows at one logical
//      chunk; the XOR spreads them over the 16 chunk positions of a 256-byte
//      bank row (d = 128: chunk ^ (row & 15); d = 64, two rows per bank row:
//      chunk ^ ((row >> 1) & 7)).
//   V: the 32 lanes of one transposed-read cycle take 64 bytes from each of 4
//      consecutive rows; the XOR moves the four 64-byte pieces apart
//      (d = 128: chunk ^ 4 (row & 3); d = 64: chunk ^ 4 ((row >> 1) & 1)).
// Every read address stays a per-lane base plus a compile-time offset.
template <int D> __device__ __forceinline__ int k_swz(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
template <int D> __device__ __forceinline__ int v_swz(int row) { return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// Pins a value at this point of the instruction stream: an empty volatile asm
// that takes and returns it, so the computation producing it stays in its
// group (the compiler may otherwise sink pure arithmetic past the groups'
// scheduling fences towards its first use).
template <typename T>
__device__ __forceinline__ void pin(T& x) { asm volatile("" : "+v"(x)); }

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

// How a kernel uses the permutation: not at all; to gather Q, K and V rows
// and scatter the output rows; or, for K and V that arrive already in
// permuted order (or dense attention, where the key order does not matter),
// to gather the Q rows and scatter the output rows only.
constexpr int PERM_NONE = 0;
constexpr int PERM_ALL = 1;
constexpr int PERM_QO = 2;

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

struct TileMeta {
  int base[4];  // first key row of each unit in the tile, in the order K and V are given
  int lim[4];   // valid keys of each unit (0: empty slot or rejected entry)
  float lw[4];  // log2 of the unit's weight
  bool full;    // every unit of the tile holds BK valid keys
};

__device__ __forceinline__ int pick4(const int (&x)[4], int u) {
  return u == 0 ? x[0] : u == 1 ? x[1] : u == 2 ? x[2] : x[3];
}

// Direct global -> LDS staging of one tile (TK keys) of K or V. A wave
// instruction moves 1 KB = RPI whole rows; lane l lands at byte 16 l of it,
// i.e. in row l / CPR at physical chunk l % CPR, which holds logical chunk
// (l % CPR) ^ swz(row). Instruction i of wave w covers tile rows
// (i NW + w) RPI .. +RPI-1, so a lane's row is i G + r0 with G = NW RPI and
// r0 = w RPI + l / CPR. G is a multiple of the swizzle periods, so the lane's
// chunk and its byte offset r0 2D + 16 chunk are the same for every i and both
// tensors' tiles: one per-lane register each for K and V, and the rest of the
// address (the unit's first row, the instruction's row step) is uniform.
// Rows of one instruction never straddle a unit (BK is a multiple of RPI).
template <int D, int NW, int TK = TILE>
struct StageGeom {
  static constexpr int CPR = D / 8;            // 16-byte chunks per row
  static constexpr int RPI = 1024 / (2 * D);   // rows per instruction
  static constexpr int G = NW * RPI;           // row step between a wave's instructions
  static constexpr int PER_WAVE = TK / G;      // instructions per wave and tile of TK keys
  static_assert(G % 16 == 0 && TK % G == 0, "swizzle periods must divide the row step");
};

template <int D, int NW, int TK = TILE>
__device__ __forceinline__ uint32_t stage_lane_offset(int wave, int lane, bool is_v) {
  using SG = StageGeom<D, NW, TK>;
  const int r0 = wave * SG::RPI + lane / SG::CPR;
  return static_cast<uint32_t>(r0 * 2 * D + 16 * ((lane % SG::CPR) ^ (is_v ? v_swz<D>(r0) : k_swz<D>(r0))));
}

// Instruction i of the full-tile path: every row valid, so the address is a
// uniform base plus the lane's fixed offset (swave: the wave index as a
// uniform value; lane_off: stage_lane_offset for this tensor).
template <int D, int NW, int BK>
__device__ __forceinline__ void stage_fast(const uint16_t* src, BSA_LDS char* dst, const TileMeta& m, int swave,
                                           uint32_t lane_off, int i) {
  using SG = StageGeom<D, NW>;
  const int row0 = i * SG::G + swave * SG::RPI;                 // first tile row of the instruction
  const int u = BK % SG::G == 0 ? i * SG::G / BK : row0 / BK;  // swave RPI < G
  const int first = pick4(m.base, u) + i * SG::G - u * BK;      // key row of the lane with r0 = 0
  const char* sp = reinterpret_cast<const char*>(src) + static_cast<size_t>(first) * (2 * D);
  pin(lane_off);  // keeps the base uniform: scalar base + 32-bit lane offset addressing
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(sp + lane_off),
                                   (BSA_LDS void*)(dst + (i * NW + swave) * 1024), 16, 0, 0);
}

// The whole tile on the general path: partial or empty units, or K and V
// gathered through perm. Rows past a unit's valid keys load a valid row of the same
// head instead (their logits are masked).
template <int D, int NW, int BK, bool PERM, bool IS_V>
__device__ __forceinline__ void stage_general(const AttendArgs& a, const uint16_t* src, BSA_LDS char* dst,
                                              const TileMeta& m, int swave, int lane) {
  using SG = StageGeom<D, NW>;
#pragma unroll
  for (int i = 0; i < SG::PER_WAVE; ++i) {
    const int row0 = i * SG::G + swave * SG::RPI;
    const int u = BK % SG::G == 0 ? i * SG::G / BK : row0 / BK;
    const int ubase = pick4(m.base, u);
    const int ulim = pick4(m.lim, u);
    const int row = row0 + lane / SG::CPR;
    const int o = row - u * BK;
    int gr;
    if constexpr (PERM) {
      bool ok = o < ulim;
      gr = gather_row<PERM>(a, ok ? ubase + o : ubase, ok);
      if (!ok) gr = 0;  // any row of this head
    } else {
      gr = ubase + min(o, max(ulim, 1) - 1);  // an empty slot has base 0: row 0
    }
    const int lc = (lane % SG::CPR) ^ (IS_V ? v_swz<D>(row) : k_swz<D>(row));
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src + static_cast<size_t>(gr) * D + lc * 8),
                                     (BSA_LDS void*)(dst + (i * NW + swave) * 1024), 16, 0, 0);
  }
}

template <int D, int NW, int BK, bool PERM, bool IS_V>
__device__ __forceinline__ void stage_one(const AttendArgs& a, const uint16_t* src, BSA_LDS char* dst,
                                          const TileMeta& m, int swave, int lane, uint32_t lane_off) {
  if (!PERM && m.full) {
#pragma unroll
    for (int i = 0; i < StageGeom<D, NW>::PER_WAVE; ++i) stage_fast<D, NW, BK>(src, dst, m, swave, lane_off, i);
  } else {
    stage_general<D, NW, BK, PERM, IS_V>(a, src, dst, m, swave, lane);
  }
}

// Instruction i of a tile's staging, without branches (K and V read in place):
// rows past a unit's valid keys load the unit's last valid key (an empty
// slot, base 0 and no keys: row 0), so the address is the unit's first row
// (uniform) plus min(row in unit, last valid row) 2D + the lane's chunk byte.
// r0 = wave RPI + lane / CPR; chunk_off = 16 ((lane % CPR) ^ swz(r0)).
template <int D, int NW, int BK>
__device__ __forceinline__ void stage_ins(const uint16_t* src, BSA_LDS char* dst, const TileMeta& m, int swave,
                                          int r0, uint32_t chunk_off, int i) {
  using SG = StageGeom<D, NW>;
  const int row0 = i * SG::G + swave * SG::RPI;
  const int u = BK % SG::G == 0 ? i * SG::G / BK : row0 / BK;
  const int c = i * SG::G - u * BK;                 // row in the unit of the lane with r0 = 0
  const int last = max(pick4(m.lim, u), 1) - 1;     // last valid row of the unit (uniform)
  const char* sp = reinterpret_cast<const char*>(src) + static_cast<size_t>(pick4(m.base, u)) * (2 * D);
  uint32_t off = static_cast<uint32_t>(min(r0 + c, last)) * (2 * D) + chunk_off;
  pin(off);  // keeps the base uniform: scalar base + 32-bit lane offset addressing
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(sp + off),
                                   (BSA_LDS void*)(dst + (i * NW + swave) * 1024), 16, 0, 0);
}

// Gathered key row of tile row r when K and V go through perm: unit r / BK, key
// r % BK -> perm[base + r % BK]; a row past the unit's valid keys, or a gather
// entry outside [0, N_pad), gives row 0 of the head (its logits are masked).
template <int BK>
__device__ __forceinline__ int tile_row_gather(const AttendArgs& a, const TileMeta& m, int r) {
  const int u = r / BK, o = r % BK;
  if (o >= pick4(m.lim, u)) return 0;
  const int g = a.perm[pick4(m.base, u) + o];
  return static_cast<unsigned>(g) < static_cast<unsigned>(a.N_pad) ? g : 0;
}

// Instruction i of a tile's staging with K and V gathered through perm: the tile's
// gathered rows come from an LDS table (rows[r] for tile row r), so the
// address is the lane's gathered row plus its fixed chunk byte.
template <int D, int NW>
__device__ __forceinline__ void stage_gathered(const uint16_t* src, BSA_LDS char* dst, const int* rows, int swave,
                                               int r0, uint32_t chunk_off, int i) {
  using SG = StageGeom<D, NW>;
  const int gr = rows[i * SG::G + r0];
  const char* sp = reinterpret_cast<const char*>(src) + static_cast<size_t>(gr) * (2 * D) + chunk_off;
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(sp),
                                   (BSA_LDS void*)(dst + (i * NW + swave) * 1024), 16, 0, 0);
}

// Rank-sorts the list chunk [c0, c0 + n) of one query block by unit index
// (ties by position) into the LDS tables; entries with an index outside
// [0, nKU) or a weight that is not a finite positive number become empty.
// The rank of entry e is the number of keys below its own plus the equal keys
// before it. A list made of a few ascending runs (a bsa_select list is two:
// the exact set, then the sample in unit order) gets it from binary searches
// of the other runs; any other list from a scan of the whole chunk.
constexpr int SORT_MAX_RUNS = 4;

template <int NT, int BK>
__device__ __forceinline__ void sort_list(const AttendArgs& a, const int32_t* idx_row, const float* w_row,
                                          int c0, int n, int* s_key, int* s_base, int* s_lim, float* s_lw,
                                          int tid) {
  __shared__ int s_nruns;                     // descents found (runs - 1)
  __shared__ int s_start[SORT_MAX_RUNS - 1];  // positions that start a run after the first, unordered
  if (tid == 0) s_nruns = 0;
  for (int e = tid; e < n; e += NT) {
    const int j = idx_row[c0 + e];
    const float wv = w_row[c0 + e];
    const bool ok = j >= 0 && j < a.nKU && wv > 0.f && wv < INFINITY;
    s_key[e] = ok ? j : 0x7FFFFFFF;
  }
  __syncthreads();
  for (int e = 1 + tid; e < n; e += NT) {
    if (s_key[e - 1] > s_key[e]) {
      const int slot = atomicAdd(&s_nruns, 1);
      if (slot < SORT_MAX_RUNS - 1) s_start[slot] = e;
    }
  }
  __syncthreads();
  const int nd = s_nruns;  // uniform
  int start[SORT_MAX_RUNS + 1];  // run r is [start[r], start[r + 1]), ascending
  const bool runs = nd < SORT_MAX_RUNS;
  if (runs) {
    start[0] = 0;
#pragma unroll
    for (int r = 1; r < SORT_MAX_RUNS; ++r) start[r] = r <= nd ? s_start[r - 1] : n;
#pragma unroll
    for (int r = 1; r < SORT_MAX_RUNS; ++r)  // insertion sort of the (at most three) starts
#pragma unroll
      for (int q = r; q > 1; --q)
        if (start[q - 1] > start[q]) {
          const int t = start[q - 1];
          start[q - 1] = start[q];
          start[q] = t;
        }
    start[SORT_MAX_RUNS] = n;
  }
  for (int e = tid; e < n; e += NT) {
    const int my = s_key[e];
    int rank = 0;
    if (runs) {
#pragma unroll
      for (int r = 0; r < SORT_MAX_RUNS; ++r) {
        const int lo = start[r], hi = start[r + 1];
        if (e >= lo && e < hi) {
          rank += e - lo;  // the run's entries before e are all <= my
        } else {
          // entries of run r below my (equal ones too when the run comes first)
          const bool before = hi <= e;
          int l = lo, h = hi;
          while (l < h) {
            const int mid = (l + h) >> 1;
            const int k2 = s_key[mid];
            if (k2 < my || (before && k2 == my)) l = mid + 1;
            else h = mid;
          }
          rank += l - lo;
        }
      }
    } else {
      for (int e2 = 0; e2 < n; ++e2) {
        const int k2 = s_key[e2];
        rank += (k2 < my || (k2 == my && e2 < e)) ? 1 : 0;
      }
    }
    const bool ok = my != 0x7FFFFFFF;
    const int b0 = ok ? my * BK : 0;
    s_base[rank] = b0;
    s_lim[rank] = ok ? max(0, min(BK, a.N - b0)) : 0;
    s_lw[rank] = ok ? __builtin_amdgcn_logf(w_row[c0 + e]) : 0.f;
  }
  __syncthreads();
}

// Description of tile t of the current list chunk. Tiles past the end
// describe empty units at row 0.
template <int BK, bool DENSE>
__device__ __forceinline__ TileMeta tile_meta(const AttendArgs& a, const int* s_base, const int* s_lim,
                                              const float* s_lw, int t, int n_entries) {
  constexpr int U = TILE / BK;
  TileMeta m;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    m.base[u] = 0;
    m.lim[u] = 0;
    m.lw[u] = 0.f;
  }
  m.full = true;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if constexpr (DENSE) {
      if (t * TILE < a.N) {
        m.base[u] = t * TILE;
        m.lim[u] = min(TILE, a.N - t * TILE);
      }
    } else {
      const int e = t * U + u;
      if (e < n_entries) {  // uniform values: keep them in scalar registers
        m.base[u] = __builtin_amdgcn_readfirstlane(s_base[e]);
        m.lim[u] = __builtin_amdgcn_readfirstlane(s_lim[e]);
        m.lw[u] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(s_lw[e])));
      }
    }
    m.full = m.full && m.lim[u] == BK;
  }
  return m;
}

// Per-lane LDS read addressing. A lane (n = lane % 32, h = lane / 32) of key
// half kh reads, for step s of S^T = K Q^T over sub-tile j, K row
// 64 kh + 32 j + n at logical chunk 2 s + h, i.e. physical chunk
// (2 s + h) ^ x with x = k_swz(row). Since (2 s + h) ^ x =
// 2 (s ^ (x >> 1)) + (h ^ (x & 1)), the byte offset within the row is
// ((32 s) ^ kx) + 16 (h ^ (x & 1)) with kx = 32 (x >> 1): one xor per read
// from two per-lane values. Likewise the transposed V reads of d-tile dt sit
// at logical chunk 4 dt + w (w = 2 g2 + c / 2) of row vrow, physical
// (4 dt + w) ^ 4 z with 4 z = v_swz(vrow), i.e. byte ((64 dt) ^ vx) + 16 w
// with vx = 64 z.
template <int D>
struct LaneOffsets {
  int kbase;  // byte of the lane's K row plus 16 (h ^ (x & 1))
  int kx;     // 32 (x >> 1)
  int vbase;  // byte of the lane's V row plus 16 w + 8 (c % 2)
  int vx;     // 64 z
};

template <int D>
__device__ __forceinline__ LaneOffsets<D> lane_offsets(int kh, int lane) {
  LaneOffsets<D> L;
  const int n = lane % 32, h = lane / 32;
  const int x = k_swz<D>(64 * kh + n);
  L.kbase = (64 * kh + n) * 2 * D + 16 * (h ^ (x & 1));
  L.kx = 32 * (x >> 1);
  const int q = lane % 16, r = q / 4, c = q % 4, g2 = (lane / 16) % 2;
  const int vrow = 64 * kh + 4 * h + r;
  L.vbase = vrow * 2 * D + 16 * (2 * g2 + c / 2) + 8 * (c % 2);
  L.vx = 16 * v_swz<D>(vrow);
  return L;
}

template <int D>
__device__ __forceinline__ int koff(const LaneOffsets<D>& L, int s) { return (32 * s) ^ L.kx; }
template <int D>
__device__ __forceinline__ int voff(const LaneOffsets<D>& L, int dt) { return (64 * dt) ^ L.vx; }

// S^T = K Q^T over the 64 keys of key half kh (the first tile of a list; the
// pipelined steps issue the same MFMAs interleaved with the softmax). Sub-tile
// j covers keys 64 kh + 32 j .. +31; accumulator register r holds key
// 8 (r/4) + 4 h + r%4 of it.
template <int D>
__device__ __forceinline__ void qk_tile(f32x16 (&S)[2], const BSA_LDS char* kslot, const LaneOffsets<D>& L,
                                        const bf16x8 (&qf)[D / 16]) {
  S[0] = f32x16{};
  S[1] = f32x16{};
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {  // the two accumulators alternate: no back-to-back dependence
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const u32x4 kv = *(const BSA_LDS u32x4*)(kslot + L.kbase + 64 * D * j + koff<D>(L, s));
      S[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kv), qf[s], S[j], 0, 0, 0);
    }
  }
}

template <int BK>
__device__ __forceinline__ void half_meta(const TileMeta& m, int kh, int (&lim)[2], int (&off)[2], float (&lw)[2]) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int u = (64 * kh + 32 * j) / BK;
    lim[j] = u == 0 ? m.lim[0] : u == 1 ? m.lim[1] : u == 2 ? m.lim[2] : m.lim[3];
    lw[j] = u == 0 ? m.lw[0] : u == 1 ? m.lw[1] : u == 2 ? m.lw[2] : m.lw[3];
    off[j] = (64 * kh + 32 * j) % BK;
  }
}

// Keys past the valid range of their unit get -inf (uniform branch; only
// tiles that hold a partial or empty unit take it). Register r of sub-tile j
// holds key off[j] + 8 (r/4) + 4 h + r%4 of its unit, so one per-lane
// threshold lim - off - 4h is compared with a constant per register.
template <int BK>
__device__ __forceinline__ bool mask_tile(f32x16 (&S)[2], const TileMeta& m, int kh, int h) {
  int lim[2], off[2];
  float lw[2];
  half_meta<BK>(m, kh, lim, off, lw);
  if (off[0] + 32 > lim[0] || off[1] + 32 > lim[1]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int thr = lim[j] - off[j] - 4 * h;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r / 4) + (r % 4) >= thr) S[j][r] = -INFINITY;
    }
    return true;
  }
  return false;
}

// Maximum of the 32 values a lane holds (a chain of 3-input maxima).
__device__ __forceinline__ float tile_max(const f32x16 (&S)[2]) {
  float mx = fmaxf(S[0][0], S[0][1]);
#pragma unroll
  for (int q2 = 1; q2 < 16; ++q2) mx = fmaxf(mx, fmaxf(S[q2 / 8][2 * (q2 % 8)], S[q2 / 8][2 * (q2 % 8) + 1]));
  return mx;
}

// Maximum of x over both 32-lane halves (they hold different keys of one row).
__device__ __forceinline__ float halves_max(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

__device__ __forceinline__ float halves_sum(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

}  // namespace attend_bf16_impl
}  // namespace bsa
