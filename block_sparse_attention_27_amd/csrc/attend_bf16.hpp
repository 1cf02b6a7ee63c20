// Weighted block-sparse flash attention (and its dense special case) on bf16
// MFMA for gfx950. Kernel template; instantiated per head dimension in
// attend_bf16_d128.hip and attend_bf16_d64.hip.
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
// Work decomposition. One workgroup per (b, h, query block) with 2*BQ/32
// waves: wave (rg, kh) owns query rows [32 rg, 32 rg + 32) and keys
// [64 kh, 64 kh + 64) of every 128-key tile; the two key halves are merged at
// the end like two partial softmaxes. Per wave and tile:
//   S^T[key][row] = K . Q^T   (A = K rows from LDS, B = Q^T in registers)
//   O^T[d][row]  += V^T . P^T (A = V^T read transposed from LDS with
//                              ds_read_b64_tr_b16, B = P^T straight from the
//                              S^T accumulators after exp and bf16 packing)
// on v_mfma_f32_32x32x16_bf16. A lane holds one query row, so the row max and
// row sum stay in the lane except for one exchange between 32-lane halves.
//
// Data movement. K and V tiles go from global memory straight into LDS
// (global_load_lds_dwordx4, no registers), double-buffered so the next tile
// streams in while the current one is computed; both are stored row-major
// with the 16-byte chunks of each row XOR-permuted so that the K reads and
// the transposed V reads are free of bank conflicts. Each lane's share of a
// staged tile sits at a fixed offset from the unit's first row, so a full
// tile costs one address add per load. The list of a query block is
// first rank-sorted by unit index so that concurrent workgroups sweep the keys
// of a head in the same order, and workgroups are mapped so that all 8 XCDs
// work on the same head at once, each on a contiguous run of query blocks.
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

constexpr int TILE = 128;           // keys per staged tile
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

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

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
  int base[4];  // first global (pre-permutation) key row of each unit in the tile
  int lim[4];   // valid keys of each unit (0: empty slot or rejected entry)
  float lw[4];  // log2 of the unit's weight
  bool full;    // every unit of the tile holds BK valid keys
};

__device__ __forceinline__ int pick4(const int (&x)[4], int u) {
  return u == 0 ? x[0] : u == 1 ? x[1] : u == 2 ? x[2] : x[3];
}

// Direct global -> LDS staging of one 128-key tile of K or V. A wave
// instruction moves 1 KB = RPI whole rows; lane l lands at byte 16 l of it,
// i.e. in row l / CPR at physical chunk l % CPR, which holds logical chunk
// (l % CPR) ^ swz(row). Instruction i of wave w covers tile rows
// (i NW + w) RPI .. +RPI-1, so a lane's row is i G + r0 with G = NW RPI and
// r0 = w RPI + l / CPR. G is a multiple of the swizzle periods, so the lane's
// chunk and its byte offset r0 2D + 16 chunk are the same for every i and both
// tensors' tiles: one per-lane register each for K and V, and the rest of the
// address (the unit's first row, the instruction's row step) is uniform.
// Rows of one instruction never straddle a unit (BK is a multiple of RPI).
template <int D, int NW>
struct StageGeom {
  static constexpr int CPR = D / 8;            // 16-byte chunks per row
  static constexpr int RPI = 1024 / (2 * D);   // rows per instruction
  static constexpr int G = NW * RPI;           // row step between a wave's instructions
  static constexpr int PER_WAVE = TILE / G;    // instructions per wave and tile
  static_assert(G % 16 == 0 && TILE % G == 0, "swizzle periods must divide the row step");
};

template <int D, int NW>
__device__ __forceinline__ uint32_t stage_lane_offset(int wave, int lane, bool is_v) {
  using SG = StageGeom<D, NW>;
  const int r0 = wave * SG::RPI + lane / SG::CPR;
  return static_cast<uint32_t>(r0 * 2 * D + 16 * ((lane % SG::CPR) ^ (is_v ? v_swz<D>(r0) : k_swz<D>(r0))));
}

// swave: the wave index as a uniform value; lane_off: stage_lane_offset for this tensor.
template <int D, int NW, int BK, bool PERM, bool IS_V>
__device__ __forceinline__ void stage_one(const AttendArgs& a, const uint16_t* src, BSA_LDS char* dst,
                                          const TileMeta& m, int swave, int lane, uint32_t lane_off) {
  using SG = StageGeom<D, NW>;
  if (!PERM && m.full) {
    // every row valid: uniform base + the lane's fixed offset, no per-lane arithmetic
#pragma unroll
    for (int i = 0; i < SG::PER_WAVE; ++i) {
      const int row0 = i * SG::G + swave * SG::RPI;  // first tile row of the instruction
      const int u = BK % SG::G == 0 ? i * SG::G / BK : row0 / BK;  // swave RPI < G
      const int first = pick4(m.base, u) + i * SG::G - u * BK;  // key row of the lane with r0 = 0
      const char* sp = reinterpret_cast<const char*>(src) + static_cast<size_t>(first) * (2 * D);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(sp + lane_off),
                                       (BSA_LDS void*)(dst + (i * NW + swave) * 1024), 16, 0, 0);
    }
    return;
  }
  // partial or empty units, or a permutation: rows past a unit's valid keys load a
  // valid row of the same head instead (their logits are masked).
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

// Rank-sorts the list chunk [c0, c0 + n) of one query block by unit index
// (ties by position) into the LDS tables; entries with an index outside
// [0, nKU) or a weight that is not a finite positive number become empty.
template <int NT, int BK>
__device__ __forceinline__ void sort_list(const AttendArgs& a, const int32_t* idx_row, const float* w_row,
                                          int c0, int n, int* s_key, int* s_base, int* s_lim, float* s_lw,
                                          int tid) {
  for (int e = tid; e < n; e += NT) {
    const int j = idx_row[c0 + e];
    const float wv = w_row[c0 + e];
    const bool ok = j >= 0 && j < a.nKU && wv > 0.f && wv < INFINITY;
    s_key[e] = ok ? j : 0x7FFFFFFF;
  }
  __syncthreads();
  for (int e = tid; e < n; e += NT) {
    const int my = s_key[e];
    int rank = 0;
    for (int e2 = 0; e2 < n; ++e2) {
      const int k2 = s_key[e2];
      rank += (k2 < my || (k2 == my && e2 < e)) ? 1 : 0;
    }
    const bool ok = my != 0x7FFFFFFF;
    const int b0 = ok ? my * BK : 0;
    s_base[rank] = b0;
    s_lim[rank] = ok ? max(0, min(BK, a.N - b0)) : 0;
    s_lw[rank] = ok ? __builtin_amdgcn_logf(w_row[c0 + e]) : 0.f;
  }
  __syncthreads();
}

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
      m.base[u] = t * TILE;
      m.lim[u] = min(TILE, a.N - t * TILE);
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

// S^T = K Q^T over the 64 keys of key half kh: sub-tile j covers keys
// 64 kh + 32 j .. +31; accumulator register r holds key 8 (r/4) + 4 h + r%4.
// Per-lane LDS read offsets. A lane (n = lane % 32, h = lane / 32) of key half
// kh reads, for step s of S^T = K Q^T over sub-tile j, K row 64 kh + 32 j + n
// at logical chunk 2 s + h: byte kbase + 64 D j + koff[s]. For the transposed
// V reads of PV step ks, d-tile dt and key group g (0: keys 16 ks + 4 h .. +3;
// 1: the same + 8) it reads at vbase + 2 D (16 ks + 8 g) + voff[dt].
template <int D>
struct LaneOffsets {
  int kbase, koff[D / 16];
  int vbase, voff[D / 32];
};

template <int D>
__device__ __forceinline__ LaneOffsets<D> lane_offsets(int kh, int lane) {
  LaneOffsets<D> L;
  const int n = lane % 32, h = lane / 32;
  L.kbase = (64 * kh + n) * 2 * D;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) L.koff[s] = 16 * ((2 * s + h) ^ k_swz<D>(64 * kh + n));
  const int q = lane % 16, r = q / 4, c = q % 4, g2 = (lane / 16) % 2;
  const int vrow = 64 * kh + 4 * h + r;
  L.vbase = vrow * 2 * D + 8 * (c % 2);
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) L.voff[dt] = 16 * ((4 * dt + 2 * g2 + c / 2) ^ v_swz<D>(vrow));
  return L;
}

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
      const u32x4 kv = *(const BSA_LDS u32x4*)(kslot + L.kbase + 64 * D * j + L.koff[s]);
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
__device__ __forceinline__ void mask_tile(f32x16 (&S)[2], const TileMeta& m, int kh, int h) {
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
  }
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

template <int D, int BQ, int BK, bool DENSE, bool PERM, bool OUT32>
__global__ __launch_bounds__(BQ * 4, 1) void attend_bf16_kernel(AttendArgs a) {
  constexpr int NRG = BQ / 32;  // row groups
  constexpr int NW = 2 * NRG;   // waves: row group x key half
  constexpr int NT = 64 * NW;
  // Four separate tile slots (K0, K1, V0, V1): each pipelined step writes one
  // K and one V slot with direct loads while it reads the other two, and the
  // slot choice is a compile-time constant there, so the compiler can see
  // that the in-flight loads never alias the reads.
  __shared__ __attribute__((aligned(1024))) char k_lds0[TILE * 2 * D];
  __shared__ __attribute__((aligned(1024))) char k_lds1[TILE * 2 * D];
  __shared__ __attribute__((aligned(1024))) char v_lds0[TILE * 2 * D];
  __shared__ __attribute__((aligned(1024))) char v_lds1[TILE * 2 * D];
  __shared__ int s_key[DENSE ? 1 : LMAX];
  __shared__ int s_base[DENSE ? 1 : LMAX];
  __shared__ int s_lim[DENSE ? 1 : LMAX];
  __shared__ float s_lw[DENSE ? 1 : LMAX];

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64;
  const int n = lane % 32, h = lane / 32;
  // wave-uniform indices held in scalar registers
  const int rg = __builtin_amdgcn_readfirstlane(wave % NRG), kh = __builtin_amdgcn_readfirstlane(wave / NRG);

  // XCD-chunked mapping: hardware workgroup g runs on XCD g % 8; XCD x takes
  // query blocks [x*qchunk, (x+1)*qchunk) of each (b, h) in turn.
  const int xg = blockIdx.x % 8, sg = blockIdx.x / 8;
  const int bh = sg / a.qchunk;
  const int qi = xg * a.qchunk + sg % a.qchunk;
  if (qi >= a.nQB) return;  // padding workgroup (uniform)

  const size_t bh_off = static_cast<size_t>(bh) * a.N_pad * D;
  const uint16_t* qb = a.q + bh_off;
  const uint16_t* kb = a.k + bh_off;
  const uint16_t* vb = a.v + bh_off;
  const size_t row_id = static_cast<size_t>(bh) * a.nQB + qi;
  const int32_t* idx_row = DENSE ? nullptr : a.idx + row_id * a.L;
  const float* w_row = DENSE ? nullptr : a.w + row_id * a.L;

  // Q^T fragments (B operand): lane (row n, half h) holds d = 16 s + 8 h .. +7.
  const int qrow = qi * BQ + 32 * rg + n;
  bool qok = qrow < a.N;
  const int qg = gather_row<PERM>(a, qrow, qok);
  bf16x8 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    qf[s] = as_bf16x8(qok ? ldg16(qb + static_cast<size_t>(qg) * D + 16 * s + 8 * h) : u32x4{0u, 0u, 0u, 0u});

  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16{};
  float m_ref = -INFINITY;  // running max of x for this row (shared by both lane halves)
  float l_part = 0.f;       // this lane's share of the weighted denominator

  // K runs one tile ahead of V so that QK of tile t+1 overlaps the softmax of tile t.
  BSA_LDS char* const K0 = (BSA_LDS char*)(k_lds0);  // address-space casts of the shared arrays
  BSA_LDS char* const K1 = (BSA_LDS char*)(k_lds1);
  BSA_LDS char* const V0 = (BSA_LDS char*)(v_lds0);
  BSA_LDS char* const V1 = (BSA_LDS char*)(v_lds1);
  const LaneOffsets<D> LO = lane_offsets<D>(kh, lane);
  const int swave = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t k_lane_off = stage_lane_offset<D, NW>(wave, lane, false);
  const uint32_t v_lane_off = stage_lane_offset<D, NW>(wave, lane, true);
  const int n_chunks = DENSE ? 1 : (a.L + LMAX - 1) / LMAX;
  for (int ck = 0; ck < n_chunks; ++ck) {
    int n_entries = 0, n_tiles;
    if constexpr (DENSE) {
      n_tiles = (a.N + TILE - 1) / TILE;
    } else {
      const int c0 = ck * LMAX;
      n_entries = min(LMAX, a.L - c0);
      if (ck > 0) __syncthreads();  // the previous chunk's tables and tiles are no longer read
      sort_list<NT, BK>(a, idx_row, w_row, c0, n_entries, s_key, s_base, s_lim, s_lw, tid);
      n_tiles = (n_entries * BK + TILE - 1) / TILE;
    }
    auto meta_of = [&](int t) { return tile_meta<BK, DENSE>(a, s_base, s_lim, s_lw, t, n_entries); };

    // prologue: K(0), V(0), K(1) in flight; S(0) = QK(0)
    const TileMeta meta0 = meta_of(0), meta1 = meta_of(1);
    stage_one<D, NW, BK, PERM, false>(a, kb, K0, meta0, swave, lane, k_lane_off);
    stage_one<D, NW, BK, PERM, true>(a, vb, V0, meta0, swave, lane, v_lane_off);
    if (n_tiles > 1) stage_one<D, NW, BK, PERM, false>(a, kb, K1, meta1, swave, lane, k_lane_off);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    f32x16 Sa[2], Sb[2];
    qk_tile<D>(Sa, K0, LO, qf);

    // One pipelined step: S_cur = QK(t) on entry, S_next = QK(t+1) on exit;
    // PAR = t & 1 selects the slots at compile time. mt and mt1 describe tiles
    // t and t+1; the step returns the description of tile t+2, which it stages.
    auto step = [&](auto par_tag, f32x16 (&Scur)[2], f32x16 (&Snext)[2], int t, const TileMeta& mt,
                    const TileMeta& mt1) -> TileMeta {
      constexpr int PAR = decltype(par_tag)::value;
      BSA_LDS char* const k_write = PAR ? K1 : K0;  // K(t+2) lands in K(t)'s slot
      BSA_LDS char* const k_read = PAR ? K0 : K1;   // K(t+1)
      BSA_LDS char* const v_write = PAR ? V0 : V1;  // V(t+1)
      BSA_LDS char* const v_read = PAR ? V1 : V0;   // V(t)
      __builtin_amdgcn_s_waitcnt(0);  // this wave's K(t+1) and V(t) loads have landed
      __syncthreads();                // ... everyone's; the K(t) and V(t-1) slots are free
      const TileMeta mt2 = meta_of(t + 2);
      if (t + 2 < n_tiles) stage_one<D, NW, BK, PERM, false>(a, kb, k_write, mt2, swave, lane, k_lane_off);
      if (t + 1 < n_tiles) stage_one<D, NW, BK, PERM, true>(a, vb, v_write, mt1, swave, lane, v_lane_off);

      // ---- branches first: mask, row max, lazy rescale of O ----
      mask_tile<BK>(Scur, mt, kh, h);
      int lim[2], off[2];
      float lw[2];
      half_meta<BK>(mt, kh, lim, off, lw);
      float mx = fmaxf(Scur[0][0], Scur[0][1]);
#pragma unroll
      for (int q2 = 1; q2 < 16; ++q2) {  // a chain of 3-input maxima over the 32 values
        const int j = q2 / 8, r = 2 * (q2 % 8);
        mx = fmaxf(mx, fmaxf(Scur[j][r], Scur[j][r + 1]));
      }
      mx = halves_max(mx) * a.c;  // c > 0
      const bool need = mx > m_ref + RESCALE_SLACK;
      const float m_new = need ? mx : m_ref;
      const float alpha = (m_ref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new);
      if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
      }
      l_part *= alpha;
      m_ref = m_new;
      const float mb = (m_ref == -INFINITY) ? 0.f : m_ref;
      const float bias0 = lw[0] - mb, bias1 = lw[1] - mb;

      // ---- straight-line block, issued in this order (sched_barrier fences):
      // group i = { QK(t+1) MFMA i, the K read four MFMAs ahead, softmax pair(s) of
      // tile t }, then the PV(t) MFMAs with their transposed V reads four ahead.
      constexpr int NQ = D / 8;                // QK MFMAs per wave and tile
      constexpr int NP = 4 * (D / 32);         // PV MFMAs per wave and tile
      constexpr int PAIRS = 16 / NQ;           // softmax pairs per group (32 values per lane)
      const BSA_LDS char* kn = k_read + LO.kbase;
      const BSA_LDS char* vt = v_read + LO.vbase;
      auto kread = [&](int i) {
        return *(const BSA_LDS u32x4*)(kn + 64 * D * (i % 2) + LO.koff[i / 2]);
      };
      auto vread = [&](int m) {
        const int ks = m / (D / 32), dt = m % (D / 32);
        const BSA_LDS char* pa = vt + 2 * D * 16 * ks + LO.voff[dt];
        const i16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((BSA_LDS i16x4*)pa);
        const i16x4 vv = __builtin_amdgcn_ds_read_tr16_b64_v4i16((BSA_LDS i16x4*)(pa + 2 * D * 8));
        const u32x2 ua = __builtin_bit_cast(u32x2, va), ub = __builtin_bit_cast(u32x2, vv);
        return u32x4{ua[0], ua[1], ub[0], ub[1]};
      };
      u32x4 kf[4], vf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) kf[i] = kread(i);
      bf16x8 pb[4];
      float lsum = 0.f;
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        const int j = i % 2, st = i / 2;
        Snext[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[i % 4]), qf[st],
                                                           st == 0 ? f32x16{} : Snext[j], 0, 0, 0);
        if (i + 4 < NQ) kf[i % 4] = kread(i + 4);
        if (i >= NQ - 4) vf[i - (NQ - 4)] = vread(i - (NQ - 4));
#pragma unroll
        for (int pp_ = 0; pp_ < PAIRS; ++pp_) {
          const int q2 = i * PAIRS + pp_;       // pair index 0..15
          const int jj = q2 / 8, r = 2 * (q2 % 8);
          const float bias = jj ? bias1 : bias0;
          const float p0 = __builtin_amdgcn_exp2f(fmaf(Scur[jj][r], a.c, bias));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(Scur[jj][r + 1], a.c, bias));
          const bf16x2 pp = {static_cast<__bf16>(p0), static_cast<__bf16>(p1)};
          lsum = __builtin_amdgcn_fdot2_f32_bf16(pp, bf16x2{static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)},
                                                 lsum, false);
          pb[2 * jj + r / 8][r % 8] = pp[0];
          pb[2 * jj + r / 8][r % 8 + 1] = pp[1];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      l_part += lsum;

      // ---- O^T += V^T P^T over 4 steps of 16 keys of this wave's half. Step ks
      // takes P registers 8 (ks%2) + e of sub-tile ks/2, i.e. keys
      // 16 ks + 8 (e/4) + 4 h + e%4; the two transposed reads of vread fetch
      // e = 0..3 and 4..7.
#pragma unroll
      for (int m = 0; m < NP; ++m) {
        const int ks = m / (D / 32), dt = m % (D / 32);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf[m % 4]), pb[ks], o[dt], 0, 0, 0);
        if (m + 4 < NP) vf[m % 4] = vread(m + 4);
        __builtin_amdgcn_sched_barrier(0);
      }
      return mt2;
    };

    int t = 0;
    TileMeta ma = meta0, mb = meta1;
    for (; t + 1 < n_tiles; t += 2) {
      const TileMeta mc = step(std::integral_constant<int, 0>{}, Sa, Sb, t, ma, mb);
      const TileMeta md = step(std::integral_constant<int, 1>{}, Sb, Sa, t + 1, mb, mc);
      ma = mc;
      mb = md;
    }
    if (t < n_tiles) step(std::integral_constant<int, 0>{}, Sa, Sb, t, ma, mb);
  }

  // ---- merge the two key halves of each row group ----
  const float l_tot = halves_sum(l_part);
  __syncthreads();  // the tile buffers are free
  // Partial O of row group rg: (D/2) x 64 floats = 128 D bytes; two row groups
  // fit one tile slot (256 D bytes), so groups 0, 1 use k_lds0 and 2, 3 k_lds1.
  static_assert(NRG <= 4, "at most four row groups");
  float* part = reinterpret_cast<float*>(rg < 2 ? k_lds0 : k_lds1) + (rg % 2) * (D / 2) * 64;
  float* pm = reinterpret_cast<float*>(v_lds0);          // [NRG][64]
  float* pl = pm + NRG * 64;
  if (kh == 1) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) part[(dt * 16 + r) * 64 + lane] = o[dt][r];
    pm[rg * 64 + lane] = m_ref;
    pl[rg * 64 + lane] = l_tot;
  }
  __syncthreads();
  if (kh == 1) return;
  const float m1 = pm[rg * 64 + lane], l1 = pl[rg * 64 + lane];
  const float mm = fmaxf(m_ref, m1);
  const float s0 = (m_ref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_ref - mm);
  const float s1 = (m1 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
  const float lsum = l_tot * s0 + l1 * s1;

  // ---- epilogue: O^T register r of d-tile dt holds d = 32 dt + 8 (r/4) + 4 h + r%4 ----
  bool ok = true;
  int orow = qrow;
  float inv = 0.f;
  if (qrow < a.N) {
    orow = gather_row<PERM>(a, qrow, ok);
    inv = lsum > 0.f ? 1.f / lsum : 0.f;
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
        for (int z = 0; z < 4; ++z) {
          const int r = 4 * g + z;
          x[z] = (o[dt][r] * s0 + part[(dt * 16 + r) * 64 + lane] * s1) * inv;
        }
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
          (qrow < a.N && lsum > 0.f) ? (mm + __builtin_amdgcn_logf(lsum)) * 0.69314718055994531f : -INFINITY;
    }
  }
}

template <int D, int BQ, int BK, bool DENSE, bool PERM, bool OUT32>
hipError_t launch_one(const AttendArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((attend_bf16_kernel<D, BQ, BK, DENSE, PERM, OUT32>), dim3(a.n_wg), dim3(BQ * 4), 0, s, a);
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
  a.qchunk = (g.nQB + 7) / 8;
  a.n_wg = 8 * a.qchunk * g.B * g.H;
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
