// Attention kernel for 128-row query blocks with two independent workgroups
// per CU. A workgroup of four waves (one per SIMD) handles one (b, h, query
// block); wave w owns query rows [32 w, 32 w + 32) and every key of the 64-key
// tiles it walks through, so no partial softmaxes are merged at the end. Two
// such workgroups share a CU (256 registers per wave, under 80 KB of LDS
// each), so the two waves on a SIMD belong to different workgroups and never
// wait at the same barrier: while one waits for its tile, the other issues.
//
// Per wave and 64-key tile (AB-Attention, Abstract and transcript on the tiled
// kernel; InstaGen, Abstract):
//   S^T[key][row] = K . Q^T   (A = K rows from LDS, B = Q^T in registers)
//   O^T[d][row]  += V^T . P^T (A = V^T read transposed from LDS with
//                              ds_read_b64_tr_b16, B = P^T straight from the
//                              S^T accumulators after exp2 and bf16 packing)
// on v_mfma_f32_32x32x16_bf16. A lane holds one query row, so the row max and
// row sum stay in the lane except for one exchange between 32-lane halves.
// The weight of a key unit enters as log2(w) in the exponent bias.
//
// Key units of 128 keys take two tiles, units of 64 one, units of 32 share a
// tile in pairs. K runs one tile ahead of V: step t computes QK(t+1) beside
// the softmax of tile t, then PV(t), while the loads of K(t+2) and V(t+1)
// stream into the two free slots.
#pragma once

#include "attend_common.hpp"

namespace bsa {
namespace attend_bf16_impl {

constexpr int T64 = 64;      // keys per staged tile
constexpr int LMAX64 = 512;  // list entries sorted and held in LDS at a time
constexpr int NW64 = 4;      // waves per workgroup (128 query rows)

// Description of 64-key tile t of the current list chunk: slot u (S = min(BK,
// 64) keys each, 64 / S slots) holds the first key row, the valid keys and
// log2(w) of the unit part it stages. Tiles past the end describe empty slots
// at row 0.
template <int BK, bool DENSE>
__device__ __forceinline__ TileMeta tile_meta64(const AttendArgs& a, const int* s_base, const int* s_lim,
                                                const float* s_lw, int t, int n_entries) {
  constexpr int S = BK < T64 ? BK : T64;
  constexpr int NS = T64 / S;     // slots per tile
  constexpr int PARTS = BK / S;   // tiles per unit
  TileMeta m;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    m.base[u] = 0;
    m.lim[u] = 0;
    m.lw[u] = 0.f;
  }
  m.full = true;
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    if constexpr (DENSE) {
      if (t * T64 < a.N) {
        m.base[u] = t * T64;
        m.lim[u] = min(T64, a.N - t * T64);
      }
    } else {
      const int slot = t * NS + u;
      const int e = slot / PARTS, part = slot % PARTS;
      if (e < n_entries) {  // uniform values: keep them in scalar registers
        m.base[u] = __builtin_amdgcn_readfirstlane(s_base[e]) + part * S;
        m.lim[u] = min(S, max(0, __builtin_amdgcn_readfirstlane(s_lim[e]) - part * S));
        m.lw[u] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(s_lw[e])));
      }
    }
    m.full = m.full && m.lim[u] == S;
  }
  return m;
}

// Instruction i of a tile's staging, without branches (K and V read in place): the
// lane's row is i G + r0 of the tile; rows past a slot's valid keys load the
// slot's last valid key (an empty slot, base 0 and no keys: row 0), so the
// address is the slot's first row (uniform) plus min(row in slot, last valid
// row) 2D + the lane's chunk byte (chunk_off = 16 ((lane % CPR) ^ swz(r0))).
template <int D, int S>
__device__ __forceinline__ void stage64_ins(const uint16_t* src, BSA_LDS char* dst, const TileMeta& m, int swave,
                                            int r0, uint32_t chunk_off, int i) {
  using SG = StageGeom<D, NW64, T64>;
  static_assert(S % SG::G == 0 || SG::G % S == 0, "slot and row step must nest");
  const int row0 = i * SG::G + swave * SG::RPI;
  const int u = S % SG::G == 0 ? i * SG::G / S : row0 / S;
  const int c = i * SG::G - u * S;               // row in the slot of the lane with r0 = 0
  const int last = max(pick4(m.lim, u), 1) - 1;  // last valid row of the slot (uniform)
  const char* sp = reinterpret_cast<const char*>(src) + static_cast<size_t>(pick4(m.base, u)) * (2 * D);
  uint32_t off = static_cast<uint32_t>(min(r0 + c, last)) * (2 * D) + chunk_off;
  pin(off);  // keeps the base uniform: scalar base + 32-bit lane offset addressing
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(sp + off),
                                   (BSA_LDS void*)(dst + (i * NW64 + swave) * 1024), 16, 0, 0);
}

// Gathered key row of tile row r when K and V go through perm: slot r / S, key
// r % S -> perm[base + r % S]; a row past the slot's valid keys, or a gather
// entry outside [0, N_pad), gives row 0 of the head (its logits are masked).
template <int S>
__device__ __forceinline__ int tile64_row_gather(const AttendArgs& a, const TileMeta& m, int r) {
  const int u = r / S, o = r % S;
  if (o >= pick4(m.lim, u)) return 0;
  const int g = a.perm[pick4(m.base, u) + o];
  return static_cast<unsigned>(g) < static_cast<unsigned>(a.N_pad) ? g : 0;
}

// The whole tile with the lookups done here (the first tiles of a chunk).
template <int D, int S, bool PERM>
__device__ __forceinline__ void stage64_direct(const AttendArgs& a, const uint16_t* src, BSA_LDS char* dst,
                                               const TileMeta& m, int swave, int r0, uint32_t chunk_off) {
  using SG = StageGeom<D, NW64, T64>;
#pragma unroll
  for (int i = 0; i < SG::PER_WAVE; ++i) {
    const int row = i * SG::G + r0;
    int gr;
    if constexpr (PERM) {
      gr = tile64_row_gather<S>(a, m, row);
    } else {
      const int u = row / S, o = row % S;
      gr = pick4(m.base, u) + min(o, max(pick4(m.lim, u), 1) - 1);
    }
    __builtin_amdgcn_global_load_lds(
        reinterpret_cast<const void*>(reinterpret_cast<const char*>(src) + static_cast<size_t>(gr) * (2 * D) + chunk_off),
        (BSA_LDS void*)(dst + (i * NW64 + swave) * 1024), 16, 0, 0);
  }
}

// Keys past the valid range of their slot get -inf (uniform branch; only
// tiles that hold a partial or empty slot take it). Register r of sub-tile j
// holds key 32 j + 8 (r/4) + 4 h + r%4 of the tile, i.e. key
// off_j + 8 (r/4) + 4 h + r%4 of slot u_j = 32 j / S.
template <int BK>
__device__ __forceinline__ bool mask_tile64(f32x16 (&S)[2], const TileMeta& m, int h) {
  constexpr int SL = BK < T64 ? BK : T64;
  int lim[2], off[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    lim[j] = pick4(m.lim, 32 * j / SL);
    off[j] = 32 * j % SL;
  }
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

// Largest shifted logit x + log2(w) of the 32 values a lane holds: sub-tile j
// belongs to slot 32 j / S, whose log-weight it carries (c > 0, so the
// maximum of the raw products scales to the maximum of x).
template <int BK>
__device__ __forceinline__ float tile_xmax64(const f32x16 (&S)[2], const TileMeta& m, float c) {
  constexpr int SL = BK < T64 ? BK : T64;
  float m0 = fmaxf(S[0][0], S[0][1]), m1 = fmaxf(S[1][0], S[1][1]);
#pragma unroll
  for (int r = 2; r < 16; r += 2) {
    m0 = fmaxf(m0, fmaxf(S[0][r], S[0][r + 1]));
    m1 = fmaxf(m1, fmaxf(S[1][r], S[1][r + 1]));
  }
  if constexpr (SL == 32) return fmaxf(fmaf(m0, c, m.lw[0]), fmaf(m1, c, m.lw[1]));
  return fmaf(fmaxf(m0, m1), c, m.lw[0]);
}

template <int D, int BK, bool DENSE, int PM, bool OUT32>
__global__ __launch_bounds__(64 * NW64, 2) void attend_t64_kernel(AttendArgs a) {
  constexpr int NT = 64 * NW64;
  constexpr bool PERM = PM == PERM_ALL;  // K and V rows gathered through perm while staging
  constexpr bool PQ = PM != PERM_NONE;   // Q rows gathered, out and lse rows scattered
  constexpr int SL = BK < T64 ? BK : T64;  // keys per slot of a tile
  constexpr int TB = T64 * 2 * D;          // bytes per staged tile
  using SG = StageGeom<D, NW64, T64>;
  // Four tile slots (K0, K1, V0, V1): each step writes one K and one V slot
  // with direct loads while it reads the other two; the slot choice is a
  // compile-time constant there.
  __shared__ __attribute__((aligned(1024))) char k_lds0[TB];
  __shared__ __attribute__((aligned(1024))) char k_lds1[TB];
  __shared__ __attribute__((aligned(1024))) char v_lds0[TB];
  __shared__ __attribute__((aligned(1024))) char v_lds1[TB];
  __shared__ int s_base[DENSE ? 1 : LMAX64];
  __shared__ int s_lim[DENSE ? 1 : LMAX64];
  __shared__ float s_lw[DENSE ? 1 : LMAX64];
  // K and V through perm: gathered key rows of tiles t+1 .. t+3, slot (t & 3)
  __shared__ int s_grow[PERM ? 4 * T64 : 1];
  static_assert(LMAX64 * 4 <= TB, "the sort keys borrow a tile slot");

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64;
  const int n = lane % 32, h = lane / 32;

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
  const int qrow = qi * 128 + 32 * wave + n;
  bool qok = qrow < a.N;
  const int qg = gather_row<PQ>(a, qrow, qok);
  bf16x8 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    qf[s] = as_bf16x8(qok ? ldg16(qb + static_cast<size_t>(qg) * D + 16 * s + 8 * h) : u32x4{0u, 0u, 0u, 0u});

  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16{};
  float m_ref = -INFINITY;  // running max of x for this row (shared by both lane halves)
  float l_part = 0.f;       // this lane's share of the weighted denominator

  BSA_LDS char* const K0 = (BSA_LDS char*)(k_lds0);  // address-space casts of the shared arrays
  BSA_LDS char* const K1 = (BSA_LDS char*)(k_lds1);
  BSA_LDS char* const V0 = (BSA_LDS char*)(v_lds0);
  BSA_LDS char* const V1 = (BSA_LDS char*)(v_lds1);
  const LaneOffsets<D> LO = lane_offsets<D>(0, lane);
  const int swave = __builtin_amdgcn_readfirstlane(wave);
  // per-lane parts of the staging addresses
  const int st_r0 = wave * SG::RPI + lane / SG::CPR;
  const uint32_t k_chunk = 16 * ((lane % SG::CPR) ^ k_swz<D>(st_r0));
  const uint32_t v_chunk = 16 * ((lane % SG::CPR) ^ v_swz<D>(st_r0));
  const int n_chunks = DENSE ? 1 : (a.L + LMAX64 - 1) / LMAX64;
  for (int ck = 0; ck < n_chunks; ++ck) {
    int n_entries = 0, n_tiles;
    if constexpr (DENSE) {
      n_tiles = (a.N + T64 - 1) / T64;
    } else {
      const int c0 = ck * LMAX64;
      n_entries = min(LMAX64, a.L - c0);
      if (ck > 0) __syncthreads();  // the previous chunk's tables and tiles are no longer read
      sort_list<NT, BK>(a, idx_row, w_row, c0, n_entries, reinterpret_cast<int*>(v_lds1), s_base, s_lim, s_lw,
                        tid);
      n_tiles = (n_entries * BK + T64 - 1) / T64;
    }
    auto meta_of = [&](int t) { return tile_meta64<BK, DENSE>(a, s_base, s_lim, s_lw, t, n_entries); };

    // prologue: K(0), V(0), K(1) in flight; S(0) = QK(0)
    const TileMeta meta0 = meta_of(0), meta1 = meta_of(1);
    stage64_direct<D, SL, PERM>(a, kb, K0, meta0, swave, st_r0, k_chunk);
    stage64_direct<D, SL, PERM>(a, vb, V0, meta0, swave, st_r0, v_chunk);
    if (n_tiles > 1) stage64_direct<D, SL, PERM>(a, kb, K1, meta1, swave, st_r0, k_chunk);
    if constexpr (PERM) {  // gathered rows of tiles 1 and 2 for the first step's staging
      if (tid < T64) {
        s_grow[1 * T64 + tid] = tile64_row_gather<SL>(a, meta1, tid);
        s_grow[2 * T64 + tid] = tile64_row_gather<SL>(a, meta_of(2), tid);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // Running-max bookkeeping on the shifted logits x + log2(w), so that no
    // exponent exceeds 2^RESCALE_SLACK whatever the weights. When a tile's
    // scores are complete, its maximum decides the transition into it:
    // rescale (need) when it exceeds the reference by more than the slack, to
    // m_new, by alpha = 2^(m_ref - m_new). The transition is applied at the top
    // of the step that computes the tile, after the previous tile's PV
    // products have landed in O.
    bool need = false;
    float m_new = m_ref, alpha = 1.f;
    auto decide = [&](float x_lane) {
      const float mx = halves_max(x_lane);
      need = mx > m_ref + RESCALE_SLACK;
      m_new = need ? mx : m_ref;
      alpha = (m_ref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new);
    };
    f32x16 Sa[2], Sb[2];
    qk_tile<D>(Sa, K0, LO, qf);
    mask_tile64<BK>(Sa, meta0, h);
    decide(tile_xmax64<BK>(Sa, meta0, a.c));

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
      // K reads for the first QK MFMAs go out first; the tile descriptions
      // (LDS reads too) complete behind them
      const BSA_LDS char* kn = k_read + LO.kbase;
      const BSA_LDS char* vt = v_read + LO.vbase;
      auto kread = [&](int i) {
        return *(const BSA_LDS u32x4*)(kn + 64 * D * (i % 2) + koff<D>(LO, i / 2));
      };
      auto vread = [&](int m) {
        const int ks = m / (D / 32), dt = m % (D / 32);
        const BSA_LDS char* pa = vt + 2 * D * 16 * ks + voff<D>(LO, dt);
        const i16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((BSA_LDS i16x4*)pa);
        const i16x4 vv = __builtin_amdgcn_ds_read_tr16_b64_v4i16((BSA_LDS i16x4*)(pa + 2 * D * 8));
        const u32x2 ua = __builtin_bit_cast(u32x2, va), ub = __builtin_bit_cast(u32x2, vv);
        return u32x4{ua[0], ua[1], ub[0], ub[1]};
      };
      u32x4 kf[4], vf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) kf[i] = kread(i);
      const TileMeta mt2 = meta_of(t + 2);
      // Staging of K(t+2) and V(t+1). With K and V gathered all of it happens
      // here, from the gathered rows the step before last looked up, and this
      // step looks up tile t+3's rows (stored at its end); otherwise one load
      // per few MFMA groups below, branch-free: past the end of the list the
      // loads fill the free slots with row 0 of the head, which nothing reads.
      int grow_next = 0;
      constexpr int PW = SG::PER_WAVE;
      if constexpr (PERM) {
        if (t + 2 < n_tiles) {
#pragma unroll
          for (int i = 0; i < PW; ++i) {
            const int gr = s_grow[((t + 2) & 3) * T64 + i * SG::G + st_r0];
            __builtin_amdgcn_global_load_lds(
                reinterpret_cast<const void*>(reinterpret_cast<const char*>(kb) + static_cast<size_t>(gr) * (2 * D) + k_chunk),
                (BSA_LDS void*)(k_write + (i * NW64 + swave) * 1024), 16, 0, 0);
          }
        }
        if (t + 1 < n_tiles) {
#pragma unroll
          for (int i = 0; i < PW; ++i) {
            const int gr = s_grow[((t + 1) & 3) * T64 + i * SG::G + st_r0];
            __builtin_amdgcn_global_load_lds(
                reinterpret_cast<const void*>(reinterpret_cast<const char*>(vb) + static_cast<size_t>(gr) * (2 * D) + v_chunk),
                (BSA_LDS void*)(v_write + (i * NW64 + swave) * 1024), 16, 0, 0);
          }
        }
        if (tid < T64 && t + 3 < n_tiles) grow_next = tile64_row_gather<SL>(a, meta_of(t + 3), tid);
      }
      constexpr int NQ = D / 8;         // QK MFMAs per wave and tile
      constexpr int NP = 4 * (D / 32);  // PV MFMAs per wave and tile
      // staging load k (K loads 0..PW-1, then V) goes with MFMA group 1 + k NQ / (2 PW): spread over
      // the QK groups, so the last loads still have the PV groups to land before the next barrier
      auto stage_k = [&](int grp) {
        if constexpr (!PERM) {
#pragma unroll
          for (int k = 0; k < 2 * PW; ++k) {
            if (1 + k * NQ / (2 * PW) != grp) continue;
            if (k < PW) stage64_ins<D, SL>(kb, k_write, mt2, swave, st_r0, k_chunk, k);
            else stage64_ins<D, SL>(vb, v_write, mt1, swave, st_r0, v_chunk, k - PW);
          }
        }
      };

      // ---- tiles with keys past a slot's end: mask S(t) and redo its maximum
      // (the previous step took it before masking); then the transition into t
      if (mask_tile64<BK>(Scur, mt, h)) decide(tile_xmax64<BK>(Scur, mt, a.c));
      if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
      }
      l_part *= alpha;
      m_ref = m_new;
      const float mb = (m_ref == -INFINITY) ? 0.f : m_ref;
      const float bias0 = mt.lw[0] - mb;
      const float bias1 = (SL == 32 ? mt.lw[1] : mt.lw[0]) - mb;

      // ---- straight-line block, issued in this order (sched_barrier fences):
      // group i = { QK(t+1) MFMA i, the K read four MFMAs ahead, softmax pair(s) of
      // tile t }, then the PV(t) MFMAs with their transposed V reads four ahead.
      constexpr int PAIRS = 16 / NQ;  // softmax pairs per group (32 values per lane)
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
          const int q2 = i * PAIRS + pp_;  // pair index 0..15
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
        stage_k(i);
        __builtin_amdgcn_sched_barrier(0);
      }
      l_part += lsum;

      // ---- O^T += V^T P^T over 4 steps of 16 keys. Step ks takes P registers
      // 8 (ks%2) + e of sub-tile ks/2, i.e. keys 16 ks + 8 (e/4) + 4 h + e%4;
      // the two transposed reads of vread fetch e = 0..3 and 4..7. Alongside,
      // the maximum of S(t+1) (before masking, which the next step applies if
      // the tile needs it) and its transition decision.
      float mx[2] = {-INFINITY, -INFINITY};  // per sub-tile: they may carry different weights
      constexpr int MS = NP - 3;
#pragma unroll
      for (int m = 0; m < NP; ++m) {
        const int ks = m / (D / 32), dt = m % (D / 32);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf[m % 4]), pb[ks], o[dt], 0, 0, 0);
        if (m + 4 < NP) vf[m % 4] = vread(m + 4);
        stage_k(NQ + m);
        if (m >= 2 && m < NP - 1) {
#pragma unroll
          for (int q = (16 * (m - 2) + MS - 1) / MS; q < (16 * (m - 1) + MS - 1) / MS; ++q) {
            mx[q / 8] = fmaxf(mx[q / 8], fmaxf(Snext[q / 8][2 * (q % 8)], Snext[q / 8][2 * (q % 8) + 1]));
            pin(mx[q / 8]);
          }
        } else if (m == NP - 1) {
          if constexpr (SL == 32) decide(fmaxf(fmaf(mx[0], a.c, mt1.lw[0]), fmaf(mx[1], a.c, mt1.lw[1])));
          else decide(fmaf(fmaxf(mx[0], mx[1]), a.c, mt1.lw[0]));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (PERM) {
        // tile t+3's slot held tile t-1, whose last reader (the staging of
        // V(t-1)) ran two steps ago; readers of the new rows come after a barrier
        if (tid < T64) s_grow[((t + 3) & 3) * T64 + tid] = grow_next;
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
    // the final steps' staging loads (into free slots) land before the slots
    // are reused by the next chunk's sort and tiles
    __builtin_amdgcn_s_waitcnt(0);
  }

  // ---- epilogue: O^T register r of d-tile dt holds d = 32 dt + 8 (r/4) + 4 h + r%4 ----
  const float lsum = halves_sum(l_part);
  bool ok = true;
  int orow = qrow;
  float inv = 0.f;
  if (qrow < a.N) {
    orow = gather_row<PQ>(a, qrow, ok);
    inv = lsum > 0.f ? 1.f / lsum : 0.f;
  }
  if constexpr (OUT32) {
    // fp32 rows go out whole: each wave stages its 32 rows (row-major, 16-byte
    // chunk c of row n at chunk c ^ (n mod CPR), conflict-free both ways) in its
    // own tile slot, then every store instruction writes 64 / CPR complete rows.
    constexpr int CPR = D / 4;  // 16-byte chunks per fp32 row
    __syncthreads();            // every wave is done with the tile slots
    char* stage = wave == 0 ? k_lds0 : wave == 1 ? k_lds1 : wave == 2 ? v_lds0 : v_lds1;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = (32 * dt + 8 * g + 4 * h) / 4;
        float4 x = make_float4(o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv, o[dt][4 * g + 2] * inv,
                               o[dt][4 * g + 3] * inv);
        *reinterpret_cast<float4*>(stage + n * (4 * D) + 16 * (c ^ (n % CPR))) = x;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    constexpr int RPS = 64 / CPR;  // rows per store instruction
#pragma unroll
    for (int z = 0; z < 32 / RPS; ++z) {
      const int rr = z * RPS + lane / CPR, c = lane % CPR;
      const int grow = qi * 128 + 32 * wave + rr;  // this lane's query row
      bool rok = true;
      int orow_r = grow;
      if (grow < a.N) orow_r = gather_row<PQ>(a, grow, rok);
      const float4 x = *reinterpret_cast<const float4*>(stage + rr * (4 * D) + 16 * (c ^ (rr % CPR)));
      if (rok) *reinterpret_cast<float4*>(static_cast<float*>(a.out) + bh_off + static_cast<size_t>(orow_r) * D + 4 * c) = x;
    }
    if (a.lse != nullptr && h == 0 && ok) {
      a.lse[static_cast<size_t>(bh) * a.N_pad + orow] =
          (qrow < a.N && lsum > 0.f) ? (m_ref + __builtin_amdgcn_logf(lsum)) * 0.69314718055994531f : -INFINITY;
    }
    return;
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
          (qrow < a.N && lsum > 0.f) ? (m_ref + __builtin_amdgcn_logf(lsum)) * 0.69314718055994531f : -INFINITY;
    }
  }
}

}  // namespace attend_bf16_impl
}  // namespace bsa
