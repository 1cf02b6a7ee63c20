// Attention kernel in which each wave owns 32 query rows: one workgroup per
// (b, h, query block) with 2 BQ / 32 waves; wave (rg, kh) owns query rows
// [32 rg, 32 rg + 32) and keys [64 kh, 64 kh + 64) of every 128-key tile; the
// two key halves are merged at the end like two partial softmaxes. Per wave
// and tile:
//   S^T[key][row] = K . Q^T   (A = K rows from LDS, B = Q^T in registers)
//   O^T[d][row]  += V^T . P^T (A = V^T read transposed from LDS with
//                              ds_read_b64_tr_b16, B = P^T straight from the
//                              S^T accumulators after exp and bf16 packing)
// on v_mfma_f32_32x32x16_bf16. A lane holds one query row, so the row max and
// row sum stay in the lane except for one exchange between 32-lane halves.
// Used for 64-row query blocks (4 waves, one per SIMD); 128-row blocks take
// attend_t64_kernel (attend_bf16_t64.hpp).
#pragma once

#include "attend_common.hpp"

namespace bsa {
namespace attend_bf16_impl {

// Largest shifted logit x + log2(w) of the 32 values a lane holds: sub-tile j
// of key half kh carries the log-weight of its unit (c > 0).
template <int BK>
__device__ __forceinline__ float tile_xmax_half(const f32x16 (&S)[2], const TileMeta& m, int kh, float c) {
  int lim[2], off[2];
  float lw[2];
  half_meta<BK>(m, kh, lim, off, lw);
  float m0 = fmaxf(S[0][0], S[0][1]), m1 = fmaxf(S[1][0], S[1][1]);
#pragma unroll
  for (int r = 2; r < 16; r += 2) {
    m0 = fmaxf(m0, fmaxf(S[0][r], S[0][r + 1]));
    m1 = fmaxf(m1, fmaxf(S[1][r], S[1][r + 1]));
  }
  return fmaxf(fmaf(m0, c, lw[0]), fmaf(m1, c, lw[1]));
}

template <int D, int BQ, int BK, bool DENSE, int PM, bool OUT32>
__global__ __launch_bounds__(BQ * 4, 1) void attend_w32_kernel(AttendArgs a) {
  constexpr bool PERM = PM == PERM_ALL;  // K and V rows gathered through perm while staging
  constexpr bool PQ = PM != PERM_NONE;   // Q rows gathered, out and lse rows scattered
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
  // K and V through perm: gathered key rows of tiles t+1 .. t+3, slot (t & 3)
  __shared__ int s_grow[PERM ? 4 * TILE : 1];

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

  // K runs one tile ahead of V so that QK of tile t+1 overlaps the softmax of tile t.
  BSA_LDS char* const K0 = (BSA_LDS char*)(k_lds0);  // address-space casts of the shared arrays
  BSA_LDS char* const K1 = (BSA_LDS char*)(k_lds1);
  BSA_LDS char* const V0 = (BSA_LDS char*)(v_lds0);
  BSA_LDS char* const V1 = (BSA_LDS char*)(v_lds1);
  const LaneOffsets<D> LO = lane_offsets<D>(kh, lane);
  const int swave = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t k_lane_off = stage_lane_offset<D, NW>(wave, lane, false);
  const uint32_t v_lane_off = stage_lane_offset<D, NW>(wave, lane, true);
  // per-lane parts of the branch-free staging addresses
  const int st_r0 = wave * StageGeom<D, NW>::RPI + lane / StageGeom<D, NW>::CPR;
  const uint32_t k_chunk = 16 * ((lane % StageGeom<D, NW>::CPR) ^ k_swz<D>(st_r0));
  const uint32_t v_chunk = 16 * ((lane % StageGeom<D, NW>::CPR) ^ v_swz<D>(st_r0));
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
    if constexpr (PERM) {  // gathered rows of tiles 1 and 2 for the first step's staging
      if (tid < TILE) {
        s_grow[1 * TILE + tid] = tile_row_gather<BK>(a, meta1, tid);
        s_grow[2 * TILE + tid] = tile_row_gather<BK>(a, meta_of(2), tid);
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
    mask_tile<BK>(Sa, meta0, kh, h);
    decide(tile_xmax_half<BK>(Sa, meta0, kh, a.c));

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
      if constexpr (PERM) {
        constexpr int PW_ = StageGeom<D, NW>::PER_WAVE;
        if (t + 2 < n_tiles) {
#pragma unroll
          for (int i = 0; i < PW_; ++i)
            stage_gathered<D, NW>(kb, k_write, s_grow + ((t + 2) & 3) * TILE, swave, st_r0, k_chunk, i);
        }
        if (t + 1 < n_tiles) {
#pragma unroll
          for (int i = 0; i < PW_; ++i)
            stage_gathered<D, NW>(vb, v_write, s_grow + ((t + 1) & 3) * TILE, swave, st_r0, v_chunk, i);
        }
        if (tid < TILE && t + 3 < n_tiles) grow_next = tile_row_gather<BK>(a, meta_of(t + 3), tid);
      }
      constexpr int PW = StageGeom<D, NW>::PER_WAVE;
      // staging load k (K loads 0..PW-1, then V) goes with MFMA group 1 + k NQ / (2 PW): spread over
      // the QK groups, so the last loads still have the PV groups to land before the next barrier
      auto stage_k = [&](int grp) {
        if constexpr (!PERM) {
#pragma unroll
          for (int k = 0; k < 2 * PW; ++k) {
            if (1 + k * (D / 8) / (2 * PW) != grp) continue;
            if (k < PW) stage_ins<D, NW, BK>(kb, k_write, mt2, swave, st_r0, k_chunk, k);
            else stage_ins<D, NW, BK>(vb, v_write, mt1, swave, st_r0, v_chunk, k - PW);
          }
        }
      };

      // ---- tiles with keys past a unit's end: mask S(t) and redo its maximum
      // (the previous step took it before masking); then the transition into t
      if (mask_tile<BK>(Scur, mt, kh, h)) decide(tile_xmax_half<BK>(Scur, mt, kh, a.c));
      if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
      }
      l_part *= alpha;
      m_ref = m_new;
      int lim[2], off[2];
      float lw[2];
      half_meta<BK>(mt, kh, lim, off, lw);
      const float mb = (m_ref == -INFINITY) ? 0.f : m_ref;
      const float bias0 = lw[0] - mb, bias1 = lw[1] - mb;

      // ---- straight-line block, issued in this order (sched_barrier fences):
      // group i = { QK(t+1) MFMA i, the K read four MFMAs ahead, softmax pair(s) of
      // tile t }, then the PV(t) MFMAs with their transposed V reads four ahead.
      constexpr int NQ = D / 8;                // QK MFMAs per wave and tile
      constexpr int NP = 4 * (D / 32);         // PV MFMAs per wave and tile
      constexpr int PAIRS = 16 / NQ;           // softmax pairs per group (32 values per lane)
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
        stage_k(i);
        __builtin_amdgcn_sched_barrier(0);
      }
      l_part += lsum;

      // ---- O^T += V^T P^T over 4 steps of 16 keys of this wave's half. Step ks
      // takes P registers 8 (ks%2) + e of sub-tile ks/2, i.e. keys
      // 16 ks + 8 (e/4) + 4 h + e%4; the two transposed reads of vread fetch
      // e = 0..3 and 4..7. Alongside, the maximum of S(t+1) (16 steps of a
      // 3-input maximum over groups 2 .. NP-2; before masking, which the next
      // step applies if the tile needs it) and its transition decision.
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
          int lim1[2], off1[2];
          float lw1[2];
          half_meta<BK>(mt1, kh, lim1, off1, lw1);
          decide(fmaxf(fmaf(mx[0], a.c, lw1[0]), fmaf(mx[1], a.c, lw1[1])));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (PERM) {
        // tile t+3's slot held tile t-1, whose last reader (the staging of
        // V(t-1)) ran two steps ago; readers of the new rows come after a barrier
        if (tid < TILE) s_grow[((t + 3) & 3) * TILE + tid] = grow_next;
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
    // are reused by the next chunk or by the merge below
    __builtin_amdgcn_s_waitcnt(0);
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
    orow = gather_row<PQ>(a, qrow, ok);
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

}  // namespace attend_bf16_impl
}  // namespace bsa
