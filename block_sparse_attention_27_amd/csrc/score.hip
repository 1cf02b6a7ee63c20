// Block scoring for gfx950: block means of Q and K, then the estimated
// attention mass of every key unit for every query block.
//
// What is computed (AB-Attention, Abstract: key blocks rated from cheap
// per-block summaries; InstaGen, Abstract: the sampling chance of a block
// follows its estimated share of attention):
//   q_mean_i = mean of the valid rows of query block i  (0 if it has none)
//   k_mean_j = mean of the n_j valid keys of unit j
//   S_ij     = n_j exp(l_ij - L_i) / sum_{valid j'} n_j' exp(l_ij' - L_i),
//   l_ij = sm_scale <q_mean_i, k_mean_j>, L_i = max over valid j; S = 0 for
//   units with no valid key.
//
// block_means_kernel streams Q and K once from HBM (16-byte loads, fp32
// accumulation, one LDS reduction per block). scores_kernel contracts the
// fp32 means in the S^T orientation (a lane holds one query block, its
// registers 16 units) on bf16 MFMAs with every value split into bf16 hi + lo
// parts (three products, fp32 accumulation: about 1e-5 relative), so each
// lane keeps its own running max and n_j-weighted sum; a second pass
// recomputes the logits (or reads them back from LDS) and writes S once,
// normalised. scores_shared_kernel does the same with each staged chunk of key
// means shared by four column tiles of a workgroup; it takes the clustering
// scorer's G representatives per block, and one representative whenever its
// grid is large enough.
#include "bsa_internal.hpp"

#include <math.h>

namespace bsa {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int MEAN_THREADS = 256;

struct MeansArgs {
  const void* q;
  const void* k;
  const int32_t* perm;
  float* q_mean;
  float* k_mean;
  float* k_var;  // nullptr, or per-dimension population variance of every key unit
  int N, N_pad, block_q, block_k, nQB, nKU, n_bh;
  int k_gather;  // 1: key rows go through perm too (0: K arrives in permuted order)
  int first;  // logical block of workgroup 0 (n_bh * nQB: key units only)
};

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }

// One workgroup per block of rows (a query block or a key unit).
template <int D, bool BF16, bool PERM>
__global__ __launch_bounds__(MEAN_THREADS) void block_means_kernel(MeansArgs a) {
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int EPC = 16 / ESZ;              // elements per 16-byte chunk
  constexpr int CH = D / EPC;                // chunks per row
  constexpr int RPP = MEAN_THREADS / CH;     // rows per pass
  __shared__ float red[RPP][D + 1];

  const int tid = threadIdx.x;
  const int nq = a.n_bh * a.nQB;
  const int lb = static_cast<int>(blockIdx.x) + a.first;
  const bool is_q = lb < nq;
  const int blk = is_q ? lb : lb - nq;
  const int per = is_q ? a.nQB : a.nKU;
  const int bs = is_q ? a.block_q : a.block_k;
  const int bh = blk / per, bi = blk % per;
  const char* base = static_cast<const char*>(is_q ? a.q : a.k) + static_cast<size_t>(bh) * a.N_pad * D * ESZ;
  const int row0 = bi * bs;
  const int nvalid = max(0, min(bs, a.N - row0));

  constexpr int MAXP = 128 / RPP;  // passes for the largest block (128 rows)
  const int cc = tid % CH, rg = tid / CH;
  u32x4 x[MAXP];
#pragma unroll
  for (int p = 0; p < MAXP; ++p) {
    const int r = rg + p * RPP;
    bool ok = r < nvalid;
    int g = row0 + r;
    if constexpr (PERM) {
      if (ok && (is_q || a.k_gather)) {
        g = a.perm[g];
        ok = static_cast<unsigned>(g) < static_cast<unsigned>(a.N_pad);
      }
    }
    x[p] = ok ? *reinterpret_cast<const u32x4*>(base + (static_cast<size_t>(g) * D + cc * EPC) * ESZ)
              : u32x4{0u, 0u, 0u, 0u};
  }
  float acc[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.f;
#pragma unroll
  for (int p = 0; p < MAXP; ++p) {
    if constexpr (BF16) {
#pragma unroll
      for (int z = 0; z < 4; ++z) {
        acc[2 * z] += bf16_lo(x[p][z]);
        acc[2 * z + 1] += bf16_hi(x[p][z]);
      }
    } else {
#pragma unroll
      for (int z = 0; z < 4; ++z) acc[z] += __uint_as_float(x[p][z]);
    }
  }
#pragma unroll
  for (int e = 0; e < EPC; ++e) red[rg][cc * EPC + e] = acc[e];
  __syncthreads();
  __shared__ float mean_s[D];
  if (tid < D) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < RPP; ++r) s += red[r][tid];
    float* out = (is_q ? a.q_mean : a.k_mean) + (static_cast<size_t>(bh) * per + bi) * D;
    const float m = nvalid > 0 ? s / static_cast<float>(nvalid) : 0.f;
    out[tid] = m;
    mean_s[tid] = m;
  }
  if (is_q || a.k_var == nullptr) return;  // whole workgroup
  // key units: population variance from the deviations of the staged rows
  __syncthreads();  // means ready; red is free
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.f;
#pragma unroll
  for (int p = 0; p < MAXP; ++p) {
    if (rg + p * RPP < nvalid) {
#pragma unroll
      for (int z = 0; z < EPC; ++z) {
        float xv;
        if constexpr (BF16) xv = (z % 2) ? bf16_hi(x[p][z / 2]) : bf16_lo(x[p][z / 2]);
        else xv = __uint_as_float(x[p][z]);
        const float dv = xv - mean_s[cc * EPC + z];
        acc[z] = fmaf(dv, dv, acc[z]);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < EPC; ++e) red[rg][cc * EPC + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < RPP; ++r) s += red[r][tid];
    a.k_var[(static_cast<size_t>(bh) * per + bi) * D + tid] = nvalid > 0 ? s / static_cast<float>(nvalid) : 0.f;
  }
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// x (8 floats) = hi + lo with hi = bf16(x) and lo = bf16(x - hi), both round
// to nearest even: |x - hi - lo| <= 2^-18 |x|.
__device__ __forceinline__ void split_bf16(f32x4 x0, f32x4 x1, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int z = 0; z < 8; ++z) {
    const float x = z < 4 ? x0[z] : x1[z - 4];
    const __bf16 h = static_cast<__bf16>(x);
    hi[z] = h;
    lo[z] = static_cast<__bf16>(x - static_cast<float>(h));
  }
}

struct ScoreArgs {
  const float* q_rep;     // [bh][nQB][G][D] query representatives (block means when G = 1)
  const int32_t* q_size;  // [bh][nQB][G] rows per representative; nullptr: weight 1 (G = 1)
  const float* k_mean;
  const float* k_var;     // STATS: per-dimension variance of every key unit
  float* S;
  int N, block_k, nQB, nKU, n_qgroups;
  float sm_scale;
};

constexpr int SC_WAVES = 8;
constexpr int SC_CACHE_CHUNKS = 20;  // units up to 640: logits stay in LDS between the passes

// One workgroup per (b, h, group of 32/G query blocks); wave w takes unit
// chunks w, w + 8, ... (32 units each). MFMA column (lane) n holds
// representative g = n % G of query block n / G. Pass 1 contracts every chunk
// and keeps, per lane, the running maximum and n_j-weighted sum of
// 2^(x - max) with x = l log2(e); the lane halves and the waves combine them.
// Pass 2 contracts the chunks again (the representatives and key means are
// small and stay in L2) or reads the logits back: from LDS when every chunk's
// fit there (up to 640 units), else, with one representative per query block,
// from S, where pass 1 left them; it scales every lane's masses by its weight
// n_g / n, sums the G lanes of a query block, and writes S once: each wave
// transposes its block through LDS so that every store instruction covers two
// contiguous 128-byte row segments of S.
// Sum over each aligned group of G consecutive lanes (G = 1, 2, 4, 8) on DPP
// moves: the quad swaps [1, 0, 3, 2] and [2, 3, 0, 1] (lane xor 1, xor 2),
// then the half-row mirror, which pairs the two quads of an 8-lane group
// once every lane of a quad holds the quad's sum.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group size");
  if constexpr (G >= 2) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  if constexpr (G >= 4) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  if constexpr (G >= 8) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  return v;
}

template <int D, int G, bool CACHE, bool STATS>
__global__ __launch_bounds__(64 * SC_WAVES) void scores_kernel(ScoreArgs a) {
  constexpr int QB = 32 / G;   // query blocks per workgroup
  __shared__ float red_m[SC_WAVES][32];
  __shared__ float red_s[SC_WAVES][32];
  __shared__ float tile[SC_WAVES][QB][33];  // one chunk of one wave: [query block][unit], padded
  // CACHE: pass 1 keeps every chunk's logits (each lane its own 16) for pass 2
  __shared__ float lcache[CACHE ? SC_CACHE_CHUNKS * 16 * 64 : 1];

  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int n = lane % 32, h = lane / 32;
  const int bh = blockIdx.x / a.n_qgroups, qg = blockIdx.x % a.n_qgroups;
  const int ib = n / G, grp = n % G;
  const int qb = qg * QB + ib;  // query block of this lane
  const bool qok = qb < a.nQB;
  const size_t rep = (static_cast<size_t>(bh) * a.nQB + (qok ? qb : 0)) * G;
  // B operand, step s of 16 dimensions: lane half h supplies dimensions
  // 16 s + 8 h .. +7, each split into bf16 hi + lo parts
  const float* qm = a.q_rep + (rep + grp) * D + 8 * h;
  // STATS: steps D/16 .. 2D/16 - 1 carry (s/2) q^2 against the key-unit variances
  constexpr int NST = (STATS ? 2 : 1) * (D / 16);
  bf16x8 qhi[NST], qlo[NST];
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    const f32x4 x0 = qok ? *reinterpret_cast<const f32x4*>(qm + 16 * st) : f32x4{0.f, 0.f, 0.f, 0.f};
    const f32x4 x1 = qok ? *reinterpret_cast<const f32x4*>(qm + 16 * st + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
    split_bf16(x0, x1, qhi[st], qlo[st]);
    if constexpr (STATS) {
      const float hs = 0.5f * a.sm_scale;
      split_bf16(hs * x0 * x0, hs * x1 * x1, qhi[D / 16 + st], qlo[D / 16 + st]);
    }
  }
  // weight n_g / n of this lane's representative; a block with no valid row
  // scores with its first (zero) representative alone
  float wgt = 1.f;
  if (a.q_size != nullptr) {
    int tot = 0, mine = 0;
#pragma unroll
    for (int x = 0; x < G; ++x) {
      const int c = qok ? a.q_size[rep + x] : 0;
      tot += c;
      mine = x == grp ? c : mine;
    }
    wgt = tot > 0 ? static_cast<float>(mine) / static_cast<float>(tot) : (grp == 0 ? 1.f : 0.f);
  }
  const float* kmb = a.k_mean + static_cast<size_t>(bh) * a.nKU * D + 8 * h;
  const float* kvb = STATS ? a.k_var + static_cast<size_t>(bh) * a.nKU * D + 8 * h : kmb;
  const int n_chunks = (a.nKU + 31) / 32;
  const float c2 = a.sm_scale * 1.4426950408889634f;  // logits in log2 units

  // x for the 32 units of chunk ch: register r holds unit j0 + 8 (r/4) + 4 h + r%4;
  // -inf for units with no valid key. <k, q> = kh.qh + kh.ql + kl.qh on bf16
  // MFMAs (fp32 accumulation): each value is hi + lo to 2^-18 relative and the
  // dropped kl.ql term is below 2^-18 of the product.
  auto logits = [&](int ch) {
    const int j0 = ch * 32;
    const int ja = j0 + n;  // A-operand row (unit) of this lane
    const bool aok = ja < a.nKU;
    f32x16 acc0 = f32x16{}, acc1 = f32x16{};
    const size_t koff_ = static_cast<size_t>(aok ? ja : 0) * D;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      // steps past D/16 read the unit's variances (STATS)
      const float* km = (st < D / 16 ? kmb : kvb) + koff_ + 16 * (st % (D / 16));
      const f32x4 x0 = aok ? *reinterpret_cast<const f32x4*>(km) : f32x4{0.f, 0.f, 0.f, 0.f};
      const f32x4 x1 = aok ? *reinterpret_cast<const f32x4*>(km + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
      bf16x8 khi, klo;
      split_bf16(x0, x1, khi, klo);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(khi, qhi[st], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(khi, qlo[st], acc1, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(klo, qhi[st], acc0, 0, 0, 0);
    }
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = j0 + 8 * (r / 4) + 4 * h + (r % 4);
      const bool valid = j < a.nKU && j * a.block_k < a.N;
      acc[r] = valid ? (acc0[r] + acc1[r]) * c2 : -INFINITY;
    }
    return acc;
  };
  auto keys_of = [&](int j) { return static_cast<float>(max(0, min(a.block_k, a.N - j * a.block_k))); };

  // Rows too long for the LDS cache with one representative per query block
  // (SPILL): pass 1 parks each lane's logits in its own query block's row of
  // S, where pass 2 reads them back (the same lane, in program order) before
  // the normalised values overwrite them, instead of contracting every chunk
  // again.
  constexpr bool SPILL = !CACHE && G == 1;
  float* const lrow = a.S + (static_cast<size_t>(bh) * a.nQB + (qok ? qb : 0)) * a.nKU;
  // 16-byte aligned rows of S (S itself need only be 4-byte aligned): four units per access
  const bool vec4 = qok && a.nKU % 4 == 0 && reinterpret_cast<uintptr_t>(a.S) % 16 == 0;

  // ---- pass 1: running maximum and weighted sum per query block
  float run_m = -INFINITY, run_s = 0.f;
  for (int ch = wave; ch < n_chunks; ch += SC_WAVES) {
    const f32x16 acc = logits(ch);
    if constexpr (CACHE) {
#pragma unroll
      for (int r = 0; r < 16; ++r) lcache[(ch * 16 + r) * 64 + lane] = acc[r];
    } else if constexpr (SPILL) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {  // registers 4 g4 .. +3: units j .. j + 3
        const int j = ch * 32 + 8 * g4 + 4 * h;
        if (vec4 && j + 3 < a.nKU) {
          *reinterpret_cast<f32x4*>(lrow + j) = f32x4{acc[4 * g4], acc[4 * g4 + 1], acc[4 * g4 + 2], acc[4 * g4 + 3]};
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (qok && j + e < a.nKU) lrow[j + e] = acc[4 * g4 + e];
        }
      }
    }
    float lmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) lmax = fmaxf(lmax, acc[r]);
    const float nm = fmaxf(run_m, lmax);
    if (nm != -INFINITY) {
      float s = run_m == -INFINITY ? 0.f : run_s * exp2f(run_m - nm);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = ch * 32 + 8 * (r / 4) + 4 * h + (r % 4);
        if (acc[r] != -INFINITY) s += keys_of(j) * exp2f(acc[r] - nm);
      }
      run_s = s;
      run_m = nm;
    }
  }
  // combine the two lane halves, then the waves
  {
    const float om = __shfl_xor(run_m, 32), os = __shfl_xor(run_s, 32);
    const float nm = fmaxf(run_m, om);
    float s = 0.f;
    if (nm != -INFINITY) {
      if (run_m != -INFINITY) s += run_s * exp2f(run_m - nm);
      if (om != -INFINITY) s += os * exp2f(om - nm);
    }
    run_m = nm;
    run_s = s;
  }
  if (h == 0) {
    red_m[wave][n] = run_m;
    red_s[wave][n] = run_s;
  }
  __syncthreads();
  float Lm = -INFINITY;
#pragma unroll
  for (int x = 0; x < SC_WAVES; ++x) Lm = fmaxf(Lm, red_m[x][n]);
  float Z = 0.f;
#pragma unroll
  for (int x = 0; x < SC_WAVES; ++x)
    if (red_m[x][n] != -INFINITY) Z += red_s[x][n] * exp2f(red_m[x][n] - Lm);
  const float invZ = Z > 0.f ? 1.f / Z : 0.f;

  // ---- pass 2: normalised scores, written row-contiguously
  const float scale = invZ * wgt;
  float* sbase = a.S + (static_cast<size_t>(bh) * a.nQB + qg * QB) * a.nKU;
  for (int ch = wave; ch < n_chunks; ch += SC_WAVES) {
    f32x16 acc;
    if constexpr (CACHE) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = lcache[(ch * 16 + r) * 64 + lane];  // written by this lane
    } else if constexpr (SPILL) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {  // written by this lane in pass 1; rows past nQB are never stored
        const int j = ch * 32 + 8 * g4 + 4 * h;
        if (vec4 && j + 3 < a.nKU) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(lrow + j);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[4 * g4 + e] = x[e];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[4 * g4 + e] = (qok && j + e < a.nKU) ? lrow[j + e] : -INFINITY;
        }
      }
    } else {
      acc = logits(ch);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int jl = 8 * (r / 4) + 4 * h + (r % 4);
      const float x = acc[r];
      float v = x == -INFINITY ? 0.f : keys_of(ch * 32 + jl) * exp2f(x - Lm) * scale;
      v = group_sum<G>(v);  // the G lanes of one query block
      if (grp == 0) tile[wave][ib][jl] = v;
    }
    // the block is exchanged between the lanes of this wave only
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int col = ch * 32 + n;
#pragma unroll
    for (int k = 0; k < QB / 2; ++k) {
      const int row = 2 * k + h;  // query block qg * QB + row
      if (qg * QB + row < a.nQB && col < a.nKU) sbase[static_cast<size_t>(row) * a.nKU + col] = tile[wave][row][n];
    }
    // the next chunk's writes to the block wait for these reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// Word 3 of a gfx9 buffer resource for raw dword accesses (data format 32):
// with stride 0 a load at an offset past the record count returns zeros and a
// store there is dropped.
constexpr int BUFFER_WORD3 = 0x00020000;

constexpr int SS_CT = 4;  // column tiles per workgroup
constexpr int SS_US = 2;  // unit halves per workgroup
constexpr int SS_LT = 36; // row stride (floats) of a wave's transposition tile: 16-byte aligned rows

// bf16 hi + lo parts of two floats, packed: hi = bf16(x), lo = bf16(x - hi)
// (one conversion per pair and part)
__device__ __forceinline__ void split2_bf16(float a, float b, uint32_t& hi, uint32_t& lo) {
  const bf16x2 h = __builtin_convertvector(f32x2{a, b}, bf16x2);
  const f32x2 hf = __builtin_convertvector(h, f32x2);
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a - hf[0], b - hf[1]}, bf16x2));
}

// One step of a reduce-scatter over lane pairs (lane, partner given by the DPP
// control): of the K values, the lane keeps the upper half when `upper` (the
// partner the lower half) and adds the partner's copy of the half it keeps.
template <int CTRL, int K>
__device__ __forceinline__ void scatter_step(float (&v)[16], bool upper) {
#pragma unroll
  for (int i = 0; i < K / 2; ++i) {
    const float keep = upper ? v[K / 2 + i] : v[i];
    const float send = upper ? v[i] : v[K / 2 + i];
    v[i] = keep + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(send), CTRL, 0xF, 0xF, false));
  }
}

// Sums v (16 values, index 4 m + e) over the G consecutive lanes of a group,
// each lane keeping 16 / G of the sums in v[0 .. 16 / G - 1]:
//   G = 1: m = i / 4, e = i % 4 (nothing to sum);
//   G = 2: m = 2 grp + i / 4, e = i % 4;  G = 4: m = grp, e = i;
//   G = 8: m = grp / 2, e = 2 (grp % 2) + i.
// The partners are lane xor 1 and xor 2 (quad permutations) and, for G = 8,
// the mirror lane 7 - i of an 8-lane half-row (it lies in the other quad).
template <int G>
__device__ __forceinline__ void group_reduce_scatter(float (&v)[16], int grp) {
  if constexpr (G == 1) {
    (void)v;
    (void)grp;
  } else if constexpr (G == 2) {
    scatter_step<0xB1, 16>(v, grp & 1);
  } else if constexpr (G == 4) {
    scatter_step<0x4E, 16>(v, grp & 2);
    scatter_step<0xB1, 8>(v, grp & 1);
  } else {
    static_assert(G == 8, "group size");
    scatter_step<0x141, 16>(v, grp & 4);
    scatter_step<0x4E, 8>(v, grp & 2);
    scatter_step<0xB1, 4>(v, grp & 1);
  }
}

// Score matrix for G representatives per query block (G >= 2; G = 1 unless
// the grid would be small and the logits fit the LDS cache of scores_kernel).
// The eight waves
// form four column tiles x two unit halves: wave (ct, us) owns MFMA columns
// (representatives) 32 ct .. 32 ct + 31 of the workgroup's 128 and the unit
// chunks us, us + 2, ... The four waves of a unit half load each chunk of 32
// key means together, split it into bf16 hi + lo parts once and keep it in
// LDS for all four column tiles: one read of the key means per four column
// tiles, where a wave of scores_kernel reads and splits every chunk itself.
// Logits are recomputed in pass 2. The key counts n_j enter as a logit offset
// log2(n_j / block_k), which is 0 for every unit but a ragged last one.
template <int D, int G>
__global__ __launch_bounds__(64 * SC_WAVES) void scores_shared_kernel(ScoreArgs a) {
  constexpr int CT = SS_CT, US = SS_US;
  static_assert(CT * US == SC_WAVES && (G == 1 || G == 2 || G == 4 || G == 8), "wave split");
  constexpr int QBT = 32 / G;       // query blocks per column tile
  constexpr int QBW = CT * QBT;     // query blocks per workgroup
  constexpr int PER = 32 * D / 4 / (64 * CT);  // float4 loads per thread and chunk
  // [buffer][unit half][hi, lo][unit][d], bf16; rows padded by 16 bytes, so
  // that the 16 lanes of a fragment read (rows n, one 16-byte slot each) fall
  // in distinct banks
  constexpr int KR = D + 8;
  __shared__ __align__(16) uint16_t kbuf[2][US][2][32 * KR];
  __shared__ float red_m[SC_WAVES][32];
  __shared__ float red_s[SC_WAVES][32];
  __shared__ __align__(16) float tile[SC_WAVES][QBT][SS_LT];

  const int tid = threadIdx.x, lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);  // uniform: chunk indices and S rows are scalar
  const int n = lane % 32, h = lane / 32;
  const int ct = wave % CT, us = wave / CT;
  // each XCD takes a contiguous range of workgroups: the ones running on an
  // XCD at a time then sweep the key means of one or two heads, which stay in
  // that XCD's L2
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = wg / a.n_qgroups, qg = wg % a.n_qgroups;
  const int ibt = n / G, grp = n % G;          // query block (in the column tile) and group of this lane
  const int qb0 = qg * QBW + ct * QBT;         // first query block of the column tile
  const int qb = qb0 + ibt;
  const bool qok = qb < a.nQB;
  const size_t rep = (static_cast<size_t>(bh) * a.nQB + (qok ? qb : 0)) * G;
  const float* qm = a.q_rep + (rep + grp) * D + 8 * h;
  // the representatives carry the scale to log2 units (sm_scale log2 e), so
  // the products are the logits
  const float c2 = a.sm_scale * 1.4426950408889634f;
  bf16x8 qhi[D / 16], qlo[D / 16];
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    const f32x4 x0 = qok ? *reinterpret_cast<const f32x4*>(qm + 16 * st) : f32x4{0.f, 0.f, 0.f, 0.f};
    const f32x4 x1 = qok ? *reinterpret_cast<const f32x4*>(qm + 16 * st + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
    split_bf16(x0 * c2, x1 * c2, qhi[st], qlo[st]);
  }
  // weight n_g / n of this lane's representative; a block with no valid row
  // scores with its first (zero) representative alone
  float wgt = 1.f;
  if (a.q_size != nullptr) {
    int tot = 0, mine = 0;
#pragma unroll
    for (int x = 0; x < G; ++x) {
      const int c = qok ? a.q_size[rep + x] : 0;
      tot += c;
      mine = x == grp ? c : mine;
    }
    wgt = tot > 0 ? static_cast<float>(mine) / static_cast<float>(tot) : (grp == 0 ? 1.f : 0.f);
  }
  // key means of this head through a buffer resource: a load past the last
  // unit (the ragged chunk, or the chunk after the last) reads zeros
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a.k_mean + static_cast<size_t>(bh) * a.nKU * D), 0, a.nKU * D * 4, BUFFER_WORD3);
  const int n_chunks = (a.nKU + 31) / 32;
  const int n_iter = (n_chunks + US - 1) / US;  // the same count for every wave: the barriers match
  // units 0 .. nV - 1 hold keys, all block_k of them but the last
  const int nV = min(a.nKU, (a.N + a.block_k - 1) / a.block_k);
  const int ch_edge = nV > 0 ? (nV - 1) / 32 : 0;  // chunks from here on hold the last valid unit or none
  const float tail = nV > 0 ? log2f(static_cast<float>(a.N - (nV - 1) * a.block_k) / static_cast<float>(a.block_k)) : 0.f;

  // staging: thread t = 64 ct + lane of unit half us takes float4 number
  // t + 64 CT p (p < PER) of the chunk's 32 x D key-mean floats
  const int gt = 64 * ct + lane;
  f32x4 xk[PER];
  auto load_chunk = [&](int ch) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const uint32_t off = static_cast<uint32_t>(ch * 32 * D + 4 * (gt + 64 * CT * p)) * 4u;
      xk[p] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0));
    }
  };
  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int idx = gt + 64 * CT * p, unit = idx / (D / 4), d4 = idx % (D / 4);
      uint32_t hi[2], lo[2];
      split2_bf16(xk[p][0], xk[p][1], hi[0], lo[0]);
      split2_bf16(xk[p][2], xk[p][3], hi[1], lo[1]);
      *reinterpret_cast<u32x2*>(&kbuf[buf][us][0][unit * KR + 4 * d4]) = u32x2{hi[0], hi[1]};
      *reinterpret_cast<u32x2*>(&kbuf[buf][us][1][unit * KR + 4 * d4]) = u32x2{lo[0], lo[1]};
    }
  };
  // products of the chunk in buffer buf with this wave's representatives
  // (kh.qh + kh.ql + kl.qh, one fp32 accumulator): the logits in log2 units.
  // The A operand is row n of the staged chunk, all 16 fragments read before
  // the first product.
  auto products = [&](int buf, f32x16& p0) {
    const uint16_t* kh = &kbuf[buf][us][0][n * KR + 8 * h];
    const uint16_t* kl = &kbuf[buf][us][1][n * KR + 8 * h];
    bf16x8 khi[D / 16], klo[D / 16];
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      khi[st] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kh + 16 * st));
      klo[st] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kl + 16 * st));
    }
    p0 = f32x16{};
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      p0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(khi[st], qhi[st], p0, 0, 0, 0);
      p0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(khi[st], qlo[st], p0, 0, 0, 0);
      p0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(klo[st], qhi[st], p0, 0, 0, 0);
    }
  };
  // x for the 32 units of chunk ch (register r: unit ch 32 + 8 (r/4) + 4 h + r%4)
  // in log2 units, with the key-count offset; -inf for units with no valid key
  auto logits = [&](int ch, const f32x16& p0) {
    f32x16 acc = p0;
    if (ch >= ch_edge) {  // uniform: the chunk of the last valid unit and any after it
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = ch * 32 + 8 * (r / 4) + 4 * h + (r % 4);
        acc[r] = j < nV - 1 ? acc[r] : (j == nV - 1 ? acc[r] + tail : -INFINITY);
      }
    }
    return acc;
  };

  // One pass over this unit half's chunks, software-pipelined. Chunk i sits
  // in buffer i & 1. After the barrier that ends iteration it - 1, iteration
  // it issues the products of chunk it + 1 between the exponentials of chunk
  // it (valu) and the staging of chunk it + 2 (loaded during iteration it - 1)
  // into the buffer chunk it left, starts the load of chunk it + 3, then
  // stores chunk it's results (store). A buffer is rewritten only behind the
  // barrier that follows the products reading it. A chunk past the last (the
  // second unit half's final chunk when the chunk count is odd, and the loads
  // and products ahead of every half's last chunk) reads zeros; its units
  // all get -inf logits, so valu adds nothing and store stores nothing for it.
  // Loads and stores are unconditional, so that the wait for a chunk's loads
  // leaves the stores of S issued after them in flight; prime issues as many
  // (dropped) stores on the way in.
  auto sweep = [&](auto&& valu, auto&& store, auto&& prime) {
    f32x16 p0;
    load_chunk(us);
    store_chunk(0);
    load_chunk(us + US);
    store_chunk(1);
    load_chunk(us + 2 * US);
    prime();
    __syncthreads();
    products(0, p0);
    f32x16 cur = logits(us, p0);
    __syncthreads();  // buffer 0 is rewritten in the first iteration
    for (int it = 0; it < n_iter; ++it) {
      const int ch = us + it * US;
      // keeps the work of chunk it below the barrier, next to the products
      // it is interleaved with (pure arithmetic may otherwise move up into
      // the previous iteration)
      asm volatile("" : "+v"(cur));
      products((it + 1) & 1, p0);
      const auto r = valu(ch, cur);
      store_chunk(it & 1);
      load_chunk(ch + 3 * US);
      // the 16 fragment reads, then each product followed by other work
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * (D / 16), 0);
#pragma unroll
      for (int x = 0; x < 3 * (D / 16); ++x) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
      }
      store(ch, r);
      cur = logits(ch + US, p0);
      __syncthreads();
    }
  };

  // ---- pass 1: running maximum and sum per representative
  float run_m = -INFINITY, run_s = 0.f;
  sweep(
      [&](int, const f32x16& acc) {
        float lmax = acc[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) lmax = fmaxf(lmax, acc[r]);
        // no branch: a chunk with no valid unit (lmax = -inf) leaves the state
        // as it is, and exp2(-inf) = 0 drops invalid units and an empty state
        const float nm = fmaxf(run_m, lmax);
        const float ns = nm == -INFINITY ? 0.f : nm;
        float sv = run_s * __builtin_amdgcn_exp2f(run_m - ns);
#pragma unroll
        for (int r = 0; r < 16; ++r) sv += __builtin_amdgcn_exp2f(acc[r] - ns);
        run_s = sv;
        run_m = nm;
        return sv;
      },
      // nothing to store; consuming the sum here keeps its exponent work
      // next to the products instead of sinking below the next chunk's mask
      [](int, float sv) { asm volatile("" ::"v"(sv)); }, [] {});
  {  // the two lane halves, then the unit halves of the column tile
    const float om = __shfl_xor(run_m, 32), os = __shfl_xor(run_s, 32);
    const float nm = fmaxf(run_m, om);
    float sv = 0.f;
    if (nm != -INFINITY) sv = run_s * __builtin_amdgcn_exp2f(run_m - nm) + os * __builtin_amdgcn_exp2f(om - nm);
    run_m = nm;
    run_s = sv;
  }
  if (h == 0) {
    red_m[wave][n] = run_m;
    red_s[wave][n] = run_s;
  }
  __syncthreads();
  float Lm = -INFINITY;
#pragma unroll
  for (int x = 0; x < US; ++x) Lm = fmaxf(Lm, red_m[x * CT + ct][n]);
  float Z = 0.f;
  if (Lm != -INFINITY) {
#pragma unroll
    for (int x = 0; x < US; ++x) Z += red_s[x * CT + ct][n] * __builtin_amdgcn_exp2f(red_m[x * CT + ct][n] - Lm);
  }
  const float invZ = Z > 0.f ? 1.f / Z : 0.f;

  // ---- pass 2: normalised scores, written row-contiguously
  const float scale = invZ * wgt;
  const float Lm0 = Lm == -INFINITY ? 0.f : Lm;  // no valid unit at all: every value is 0
  // the column tile's rows of S through a buffer resource that ends at its
  // last valid query block; stores past it, or flagged with an offset beyond
  // any record, are dropped
  const int rows_valid = max(0, min(QBT, a.nQB - qb0));
  const uint64_t sb = reinterpret_cast<uint64_t>(a.S + (static_cast<size_t>(bh) * a.nQB + min(qb0, a.nQB)) * a.nKU);
  // uniform: a scalar resource. readfirstlane returns int: each half goes
  // through uint32_t, so that the low half is not sign-extended into the high
  const uint64_t sb_u =
      (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(sb >> 32)))) << 32) |
      static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(sb & 0xffffffffu))));
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<float*>(sb_u), 0, __builtin_amdgcn_readfirstlane(rows_valid * a.nKU * 4), BUFFER_WORD3);
  float* trow = &tile[wave][ibt][0];
  struct Sums {
    float v[16];
  };
  sweep(
      [&](int, const f32x16& acc) {
        Sums o;
#pragma unroll
        for (int r = 0; r < 16; ++r) o.v[r] = __builtin_amdgcn_exp2f(acc[r] - Lm0) * scale;  // exp2(-inf) = 0
        group_reduce_scatter<G>(o.v, grp);  // sums over the G representatives of the query block
        return o;
      },
      [&](int ch, const Sums& o) {
        // the lane's sums are consecutive units of its query block's row
        if constexpr (G == 1) {
#pragma unroll
          for (int m = 0; m < 4; ++m)
            *reinterpret_cast<f32x4*>(trow + 8 * m + 4 * h) = f32x4{o.v[4 * m], o.v[4 * m + 1], o.v[4 * m + 2], o.v[4 * m + 3]};
        } else if constexpr (G == 2) {
          *reinterpret_cast<f32x4*>(trow + 16 * grp + 4 * h) = f32x4{o.v[0], o.v[1], o.v[2], o.v[3]};
          *reinterpret_cast<f32x4*>(trow + 16 * grp + 8 + 4 * h) = f32x4{o.v[4], o.v[5], o.v[6], o.v[7]};
        } else if constexpr (G == 4) {
          *reinterpret_cast<f32x4*>(trow + 8 * grp + 4 * h) = f32x4{o.v[0], o.v[1], o.v[2], o.v[3]};
        } else {
          *reinterpret_cast<f32x2*>(trow + 8 * (grp / 2) + 4 * h + 2 * (grp % 2)) = f32x2{o.v[0], o.v[1]};
        }
        // the block is exchanged between the lanes of this wave only
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int col = ch * 32 + n;
#pragma unroll
        for (int k = 0; k < QBT / 2; ++k) {
          const int row = 2 * k + h;  // query block qb0 + row
          const uint32_t off = col < a.nKU ? static_cast<uint32_t>(row * a.nKU + col) * 4u : 0x80000000u;
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(tile[wave][row][n]), srs, off, 0, 0);
        }
        // the next chunk's writes to the block wait for these reads
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      },
      [&] {
        // as many stores as a chunk issues, all dropped (offset beyond any record)
#pragma unroll
        for (int k = 0; k < QBT / 2; ++k) __builtin_amdgcn_raw_buffer_store_b32(0u, srs, 0x80000000u + 4u * k, 0, 0);
      });
}

}  // namespace

hipError_t launch_block_means(const Geometry& g, const void* q, const void* k, const int32_t* perm,
                              float* q_mean, float* k_mean, float* k_var, bool keys_only, hipStream_t s) {
  MeansArgs a;
  a.q = q;
  a.k = k;
  a.perm = perm;
  a.q_mean = q_mean;
  a.k_mean = k_mean;
  a.k_var = k_var;
  a.N = g.N;
  a.N_pad = g.N_pad;
  a.block_q = g.block_q;
  a.block_k = g.block_k;
  a.nQB = g.nQB;
  a.nKU = g.nKU;
  a.n_bh = g.B * g.H;
  a.first = keys_only ? a.n_bh * g.nQB : 0;
  const dim3 grid(a.n_bh * ((keys_only ? 0 : g.nQB) + g.nKU));
  const bool p = perm != nullptr;
  a.k_gather = p && !g.kv_permuted;
#define BSA_MEANS(D, BF, P) hipLaunchKernelGGL((block_means_kernel<D, BF, P>), grid, dim3(MEAN_THREADS), 0, s, a)
  if (g.d == 128) {
    if (g.bf16) { if (p) BSA_MEANS(128, true, true); else BSA_MEANS(128, true, false); }
    else { if (p) BSA_MEANS(128, false, true); else BSA_MEANS(128, false, false); }
  } else {
    if (g.bf16) { if (p) BSA_MEANS(64, true, true); else BSA_MEANS(64, true, false); }
    else { if (p) BSA_MEANS(64, false, true); else BSA_MEANS(64, false, false); }
  }
#undef BSA_MEANS
  return hipGetLastError();
}

hipError_t launch_scores(const Geometry& g, int groups, const float* q_rep, const int32_t* q_size,
                         const float* k_mean, const float* k_var, float* S, hipStream_t s) {
  ScoreArgs a;
  a.q_rep = q_rep;
  a.q_size = q_size;
  a.k_mean = k_mean;
  a.k_var = k_var;
  a.S = S;
  a.N = g.N;
  a.block_k = g.block_k;
  a.nQB = g.nQB;
  a.nKU = g.nKU;
  const int per_wg = 32 / groups;
  a.n_qgroups = (g.nQB + per_wg - 1) / per_wg;
  a.sm_scale = g.sm_scale;
  const dim3 grid(g.B * g.H * a.n_qgroups), block(64 * SC_WAVES);
  const bool cache = (g.nKU + 31) / 32 <= SC_CACHE_CHUNKS;
  if (k_var != nullptr) {  // statistics-aware scoring: one representative per query block
    if (groups != 1) return hipErrorInvalidValue;
    if (g.d == 128) {
      if (cache) hipLaunchKernelGGL((scores_kernel<128, 1, true, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((scores_kernel<128, 1, false, true>), grid, block, 0, s, a);
    } else {
      if (cache) hipLaunchKernelGGL((scores_kernel<64, 1, true, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((scores_kernel<64, 1, false, true>), grid, block, 0, s, a);
    }
    return hipGetLastError();
  }
  // the kernel that shares each staged chunk of key means between four
  // column tiles: two or more representatives per query block; one when the
  // logits do not fit the LDS cache, or when its grid still has 64 or more
  // workgroups (below that, scores_kernel's four times larger grid is faster)
  const int per_wg_shared = SS_CT * 32 / groups;
  const dim3 grid_shared(g.B * g.H * ((g.nQB + per_wg_shared - 1) / per_wg_shared));
  ScoreArgs as = a;
  as.n_qgroups = (g.nQB + per_wg_shared - 1) / per_wg_shared;
  const bool shared_one = !cache || grid_shared.x >= 64;
#define BSA_SCORES(D, G)                                                                                \
  if (G > 1 || shared_one) hipLaunchKernelGGL((scores_shared_kernel<D, G>), grid_shared, block, 0, s, as); \
  else if (cache) hipLaunchKernelGGL((scores_kernel<D, G, true, false>), grid, block, 0, s, a);         \
  else hipLaunchKernelGGL((scores_kernel<D, G, false, false>), grid, block, 0, s, a)
#define BSA_SCORES_G(D)                      \
  switch (groups) {                          \
    case 1: BSA_SCORES(D, 1); break;         \
    case 2: BSA_SCORES(D, 2); break;         \
    case 4: BSA_SCORES(D, 4); break;         \
    case 8: BSA_SCORES(D, 8); break;         \
    default: return hipErrorInvalidValue;    \
  }
  if (g.d == 128) {
    BSA_SCORES_G(128)
  } else {
    BSA_SCORES_G(64)
  }
#undef BSA_SCORES_G
#undef BSA_SCORES
  return hipGetLastError();
}

}  // namespace bsa
