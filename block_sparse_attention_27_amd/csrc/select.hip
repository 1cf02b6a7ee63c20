// Block selection for gfx950: exact top-k set plus a fixed-size systematic
// sample weighted by inverse inclusion probability, one workgroup per
// (b, h, query block).
//
// What is computed (InstaGen, Abstract: exact set computed in full, the rest
// represented by a sample drawn in proportion to estimated attention and
// reweighted by inverse sampling probability, one sample per query cluster;
// AB-Attention transcript: inclusion probabilities with certain inclusion for
// the strongest blocks, a fixed number of distinct blocks, probability 1/4 ->
// weight 4):
//   1. exact set K = the k valid units with the largest score (ties: lower
//      index; NaN/zero/negative scores count as 0, +inf as FLT_MAX);
//   2. on the rest R, integer scores q_j = max(1, floor(s_j 2^(20 - e))) with
//      e the binary exponent of max_R s; exact water-filling of
//      pi_j = min(1, c q_j), sum_R pi_j = m; pi in 32-bit fixed point with
//      floor(2^32 fl64((m-t) q_j) / fl64(Q_U)) and the integer shortfall paid
//      as +1 to the first uncapped units, so sum_R pi_int = m 2^32 exactly;
//   3. systematic sampling over R in index order from the offset
//      u = Philox4x32-10((i, h, b, 0), seed) word 0;
//   4. emit K ascending with w = 1, then sample slot s -> its unit with
//      w = fp32(2^32 / pi_int).
// Every sum is an integer sum, so the result is independent of reduction
// order and bit-identical to the CPU definition. The only floating-point
// operations are two correctly rounded fp64 divisions and one fp64 -> fp32
// rounding.
//
// Layout: thread t owns the E consecutive units [t E, t E + E), so exclusive
// scans give ranks in unit order directly. Rows of up to 1024 valid units take
// one wave each (ballot counts, DPP sums and scans, no barriers); longer rows take a
// 256-thread workgroup.
#include "bsa_internal.hpp"

namespace bsa {
namespace {

constexpr int SEL_THREADS = 256;
constexpr int SEL_WAVES = SEL_THREADS / 64;
constexpr int FS = 20;  // score quantisation bits

struct SelectArgs {
  const float* S;
  int32_t* idx;
  float* w;
  int H, nQB, nKU, nV, k, m;
  uint32_t seed_lo, seed_hi;
};

// Philox4x32-10 (Salmon et al., SC'11): word 0 of the output block.
__device__ __forceinline__ uint32_t philox_word0(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                 uint32_t k0, uint32_t k1) {
  constexpr uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  constexpr uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += W0;
      k1 += W1;
    }
    const uint32_t lo0 = M0 * c0, hi0 = __umulhi(M0, c0);
    const uint32_t lo1 = M1 * c2, hi1 = __umulhi(M1, c2);
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return c0;
}

// NaN, zero and negatives -> 0; +inf -> FLT_MAX; other values keep their bits
// (monotone in the value for non-negative floats).
__device__ __forceinline__ uint32_t sanitize(uint32_t b) {
  if (b >> 31) return 0u;
  if ((b & 0x7F800000u) == 0x7F800000u) return (b & 0x007FFFFFu) ? 0u : 0x7F7FFFFFu;
  return b;
}

// e such that the value of bits x (> 0, finite) is f 2^e with f in [0.5, 1).
__device__ __forceinline__ int frexp_exp(uint32_t x) {
  const int E = static_cast<int>(x >> 23);
  if (E > 0) return E - 126;
  const uint32_t mant = x & 0x007FFFFFu;
  return (32 - __clz(mant)) - 149;
}

// floor(value(x) 2^(FS - e)), at least 1; exact integer arithmetic.
__device__ __forceinline__ uint32_t quantise(uint32_t x, int e) {
  if (x == 0u) return 1u;
  const int E = static_cast<int>(x >> 23);
  const uint64_t sig = E ? ((x & 0x007FFFFFu) | 0x00800000u) : (x & 0x007FFFFFu);
  const int shift = (E ? E : 1) - 150 + FS - e;
  uint64_t q;
  if (shift >= 0) q = sig << shift;
  else if (shift > -64) q = sig >> (-shift);
  else q = 0;
  return q > 0 ? static_cast<uint32_t>(q) : 1u;
}

// Cross-lane steps on DPP moves, which stay in the VALU (a lane shuffle is an
// LDS round trip). Rows of the wave are its four 16-lane groups. A lane whose
// DPP source is outside its row, or whose row is masked off, receives 0.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, ROWS, 0xF, false));
}
template <int CTRL, int ROWS = 0xF, typename T>
__device__ __forceinline__ T dpp(T v) {
  if constexpr (sizeof(T) == 8) {
    return (static_cast<uint64_t>(dpp32<CTRL, ROWS>(static_cast<uint32_t>(v >> 32))) << 32) |
           dpp32<CTRL, ROWS>(static_cast<uint32_t>(v));
  } else {
    return static_cast<T>(dpp32<CTRL, ROWS>(static_cast<uint32_t>(v)));
  }
}
template <typename T>
__device__ __forceinline__ T lane_value(T v, int l) {
  if constexpr (sizeof(T) == 8) {
    return (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v >> 32), l))) << 32) |
           static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v)), l));
  } else {
    return static_cast<T>(__builtin_amdgcn_readlane(static_cast<int>(v), l));
  }
}
// Sum over the wave, in every lane: quad swaps, the half-row and row mirrors
// (every lane then holds its row's sum), then the four rows in scalars.
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
  v += dpp<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x140>(v);  // row_mirror
  return lane_value(v, 0) + lane_value(v, 16) + lane_value(v, 32) + lane_value(v, 48);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp<0xB1>(v));
  v = max(v, dpp<0x4E>(v));
  v = max(v, dpp<0x141>(v));
  v = max(v, dpp<0x140>(v));
  return max(max(lane_value(v, 0), lane_value(v, 16)), max(lane_value(v, 32), lane_value(v, 48)));
}
// Inclusive prefix sum over lanes: shifts by 1, 2, 4, 8 within each row, then
// the last lane of row 0 (2) is added to row 1 (3), and lane 31 to rows 2, 3.
__device__ __forceinline__ uint64_t wave_inclusive_scan(uint64_t x) {
  x += dpp<0x111>(x);       // row_shr:1
  x += dpp<0x112>(x);       // row_shr:2
  x += dpp<0x114>(x);       // row_shr:4
  x += dpp<0x118>(x);       // row_shr:8
  x += dpp<0x142, 0xA>(x);  // row_bcast:15 into rows 1 and 3
  x += dpp<0x143, 0xC>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}

template <typename T>
__device__ __forceinline__ T block_sum(T v, T* red) {
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  v = wave_sum(v);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  T t = 0;
#pragma unroll
  for (int x = 0; x < SEL_WAVES; ++x) t += red[x];
  __syncthreads();
  return t;
}

__device__ __forceinline__ uint32_t block_max(uint32_t v, uint32_t* red) {
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  v = wave_max_u32(v);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (int x = 0; x < SEL_WAVES; ++x) t = max(t, red[x]);
  __syncthreads();
  return t;
}

// Exclusive prefix over threads in index order; `total` receives the block sum.
__device__ __forceinline__ uint64_t block_exscan(uint64_t v, uint64_t* red, uint64_t& total) {
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const uint64_t x = wave_inclusive_scan(v);
  if (lane == 63) red[wave] = x;
  __syncthreads();
  uint64_t before = 0, tot = 0;
#pragma unroll
  for (int z = 0; z < SEL_WAVES; ++z) {
    const uint64_t r = red[z];
    if (z < wave) before += r;
    tot += r;
  }
  __syncthreads();
  total = tot;
  return before + x - v;
}

template <int E>
__global__ __launch_bounds__(SEL_THREADS) void select_kernel(SelectArgs a) {
  __shared__ uint32_t sbits[SEL_THREADS * E];
  __shared__ uint64_t red64[SEL_WAVES];
  __shared__ uint32_t red32[SEL_WAVES];
  __shared__ uint32_t cnt2[2][SEL_WAVES];  // per-wave counts, alternating buffers

  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  const int i = row % a.nQB, bh = row / a.nQB;
  const int hd = bh % a.H, b = bh / a.H;
  const float* srow = a.S + static_cast<size_t>(row) * a.nKU;
  const int L = a.k + a.m;
  int32_t* irow = a.idx + static_cast<size_t>(row) * L;
  float* wrow = a.w + static_cast<size_t>(row) * L;

  {  // every load of the row in flight at once (coalesced), then through LDS to the unit owners
    uint32_t v[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int x = tid + e * SEL_THREADS;
      v[e] = x < a.nV ? __float_as_uint(srow[x]) : 0u;
    }
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (tid + e * SEL_THREADS < a.nV) sbits[tid + e * SEL_THREADS] = v[e];
  }
  __syncthreads();

  uint32_t key[E];
  bool valid[E], inK[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = tid * E + e;
    valid[e] = j < a.nV;
    key[e] = valid[e] ? sanitize(sbits[j]) : 0u;
    inK[e] = false;
  }

  // ---- 1. exact set: T = k-th largest key, ties by lower index ----
  if (a.k > 0) {
    // counts from ballots (cand >= 1 and invalid units hold key 0); one
    // barrier per bit: a buffer is rewritten two bits later, after every
    // thread has passed the barrier that follows its reads
    const int wave = tid / 64;
    uint32_t T = 0;
    for (int bit = 30; bit >= 0; --bit) {
      const uint32_t cand = T | (1u << bit);
      uint32_t c = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) c += __popcll(__ballot(key[e] >= cand));
      if (tid % 64 == 0) cnt2[bit & 1][wave] = c;
      __syncthreads();
      uint32_t tot = 0;
#pragma unroll
      for (int x = 0; x < SEL_WAVES; ++x) tot += cnt2[bit & 1][x];
      if (tot >= static_cast<uint32_t>(a.k)) T = cand;
    }
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      gt += (valid[e] && key[e] > T) ? 1u : 0u;
      eq += (valid[e] && key[e] == T) ? 1u : 0u;
    }
    const uint32_t need = static_cast<uint32_t>(a.k) - block_sum(gt, red32);
    uint64_t eq_total;
    uint32_t r = static_cast<uint32_t>(block_exscan(eq, red64, eq_total));
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (!valid[e]) continue;
      if (key[e] > T) {
        inK[e] = true;
      } else if (key[e] == T) {
        inK[e] = r < need;
        ++r;
      }
    }
  }

  bool inR[E], capped[E];
  uint64_t pi[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    inR[e] = valid[e] && !inK[e];
    capped[e] = false;
    pi[e] = 0;
  }

  uint64_t delta = 0;
  if (a.m > 0) {
    // ---- 2a. quantised scores over R ----
    uint32_t mx = 0;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (inR[e]) mx = max(mx, key[e]);
    mx = block_max(mx, red32);
    uint32_t q[E];
    const int ex = mx ? frexp_exp(mx) : 0;
    uint64_t qsum = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      q[e] = inR[e] ? (mx ? quantise(key[e], ex) : 1u) : 0u;
      qsum += q[e];
    }
    uint64_t QU = block_sum(qsum, red64);

    // ---- 2b. water-filling on exact integers ----
    uint64_t t = 0;
    while (true) {
      const uint64_t mt = static_cast<uint64_t>(a.m) - t;
      uint64_t packed = 0;  // (count << 40) | sum of q
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (inR[e] && !capped[e] && mt * q[e] >= QU) {
          capped[e] = true;
          packed += (1ull << 40) + q[e];
        }
      }
      packed = block_sum(packed, red64);
      const uint64_t cnt = packed >> 40;
      if (cnt == 0) break;
      t += cnt;
      QU -= packed & ((1ull << 40) - 1);
    }

    // ---- 2c. fixed-point pi ----
    // (m - t) q_j < 2^33 and Q_U < 2^33 are exact in fp64, and so is their
    // product form below; an uncapped unit has (m - t) q_j < Q_U, so its
    // correctly rounded ratio is below 1 and 2^32 ratio fits 32 bits.
    const uint64_t mt = static_cast<uint64_t>(a.m) - t;
    const double mt_d = static_cast<double>(static_cast<uint32_t>(mt));
    const double qu_d = static_cast<double>(QU);
    uint64_t usum = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (!inR[e]) continue;
      if (capped[e]) {
        pi[e] = 1ull << 32;
      } else {
        const double ratio = (mt_d * static_cast<double>(q[e])) / qu_d;
        pi[e] = static_cast<uint32_t>(ratio * 4294967296.0);
        usum += pi[e];
      }
    }
    delta = (mt << 32) - block_sum(usum, red64);
  }

  // ---- ranks in unit order: K (high word) and uncapped R (low word) ----
  uint32_t nk = 0, nu = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    nk += inK[e] ? 1u : 0u;
    nu += (inR[e] && !capped[e]) ? 1u : 0u;
  }
  uint64_t rk_total;
  const uint64_t rk = block_exscan((static_cast<uint64_t>(nk) << 32) | nu, red64, rk_total);
  uint32_t kpos = static_cast<uint32_t>(rk >> 32);
  uint32_t upos = static_cast<uint32_t>(rk);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = tid * E + e;
    if (inK[e]) {
      irow[kpos] = j;
      wrow[kpos] = 1.0f;
      ++kpos;
    }
    if (a.m > 0 && inR[e] && !capped[e]) {
      if (upos < delta) pi[e] += 1;
      ++upos;
    }
  }

  if (a.m > 0) {
    // ---- 3. systematic sample over the cumulative pi axis ----
    uint64_t psum = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) psum += pi[e];
    uint64_t ptotal;
    uint64_t c = block_exscan(psum, red64, ptotal);
    const uint64_t u = philox_word0(static_cast<uint32_t>(i), static_cast<uint32_t>(hd),
                                    static_cast<uint32_t>(b), 0u, a.seed_lo, a.seed_hi);
    auto below = [u](uint64_t x) -> uint64_t { return x > u ? ((x - u - 1) >> 32) + 1 : 0; };
    // every key is in registers and the exscan's barriers have passed: the
    // staging array hands pi - 1 of each sampled slot (1 <= pi <= 2^32) to the
    // thread that writes its weight (k + m <= nV slots)
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (!inR[e]) continue;
      const uint64_t c0 = c;
      c += pi[e];
      const uint64_t n0 = below(c0), n1 = below(c);
      if (n1 > n0 && n0 < static_cast<uint64_t>(a.m)) {  // n0 < m always holds when sum pi = m 2^32
        irow[a.k + static_cast<int>(n0)] = tid * E + e;
        sbits[n0] = static_cast<uint32_t>(pi[e] - 1);
      }
    }
    __syncthreads();
    for (int x = tid; x < a.m; x += SEL_THREADS)
      wrow[a.k + x] = static_cast<float>(4294967296.0 / (static_cast<double>(sbits[x]) + 1.0));
  }
}

// ---- one wave per row (up to 64 E valid units) --------------------------
// The same computation with every reduction inside one wave: counts from
// ballots, sums and scans from DPP moves, no workgroup barriers. Lane t
// owns units [t E, t E + E).
constexpr int SELW_WAVES = 4;

// Exclusive prefix over lanes; `total` receives the wave sum.
__device__ __forceinline__ uint64_t wave_exscan(uint64_t v, uint64_t& total) {
  const uint64_t x = wave_inclusive_scan(v);
  total = lane_value(x, 63);
  return x - v;
}

template <int E>
__global__ __launch_bounds__(64 * SELW_WAVES) void select_wave_kernel(SelectArgs a, int rows) {
  __shared__ uint32_t sbits[SELW_WAVES][64 * E];
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int row = blockIdx.x * SELW_WAVES + wave;
  if (row >= rows) return;  // whole wave; nothing below synchronises across waves
  const int i = row % a.nQB, bh = row / a.nQB;
  const int hd = bh % a.H, b = bh / a.H;
  const float* srow = a.S + static_cast<size_t>(row) * a.nKU;
  const int L = a.k + a.m;
  int32_t* irow = a.idx + static_cast<size_t>(row) * L;
  float* wrow = a.w + static_cast<size_t>(row) * L;

  uint32_t* sb = sbits[wave];
  {  // every load of the row in flight at once (coalesced), then through LDS to the unit owners
    uint32_t v[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int x = lane + 64 * e;
      v[e] = x < a.nV ? __float_as_uint(srow[x]) : 0u;
    }
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (lane + 64 * e < a.nV) sb[lane + 64 * e] = v[e];
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  uint32_t key[E];
  bool valid[E], inK[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = lane * E + e;
    const uint32_t raw = sb[j];  // inside the wave's slice; ignored past nV
    valid[e] = j < a.nV;
    key[e] = valid[e] ? sanitize(raw) : 0u;
    inK[e] = false;
  }

  // ---- 1. exact set ----
  if (a.k > 0) {
    uint32_t T = 0;
    for (int bit = 30; bit >= 0; --bit) {
      const uint32_t cand = T | (1u << bit);
      uint32_t c = 0;  // cand >= 1, and invalid units hold key 0
#pragma unroll
      for (int e = 0; e < E; ++e) c += __popcll(__ballot(key[e] >= cand));
      if (c >= static_cast<uint32_t>(a.k)) T = cand;
    }
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      gt += __popcll(__ballot(valid[e] && key[e] > T));
      eq += (valid[e] && key[e] == T) ? 1u : 0u;
    }
    const uint32_t need = static_cast<uint32_t>(a.k) - gt;
    uint64_t eq_total;
    uint32_t r = static_cast<uint32_t>(wave_exscan(eq, eq_total));
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (!valid[e]) continue;
      if (key[e] > T) {
        inK[e] = true;
      } else if (key[e] == T) {
        inK[e] = r < need;
        ++r;
      }
    }
  }

  bool inR[E], capped[E];
  uint64_t pi[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    inR[e] = valid[e] && !inK[e];
    capped[e] = false;
    pi[e] = 0;
  }

  uint64_t delta = 0;
  if (a.m > 0) {
    // ---- 2a. quantised scores over R ----
    uint32_t mx = 0;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (inR[e]) mx = max(mx, key[e]);
    mx = wave_max_u32(mx);
    uint32_t q[E];
    const int ex = mx ? frexp_exp(mx) : 0;
    uint64_t qsum = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      q[e] = inR[e] ? (mx ? quantise(key[e], ex) : 1u) : 0u;
      qsum += q[e];
    }
    uint64_t QU = wave_sum(qsum);

    // ---- 2b. water-filling on exact integers ----
    uint64_t t = 0;
    while (true) {
      const uint64_t mt = static_cast<uint64_t>(a.m) - t;
      uint64_t qcap = 0;
      uint32_t cnt = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const bool cap = inR[e] && !capped[e] && mt * q[e] >= QU;
        cnt += __popcll(__ballot(cap));
        if (cap) {
          capped[e] = true;
          qcap += q[e];
        }
      }
      if (cnt == 0) break;
      t += cnt;
      QU -= wave_sum(qcap);
    }

    // ---- 2c. fixed-point pi ----
    // (m - t) q_j < 2^33 and Q_U < 2^31 are exact in fp64, and so is their
    // product form below; an uncapped unit has (m - t) q_j < Q_U, so its
    // correctly rounded ratio is below 1 and 2^32 ratio fits 32 bits.
    const uint64_t mt = static_cast<uint64_t>(a.m) - t;
    const double mt_d = static_cast<double>(static_cast<uint32_t>(mt));
    const double qu_d = static_cast<double>(QU);
    uint64_t usum = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (!inR[e]) continue;
      if (capped[e]) {
        pi[e] = 1ull << 32;
      } else {
        const double ratio = (mt_d * static_cast<double>(q[e])) / qu_d;
        pi[e] = static_cast<uint32_t>(ratio * 4294967296.0);
        usum += pi[e];
      }
    }
    delta = (mt << 32) - wave_sum(usum);
  }

  // ---- ranks in unit order: K (high word) and uncapped R (low word) ----
  uint32_t nk = 0, nu = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    nk += inK[e] ? 1u : 0u;
    nu += (inR[e] && !capped[e]) ? 1u : 0u;
  }
  uint64_t rk_total;
  const uint64_t rk = wave_exscan((static_cast<uint64_t>(nk) << 32) | nu, rk_total);
  uint32_t kpos = static_cast<uint32_t>(rk >> 32);
  uint32_t upos = static_cast<uint32_t>(rk);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = lane * E + e;
    if (inK[e]) {
      irow[kpos] = j;
      wrow[kpos] = 1.0f;
      ++kpos;
    }
    if (a.m > 0 && inR[e] && !capped[e]) {
      if (upos < delta) pi[e] += 1;
      ++upos;
    }
  }

  if (a.m > 0) {
    // ---- 3. systematic sample over the cumulative pi axis ----
    uint64_t psum = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) psum += pi[e];
    uint64_t ptotal;
    uint64_t c = wave_exscan(psum, ptotal);
    const uint64_t u = philox_word0(static_cast<uint32_t>(i), static_cast<uint32_t>(hd),
                                    static_cast<uint32_t>(b), 0u, a.seed_lo, a.seed_hi);
    auto below = [u](uint64_t x) -> uint64_t { return x > u ? ((x - u - 1) >> 32) + 1 : 0; };
    // every key is in registers now: the slice is reused to hand pi - 1 of
    // each sampled slot (1 <= pi <= 2^32) to the lane that writes its weight
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (!inR[e]) continue;
      const uint64_t c0 = c;
      c += pi[e];
      const uint64_t n0 = below(c0), n1 = below(c);
      if (n1 > n0 && n0 < static_cast<uint64_t>(a.m)) {  // k + m <= nV <= 64 E slots
        irow[a.k + static_cast<int>(n0)] = lane * E + e;
        sb[n0] = static_cast<uint32_t>(pi[e] - 1);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int x = lane; x < a.m; x += 64)
      wrow[a.k + x] = static_cast<float>(4294967296.0 / (static_cast<double>(sb[x]) + 1.0));
  }
}

}  // namespace

hipError_t launch_select(const Geometry& g, int k_exact, int m_sample, const float* S, int32_t* idx,
                         float* w, hipStream_t s) {
  SelectArgs a;
  a.S = S;
  a.idx = idx;
  a.w = w;
  a.H = g.H;
  a.nQB = g.nQB;
  a.nKU = g.nKU;
  a.nV = g.n_valid_units;
  a.k = k_exact;
  a.m = m_sample;
  a.seed_lo = static_cast<uint32_t>(g.seed);
  a.seed_hi = static_cast<uint32_t>(g.seed >> 32);
  const int rows = g.B * g.H * g.nQB;
  const dim3 wgrid((rows + SELW_WAVES - 1) / SELW_WAVES), wblock(64 * SELW_WAVES);
  const int per_lane = (a.nV + 63) / 64;
  if (per_lane <= 16) {
    if (per_lane <= 4) hipLaunchKernelGGL((select_wave_kernel<4>), wgrid, wblock, 0, s, a, rows);
    else if (per_lane <= 6) hipLaunchKernelGGL((select_wave_kernel<6>), wgrid, wblock, 0, s, a, rows);
    else if (per_lane <= 8) hipLaunchKernelGGL((select_wave_kernel<8>), wgrid, wblock, 0, s, a, rows);
    else if (per_lane <= 10) hipLaunchKernelGGL((select_wave_kernel<10>), wgrid, wblock, 0, s, a, rows);
    else if (per_lane <= 12) hipLaunchKernelGGL((select_wave_kernel<12>), wgrid, wblock, 0, s, a, rows);
    else hipLaunchKernelGGL((select_wave_kernel<16>), wgrid, wblock, 0, s, a, rows);
    return hipGetLastError();
  }
  const dim3 grid(rows), block(SEL_THREADS);
  if (a.nV <= 8 * SEL_THREADS) hipLaunchKernelGGL((select_kernel<8>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((select_kernel<16>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace bsa
