// Block selection for gfx950: exact top-k set plus a fixed-size systematic
// sample weighted by inverse inclusion probability, one workgroup per
// (b, h, query block).
//
// What is computed (InstaGen, Abstract: the highest-scoring blocks are kept
// whole, the others enter by a draw whose chance follows their estimated
// attention and are scaled by one over that chance, with one draw per query
// cluster; AB-Attention transcript: inclusion probabilities with certain
// inclusion for the strongest blocks, a fixed number of distinct blocks,
// probability 1/4 -> weight 4):
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
// order and bit-identical to the CPU definition. Besides exact power-of-two
// scalings and conversions, the only floating-point operations are two
// correctly rounded fp64 divisions and one fp64 -> fp32 rounding.
//
// Layout: thread t owns the E consecutive units [t E, t E + E), so exclusive
// scans give ranks in unit order directly. Rows of up to 1024 valid units take
// one wave each (ballot counts, DPP sums and scans, no barriers); longer rows take a
// 256-thread workgroup. The threshold of the exact set is found bit by bit,
// most significant first, below the bits that every key shares: the top 12
// bits over every key, the low 19 over the few keys that share the
// threshold's top bits, gathered into LDS (one wave finishes them without
// barriers).
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

// floor(value(x) 2^(FS - e)), at least 1. x is at most the maximum whose
// exponent is e, so value(x) < 2^e and the scaled value is below 2^FS: scaling
// by a power of two is exact unless the result underflows, and a result that
// small is far below 1, whose floor (0) gives 1 either way. The conversion
// truncates, which is the floor of a non-negative value.
__device__ __forceinline__ uint32_t quantise(uint32_t x, int e) {
  const float v = __builtin_amdgcn_ldexpf(__uint_as_float(x), FS - e);
  return max(1u, static_cast<uint32_t>(v));
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

// Workgroup reductions with one barrier each: every reduction writes the
// half of its buffer given by a parity that flips at every reduction, so a
// half is rewritten only after the next reduction's barrier, which every
// thread reaches after its reads of this one.
struct BlockRed {
  uint64_t r64[2][SEL_WAVES];
  uint32_t r32[2][SEL_WAVES];
};

template <typename T>
__device__ __forceinline__ T* red_half(BlockRed& r, int par) {
  if constexpr (sizeof(T) == 8) return r.r64[par];
  else return r.r32[par];
}

template <typename T>
__device__ __forceinline__ T block_sum(T v, BlockRed& r, int& par) {
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  T* red = red_half<T>(r, par);
  par ^= 1;
  v = wave_sum(v);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  T t = 0;
#pragma unroll
  for (int x = 0; x < SEL_WAVES; ++x) t += red[x];
  return t;
}

__device__ __forceinline__ uint32_t block_max(uint32_t v, BlockRed& r, int& par) {
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  uint32_t* red = r.r32[par];
  par ^= 1;
  v = wave_max_u32(v);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (int x = 0; x < SEL_WAVES; ++x) t = max(t, red[x]);
  return t;
}

// Exclusive prefix over threads in index order; `total` receives the block sum.
__device__ __forceinline__ uint64_t block_exscan(uint64_t v, BlockRed& r, int& par, uint64_t& total) {
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  uint64_t* red = r.r64[par];
  par ^= 1;
  const uint64_t x = wave_inclusive_scan(v);
  if (lane == 63) red[wave] = x;
  __syncthreads();
  uint64_t before = 0, tot = 0;
#pragma unroll
  for (int z = 0; z < SEL_WAVES; ++z) {
    const uint64_t rz = red[z];
    if (z < wave) before += rz;
    tot += rz;
  }
  total = tot;
  return before + x - v;
}

// Every key lies between the smallest and the largest, so all of them (and
// the k-th largest) share the bits above the highest bit where those two
// differ: the bitwise search starts below it, from that common prefix.
// Returns the highest differing bit (-1 when every key is equal) and sets T.
__device__ __forceinline__ int common_prefix(uint32_t kmin, uint32_t kmax, uint32_t& T) {
  const uint32_t diff = kmin ^ kmax;
  const int top = diff ? 31 - __clz(diff) : -1;
  T = top >= 0 ? kmax & ~((2u << top) - 1u) : kmax;  // top = 31 cannot occur: keys are below 2^31
  return top;
}

// ceil(x / d) for d >= 1: the smallest q with d q >= x.
__device__ __forceinline__ uint32_t level(uint32_t x, uint32_t d) { return x / d + (x % d != 0u ? 1u : 0u); }

// The threshold search of the exact set runs in two phases: the top bits
// 30..SPLIT over every key, then the low SPLIT bits over the keys that share
// the threshold's top bits ("in play"), compacted into LDS. For the largest
// prefix P with at least k keys >= P, fewer than k keys lie above P's bin, so
// the low bits are the search for the (k - above)-th largest in-play key.
constexpr int SPLIT = 19;      // top 12 bits: the exponent and 4 mantissa bits
constexpr int PLAY_MAX = 256;  // in-play keys one wave finishes (4 per lane); more take the block loop

// Six waves per SIMD (at most 80 registers): the kernel is bound by vector
// ALU issue, and more resident rows hide the latency of its barriers.
template <int E>
__global__ __launch_bounds__(SEL_THREADS) __attribute__((amdgpu_waves_per_eu(6))) void select_kernel(SelectArgs a) {
  static_assert(PLAY_MAX <= SEL_THREADS * E, "the in-play keys borrow the row's staging array");
  __shared__ uint32_t sbits[SEL_THREADS * E];
  __shared__ BlockRed red;
  __shared__ uint32_t cnt2[2][SEL_WAVES];  // per-wave counts, alternating buffers
  __shared__ uint32_t t_bcast;
  int par = 0;  // reduction buffer half (uniform)

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
      v[e] = __float_as_uint(srow[min(x, a.nV - 1)]);  // past nV: a copy, never used
    }
#pragma unroll
    for (int e = 0; e < E; ++e) sbits[tid + e * SEL_THREADS] = v[e];
  }
  __syncthreads();

  // Per-unit state stays small: validity is recomputed from the unit index,
  // the exact set is a bit mask (bit e: unit tid E + e), the capped units are
  // the units of R at or above the water level, and pi (1 <= pi <= 2^32 on R)
  // is held as pi - 1 in 32 bits.
  const int j0 = tid * E;
  auto valid = [&](int e) { return j0 + e < a.nV; };
  uint32_t key[E];
  uint32_t fK = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) key[e] = valid(e) ? sanitize(sbits[j0 + e]) : 0u;

  // ---- 1. exact set: T = k-th largest key, ties by lower index ----
  if (a.k > 0) {
    // counts from ballots (cand >= 1 and invalid units hold key 0); one
    // barrier per bit: a buffer is rewritten two bits later, after every
    // thread has passed the barrier that follows its reads
    const int wave = tid / 64, lane = tid % 64;
    uint32_t kmax = 0, kmin = 0xFFFFFFFFu;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      kmax = max(kmax, valid(e) ? key[e] : 0u);
      kmin = min(kmin, valid(e) ? key[e] : 0xFFFFFFFFu);
    }
    {  // both extremes in one reduction: the maximum of the keys and of their complements
      kmax = wave_max_u32(kmax);
      kmin = ~wave_max_u32(~kmin);
      uint64_t* rr = red.r64[par];
      par ^= 1;
      if (lane == 0) rr[wave] = (static_cast<uint64_t>(kmax) << 32) | ~kmin;
      __syncthreads();
      uint32_t m0 = 0, m1 = 0;
#pragma unroll
      for (int x = 0; x < SEL_WAVES; ++x) {
        m0 = max(m0, static_cast<uint32_t>(rr[x] >> 32));
        m1 = max(m1, static_cast<uint32_t>(rr[x]));
      }
      kmax = m0;
      kmin = ~m1;
    }
    uint32_t T;
    const int top_bit = common_prefix(kmin, kmax, T);
    auto block_bits = [&](int top, int low) {
      for (int bit = top; bit >= low; --bit) {
        const uint32_t cand = T | (1u << bit);
        uint32_t c = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) c += __popcll(__ballot(key[e] >= cand));
        if (lane == 0) cnt2[bit & 1][wave] = c;
        __syncthreads();
        uint32_t tot = 0;
#pragma unroll
        for (int x = 0; x < SEL_WAVES; ++x) tot += cnt2[bit & 1][x];
        if (tot >= static_cast<uint32_t>(a.k)) T = cand;
      }
    };
    block_bits(top_bit, SPLIT);
    // keys above T's bin, and the keys in it (hi may be 2^31: no key reaches it)
    const uint32_t hi = T + (1u << SPLIT);
    uint32_t n_above = 0, n_play = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      n_above += (valid(e) && key[e] >= hi) ? 1u : 0u;
      n_play += (valid(e) && key[e] >= T && key[e] < hi) ? 1u : 0u;
    }
    uint64_t tot;
    const uint64_t pos = block_exscan((static_cast<uint64_t>(n_above) << 32) | n_play, red, par, tot);
    const uint32_t above = static_cast<uint32_t>(tot >> 32), play = static_cast<uint32_t>(tot);
    if (play <= static_cast<uint32_t>(PLAY_MAX)) {
      // every key is in registers and the exscan's barrier has passed: the
      // staging array takes the in-play keys
      uint32_t p = static_cast<uint32_t>(pos);
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (valid(e) && key[e] >= T && key[e] < hi) sbits[p++] = key[e];
      __syncthreads();
      if (wave == 0) {
        const uint32_t need = static_cast<uint32_t>(a.k) - above;  // >= 1
        uint32_t ck[PLAY_MAX / 64];
#pragma unroll
        for (int z = 0; z < PLAY_MAX / 64; ++z) {
          const uint32_t x = static_cast<uint32_t>(lane + 64 * z);
          ck[z] = x < play ? sbits[x] : 0u;  // padding 0 never reaches cand >= 1
        }
        for (int bit = min(SPLIT - 1, top_bit); bit >= 0; --bit) {
          const uint32_t cand = T | (1u << bit);
          uint32_t c = 0;
#pragma unroll
          for (int z = 0; z < PLAY_MAX / 64; ++z) c += __popcll(__ballot(ck[z] >= cand));
          if (c >= need) T = cand;
        }
        if (lane == 0) t_bcast = T;
      }
      __syncthreads();
      T = t_bcast;
    } else {
      block_bits(min(SPLIT - 1, top_bit), 0);
    }
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      gt += (valid(e) && key[e] > T) ? 1u : 0u;
      eq += (valid(e) && key[e] == T) ? 1u : 0u;
    }
    // one scan: the count above T (high word, total only) and the ranks of the keys equal to T
    uint64_t ge_total;
    const uint64_t ge = block_exscan((static_cast<uint64_t>(gt) << 32) | eq, red, par, ge_total);
    const uint32_t need = static_cast<uint32_t>(a.k) - static_cast<uint32_t>(ge_total >> 32);
    uint32_t r = static_cast<uint32_t>(ge);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (!valid(e)) continue;
      if (key[e] > T) {
        fK |= 1u << e;
      } else if (key[e] == T) {
        if (r < need) fK |= 1u << e;
        ++r;
      }
    }
  }
  auto inR = [&](int e) { return valid(e) && ((fK >> e) & 1u) == 0u; };

  // ---- 2. inclusion probabilities on R (valid and not in K) ----
  // q: quantised scores on R, 1 <= q < 2^FS, and 0 elsewhere, so that with at
  // most 4096 valid units every sum of q fits 32 bits. thr: the water level;
  // the capped units (pi = 1) are the units of R with q >= thr.
  uint32_t q[E];
#pragma unroll
  for (int e = 0; e < E; ++e) q[e] = 0u;
  uint32_t thr = 0xFFFFFFFFu, delta = 0;
  uint32_t pim1[E];  // pi - 1 on R (pi in [1, 2^32]), before the shortfall
  // this thread's uncapped units, capped units and sum of pi over the uncapped ones
  uint32_t nu = 0, ncap = 0;
  uint64_t usum = 0;
  if (a.m > 0) {
    // ---- 2a. quantised scores over R ----
    uint32_t mx = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) mx = max(mx, inR(e) ? key[e] : 0u);
    mx = block_max(mx, red, par);
    const int ex = mx ? frexp_exp(mx) : 0;
    uint32_t qsum = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      q[e] = inR(e) ? (mx ? quantise(key[e], ex) : 1u) : 0u;
      qsum += q[e];
    }
    const uint32_t QR = block_sum(qsum, red, par);

    // ---- 2b. water-filling on exact integers ----
    // A unit of R is capped once (m - t) q_j >= Q_U, i.e. once q_j reaches the
    // level ceil(Q_U / (m - t)), with t the capped units and Q_U the sum of q
    // over the others. Capping the units at or above the level can only lower
    // it, so after every round the capped units are exactly those with q at or
    // above the current level: a round is one compare per unit and one sum,
    // until a round caps nothing new.
    uint32_t t = 0, QU = QR;
    thr = level(QU, static_cast<uint32_t>(a.m));
    while (true) {
      uint32_t cnt = 0, qs = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const bool cap = q[e] >= thr;  // q = 0 outside R never reaches thr >= 1
        cnt += cap ? 1u : 0u;
        qs += cap ? q[e] : 0u;
      }
      const uint64_t tot = block_sum((static_cast<uint64_t>(cnt) << 40) | qs, red, par);
      const uint32_t nt = static_cast<uint32_t>(tot >> 40);
      if (nt == t) break;
      t = nt;
      QU = QR - static_cast<uint32_t>(tot & ((1ull << 40) - 1));
      if (t >= static_cast<uint32_t>(a.m)) break;  // R is all capped (t = m = |R|)
      thr = level(QU, static_cast<uint32_t>(a.m) - t);
    }

    // ---- 2c. fixed-point pi ----
    // (m - t) q_j < 2^32 and Q_U < 2^32 are exact in fp64; an uncapped unit has
    // (m - t) q_j < Q_U, so its correctly rounded ratio is below 1 and 2^32
    // ratio fits 32 bits (>= 1).
    const uint32_t mt = static_cast<uint32_t>(a.m) - t;
    const double mt_d = static_cast<double>(mt), qu_d = static_cast<double>(QU);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      pim1[e] = 0xFFFFFFFFu;  // capped: pi = 2^32
      ncap += q[e] >= thr ? 1u : 0u;
      if (q[e] != 0u && q[e] < thr) {
        const double ratio = (mt_d * static_cast<double>(q[e])) / qu_d;
        const uint32_t pv = static_cast<uint32_t>(ratio * 4294967296.0);
        pim1[e] = pv - 1u;
        usum += pv;
        ++nu;
      }
    }
    // below the number of uncapped units: the floors lose less than 1 each
    delta = static_cast<uint32_t>((static_cast<uint64_t>(mt) << 32) - block_sum(usum, red, par));
  }

  // ---- ranks in unit order: K (high word) and uncapped R (low word) ----
  uint64_t rk_total;
  const uint64_t rk = block_exscan((static_cast<uint64_t>(__popc(fK)) << 32) | nu, red, par, rk_total);
  {  // the exact set, ascending, with w = 1
    uint32_t kpos = static_cast<uint32_t>(rk >> 32);
    for (uint32_t f = fK; f != 0u; f &= f - 1u, ++kpos) {
      irow[kpos] = j0 + __builtin_ctz(f);
      wrow[kpos] = 1.0f;
    }
  }

  if (a.m > 0) {
    // The shortfall delta goes as +1 to the uncapped units of rank < delta; the
    // uncapped units of this thread hold ranks u0 .. u0 + nu - 1. The sum of pi
    // over its units of R follows without another pass: the uncapped pi, the
    // shortfall it receives, and 2^32 for every capped unit.
    const uint32_t u0 = static_cast<uint32_t>(rk);
    const uint32_t n_short = min(nu, delta > u0 ? delta - u0 : 0u);
    const uint64_t psum = usum + n_short + (static_cast<uint64_t>(ncap) << 32);

    // ---- 3. systematic sample over the cumulative pi axis: slot s sits at
    // u + s 2^32. This thread's units cover [c, c + psum); np is the first slot
    // at or above the running end c, and since pi <= 2^32 a unit holds at most
    // one slot (units outside R add nothing and hold none) ----
    uint64_t ptotal;
    uint64_t c = block_exscan(psum, red, par, ptotal);
    const uint64_t u = philox_word0(static_cast<uint32_t>(i), static_cast<uint32_t>(hd),
                                    static_cast<uint32_t>(b), 0u, a.seed_lo, a.seed_hi);
    uint32_t n = c > u ? static_cast<uint32_t>(((c - u - 1) >> 32) + 1) : 0u;  // slots below c
    uint64_t np = u + (static_cast<uint64_t>(n) << 32);
    // every key is in registers and the exscan's barrier has passed: the
    // staging array hands pi - 1 of each sampled slot (1 <= pi <= 2^32) to the
    // thread that writes its weight (k + m <= nV slots)
    uint32_t upos = u0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool unc = q[e] != 0u && q[e] < thr;
      const uint32_t pe = pim1[e] + ((unc && upos < delta) ? 1u : 0u);  // pi - 1 with the shortfall
      upos += unc ? 1u : 0u;
      c += q[e] != 0u ? static_cast<uint64_t>(pe) + 1u : 0u;
      if (c > np) {
        if (n < static_cast<uint32_t>(a.m)) {  // always, when sum pi = m 2^32
          irow[a.k + static_cast<int>(n)] = j0 + e;
          sbits[n] = pe;
        }
        ++n;
        np += 1ull << 32;
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
      v[e] = __float_as_uint(srow[min(x, a.nV - 1)]);  // past nV: a copy, never used
    }
#pragma unroll
    for (int e = 0; e < E; ++e) sb[lane + 64 * e] = v[e];
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // Small per-unit state, as in select_kernel: validity from the unit index,
  // a bit mask for the exact set, the water level for the capped units, pi - 1
  // in 32 bits.
  const int j0 = lane * E;
  auto valid = [&](int e) { return j0 + e < a.nV; };
  uint32_t key[E];
  uint32_t fK = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t raw = sb[j0 + e];  // inside the wave's slice; ignored past nV
    key[e] = valid(e) ? sanitize(raw) : 0u;
  }

  // ---- 1. exact set: the top bits over every key, the low bits over the
  // keys in the threshold's bin (compacted into the wave's slice) ----
  if (a.k > 0) {
    uint32_t kmax = 0, kmin = 0xFFFFFFFFu;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      kmax = max(kmax, valid(e) ? key[e] : 0u);
      kmin = min(kmin, valid(e) ? key[e] : 0xFFFFFFFFu);
    }
    uint32_t T;
    const int top_bit = common_prefix(~wave_max_u32(~kmin), wave_max_u32(kmax), T);
    for (int bit = top_bit; bit >= SPLIT; --bit) {
      const uint32_t cand = T | (1u << bit);
      uint32_t c = 0;  // cand >= 1, and invalid units hold key 0
#pragma unroll
      for (int e = 0; e < E; ++e) c += __popcll(__ballot(key[e] >= cand));
      if (c >= static_cast<uint32_t>(a.k)) T = cand;
    }
    {
      const uint32_t hi = T + (1u << SPLIT);  // may be 2^31: no key reaches it
      uint32_t above = 0, n_play = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        above += __popcll(__ballot(valid(e) && key[e] >= hi));
        n_play += (valid(e) && key[e] >= T && key[e] < hi) ? 1u : 0u;
      }
      uint64_t play64;
      uint32_t p = static_cast<uint32_t>(wave_exscan(n_play, play64));
      const uint32_t play = static_cast<uint32_t>(play64);  // <= nV <= 64 E: fits the slice
      // every key is in registers: the slice takes the in-play keys
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (valid(e) && key[e] >= T && key[e] < hi) sb[p++] = key[e];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const uint32_t need = static_cast<uint32_t>(a.k) - above;  // >= 1
      const int chunks = static_cast<int>((play + 63) / 64);   // uniform
      uint32_t ck[E];
#pragma unroll
      for (int z = 0; z < E; ++z) {
        const uint32_t x = static_cast<uint32_t>(lane + 64 * z);
        ck[z] = (z < chunks && x < play) ? sb[x] : 0u;  // padding 0 never reaches cand >= 1
      }
      for (int bit = min(SPLIT - 1, top_bit); bit >= 0; --bit) {
        const uint32_t cand = T | (1u << bit);
        uint32_t c = 0;
#pragma unroll
        for (int z = 0; z < E; ++z)
          if (z < chunks) c += __popcll(__ballot(ck[z] >= cand));
        if (c >= need) T = cand;
      }
    }
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      gt += __popcll(__ballot(valid(e) && key[e] > T));
      eq += (valid(e) && key[e] == T) ? 1u : 0u;
    }
    const uint32_t need = static_cast<uint32_t>(a.k) - gt;
    uint64_t eq_total;
    uint32_t r = static_cast<uint32_t>(wave_exscan(eq, eq_total));
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (!valid(e)) continue;
      if (key[e] > T) {
        fK |= 1u << e;
      } else if (key[e] == T) {
        if (r < need) fK |= 1u << e;
        ++r;
      }
    }
  }
  auto inR = [&](int e) { return valid(e) && ((fK >> e) & 1u) == 0u; };

  // ---- 2. inclusion probabilities on R, as in select_kernel ----
  uint32_t q[E];
#pragma unroll
  for (int e = 0; e < E; ++e) q[e] = 0u;
  uint32_t thr = 0xFFFFFFFFu, delta = 0;
  uint32_t pim1[E];  // pi - 1 on R (pi in [1, 2^32]), before the shortfall
  uint32_t nu = 0, ncap = 0;
  uint64_t usum = 0;
  if (a.m > 0) {
    // ---- 2a. quantised scores over R ----
    uint32_t mx = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) mx = max(mx, inR(e) ? key[e] : 0u);
    mx = wave_max_u32(mx);
    const int ex = mx ? frexp_exp(mx) : 0;
    uint32_t qsum = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      q[e] = inR(e) ? (mx ? quantise(key[e], ex) : 1u) : 0u;
      qsum += q[e];
    }
    const uint32_t QR = wave_sum(qsum);

    // ---- 2b. water-filling on exact integers: rounds of one compare per unit ----
    uint32_t t = 0, QU = QR;
    thr = level(QU, static_cast<uint32_t>(a.m));
    while (true) {
      uint32_t cnt = 0, qs = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const bool cap = q[e] >= thr;
        cnt += __popcll(__ballot(cap));
        qs += cap ? q[e] : 0u;
      }
      if (cnt == t) break;
      t = cnt;
      QU = QR - wave_sum(qs);
      if (t >= static_cast<uint32_t>(a.m)) break;
      thr = level(QU, static_cast<uint32_t>(a.m) - t);
    }

    // ---- 2c. fixed-point pi ----
    const uint32_t mt = static_cast<uint32_t>(a.m) - t;
    const double mt_d = static_cast<double>(mt), qu_d = static_cast<double>(QU);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      pim1[e] = 0xFFFFFFFFu;  // capped: pi = 2^32
      ncap += q[e] >= thr ? 1u : 0u;
      if (q[e] != 0u && q[e] < thr) {
        const double ratio = (mt_d * static_cast<double>(q[e])) / qu_d;
        const uint32_t pv = static_cast<uint32_t>(ratio * 4294967296.0);
        pim1[e] = pv - 1u;
        usum += pv;
        ++nu;
      }
    }
    delta = static_cast<uint32_t>((static_cast<uint64_t>(mt) << 32) - wave_sum(usum));
  }

  // ---- ranks in unit order: K (high word) and uncapped R (low word) ----
  uint64_t rk_total;
  const uint64_t rk = wave_exscan((static_cast<uint64_t>(__popc(fK)) << 32) | nu, rk_total);
  {
    uint32_t kpos = static_cast<uint32_t>(rk >> 32);
    for (uint32_t f = fK; f != 0u; f &= f - 1u, ++kpos) {
      irow[kpos] = j0 + __builtin_ctz(f);
      wrow[kpos] = 1.0f;
    }
  }

  if (a.m > 0) {
    // the sum of pi over this lane's units of R without another pass, as in select_kernel
    const uint32_t u0 = static_cast<uint32_t>(rk);
    const uint32_t n_short = min(nu, delta > u0 ? delta - u0 : 0u);
    const uint64_t psum = usum + n_short + (static_cast<uint64_t>(ncap) << 32);

    // ---- 3. systematic sample over the cumulative pi axis ----
    uint64_t ptotal;
    uint64_t c = wave_exscan(psum, ptotal);
    const uint64_t u = philox_word0(static_cast<uint32_t>(i), static_cast<uint32_t>(hd),
                                    static_cast<uint32_t>(b), 0u, a.seed_lo, a.seed_hi);
    uint32_t n = c > u ? static_cast<uint32_t>(((c - u - 1) >> 32) + 1) : 0u;
    uint64_t np = u + (static_cast<uint64_t>(n) << 32);
    // every key is in registers now: the slice is reused to hand pi - 1 of
    // each sampled slot (1 <= pi <= 2^32) to the lane that writes its weight
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    uint32_t upos = u0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool unc = q[e] != 0u && q[e] < thr;
      const uint32_t pe = pim1[e] + ((unc && upos < delta) ? 1u : 0u);  // pi - 1 with the shortfall
      upos += unc ? 1u : 0u;
      c += q[e] != 0u ? static_cast<uint64_t>(pe) + 1u : 0u;
      if (c > np) {
        if (n < static_cast<uint32_t>(a.m)) {  // k + m <= nV <= 64 E slots
          irow[a.k + static_cast<int>(n)] = j0 + e;
          sb[n] = pe;
        }
        ++n;
        np += 1ull << 32;
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
