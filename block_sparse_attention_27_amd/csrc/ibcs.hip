// Intra-block query clustering for gfx950: Lloyd's k-means of every query
// block's valid rows into G groups.
//
// What is computed (AB-Attention, Abstract: the Intra-Block Clustering
// Selector clusters the queries of each query block only, with no token
// permutation; podcast transcript, the passage on how blocks are chosen:
// similar queries are grouped, each group has a representative and a weight
// from its size). The pages fix no algorithm; this is the reading the library
// takes:
//   * the group decisions use exact integers: q_int = rint(q 2^s), s = 11 - e
//     with max |q| over the block = f 2^e, f in [0.5, 1), so |q_int| <= 2^11
//     and a squared distance over d <= 128 dimensions is an exact unsigned
//     32-bit sum (at most 2^31);
//   * the initial centroid of group g is q_int of row floor(g n / G) of the
//     block (n valid rows, in the block's own order after the optional
//     gather);
//   * an iteration assigns every row to the nearest centroid (ties: the lower
//     group), then sets every centroid to the rounded mean of its rows,
//     floor((2 sum + n_g) / (2 n_g)); a group with no rows keeps its centroid;
//   * after T iterations the kernel writes each group's row count n_g and its
//     representative, the fp32 mean of its rows' original values (zero for an
//     empty group).
// Every decision is integer arithmetic, so the counts are bit-identical to
// the definition on any hardware. The score kernel turns the output into S as
// the mixture, by n_g / n, of every group's n_j-weighted softmax over the key
// units.
//
// One workgroup (512 threads) per (b, h, query block). The block's rows are
// staged once in LDS in their input type, next to their 16-bit fixed-point
// copies. A distance is |q|^2 + |c|^2 - 2 <q, c> with the inner product on
// v_dot2_i32_i16 (two dimensions per instruction, exact); TPR threads share a
// row and every centroid read is an LDS broadcast. For the centroid sums a
// thread owns one column of a range of rows; all lanes of a wave walk the same
// rows, so a row's group is wave-uniform and each row costs one add into the
// right register. The final fp32 means use a fixed order, so the output is
// deterministic.
#include "bsa_internal.hpp"

namespace bsa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int CL_THREADS = 512;

struct ClusterArgs {
  const void* q;
  const int32_t* perm;
  float* q_cent;
  int32_t* q_size;
  int N, N_pad, nQB, iters;
};

template <bool BF16>
struct Stage;
template <>
struct Stage<true> {
  typedef uint16_t T;
  static __device__ __forceinline__ float get(T x) { return __uint_as_float(static_cast<uint32_t>(x) << 16); }
};
template <>
struct Stage<false> {
  typedef float T;
  static __device__ __forceinline__ float get(T x) { return x; }
};

constexpr int FIXED_BITS = 11;

typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// the two int16 halves of a 32-bit word (taken by value: a bit cast of a
// vector-element lvalue would read the vector's first element)
__device__ __forceinline__ s16x2 as_s16x2(int v) { return __builtin_bit_cast(s16x2, v); }

// sum of the 8 products of two 16-byte runs of int16
__device__ __forceinline__ int dot8(i32x4 x, i32x4 y, int acc) {
#pragma unroll
  for (int z = 0; z < 4; ++z) acc = __builtin_amdgcn_sdot2(as_s16x2(x[z]), as_s16x2(y[z]), acc, false);
  return acc;
}

template <int D, int BQ, int G, bool BF16, bool PERM>
__global__ __launch_bounds__(CL_THREADS) void block_clusters_kernel(ClusterArgs a) {
  typedef typename Stage<BF16>::T T;
  constexpr int ESZ = sizeof(T);
  constexpr int EPC = 16 / ESZ;              // elements per 16-byte chunk
  constexpr int CH = D / EPC;                // chunks per row
  constexpr int RPP = CL_THREADS / CH;       // rows staged per pass
  constexpr int LD = D + EPC;                // padded LDS row (elements)
  constexpr int LDI = D + 8;                 // padded fixed-point row (int16)
  constexpr int TPR = CL_THREADS / BQ;       // threads per row in the distance step
  constexpr int DP = D / TPR;                // dimensions per distance thread
  constexpr int PARTS = CL_THREADS / D;      // row ranges in the sum steps
  constexpr int RP = BQ / PARTS;             // rows per range
  constexpr int NPART = (TPR * BQ * G > PARTS * G * D) ? TPR * BQ * G : PARTS * G * D;
  static_assert(DP % 8 == 0 && RP * PARTS == BQ && D <= 128, "tiling");

  __shared__ __align__(16) T rows[BQ][LD];
  __shared__ __align__(16) short qi[BQ][LDI];  // fixed-point rows
  __shared__ __align__(16) short ci[G][D];     // fixed-point centroids
  __shared__ int qq[BQ];                        // |q_int|^2 per row
  __shared__ int cc2[G];                        // |c_int|^2 per centroid
  __shared__ union {
    int ip[NPART];       // partial inner products
    float fsum[NPART];   // partial sums of the original values
  } part;
  constexpr int NW = (BQ + 63) / 64;  // waves that hold rows in the assignment step
  __shared__ int rowlist[BQ];         // rows ordered by group, ascending within a group
  __shared__ int wcnt[NW][G];         // rows of each group per assignment wave
  __shared__ float wmax[CL_THREADS / 64];

  const int tid = threadIdx.x;
  const int blk = blockIdx.x;  // (bh, i)
  const int bh = blk / a.nQB, i = blk % a.nQB;
  const int row0 = i * BQ;
  const int n = max(0, min(BQ, a.N - row0));
  float* cout = a.q_cent + static_cast<size_t>(blk) * G * D;
  int32_t* sout = a.q_size + static_cast<size_t>(blk) * G;
  if (n == 0) {  // whole workgroup: a block with no valid row has no groups
    for (int x = tid; x < G * D; x += CL_THREADS) cout[x] = 0.f;
    if (tid < G) sout[tid] = 0;
    return;
  }

  // ---- stage the valid rows (all loads in flight at once); largest magnitude
  const char* base = static_cast<const char*>(a.q) + static_cast<size_t>(bh) * a.N_pad * D * ESZ;
  constexpr int MAXP = BQ / RPP;  // staging passes for a full block
  const int cc = tid % CH, rg = tid / CH;
  u32x4 xr[MAXP];
#pragma unroll
  for (int pp = 0; pp < MAXP; ++pp) {
    const int r = rg + pp * RPP;
    int gr = row0 + r;
    bool ok = r < n;
    if constexpr (PERM) {
      if (ok) {
        gr = a.perm[gr];
        ok = static_cast<unsigned>(gr) < static_cast<unsigned>(a.N_pad);  // a bad gather entry reads as a zero row
      }
    }
    xr[pp] = ok ? *reinterpret_cast<const u32x4*>(base + (static_cast<size_t>(gr) * D + cc * EPC) * ESZ)
                : u32x4{0u, 0u, 0u, 0u};
  }
  float mx = 0.f;
#pragma unroll
  for (int pp = 0; pp < MAXP; ++pp) {
    const int r = rg + pp * RPP;
    if (r < n) *reinterpret_cast<u32x4*>(&rows[r][cc * EPC]) = xr[pp];
    const T* xv = reinterpret_cast<const T*>(&xr[pp]);
#pragma unroll
    for (int z = 0; z < EPC; ++z) mx = fmaxf(mx, fabsf(Stage<BF16>::get(xv[z])));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if (tid % 64 == 0) wmax[tid / 64] = mx;
  __syncthreads();  // per-wave maxima ready
  mx = wmax[0];
#pragma unroll
  for (int x = 1; x < CL_THREADS / 64; ++x) mx = fmaxf(mx, wmax[x]);
  int ex = 0;
  if (mx > 0.f) frexpf(mx, &ex);
  const int sh = mx > 0.f ? FIXED_BITS - ex : 0;

  // ---- fixed-point copies (|q_int| <= 2^11) from the staged registers.
  // x 2^sh is exact, and adding 1.5 2^23 rounds it to the nearest integer
  // (ties to even) in the last place of a float in [2^23, 2^24), whose bits
  // minus those of 1.5 2^23 are that integer.
  constexpr float MAGIC = 12582912.f;  // 1.5 2^23
#pragma unroll
  for (int pp = 0; pp < MAXP; ++pp) {
    const int r = rg + pp * RPP;
    if (r < n) {
      const T* xv = reinterpret_cast<const T*>(&xr[pp]);
      uint32_t w[EPC / 2];
#pragma unroll
      for (int z = 0; z < EPC / 2; ++z) {
        const uint32_t i0 = __float_as_uint(ldexpf(Stage<BF16>::get(xv[2 * z]), sh) + MAGIC) - 0x4B400000u;
        const uint32_t i1 = __float_as_uint(ldexpf(Stage<BF16>::get(xv[2 * z + 1]), sh) + MAGIC) - 0x4B400000u;
        w[z] = (i0 & 0xFFFFu) | (i1 << 16);
      }
      if constexpr (EPC == 8) {
        *reinterpret_cast<u32x4*>(&qi[r][cc * EPC]) = u32x4{w[0], w[1], w[2], w[3]};
      } else {
#pragma unroll
        for (int z = 0; z < EPC / 2; ++z) *reinterpret_cast<uint32_t*>(&qi[r][cc * EPC + 2 * z]) = w[z];
      }
    }
  }
  __syncthreads();  // rows and fixed-point rows ready
  for (int x = tid; x < G * D; x += CL_THREADS) ci[x / D][x % D] = qi[((x / D) * n) / G][x % D];
  if (tid < G) cc2[tid] = 0;
  __syncthreads();
  // |c_int|^2 of every centroid: column tid of each, summed per wave, then across waves
  auto centroid_squares = [&]() {
    if (tid < D) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int c = ci[g][tid];
        int v = c * c;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
        if (tid % 64 == 0) atomicAdd(&cc2[g], v);
      }
    }
  };
  centroid_squares();

  const int dr = tid % BQ, dp = tid / BQ;   // distance step: row dr, dimensions [dp DP, dp DP + DP)
  const int uj = tid % D, up = tid / D;     // sum steps: column uj, rows [up RP, up RP + RP)
  const int r1 = min(n, up * RP + RP);
  {  // |q_int|^2 per row
    int acc = 0;
    if (dr < n) {
#pragma unroll
      for (int e = 0; e < DP; e += 8) {
        const i32x4 x = *reinterpret_cast<const i32x4*>(&qi[dr][dp * DP + e]);
        acc = dot8(x, x, acc);
      }
    }
    part.ip[dp * BQ + dr] = acc;
  }
  __syncthreads();
  if (tid < n) {
    int s = 0;
#pragma unroll
    for (int x = 0; x < TPR; ++x) s += part.ip[x * BQ + tid];
    qq[tid] = s;
  }

  int cnt_s[G], off_s[G];  // group sizes and rowlist offsets of the last assignment
  for (int it = 0; it < a.iters; ++it) {
    __syncthreads();  // centroids and |q|^2 ready
    {
      int acc[G];
#pragma unroll
      for (int g = 0; g < G; ++g) acc[g] = 0;
#pragma unroll
      for (int e = 0; e < DP; e += 8) {
        const int j0 = dp * DP + e;
        const i32x4 x = *reinterpret_cast<const i32x4*>(&qi[dr][j0]);
#pragma unroll
        for (int g = 0; g < G; ++g) acc[g] = dot8(x, *reinterpret_cast<const i32x4*>(&ci[g][j0]), acc[g]);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) part.ip[(dp * BQ + dr) * G + g] = acc[g];
    }
    __syncthreads();  // partial inner products ready
    int myl = G, rank = 0;  // group of row tid (G: no row) and its rank among the wave's rows of that group
    if (tid < 64 * NW) {    // whole waves
      if (tid < n) {
        uint32_t best = 0u;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          int ip = 0;
#pragma unroll
          for (int x = 0; x < TPR; ++x) ip += part.ip[(x * BQ + tid) * G + g];
          // |q - c|^2 in [0, 2^31]: exact in unsigned 32-bit arithmetic
          const uint32_t d2 = static_cast<uint32_t>(qq[tid]) + static_cast<uint32_t>(cc2[g]) - 2u * static_cast<uint32_t>(ip);
          if (g == 0 || d2 < best) {  // strict: ties keep the lower group
            best = d2;
            myl = g;
          }
        }
      }
      const uint64_t below = (1ull << (tid % 64)) - 1ull;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const uint64_t m = __ballot(myl == g);
        if (myl == g) rank = __popcll(m & below);
        if (tid % 64 == 0) wcnt[tid / 64][g] = __popcll(m);
      }
    }
    __syncthreads();  // group counts per wave ready
    int cnt[G], off[G];  // rows per group and the group's first position in rowlist
#pragma unroll
    for (int g = 0; g < G; ++g) {
      cnt[g] = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) cnt[g] += wcnt[w][g];
      off[g] = g == 0 ? 0 : off[g - 1] + cnt[g - 1];
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      cnt_s[g] = cnt[g];
      off_s[g] = off[g];
    }
    if (tid < n) {
      int pos = rank;
#pragma unroll
      for (int g = 0; g < G; ++g) pos += g == myl ? off[g] : 0;
#pragma unroll
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int g = 0; g < G; ++g) pos += (w < tid / 64 && g == myl) ? wcnt[w][g] : 0;
      rowlist[pos] = tid;
    }
    __syncthreads();  // rowlist ready
    {
      // fixed-point sums per group over this thread's column and position range
      const int p0 = up * RP;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int lo = max(p0, off[g]), hi = min(r1, off[g] + cnt[g]);
        int acc = 0;
        const short* qcol = &qi[0][0] + uj;
#pragma unroll 4
        for (int x = lo; x < hi; ++x) acc += qcol[__umul24(rowlist[x], LDI)];
        part.ip[(up * G + g) * D + uj] = acc;
      }
    }
    if (tid < G) cc2[tid] = 0;
    __syncthreads();  // partial sums ready
    if (tid < D) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int c = cnt[g];
        if (c > 0) {
          int sum = 0;
#pragma unroll
          for (int x = 0; x < PARTS; ++x) sum += part.ip[(x * G + g) * D + tid];
          // rounded mean, halves up: floor((2 s + c) / (2 c)). The exact quotient is
          // k + f / (2c) with f an integer, so (num + 1/2) / (2c) sits at least 1/512
          // inside [k, k + 1); its fp32 value (|num| < 2^20, one rcp and one multiply)
          // is within 4e-4 of it, and the floor is exact.
          const int num = 2 * sum + c;
          const float y = (static_cast<float>(num) + 0.5f) * __builtin_amdgcn_rcpf(static_cast<float>(2 * c));
          ci[g][tid] = static_cast<short>(static_cast<int>(floorf(y)));
        }
      }
    }
    centroid_squares();  // each column is read by the thread that wrote it
    // the next iteration's first barrier publishes the centroids and their squares
  }
  __syncthreads();  // the last update's reads of the partial sums are done

  // ---- representatives: fp32 means of the original rows of every group, in
  // rowlist order (fixed), so the result is deterministic
  {
    const int p0 = up * RP;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int lo = max(p0, off_s[g]), hi = min(r1, off_s[g] + cnt_s[g]);
      float acc = 0.f;
      const T* rcol = &rows[0][0] + uj;
#pragma unroll 4
      for (int x = lo; x < hi; ++x) acc += Stage<BF16>::get(rcol[__umul24(rowlist[x], LD)]);
      part.fsum[(up * G + g) * D + uj] = acc;
    }
  }
  __syncthreads();
  if (tid < D) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int c = cnt_s[g];
      float sum = 0.f;
#pragma unroll
      for (int x = 0; x < PARTS; ++x) sum += part.fsum[(x * G + g) * D + tid];
      cout[g * D + tid] = c > 0 ? sum / static_cast<float>(c) : 0.f;
    }
  }
  if (tid < G) sout[tid] = cnt_s[tid];
}

}  // namespace

hipError_t launch_block_clusters(const Geometry& g, int groups, int iters, const void* q,
                                 const int32_t* perm, float* q_cent, int32_t* q_size, hipStream_t s) {
  ClusterArgs a;
  a.q = q;
  a.perm = perm;
  a.q_cent = q_cent;
  a.q_size = q_size;
  a.N = g.N;
  a.N_pad = g.N_pad;
  a.nQB = g.nQB;
  a.iters = iters;
  const dim3 grid(g.B * g.H * g.nQB), block(CL_THREADS);
  const bool p = perm != nullptr;
#define BSA_CL(D, BQ, G, BF, P) hipLaunchKernelGGL((block_clusters_kernel<D, BQ, G, BF, P>), grid, block, 0, s, a)
#define BSA_CL_P(D, BQ, G, BF) \
  if (p) BSA_CL(D, BQ, G, BF, true); else BSA_CL(D, BQ, G, BF, false)
#define BSA_CL_T(D, BQ, G) \
  if (g.bf16) { BSA_CL_P(D, BQ, G, true); } else { BSA_CL_P(D, BQ, G, false); }
#define BSA_CL_G(D, BQ)                                   \
  switch (groups) {                                       \
    case 1: BSA_CL_T(D, BQ, 1) break;                     \
    case 2: BSA_CL_T(D, BQ, 2) break;                     \
    case 4: BSA_CL_T(D, BQ, 4) break;                     \
    case 8: BSA_CL_T(D, BQ, 8) break;                     \
    default: return hipErrorInvalidValue;                 \
  }
  if (g.d == 128) {
    if (g.block_q == 128) { BSA_CL_G(128, 128) } else { BSA_CL_G(128, 64) }
  } else {
    if (g.block_q == 128) { BSA_CL_G(64, 128) } else { BSA_CL_G(64, 64) }
  }
#undef BSA_CL_G
#undef BSA_CL_T
#undef BSA_CL_P
#undef BSA_CL
  return hipGetLastError();
}

}  // namespace bsa
