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
// One workgroup (256 threads) per (b, h, query block). The block's rows are
// staged once in LDS in their input type, next to their 16-bit fixed-point
// copies. A distance is |q|^2 + |c|^2 - 2 <q, c> with the inner product on
// v_dot2_i32_i16 (two dimensions per instruction, exact); TPR threads share a
// row and every centroid read is an LDS broadcast. The centroid sums are
// integer LDS atomics (exact, so their order does not matter); the final fp32
// means use a fixed order, so the output is deterministic.
#include "bsa_internal.hpp"

namespace bsa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int CL_THREADS = 256;

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
  __shared__ int sums[G][D];                    // centroid sums (atomics)
  __shared__ int qq[BQ];                        // |q_int|^2 per row
  __shared__ int ccp[TPR][G];                   // |c_int|^2 per distance part
  __shared__ union {
    int ip[NPART];       // partial inner products
    float fsum[NPART];   // partial sums of the original values
  } part;
  __shared__ int lab[BQ];
  __shared__ int cnt[G];
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

  // ---- fixed-point copies (|q_int| <= 2^11) from the staged registers
#pragma unroll
  for (int pp = 0; pp < MAXP; ++pp) {
    const int r = rg + pp * RPP;
    if (r < n) {
      const T* xv = reinterpret_cast<const T*>(&xr[pp]);
      short v[EPC];
#pragma unroll
      for (int z = 0; z < EPC; ++z) v[z] = static_cast<short>(__float2int_rn(ldexpf(Stage<BF16>::get(xv[z]), sh)));
#pragma unroll
      for (int z = 0; z < EPC; ++z) qi[r][cc * EPC + z] = v[z];
    }
  }
  __syncthreads();  // rows and fixed-point rows ready
  for (int x = tid; x < G * D; x += CL_THREADS) ci[x / D][x % D] = qi[((x / D) * n) / G][x % D];

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

  for (int it = 0; it < a.iters; ++it) {
    if (tid < G) cnt[tid] = 0;
    for (int x = tid; x < G * D; x += CL_THREADS) sums[x / D][x % D] = 0;
    __syncthreads();  // centroids and |q|^2 ready; counts and sums cleared
    {
      int acc[G], cacc[G];
#pragma unroll
      for (int g = 0; g < G; ++g) acc[g] = cacc[g] = 0;
#pragma unroll
      for (int e = 0; e < DP; e += 8) {
        const int j0 = dp * DP + e;
        const i32x4 x = *reinterpret_cast<const i32x4*>(&qi[dr][j0]);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const i32x4 c = *reinterpret_cast<const i32x4*>(&ci[g][j0]);  // broadcast
          acc[g] = dot8(x, c, acc[g]);
          cacc[g] = dot8(c, c, cacc[g]);
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) part.ip[(dp * BQ + dr) * G + g] = acc[g];
      if (dr == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) ccp[dp][g] = cacc[g];
      }
    }
    __syncthreads();  // partial inner products ready
    if (tid < n) {
      uint32_t best = 0u;
      int bg = 0;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        int ip = 0, cc = 0;
#pragma unroll
        for (int x = 0; x < TPR; ++x) {
          ip += part.ip[(x * BQ + tid) * G + g];
          cc += ccp[x][g];
        }
        // |q - c|^2 in [0, 2^31]: exact in unsigned 32-bit arithmetic
        const uint32_t d2 = static_cast<uint32_t>(qq[tid]) + static_cast<uint32_t>(cc) - 2u * static_cast<uint32_t>(ip);
        if (g == 0 || d2 < best) {  // strict: ties keep the lower group
          best = d2;
          bg = g;
        }
      }
      lab[tid] = bg;
      atomicAdd(&cnt[bg], 1);
    }
    __syncthreads();  // labels and counts ready
#pragma unroll 8
    for (int r = up * RP; r < r1; ++r) atomicAdd(&sums[lab[r]][uj], static_cast<int>(qi[r][uj]));
    __syncthreads();  // sums ready
    if (tid < D) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int c = cnt[g];
        if (c > 0) {
          // rounded mean, halves up: floor((2 s + c) / (2 c)) with a floored division
          const int num = 2 * sums[g][tid] + c, den = 2 * c;
          int qv = num / den;
          if (num % den != 0 && num < 0) --qv;
          ci[g][tid] = static_cast<short>(qv);
        }
      }
    }
    __syncthreads();  // centroids moved
  }

  // ---- representatives: fp32 means of the original rows of every group
  {
    float acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = 0.f;
#pragma unroll 8
    for (int r = up * RP; r < r1; ++r) {
      const float x = Stage<BF16>::get(rows[r][uj]);
      const int l = lab[r];
#pragma unroll
      for (int g = 0; g < G; ++g) acc[g] += l == g ? x : 0.f;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) part.fsum[(up * G + g) * D + uj] = acc[g];
  }
  __syncthreads();
  if (tid < D) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int c = cnt[g];
      float s = 0.f;
#pragma unroll
      for (int x = 0; x < PARTS; ++x) s += part.fsum[(x * G + g) * D + tid];
      cout[g * D + tid] = c > 0 ? s / static_cast<float>(c) : 0.f;
    }
  }
  if (tid < G) sout[tid] = cnt[tid];
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
