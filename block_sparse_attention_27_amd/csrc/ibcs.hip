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
// staged once in LDS in their input type, next to their fixed-point copies
// held as f16 (every integer of magnitude up to 2^11 is exact in f16). The two
// contractions of an iteration run on the matrix cores, exactly:
//   * the inner products <q, c_g> on f16 MFMA, once with the low six bits of
//     every centroid entry (c & 63) and once with the rest (c >> 6): each
//     partial sum is an integer below 2^24 in magnitude, so the fp32
//     accumulator holds it exactly, and <q, c> = 64 high + low in int32;
//   * the centroid sums as a one-hot (groups x rows) matrix times the
//     fixed-point rows on f16 MFMA (sums below 2^18: exact).
// The nearest centroid minimises |c|^2 - 2 <q, c>, the squared distance less
// the row's own |q|^2. The final fp32 means of bf16 rows are the one-hot matrix
// times the rows on bf16 MFMA with fp32 sums in a fixed order, so the output
// is deterministic; fp32 rows take a plain loop in row order.
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

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
#define BSA_LDS __attribute__((address_space(3)))

// Operand layouts of v_mfma_f32_32x32x16_{f16,bf16} (64 lanes, l = lane,
// n = l % 32, h = l / 32): A (32 x 16) lane l holds A[n][8 h + e], B (16 x 32)
// holds B[8 h + e][n], e = 0..7; accumulator register r holds C[8 (r/4) +
// 4 h + r%4][n].
//
// Eight values of one column over rows of a row-major 16-bit LDS array come
// from two ds_read_b64_tr_b16: in each 16-lane group, lane q gives the address
// of row q / 4, columns 4 (q % 4) .. +3 of a 4 x 16 block and receives column q
// of it (4 rows). Lane l thus gets rows r0 + 4 h + {0..3} and r0 + 8 + 4 h +
// {0..3} of column c0 + n: element e of the operand is row
// r0 + (e < 4 ? 4 h + e : 8 + 4 h + e - 4), and the other operand of the
// product uses the same row order.
template <int LDE>
__device__ __forceinline__ u32x4 column8(const uint16_t* base, int r0, int c0, int lane) {
  const int q = lane % 16, g2 = (lane / 16) % 2, h = lane / 32;
  const uint16_t* p = base + (r0 + 4 * h + q / 4) * LDE + c0 + 16 * g2 + 4 * (q % 4);
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((BSA_LDS i16x4*)(p));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((BSA_LDS i16x4*)(p + 8 * LDE));
  const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
  return u32x4{ua[0], ua[1], ub[0], ub[1]};
}

// The matching eight entries of one row of a row-major 16-bit array: columns
// r0 + 4 h + {0..3} and r0 + 8 + 4 h + {0..3} (zero when the row is absent).
__device__ __forceinline__ u32x4 row8_tr_order(const uint16_t* row, int r0, int lane, bool present) {
  const int h = lane / 32;
  const u32x2 a = *reinterpret_cast<const u32x2*>(row + r0 + 4 * h);
  const u32x2 b = *reinterpret_cast<const u32x2*>(row + r0 + 8 + 4 * h);
  return present ? u32x4{a[0], a[1], b[0], b[1]} : u32x4{0u, 0u, 0u, 0u};
}

// Wave-wide sum and maximum on DPP moves (no LDS round trip): two quad
// swaps, the half-row mirror and the row mirror leave every lane of a 16-lane
// row with the row's result; the four rows are combined in scalar registers.
__device__ __forceinline__ int dpp_row_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1, 0, 3, 2]
  v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2, 3, 0, 1]
  v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
  v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);  // row_mirror
  return v;
}
__device__ __forceinline__ int wave_sum(int v) {
  v = dpp_row_sum(v);
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) + __builtin_amdgcn_readlane(v, 32) +
         __builtin_amdgcn_readlane(v, 48);
}
template <int CTRL>
__device__ __forceinline__ float dpp_max(float v) {
  return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false)));
}
__device__ __forceinline__ float wave_max(float v) {
  v = dpp_max<0x140>(dpp_max<0x141>(dpp_max<0x4E>(dpp_max<0xB1>(v))));
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

template <int D, int BQ, int G, bool BF16, bool PERM>
__global__ __launch_bounds__(CL_THREADS, BF16 ? (G <= 4 ? 6 : 5) : 1) void block_clusters_kernel(ClusterArgs a) {
  typedef typename Stage<BF16>::T T;
  constexpr int ESZ = sizeof(T);
  constexpr int EPC = 16 / ESZ;              // elements per 16-byte chunk
  constexpr int CH = D / EPC;                // chunks per row
  constexpr int RPP = CL_THREADS / CH;       // rows staged per pass
  constexpr int MAXP = BQ / RPP;             // staging passes for a full block
  constexpr int LR = D + EPC;                // padded staged row (elements)
  constexpr int LQ = D + 8;                  // padded fixed-point row (f16)
  constexpr int LO = BQ + 8;                 // padded one-hot row
  constexpr int NWV = CL_THREADS / 64;       // waves
  constexpr int MT = BQ / 32;                // distance products: row tiles (x {low, high} parts)
  constexpr int NT = D / 32;                 // sums: column tiles
  constexpr int SPL = NWV / NT;              // sums: waves per column tile (row ranges)
  constexpr int KPW = BQ / 16 / SPL;         // sums: 16-row steps per wave
  constexpr int PARTS = CL_THREADS / D;      // fp32 means: row ranges
  constexpr int RP = BQ / PARTS;             // fp32 means: rows per range
  constexpr int LP = BQ + 1;                 // inner products: [part][group][row], padded rows
  constexpr int NPART_A = 2 * G * LP > SPL * G * D ? 2 * G * LP : SPL * G * D;
  constexpr int NPART = (!BF16 && PARTS * G * D > NPART_A) ? PARTS * G * D : NPART_A;
  static_assert(2 * MT <= NWV && KPW >= 1 && SPL * KPW * 16 == BQ && D % 32 == 0 && D <= 128, "tiling");
  static_assert(G <= 8, "one-hot rows of at most 8 groups sit in registers 0..3 of both lane halves");

  // fp32 rows stay in LDS for the final means; bf16 rows are read again from
  // global memory there (the block was just read: L2), which leaves room for
  // three workgroups per CU (six waves per SIMD: the bound above; eight groups
  // take five, two workgroups)
  __shared__ __align__(16) T rows[BF16 ? 1 : BQ][LR];  // the block's rows (zero past n)
  __shared__ int grow[BQ];                            // global row of every block row (-1: none)
  __shared__ __align__(16) _Float16 qh[BQ][LQ];       // fixed-point rows as exact f16 integers
  __shared__ __align__(16) _Float16 chl[2][G][D];     // centroid parts: c & 63 and c >> 6
  __shared__ short ci[G][D];                          // fixed-point centroids
  __shared__ __align__(16) _Float16 ohh[G][LO];       // one-hot of the assignment (f16)
  __shared__ __align__(16) uint16_t ohb[BF16 ? G : 1][LO];  // the same as bf16 bits
  __shared__ int lab[BF16 ? 1 : BQ];                  // group of each row (fp32 means)
  __shared__ int cc2[G];                              // |c_int|^2 per centroid
  __shared__ __align__(16) float part[NPART];         // inner products / partial sums
  constexpr int NW = (BQ + 63) / 64;                  // waves that hold rows in the assignment step
  __shared__ int wcnt[NW][G];
  __shared__ float wmax[NWV];

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64, ln = lane % 32, lh = lane / 32;
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

  // ---- stage the rows (all loads in flight at once; zeros past n); largest magnitude
  const char* base = static_cast<const char*>(a.q) + static_cast<size_t>(bh) * a.N_pad * D * ESZ;
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
    if (cc == 0) grow[r] = ok ? gr : -1;
  }
  float mx = 0.f;
#pragma unroll
  for (int pp = 0; pp < MAXP; ++pp) {
    const int r = rg + pp * RPP;
    if constexpr (!BF16) *reinterpret_cast<u32x4*>(&rows[r][cc * EPC]) = xr[pp];
    const T* xv = reinterpret_cast<const T*>(&xr[pp]);
#pragma unroll
    for (int z = 0; z < EPC; ++z) mx = fmaxf(mx, fabsf(Stage<BF16>::get(xv[z])));
  }
  mx = wave_max(mx);
  if (lane == 0) wmax[wave] = mx;
  __syncthreads();  // per-wave maxima ready
  mx = wmax[0];
#pragma unroll
  for (int x = 1; x < NWV; ++x) mx = fmaxf(mx, wmax[x]);
  int ex = 0;
  frexpf(mx, &ex);  // a block of zeros (mx = 0) keeps ex = 0: any shift leaves its zeros
  const int sh = FIXED_BITS - ex;

  // ---- fixed-point copies: x 2^sh is exact and rint rounds it to the nearest
  // integer (ties to even); |q_int| <= 2^11 is exact in f16
#pragma unroll
  for (int pp = 0; pp < MAXP; ++pp) {
    const int r = rg + pp * RPP;
    const T* xv = reinterpret_cast<const T*>(&xr[pp]);
#pragma unroll
    for (int z = 0; z < EPC; ++z) qh[r][cc * EPC + z] = static_cast<_Float16>(__builtin_rintf(ldexpf(Stage<BF16>::get(xv[z]), sh)));
  }
  __syncthreads();  // rows and fixed-point rows ready
  for (int x = tid; x < G * D; x += CL_THREADS) {
    const int g = x / D, d = x % D;
    const int c = static_cast<int>(static_cast<float>(qh[(g * n) / G][d]));
    ci[g][d] = static_cast<short>(c);
    chl[0][g][d] = static_cast<_Float16>(c & 63);
    chl[1][g][d] = static_cast<_Float16>(c >> 6);
  }
  if (tid < G) cc2[tid] = 0;
  __syncthreads();
  // |c_int|^2 of every centroid: column tid of each, summed per wave, then across waves
  auto centroid_squares = [&]() {
    if (tid < D) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int c = ci[g][tid];
        const int v = wave_sum(c * c);  // whole waves: D is a multiple of 64
        if (lane == 0) atomicAdd(&cc2[g], v);
      }
    }
  };
  centroid_squares();

  int cnt[G];  // group sizes of the last assignment
  for (int it = 0; it < a.iters; ++it) {
    __syncthreads();  // centroids, their parts and |c|^2 ready
    // ---- inner products <q, c_g> on f16 MFMA, once with the low and once with
    // the high centroid part: every partial sum is an integer below 2^24 in
    // magnitude (128 x 2^11 x 63 and 128 x 2^11 x 32), so fp32 holds it exactly
    if (wave < 2 * MT) {
      const int mt = wave % MT, pt = wave / MT;
      const bool gok = ln < G;
      const _Float16* ar = &qh[32 * mt + ln][8 * lh];
      const _Float16* br = &chl[pt][gok ? ln : 0][8 * lh];
      f32x16 acc = {};
      // operands of two steps are read before their products: one LDS round trip per two MFMAs
      constexpr int KB = 2;
#pragma unroll
      for (int k0 = 0; k0 < D / 16; k0 += KB) {
        u32x4 au[KB], bu[KB];
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) {
          au[kk] = *reinterpret_cast<const u32x4*>(ar + 16 * (k0 + kk));
          bu[kk] = *reinterpret_cast<const u32x4*>(br + 16 * (k0 + kk));
        }
#pragma unroll
        for (int kk = 0; kk < KB; ++kk)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, au[kk]),
                                                       __builtin_bit_cast(f16x8, gok ? bu[kk] : u32x4{0u, 0u, 0u, 0u}),
                                                       acc, 0, 0, 0);
      }
      if (gok) {
#pragma unroll
        for (int r = 0; r < 16; ++r) part[(pt * G + ln) * LP + 32 * mt + 8 * (r / 4) + 4 * lh + r % 4] = acc[r];
      }
    }
    __syncthreads();  // inner products ready
    // ---- assignment: |q - c|^2 = |q|^2 + |c|^2 - 2 <q, c>, and |q|^2 is the
    // same for every group, so the nearest centroid minimises |c|^2 - 2 <q, c>
    // (exact in int32: |c|^2 <= 2^29, |<q, c>| <= 2^29); ties keep the lower group
    if (tid < 64 * NW) {  // whole waves
      int myl = G;
      if (tid < n) {
        int best = 0;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const int ip = 64 * static_cast<int>(part[(G + g) * LP + tid]) + static_cast<int>(part[g * LP + tid]);
          const int sc = cc2[g] - 2 * ip;
          if (g == 0 || sc < best) {
            best = sc;
            myl = g;
          }
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const uint64_t m = __ballot(myl == g);
        if (lane == 0) wcnt[wave][g] = __popcll(m);
      }
      if (tid < BQ) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          ohh[g][tid] = static_cast<_Float16>(myl == g ? 1.f : 0.f);
          if constexpr (BF16) ohb[g][tid] = myl == g ? 0x3F80u : 0u;
        }
        if constexpr (!BF16) lab[tid] = myl;
      }
    }
    __syncthreads();  // one-hot rows and counts ready; the assignment's reads of |c|^2 are done
    if (tid < G) cc2[tid] = 0;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      cnt[g] = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) cnt[g] += wcnt[w][g];
    }
    // ---- centroid sums on f16 MFMA: one-hot (groups x rows) times the
    // fixed-point rows; sums stay below 2^18 in magnitude, exact in fp32.
    // Wave w: columns 32 (w % NT) .., rows 16 KPW (w / NT) ..
    {
      const int nt = wave % NT, kp = wave / NT;
      const bool gok = ln < G;
      f32x16 acc = {};
#pragma unroll
      for (int kk = 0; kk < KPW; ++kk) {
        const int r0 = 16 * (kp * KPW + kk);
        const u32x4 au = row8_tr_order(reinterpret_cast<const uint16_t*>(&ohh[gok ? ln : 0][0]), r0, lane, gok);
        const u32x4 bu = column8<LQ>(reinterpret_cast<const uint16_t*>(&qh[0][0]), r0, 32 * nt, lane);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, au), __builtin_bit_cast(f16x8, bu), acc,
                                                     0, 0, 0);
      }
      // register r holds group 8 (r/4) + 4 lh + r % 4: groups below 8 are in registers 0..3
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int g = 4 * lh + r;
        if (g < G) part[(kp * G + g) * D + 32 * nt + ln] = acc[r];
      }
    }
    __syncthreads();  // partial sums ready
    if (tid < D) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int c = cnt[g];
        if (c > 0) {
          float fs = 0.f;
#pragma unroll
          for (int x = 0; x < SPL; ++x) fs += part[(x * G + g) * D + tid];
          const int sum = static_cast<int>(fs);
          // rounded mean, halves up: floor((2 s + c) / (2 c)). The exact quotient is
          // k + f / (2c) with f an integer, so (num + 1/2) / (2c) sits at least 1/512
          // inside [k, k + 1); its fp32 value (|num| < 2^20, one rcp and one multiply)
          // is within 4e-4 of it, and the floor is exact.
          const int num = 2 * sum + c;
          const float y = (static_cast<float>(num) + 0.5f) * __builtin_amdgcn_rcpf(static_cast<float>(2 * c));
          const int cn = static_cast<int>(floorf(y));
          ci[g][tid] = static_cast<short>(cn);
          chl[0][g][tid] = static_cast<_Float16>(cn & 63);
          chl[1][g][tid] = static_cast<_Float16>(cn >> 6);
        }
      }
    }
    centroid_squares();  // each column is read by the thread that wrote it
    // the next iteration's first barrier publishes the centroids and their squares
  }
  __syncthreads();  // the last update's reads of the partial sums are done

  // ---- representatives: fp32 means of the original rows of every group
  if constexpr (BF16) {
    // one-hot times the bf16 rows on MFMA with fp32 sums (a fixed order:
    // deterministic). The rows are read again (the block was read at the
    // start: L2) with the staging's 16-byte loads into the fixed-point rows'
    // LDS, free after the last iteration, and the B operand of a 16-row step
    // (column 32 nt + n of rows r0 + {4 h .. 4 h + 3, 8 + 4 h .. 8 + 4 h + 3},
    // the row order of the one-hot operand) comes from the transposing reads
    // of the centroid sums.
    uint16_t* rb = reinterpret_cast<uint16_t*>(&qh[0][0]);
#pragma unroll
    for (int pp = 0; pp < MAXP; ++pp) {
      const int r = rg + pp * RPP;
      const int gr = grow[r];
      const u32x4 x = gr >= 0 ? *reinterpret_cast<const u32x4*>(base + (static_cast<size_t>(gr) * D + cc * EPC) * ESZ)
                              : u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(rb + r * LQ + cc * EPC) = x;
    }
    __syncthreads();  // the rows are staged
    const int nt = wave % NT, kp = wave / NT;
    const bool gok = ln < G;
    f32x16 acc = {};
#pragma unroll
    for (int kk = 0; kk < KPW; ++kk) {
      const int r0 = 16 * (kp * KPW + kk);
      const u32x4 au = row8_tr_order(&ohb[gok ? ln : 0][0], r0, lane, gok);
      const u32x4 bu = column8<LQ>(rb, r0, 32 * nt, lane);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, au), __builtin_bit_cast(bf16x8, bu), acc,
                                                    0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int g = 4 * lh + r;
      if (g < G) part[(kp * G + g) * D + 32 * nt + ln] = acc[r];
    }
    __syncthreads();
    if (tid < D) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float sum = 0.f;
#pragma unroll
        for (int x = 0; x < SPL; ++x) sum += part[(x * G + g) * D + tid];
        cout[g * D + tid] = cnt[g] > 0 ? sum / static_cast<float>(cnt[g]) : 0.f;
      }
    }
  } else {
    // fp32 rows: thread (column uj, rows [up RP, up RP + RP)) walks its rows in order
    const int uj = tid % D, up = tid / D;
    float acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = 0.f;
    for (int r = up * RP; r < min(n, up * RP + RP); ++r) {
      const float x = Stage<BF16>::get(rows[r][uj]);
      const int l = lab[r];
#pragma unroll
      for (int g = 0; g < G; ++g) acc[g] += l == g ? x : 0.f;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) part[(up * G + g) * D + uj] = acc[g];
    __syncthreads();
    if (tid < D) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float sum = 0.f;
#pragma unroll
        for (int x = 0; x < PARTS; ++x) sum += part[(x * G + g) * D + tid];
        cout[g * D + tid] = cnt[g] > 0 ? sum / static_cast<float>(cnt[g]) : 0.f;
      }
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
