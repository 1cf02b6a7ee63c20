/*
 * bsa.h -- weighted dynamic block-sparse attention for video DiTs on AMD
 * Instinct MI355X (gfx950). C ABI of libbsa.so.
 *
 * The method (InstaGen, "Group-Shared Importance Sampling for Fast Video
 * Generation", Abstract; AB-Attention, "Accurate Block Attention", Abstract
 * and the transcript's sections on inclusion-probability sampling and the
 * tiled kernel): every query block scores the key blocks from block summaries,
 * keeps the top-scoring ones as an exact set, draws a fixed-size sample of
 * the rest with chances that follow the estimated attention, and runs one sparse
 * attention pass in which every sampled block is reweighted by the inverse of
 * its inclusion probability in both the softmax numerator and denominator.
 *
 * Pipeline: bsa_score (or bsa_score_ibcs, bsa_score_stats) -> bsa_select ->
 * bsa_attend.
 * bsa_attend_dense is plain dense attention built on the same tiling, for
 * timing and checking.
 *
 * Conventions shared by every call
 *   Layout     Q, K, V and out are contiguous row-major [B][H][N_pad][d]
 *              (element type `dtype`); S is [B][H][nQB][nKU] fp32; idx and w
 *              are [B][H][nQB][k_exact + m_sample] (int32 / fp32); lse is
 *              [B][H][N_pad] fp32. nQB = N_pad / block_q, nKU = N_pad / block_k.
 *   Validity   Rows r < N are tokens, rows N..N_pad-1 are padding. Padding rows
 *              of Q, K and V are never read (their contents do not matter);
 *              padding rows of out are written as zeros and their lse as -inf.
 *              Key unit j holds keys [j*block_k, (j+1)*block_k) and is valid
 *              when j*block_k < N; a partly filled tail unit uses only its
 *              keys below N.
 *   Permutation perm, when not NULL, is int32[N_pad] on the device: the
 *              computation runs on the gathered rows X'[r] = X[perm[r]] for
 *              Q, K and V alike, and row r of the result is written to row
 *              perm[r] of out (and lse). perm must map 0..N-1 onto 0..N-1;
 *              entries r >= N are not read. An entry outside [0, N_pad) is
 *              never dereferenced (no out-of-bounds access) but the result is
 *              then unspecified. With kv_permuted = 1 the caller passes K and
 *              V already gathered (K' and V', as bsa_permute_rows writes
 *              them) and only Q and out go through perm; the results are the
 *              same, and the sparse pass reads each key unit as one run of
 *              contiguous rows instead of gathering it row by row.
 *   Memory     All array arguments are device pointers owned by the caller;
 *              Q/K/V/out must be 16-byte aligned, the others 4-byte aligned.
 *              The library allocates nothing, keeps no state between calls and
 *              may be called from several host threads on different streams.
 *   Execution  Every call only enqueues work on `stream` and returns; the
 *              caller synchronises. Calls on one stream run in order.
 *   Errors     Invalid arguments return BSA_ERR_INVALID_ARG before anything is
 *              launched; shapes the kernels do not implement return
 *              BSA_ERR_UNSUPPORTED; a failed launch returns BSA_ERR_HIP.
 *              Faults inside a kernel surface at the caller's synchronisation.
 */
#ifndef BSA_H
#define BSA_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BSA_ABI_VERSION 7

typedef enum bsa_status {
  BSA_OK = 0,
  BSA_ERR_INVALID_ARG = 1,
  BSA_ERR_UNSUPPORTED = 2,
  BSA_ERR_HIP = 3
} bsa_status;

typedef enum bsa_dtype {
  BSA_BF16 = 0, /* bfloat16 Q/K/V/out, bf16 MFMA with fp32 accumulation */
  BSA_FP32 = 1  /* float Q/K/V/out, fp32 arithmetic throughout */
} bsa_dtype;

/* The problem statement shared by all calls (InstaGen, Abstract: Q/K/V, a
 * block size, an exact-set size, a sample size and a random seed). */
typedef struct bsa_problem {
  int32_t B, H;       /* batch, heads (>= 1) */
  int32_t N;          /* valid tokens, 1 <= N <= N_pad */
  int32_t N_pad;      /* padded rows; a multiple of block_q and of block_k */
  int32_t d;          /* head dimension: 64 or 128 */
  int32_t block_q;    /* query-block rows: 64 or 128 */
  int32_t block_k;    /* key-unit rows: 32, 64 or 128 (4, 2 or 1 per 128-key tile) */
  int32_t k_exact;    /* exact-set size k >= 0 */
  int32_t m_sample;   /* sample size m >= 0; 1 <= k+m <= number of valid units */
  int32_t dtype;      /* bsa_dtype of Q, K, V */
  int32_t out_fp32;   /* 0: out has the element type of Q; 1: out is fp32 (always fp32 for BSA_FP32) */
  int32_t kv_permuted; /* 0: K and V in token order; 1: K and V given as K' = K[perm],
                          V' = V[perm] (needs perm in every call that takes one) */
  uint64_t seed;      /* sampler seed (Philox4x32-10 key) */
  float sm_scale;     /* logit = sm_scale * <q, k>; finite and > 0 */
} bsa_problem;

/* Returns BSA_ABI_VERSION. */
int32_t bsa_abi_version(void);

/* Static text for a bsa_status value (never NULL). */
const char* bsa_status_string(int32_t status);

/*
 * bsa_score -- block summaries and estimated attention per key unit.
 * (AB-Attention, Abstract: key blocks rated from cheap per-block summaries;
 * InstaGen, Abstract: the sampling chance of a block follows its estimated
 * share of attention.)
 *
 *   q_mean[b,h,i,:] = mean of the valid rows of query block i      (fp32, out)
 *   k_mean[b,h,j,:] = mean of the n_j valid keys of unit j          (fp32, out)
 *   S[b,h,i,j] = n_j exp(l_ij) / sum_{valid j'} n_j' exp(l_ij'),
 *       l_ij = sm_scale <q_mean_i, k_mean_j>;  S = 0 for invalid units.
 * A query block with no valid row has q_mean = 0. Uses q, k (dtype), perm
 * (optional, see above). q_mean is [B][H][nQB][d], k_mean [B][H][nKU][d];
 * both are written (the caller owns them; 16-byte aligned). One head's key
 * means are read as one 32-bit-addressed range: nKU * d * 4 above 2^31 - 1
 * bytes (more than 4,194,303 key units at d = 128) gives BSA_ERR_UNSUPPORTED,
 * here and in bsa_score_stats and bsa_score_ibcs.
 */
bsa_status bsa_score(const bsa_problem* p, const void* q, const void* k, const int32_t* perm,
                     float* S, float* q_mean, float* k_mean, hipStream_t stream);

/*
 * bsa_score_ibcs -- the same score matrix from several representatives per
 * query block: intra-block query clustering. (AB-Attention, Abstract: the
 * Intra-Block Clustering Selector clusters queries only within each query
 * block, without permuting tokens; transcript, the passage on choosing
 * blocks: every group of similar queries gets a representative and a weight
 * from its size, and the representatives score the key blocks.)
 *
 * Per query block with n > 0 valid rows, Lloyd's k-means with `groups`
 * groups and `iters` iterations on fixed-point copies of the rows, so that
 * every assignment is an exact integer decision:
 *   q_int = rint(q 2^s) (nearest, ties to even), s = 11 - e, where the
 *       block's largest |q| is f 2^e with f in [0.5, 1); |q_int| <= 2^11;
 *   initial centroid g = q_int of row floor(g n / groups) of the block (after
 *       the optional gather);
 *   each iteration assigns every row to the centroid at the smallest exact
 *       integer squared distance (ties: lower group), then moves every
 *       non-empty group's centroid to floor((2 sum + n_g) / (2 n_g)), the
 *       rounded mean of its rows' q_int (an empty group keeps its centroid).
 * q_cent is the mean of the members' original values after the last
 * assignment (fp32), and n_g the group's row count. Then
 *   S[b,h,i,j] = sum_g (n_g / n) n_j exp(l_gj) / sum_{valid j'} n_j' exp(l_gj'),
 *       l_gj = sm_scale <q_cent_ig, k_mean_j>;  S = 0 for invalid units.
 * Group sizes are reproducible bit for bit. They equal those of plain fp64
 * Lloyd k-means on the raw rows (same start, same iterations) whenever every
 * assignment's distance margin exceeds the rounding bound
 * 6 e sqrt(d D) + 9 e^2 d, e = 2^-(s+1); where the margins are smaller the two
 * readings can group a row differently.
 * A query block with no valid row scores like bsa_score's (one zero
 * representative, weight 1) and reports zero centroids and sizes. With
 * groups = 1 the result is bsa_score's.
 *   groups    1, 2, 4 or 8;  iters  1..16 (else BSA_ERR_INVALID_ARG)
 *   q_cent    [B][H][nQB][groups][d] fp32, out (16-byte aligned)
 *   q_size    [B][H][nQB][groups] int32, out: rows per group, n_g
 *   k_mean    [B][H][nKU][d] fp32, out, as in bsa_score
 */
bsa_status bsa_score_ibcs(const bsa_problem* p, int32_t groups, int32_t iters, const void* q, const void* k,
                          const int32_t* perm, float* S, float* q_cent, int32_t* q_size, float* k_mean,
                          hipStream_t stream);

/*
 * bsa_score_stats -- statistics-aware scoring of the key units. (Veda,
 * Abstract: tile selection as reconstruction of full attention, with
 * statistics-aware tile scoring.) Each key unit is scored by the attention
 * mass its keys would get if they were Gaussian with the unit's per-dimension
 * mean and variance:
 *   k_var[b,h,j,:] = population variance of the n_j valid keys of unit j   (fp32, out)
 *   l_ij = s <q_mean_i, k_mean_j> + (s^2 / 2) <q_mean_i^2, k_var_j>,  s = sm_scale,
 *   S[b,h,i,j] = n_j exp(l_ij) / sum_{valid j'} n_j' exp(l_ij');  S = 0 for invalid units.
 * A unit of identical keys scores as in bsa_score. q_mean, k_mean as in
 * bsa_score; k_var is [B][H][nKU][d] (16-byte aligned).
 */
bsa_status bsa_score_stats(const bsa_problem* p, const void* q, const void* k, const int32_t* perm, float* S,
                           float* q_mean, float* k_mean, float* k_var, hipStream_t stream);

/*
 * bsa_select -- exact set plus fixed-size weighted sample, per (b, h, i).
 * (InstaGen, Abstract: exact set plus a weighted sample, one sample shared by
 * a query cluster; AB-Attention transcript: inclusion probabilities, a fixed
 * number of distinct blocks, and 1/pi weights -- probability 1/4 counts 4x.)
 *
 * For each row of S (only the valid units 0..ceil(N/block_k)-1 are read):
 *   1. exact set: the k valid units with the largest score (ties: lower
 *      index); NaN, zero and negative scores count as 0, +inf as FLT_MAX;
 *   2. the other valid units R get inclusion probabilities
 *      pi_j = min(1, c s_j) with sum_R pi_j = m, computed bit-reproducibly:
 *      scores quantised to 20-bit integers relative to the row maximum
 *      (minimum 1), exact integer water-filling for c, pi in 32-bit fixed
 *      point summing to exactly m * 2^32;
 *   3. systematic sampling over R in ascending unit order with offset
 *      u = word 0 of Philox4x32-10(counter = (i, h, b, 0),
 *      key = (seed & 0xffffffff, seed >> 32)) gives exactly m distinct units.
 * Output row: idx[0..k) = exact set ascending, w = 1; idx[k + s] = the unit
 * drawn by the s-th sample point, w = fp32(2^32 / pi_int) (1 for units with
 * pi = 1). Results are bit-identical to the reference definition for any
 * input S. Needs ceil(N/block_k) <= 4096.
 */
bsa_status bsa_select(const bsa_problem* p, const float* S, int32_t* idx, float* w,
                      hipStream_t stream);

/*
 * bsa_permute_rows -- x_perm[b][h][r] = x[b][h][perm[r]] for r < N; rows
 * N .. N_pad-1 of x_perm are written as zeros, and so is a row whose perm
 * entry lies outside [0, N_pad).
 * (InstaGen, Abstract: permuted block-sparse attention computes blocks of an
 * attention matrix whose tokens have been reordered by semantic similarity.)
 * Puts K and V into the permuted order once, for calls with kv_permuted = 1.
 * x and x_perm are [B][H][N_pad][d] of `dtype`, 16-byte aligned device
 * buffers owned by the caller, and must not overlap; perm is required. Uses B,
 * H, N, N_pad, d and dtype of p (the other fields are checked as in every
 * call but not used). A pure copy of bytes: bit-exact. Errors: a null or
 * misaligned pointer, a missing perm or overlapping buffers give
 * BSA_ERR_INVALID_ARG; more than 2^31 - 1024 16-byte chunks per (b, h), or a
 * grid beyond 2^32 work-items, give BSA_ERR_UNSUPPORTED.
 */
bsa_status bsa_permute_rows(const bsa_problem* p, const void* x, const int32_t* perm, void* x_perm,
                            hipStream_t stream);

/*
 * bsa_attend -- one weighted block-sparse attention pass.
 * (AB-Attention, Abstract and transcript: the weights enter numerator and
 * denominator alike -- equivalently the sampled logits are shifted by ln w
 * before the softmax -- and small key blocks are gathered into full
 * matrix-core tiles; InstaGen, Abstract: sampled keys kept block-shaped.)
 *
 * For every valid query row r of block i, over the list entries (j, w_j) of
 * that block and the valid keys t of unit j, with a_rt = sm_scale <q_r, k_t>:
 *   out_r = sum_j w_j sum_t exp(a_rt) v_t / sum_j w_j sum_t exp(a_rt)
 *   lse_r = ln(sum_j w_j sum_t exp(a_rt))
 * The list is used as given (a repeated entry counts twice); entries with an
 * index outside [0, nKU) or a weight that is not a finite number > 0
 * contribute nothing. Any finite positive weight is accepted (the running
 * maximum of the online softmax is kept on the weighted logits, so no
 * intermediate exceeds 2^8 times the largest weighted term).
 * idx/w may come from bsa_select or from the caller (e.g. a plan reused across
 * denoising steps). lse may be NULL.
 * Output type and accuracy: out is fp32 when out_fp32 is 1 or dtype is
 * BSA_FP32, else bf16. For bf16 Q/K/V the fp32 output stays within 2e-3
 * relative L2 of the exact (fp64) result on the layers this library is
 * tested on (P is rounded to bf16 for the matrix cores: about 1.6e-3). A
 * bf16 out is that fp32 result rounded to nearest even, bit for bit; the
 * rounding adds about 1.7e-3 relative RMS of its own, so the bf16 output
 * measures about 2.3e-3 relative L2 against the exact result (bounded by
 * 2.5e-3 in the tests).
 */
bsa_status bsa_attend(const bsa_problem* p, const void* q, const void* k, const void* v,
                      const int32_t* perm, const int32_t* idx, const float* w, void* out,
                      float* lse, hipStream_t stream);

/*
 * bsa_attend_dense -- masked softmax(sm_scale Q K^T) V over the N valid keys,
 * same layouts, permutation, outputs and accuracy as bsa_attend (k_exact,
 * m_sample and seed are ignored). It is full self-attention, the baseline the
 * pages measure their sparse methods against (InstaGen, Abstract: speedup over
 * the dense model; AB-Attention, Abstract: the share of attention skipped),
 * and the limit the weighted pass reproduces when every valid unit is listed.
 * The timing and accuracy reference for the sparse pass.
 */
bsa_status bsa_attend_dense(const bsa_problem* p, const void* q, const void* k, const void* v,
                            const int32_t* perm, void* out, float* lse, hipStream_t stream);

/*
 * bsa_mfma_ceiling -- a measurement aid, not a step of the method: the
 * sustained rate of the bf16 matrix cores on this chip, against which the
 * attention kernels' rates can be read. Under a long matrix load the chip
 * runs well below its top clock, at or near its socket power limit, so the
 * published bf16 peak (at the top clock) is not reached even by a kernel that
 * does nothing else.
 *
 * Launches n_wg workgroups of 4 waves (two per CU, as bsa_attend's kernel);
 * every wave runs `iters` rounds of 8 independent v_mfma_f32_32x32x16_bf16 on
 * register operands, so the launch performs n_wg * 4 * iters * 8 * 32768
 * floating-point operations and touches memory only to write `out`.
 *   out  device, caller-owned, 4-byte aligned, n_wg * 256 floats: thread t of
 *        workgroup g writes out[g * 256 + t] = 8 iters sum_r C[i_r][l % 32],
 *        the sum of its accumulators, where lane l = t % 64 holds the A
 *        fragment a_e = bf16(0.001 (l + e)) and the B fragment
 *        b_e = bf16(0.002 (l - e)), e = 0..7, C = A B is their 32x32 product
 *        (A[i][k] from lane i + 32 (k / 8), element k % 8; B[k][j] from lane
 *        j + 32 (k / 8)), and i_r = 8 (r / 4) + 4 (l / 32) + r % 4.
 * Time the launch with events on `stream` and divide the operations by it.
 * Errors: out NULL or misaligned, iters < 1 or n_wg < 1 give
 * BSA_ERR_INVALID_ARG (nothing launched); a failed launch BSA_ERR_HIP.
 */
bsa_status bsa_mfma_ceiling(float* out, int32_t iters, int32_t n_wg, hipStream_t stream);

/*
 * bsa_mfma_ceiling_random -- the same measurement aid on data that changes
 * from one product to the next. A product's energy depends on how many
 * operand bits toggle, and at the power limit energy sets the clock, so
 * constant operands overstate what products over real data can sustain.
 *
 * Same launch and operation count as bsa_mfma_ceiling. Thread t of workgroup
 * g (n = 256 g + t, lane l = t % 64) holds four A fragments
 * a_f[e] = bf16(v(64 n + 8 f + e)) and four B fragments
 * b_f[e] = bf16(v(64 n + 32 + 8 f + e + l)), f = 0..3, e = 0..7, where v(x)
 * in [-2, 2) is the top 24 bits of Wellons' lowbias32 hash of x as a
 * fraction, times 4, minus 2. Round 4 j + u multiplies into chain c
 * (c = 0..7) the fragments a_((c + u) mod 4) and b_((c / 2 + 3 u) mod 4).
 *   out  as for bsa_mfma_ceiling: the sum of the thread's 8 x 16 accumulators
 *        (C[i_r][l % 32] summed over its rows i_r, over every round and chain).
 * Errors: out NULL or misaligned, iters < 4 or not a multiple of 4, n_wg < 1
 * or above 2^18 give BSA_ERR_INVALID_ARG (nothing launched); a failed launch
 * BSA_ERR_HIP.
 */
bsa_status bsa_mfma_ceiling_random(float* out, int32_t iters, int32_t n_wg, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BSA_H */
