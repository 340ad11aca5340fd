/*
 * nmsparse.h -- C ABI of the MI355X (gfx950) library for semi-structured
 * sparse feed-forward matmuls: magnitude N:M and V:N:M pruning, compression
 * to values plus packed position metadata, and the sparse x dense products of
 * the FFN forward pass and of the double-pruned backward pass.
 *
 * Sources (page title, section):
 *   "Success story: ESPLAG" (inno4scale) -- Highlights, Research Topic,
 *       Solution: semi-structured N:M magnitude pruning, a compressed storage
 *       format (VENOM) and an SpMM kernel library; figures 1-3 (the formats)
 *       are missing from the page.
 *   "To 2:4 Sparsity and Beyond: Neuron-level Activation Function to
 *       Accelerate LLM Pre-Training" -- abstract: 2:4 weights and v:n:m
 *       (Venom) activations in every FFN matmul.
 *   NSF PAR award 2340011 listing -- SLOPE abstract: the backward pass uses
 *       the transposed weight re-pruned with N:M ("double pruned"); lazy
 *       low-rank adapters join the sparse weight late in pre-training.
 *   "Sparser, Faster, Lighter Transformer Language Models" -- Methodologie:
 *       ReLU activations, the FFN as the dominant cost.
 *
 * Conventions shared by every call
 *   - Matrices are row-major.  Leading dimensions (lda, ldb, ...) count
 *     elements, not bytes, and must be >= the row width.
 *   - Groups are M consecutive elements along the reduction dimension K of the
 *     left (sparse) operand, starting at column 0.  K must be a multiple of M.
 *   - Selection keeps the N largest magnitudes of a group; on equal magnitude
 *     the lower position wins.  A group always keeps exactly N elements, zeros
 *     included.  +0.0 and -0.0 have equal magnitude.
 *   - Compressed form of an R x K matrix, N:M:
 *       values [R][(K/M)*N]  kept elements in ascending position, raw bits of
 *                            the input dtype (signed zeros preserved);
 *       meta   [R][ceil((K/M)*N*b/8)] bytes, b = ceil(log2 M): per row one
 *                            LSB-first bit stream of b-bit positions, survivor
 *                            s of group g at bit (g*N + s)*b.  For 2:4 this is
 *                            one nibble p0 | p1 << 2 per group, even groups in
 *                            the low nibble (ceil(K/8) bytes per row).
 *   - V:N:M form (N = 2): per V-row block and M-column group the 4 columns with
 *     the largest block L1 norm (fp64, rows summed top to bottom) are kept,
 *     then 2 of those 4 per row by magnitude:
 *       colsel [R/V][K/M][4] u8  the 4 kept columns of each group, ascending;
 *       values [R][(K/M)*2]       kept elements;
 *       meta   [R][ceil(K/M/2)]   2:4 nibbles j0 | j1 << 2 over j = 0..3,
 *                                 j indexing the group's colsel entries.
 *   - Device pointers: every array argument is device memory owned by the
 *     caller, naturally aligned for its element type.  Outputs are fully
 *     overwritten and must not overlap inputs.  The library allocates nothing
 *     and keeps no state: calls are reentrant and thread-safe -- except
 *     spmm_nm_general_noalloc, whose calls share a fixed scratch buffer per
 *     GPU (see there).
 *   - Streams: `stream` is a hipStream_t (NULL = the null stream).  Every call
 *     is asynchronous on that stream; argument errors are returned before
 *     anything is launched.  No call allocates, clears memory with a memset or
 *     synchronises, so a sequence of calls on one stream can be captured into a
 *     HIP graph and replayed.
 *   - Floating point: products accumulate in fp32 and are written as fp32,
 *     except where a call states a bf16 result (rounded to nearest even).
 *   - Errors: NM_ERR_NULL for a NULL required pointer, NM_ERR_SHAPE for
 *     non-positive sizes, sizes that are not multiples of the group/block, or
 *     a leading dimension below the row width, NM_ERR_UNSUPPORTED for a dtype
 *     or (N, M, V) the call does not implement, NM_ERR_ALIGN for a pointer
 *     that is not aligned to its element size, NM_ERR_HIP when the launch
 *     fails (nm_last_hip_error() names the HIP error), NM_ERR_TOO_LARGE when
 *     an operand does not fit a fixed scratch buffer (spmm_nm_general_noalloc).
 */
#ifndef NMSPARSE_H
#define NMSPARSE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NM_OK = 0,
  NM_ERR_NULL = 1,
  NM_ERR_SHAPE = 2,
  NM_ERR_UNSUPPORTED = 3,
  NM_ERR_ALIGN = 4,
  NM_ERR_HIP = 5,
  NM_ERR_TOO_LARGE = 6
} nm_status;

typedef enum { NM_F32 = 0, NM_BF16 = 1 } nm_dtype;

/* A hipStream_t, passed as an opaque pointer (NULL = the null stream). */
typedef void* nm_stream;

/*
 * nm_prune -- magnitude N:M pruning along K ("Success story: ESPLAG",
 * Highlights and Solution; "To 2:4 Sparsity and Beyond", abstract).
 *   A     [R][lda]    fp32 or bf16 input (dt)
 *   mask  [R][ldmask] u8 output: 1 where kept, 0 elsewhere (columns 0..K-1)
 * N:M: M in {4, 8, 16}, 1 <= N < M.
 */
nm_status nm_prune(nm_dtype dt, const void* A, int64_t lda, int64_t R, int64_t K, int N, int M,
                   uint8_t* mask, int64_t ldmask, nm_stream stream);

/*
 * nm_compress -- gather the kept elements of each group in ascending position
 * and pack their positions ("Success story: ESPLAG", Solution: compressed
 * storage format).
 *   A          [R][lda] input; mask [R][ldmask] u8 (nonzero = kept)
 *   values     [R][(K/M)*N] output, dtype dt
 *   meta       [R][ceil((K/M)*N*b/8)] u8 output
 *   bad_groups nullable device int32: incremented (never reset) by the number
 *              of groups whose mask keeps a count other than N.  Such a group
 *              is stored as +0.0 values at positions 0..N-1.
 */
nm_status nm_compress(nm_dtype dt, const void* A, int64_t lda, const uint8_t* mask, int64_t ldmask,
                      int64_t R, int64_t K, int N, int M, void* values, uint8_t* meta,
                      int32_t* bad_groups, nm_stream stream);

/*
 * nm_prune_compress -- nm_prune and nm_compress in one call: the N:M magnitude
 * selection of A ("Success story: ESPLAG", Highlights and Solution: pruning to
 * N:M and its compressed storage) written both as the mask and as values +
 * metadata.  Outputs are byte-identical to nm_prune followed by nm_compress.
 *   A [R][lda], mask [R][ldmask] u8 output, values [R][(K/M)*N] and
 *   meta [R][ceil((K/M)*N*ceil(log2 M)/8)] outputs, dtype dt.
 * 2:4 with 16-byte aligned rows (A, mask, values) and K % 16 == 0 runs as one
 * pass over A; other calls run the two passes.  Errors as for nm_compress.
 */
nm_status nm_prune_compress(nm_dtype dt, const void* A, int64_t lda, int64_t R, int64_t K, int N,
                            int M, uint8_t* mask, int64_t ldmask, void* values, uint8_t* meta,
                            nm_stream stream);

/*
 * nm_prune_compress_transpose -- nm_prune_compress of A and nm_transpose of B
 * in one launch: the two passes that prepare the 2:4 product of an FFN layer
 * ("Success story: ESPLAG", Solution: the weight pruned to 2:4 and stored
 * compressed; the activations then feed spmm_nm_t K-contiguous).
 *   A, mask, values, meta as for nm_prune_compress;
 *   B [KB][ldb] dense input, Bt [Nc][ldbt] output (ldbt >= KB): Bt[c][k] = B[k][c].
 * Outputs are byte-identical to nm_prune_compress followed by nm_transpose.
 * bf16 only (NM_ERR_UNSUPPORTED otherwise).  2:4 with the single-pass layout of
 * nm_prune_compress runs as one kernel; other calls run the two kernels.
 * Bt must not overlap B; no output may overlap an input.  Errors as for the
 * two calls.
 */
nm_status nm_prune_compress_transpose(nm_dtype dt, const void* A, int64_t lda, int64_t R,
                                      int64_t K, int N, int M, uint8_t* mask, int64_t ldmask,
                                      void* values, uint8_t* meta, const void* B, int64_t ldb,
                                      int64_t KB, int64_t Nc, void* Bt, int64_t ldbt,
                                      nm_stream stream);

/*
 * nm_decompress -- inverse of nm_compress: dense A_out [R][lda] with +0.0 at
 * every position that is not kept.
 */
nm_status nm_decompress(nm_dtype dt, const void* values, const uint8_t* meta, int64_t R, int64_t K,
                        int N, int M, void* A_out, int64_t lda, nm_stream stream);

/*
 * spmm_nm -- C = decompress(values, meta) * B for a 2:4 left operand
 * ("Success story: ESPLAG", Research Topic: the SpMM; "To 2:4 Sparsity and
 * Beyond", abstract: 2:4 weights in every FFN matmul).
 *   values [R][K/2], meta [R][ceil(K/8)] (2:4 form of an R x K matrix), dtype dt
 *   B      [K][ldb] dense, dtype dt
 *   C      [R][ldc] fp32 output, C[r][n] for n < Nc
 * K must be a multiple of 4.
 */
nm_status spmm_nm(nm_dtype dt, const void* values, const uint8_t* meta, int64_t R, int64_t K,
                  const void* B, int64_t ldb, int64_t Nc, float* C, int64_t ldc, nm_stream stream);

/*
 * spmm_nm_t -- spmm_nm with the dense operand given K-contiguous:
 * C[r][n] = sum_k decompress(values, meta)[r][k] * Bt[n][k]
 * ("Success story: ESPLAG", Research Topic: the SpMM of a 2:4 layer).
 *   values [R][K/2], meta [R][ceil(K/8)] (2:4 form of an R x K matrix), dtype dt
 *   Bt     [Nc][ldbt] dense, dtype dt: row n holds column n of B (the token-major
 *          activation layout of an FFN, [tokens][d_model])
 *   C      [R][ldc] fp32 output, C[r][n] for n < Nc
 * K must be a multiple of 4.  Errors as for spmm_nm.  The pipelined bf16 kernel
 * runs when K % 256 == 0, ldbt % 8 == 0 and values, meta and Bt are 16-byte
 * aligned; other calls take a slower general kernel.
 */
nm_status spmm_nm_t(nm_dtype dt, const void* values, const uint8_t* meta, int64_t R, int64_t K,
                    const void* Bt, int64_t ldbt, int64_t Nc, float* C, int64_t ldc, nm_stream stream);

/*
 * spmm_nm_t_out_bf16 -- spmm_nm_t with a bf16 result: each fp32 sum is rounded
 * to the nearest bf16, ties to even, as it is stored.  The output an FFN's
 * up-projection hands to the next step in bf16 (the activations that
 * prune_act_venom selects from; "To 2:4 Sparsity and Beyond", abstract).
 *   values, meta, Bt as for spmm_nm_t (dtype dt, bf16 or fp32 products);
 *   C [R][ldc] bf16 output (uint16 bit patterns), C[r][n] for n < Nc.
 * Errors as for spmm_nm_t (C aligned to 2 bytes).
 */
nm_status spmm_nm_t_out_bf16(nm_dtype dt, const void* values, const uint8_t* meta, int64_t R,
                             int64_t K, const void* Bt, int64_t ldbt, int64_t Nc, void* C,
                             int64_t ldc, nm_stream stream);

/*
 * spmm_nm_t_lowrank -- spmm_nm_t of a 2:4 weight plus a low-rank adapter,
 * applied lazily (SLOPE abstract, NSF PAR award 2340011: low-rank adapters
 * joined to the sparse weight late in pre-training).  The adapted weight
 * W_s + U Vt is never formed:
 *   Tt[n][j] = sum_k Bt[n][k] * Vt[j][k]                   (adapter's inner activations)
 *   C[r][n]  = sum_k decompress(values, meta)[r][k] * Bt[n][k] + sum_j U[r][j] * Tt[n][j]
 *   values, meta, Bt as for spmm_nm_t (dtype dt)
 *   U      [R][ldu] dense, dtype dt, ldu >= rank
 *   Vt     [rank][ldvt] dense, dtype dt, ldvt >= K
 *   Tt     [Nc][rank] fp32 output, contiguous (row n holds the rank inner
 *          activations of column n of B; caller-allocated, kept for the
 *          adapter's backward)
 *   C      [R][ldc] fp32 output, C[r][n] for n < Nc
 * Two launches on the stream.  K must be a multiple of 4 and 0 < rank <= 2^20;
 * no output may overlap an input or the other output.  Errors as for
 * spmm_nm_t (U and Vt aligned to their element size, Tt and C to 4 bytes).
 * With bf16, rank % 16 == 0, K % 16 == 0, ldbt, ldvt and ldu multiples of 8
 * and Bt, Vt, U and Tt 16-byte aligned, Tt comes from matrix instructions and
 * the adapter term is added inside the pipelined SpMM (when that kernel's own
 * conditions hold) as extra steps after the sparse ones; each Tt value then
 * enters that term as two bf16 parts (about 16 significant bits).  Other calls
 * take plain fp32 kernels after the SpMM.
 */
nm_status spmm_nm_t_lowrank(nm_dtype dt, const void* values, const uint8_t* meta, int64_t R,
                            int64_t K, const void* Bt, int64_t ldbt, int64_t Nc, const void* U,
                            int64_t ldu, const void* Vt, int64_t ldvt, int64_t rank, float* Tt,
                            float* C, int64_t ldc, nm_stream stream);

/*
 * spmm_nm_t_relu_venom -- an FFN up-projection whose activations leave the
 * kernel already pruned ("To 2:4 Sparsity and Beyond", abstract: 2:4 weights
 * and v:n:m activations in the FFN; "Sparser, Faster, Lighter Transformer
 * Language Models", Methodologie: ReLU).  With C = decompress(values, meta) Bt^T
 * as in spmm_nm_t ([R][Nc]: R the FFN width, Nc the tokens), the activations
 * h = ReLU(bf16(C))^T [Nc][R] (each fp32 sum rounded to nearest even, then
 * every value <= 0 made +0.0) are pruned to V:N:M along R with V-blocks of
 * tokens, exactly as prune_act_venom(h, V, M, apply_relu) would, and only the
 * compressed form is written: h is never stored.
 *   values, meta, Bt as for spmm_nm_t, bf16 only
 *   h_values [Nc][(R/M)*2] bf16, h_meta [Nc][ceil((R/M)/2)], h_colsel
 *            [Nc/V][R/M][4]: the outputs of prune_act_venom for h
 * V in {64, 128, 256} and M in {4, 8, 16} (NM_ERR_UNSUPPORTED otherwise, and
 * for dtypes other than bf16); R % 256 == 0, Nc % 256 == 0, K % 256 == 0, ldbt % 8 == 0,
 * values, meta and Bt 16-byte aligned, values and Bt each below 4 GiB,
 * h_values 16-byte and h_meta, h_colsel 4-byte aligned (NM_ERR_UNSUPPORTED
 * otherwise: compose spmm_nm_t_out_bf16,
 * nm_transpose and prune_act_venom instead).  NM_ERR_SHAPE for non-positive
 * sizes, K % 4 != 0, ldbt < K, R % M != 0 or Nc % V != 0.
 */
nm_status spmm_nm_t_relu_venom(nm_dtype dt, const void* values, const uint8_t* meta, int64_t R,
                               int64_t K, const void* Bt, int64_t ldbt, int64_t Nc, int V, int M,
                               void* h_values, uint8_t* h_meta, uint8_t* h_colsel,
                               nm_stream stream);

/*
 * spmm_nm_general -- spmm_nm_t for any N:M form nm_compress writes ("Success
 * story: ESPLAG", Solution: N:M patterns beyond 2:4):
 * C[r][n] = sum_k decompress(values, meta, N, M)[r][k] * Bt[n][k]
 *   values [R][(K/M)*N], meta [R][ceil((K/M)*N*ceil(log2 M)/8)] (the layout of
 *          nm_compress), dtype dt
 *   Bt     [Nc][ldbt] dense, dtype dt (K-contiguous, as for spmm_nm_t)
 *   C      [R][ldc] fp32 output
 *   work   optional device memory of work_bytes bytes, 16-byte aligned, that
 *          must not overlap any other argument (NULL allowed)
 * M in {4, 8, 16}, 1 <= N < M, K % M == 0.  When N <= 2 every aligned run of
 * 4 columns holds at most two survivors: with work of at least
 * nm_general_work_bytes(dt, R, K, N, M) bytes the matrix is rewritten there
 * in 2:4 form (runs padded with +0.0) and spmm_nm_t computes the product; 2:4
 * itself goes to spmm_nm_t directly.  With N > 2 (bf16, K % 64 == 0, ldbt % 8
 * == 0, ldc % 4 == 0, 16-byte aligned Bt and C) the work memory receives the
 * matrix as dense bf16 rows [R][K] and a dense matrix-core GEMM computes the
 * product.  Other calls, and any without enough work memory, take a plain SIMT
 * kernel.  Errors as for spmm_nm_t, plus
 * NM_ERR_UNSUPPORTED for an N:M outside the set above and NM_ERR_SHAPE for
 * K % M != 0 or work_bytes < 0.
 */
nm_status spmm_nm_general(nm_dtype dt, const void* values, const uint8_t* meta, int64_t R,
                          int64_t K, int N, int M, const void* Bt, int64_t ldbt, int64_t Nc,
                          float* C, int64_t ldc, void* work, int64_t work_bytes,
                          nm_stream stream);

/*
 * sddmm_venom -- gradient reaching V:N:M activations through a down-projection
 * ("To 2:4 Sparsity and Beyond", abstract: v:n:m activations in every FFN
 * matmul).  For Y = h_s . W_down with h_s the V:N:M form (prune_act_venom,
 * apply_relu) of h = ReLU(z) [T][F]:
 *   dz[t][2g+s] = sum_c dY[t][c] * W_down[g*M + colsel[t/V][g][j_s]][c]
 *                 (times [h_values[t][2g+s] > 0] when apply_relu)
 * i.e. dY . W_down^T at the entries h_s keeps -- the only ones through which
 * the gradient flows -- gated by ReLU's derivative.
 *   dY       [T][lddy] dtype dt         W_down [F][ldw] dtype dt (Nc columns)
 *   h_values [T][(F/M)*2], h_meta [T][ceil(F/M/2)], h_colsel [T/V][F/M][4]:
 *            h_s as prune_act_venom writes it (N = 2, 4 kept columns per group)
 *   dz       [T][(F/M)*2] fp32 output, aligned with h_values
 *   dYt      optional (NULL allowed, bf16 only): dYt [Nc][lddyt] receives
 *            dY^T, the operand spmm_venom_tn takes
 * M in {4, 8, 16}, 1 <= V <= 256, F % M == 0, T % V == 0.  bf16 with
 * V % 128 == 0, Nc % 64 == 0 and 16-byte aligned rows runs the pipelined
 * matrix-core kernel (B rows gathered per V-block); other calls a SIMT kernel
 * (then dYt by nm_transpose).  Errors as for sddmm_nm.
 */
nm_status sddmm_venom(nm_dtype dt, const void* dY, int64_t lddy, const void* W_down, int64_t ldw,
                      int64_t T, int64_t F, int64_t Nc, int V, int M, const void* h_values,
                      const uint8_t* h_meta, const uint8_t* h_colsel, int apply_relu, float* dz,
                      void* dYt, int64_t lddyt, nm_stream stream);

/*
 * spmm_venom_tn -- weight gradient of the same down-projection:
 *   dW[k][c] = sum_t h_s[t][k] * dY[t][c]      (h_s^T . dY)
 *   h_values, h_meta, h_colsel: h_s [T][F] in V:N:M form (as for sddmm_venom)
 *   dYt  [Nc][lddyt] dY^T, dtype dt (token index contiguous)
 *   dW   [F][lddw] fp32 output
 *   work optional device memory of work_bytes bytes, 16-byte aligned, not
 *        overlapping any argument (NULL allowed)
 * The reduction runs over tokens and every V-block of tokens keeps a different
 * half of each group's rows, so the product has no empty blocks for the matrix
 * instructions to skip.  bf16 with work of at least
 * nm_venom_tn_work_bytes(dt, T, F) bytes, T % 64 == 0, lddyt % 8 == 0,
 * lddw % 4 == 0 and 16-byte aligned operands writes h_s^T densely into work
 * and runs a matrix-core NT GEMM; other calls a SIMT kernel on the compressed
 * form.  Errors as for spmm_venom, plus NM_ERR_SHAPE for work_bytes < 0.
 */
nm_status spmm_venom_tn(nm_dtype dt, const void* h_values, const uint8_t* h_meta,
                        const uint8_t* h_colsel, int64_t T, int64_t F, int V, int M,
                        const void* dYt, int64_t lddyt, int64_t Nc, float* dW, int64_t lddw,
                        void* work, int64_t work_bytes, nm_stream stream);

/* Work bytes spmm_venom_tn uses for T tokens and F columns of h (host only; 0 = none). */
int64_t nm_venom_tn_work_bytes(nm_dtype dt, int64_t T, int64_t F);

/*
 * spmm_nm_general_noalloc -- spmm_nm_general for callers that cannot allocate
 * device memory (code under stream capture, tight serving loops, harnesses that
 * forbid allocation): the same product and kernels, with the work memory (the
 * 2:4 rewrite or the dense rows) held in a fixed 64 MiB scratch buffer that the library keeps in each GPU's memory
 * for the life of the process (nm_general_scratch_bytes() gives the size).
 * The call allocates nothing and takes no work argument; the caller still
 * passes inputs and outputs as for spmm_nm_general.  Every call on one GPU
 * shares that buffer: calls that overlap on one GPU (two streams, or two host
 * threads) race and must be serialised by the caller.  Nothing in the buffer
 * needs clearing between calls.  Errors as for spmm_nm_general, plus
 * NM_ERR_TOO_LARGE, returned before any launch, when the rewrite needs more
 * than the buffer holds (nm_general_work_bytes(dt, R, K, N, M) >
 * nm_general_scratch_bytes()).
 */
nm_status spmm_nm_general_noalloc(nm_dtype dt, const void* values, const uint8_t* meta, int64_t R,
                                  int64_t K, int N, int M, const void* Bt, int64_t ldbt, int64_t Nc,
                                  float* C, int64_t ldc, nm_stream stream);

/*
 * nm_gmp_n_at -- host only: the N:M pattern a gradual magnitude pruning
 * schedule has in effect at a training step ("Success story: ESPLAG",
 * Highlights and Research Topic: semi-structured gradual magnitude pruning;
 * "To 2:4 Sparsity and Beyond", abstract: sparse steps, then regular dense
 * steps towards the end).  The pages give no schedule; the one implemented:
 *   - dense (returns M) before t_begin and, when t_dense >= 0, from t_dense on;
 *   - pruning events at t_begin + e*interval for e = 0 .. E-1,
 *     E = (t_end - t_begin) / interval + 1;
 *   - after event e the pattern is N_e : M with
 *     N_e = M - ceil((M - n_final) * (e + 1) / E), falling linearly to n_final
 *     at the last event and held until the dense switch.
 * *prune_now (nullable) is set to 1 when `step` is a pruning event: the caller
 * then magnitude-prunes its current weight to N_e:M (nm_prune_compress) and
 * keeps the pruned entries at zero.  Returns -1 for invalid parameters
 * (M not in {4, 8, 16}, n_final outside 1 .. M-1, t_begin < 0,
 * t_end < t_begin, interval < 1).
 */
int nm_gmp_n_at(int M, int n_final, int64_t t_begin, int64_t t_end, int64_t interval,
                int64_t t_dense, int64_t step, int* prune_now);

/* Bytes of the fixed scratch buffer of spmm_nm_general_noalloc (host only). */
int64_t nm_general_scratch_bytes(void);

/*
 * nm_general_work_bytes -- host only: the work bytes spmm_nm_general uses for
 * an R x K matrix in N:M form (0 when it uses none, or for invalid arguments).
 */
int64_t nm_general_work_bytes(nm_dtype dt, int64_t R, int64_t K, int N, int M);

/*
 * nm_transpose -- dst[c][r] = src[r][c] for an R x Cn matrix: turns a row-major
 * dense operand B [K][Nc] into the K-contiguous form spmm_nm_t takes.
 *   src [R][lds], dst [Cn][ldd] (ldd >= R), dtype dt; dst must not overlap src.
 * bf16 only (NM_ERR_UNSUPPORTED for other dtypes).
 */
nm_status nm_transpose(nm_dtype dt, const void* src, int64_t lds, int64_t R, int64_t Cn, void* dst,
                       int64_t ldd, nm_stream stream);

/*
 * prune_act_venom -- V:N:M prune (N = 2) and compress in one pass, optionally
 * after ReLU ("To 2:4 Sparsity and Beyond", abstract: v:n:m activations;
 * "Sparser, Faster, Lighter Transformer Language Models", Methodologie: ReLU;
 * "Success story: ESPLAG", Solution: VENOM format).
 *   Z       [R][ldz] input, dtype dt
 *   apply_relu  nonzero: select on h = ReLU(Z) (every z <= 0, and -0.0,
 *               becomes +0.0) and store h's values
 *   values  [R][(K/M)*2], meta [R][ceil(K/M/2)], colsel [R/V][K/M][4] outputs
 *   mask    nullable [R][ldmask] u8 output: 1 at the 2 kept columns per group
 * M in {4, 8, 16}; 1 <= V <= 256; R % V == 0; K % M == 0.
 */
nm_status prune_act_venom(nm_dtype dt, const void* Z, int64_t ldz, int64_t R, int64_t K, int V,
                          int M, int apply_relu, void* values, uint8_t* meta, uint8_t* colsel,
                          uint8_t* mask, int64_t ldmask, nm_stream stream);

/*
 * spmm_venom -- C = decompress_venom(values, meta, colsel) * B:
 * C[r][n] = sum_g sum_s values[r][2g+s] * B[g*M + colsel[r/V][g][j_s]][n]
 * ("To 2:4 Sparsity and Beyond", abstract; "Success story: ESPLAG",
 * Solution: VENOM format and its SpMM).
 *   B [K][ldb] dense, dtype dt; C [R][ldc] fp32 output.
 * M in {4, 8, 16}; 1 <= V <= 256; R % V == 0; K % M == 0.
 */
nm_status spmm_venom(nm_dtype dt, const void* values, const uint8_t* meta, const uint8_t* colsel,
                     int64_t R, int64_t K, int V, int M, const void* B, int64_t ldb, int64_t Nc,
                     float* C, int64_t ldc, nm_stream stream);

/*
 * nm_reprune_t -- double pruning (NSF PAR award 2340011, SLOPE abstract): the
 * 2:4-compressed W_s [R x K] is decompressed with +0.0 fill, transposed to
 * [K x R], pruned 2:4 by magnitude along R and compressed.
 *   values [R][K/2], meta [R][ceil(K/8)]      input (2:4 along K)
 *   values_t [K][R/2], meta_t [K][ceil(R/8)]  output (2:4 along R)
 * R and K must be multiples of 4.
 */
nm_status nm_reprune_t(nm_dtype dt, const void* values, const uint8_t* meta, int64_t R, int64_t K,
                       void* values_t, uint8_t* meta_t, nm_stream stream);

/*
 * nm_reprune_t_transpose -- nm_reprune_t of W_s and nm_transpose of X in one
 * launch: the two passes of a double-pruned training step (NSF PAR award
 * 2340011, SLOPE abstract: the transposed weight re-pruned for the backward
 * pass; the layer input then feeds spmm_nm_t K-contiguous) that touch
 * disjoint data.
 *   values, meta, R, K, values_t, meta_t as for nm_reprune_t;
 *   X [RX][ldx] dense input, Xt [CX][ldxt] output (ldxt >= RX): Xt[c][r] = X[r][c].
 * Outputs are byte-identical to nm_reprune_t followed by nm_transpose.  bf16
 * only (NM_ERR_UNSUPPORTED otherwise).  With R and K multiples of 128 and the
 * re-prune's aligned layout the two run as one kernel; otherwise as the two
 * kernels.  No output may overlap an input.  Errors as for the two calls.
 */
nm_status nm_reprune_t_transpose(nm_dtype dt, const void* values, const uint8_t* meta, int64_t R,
                                 int64_t K, void* values_t, uint8_t* meta_t, const void* X,
                                 int64_t ldx, int64_t RX, int64_t CX, void* Xt, int64_t ldxt,
                                 nm_stream stream);

/*
 * nm_mfma_rate_probe -- a measurement aid, not a step of the sparse path: a
 * chip-wide loop of independent bf16 matrix instructions on register operands
 * (kind 0: v_mfma_f32_32x32x16_bf16; kind 1: v_smfmac_f32_32x32x32_bf16, 2:4),
 * eight accumulators per wave, two waves per SIMD on 256 CUs, no memory traffic.
 * Timed by the caller (events around it on `stream`), it gives the matrix rate
 * the chip sustains under its power limit, the reference the benchmark reports
 * next to the nominal peak.
 *   iters  loop count per wave (1 .. 2^24)
 *   sink   device fp32 [512 * 256]: one value per thread, written so that
 *          nothing is optimised away (its contents mean nothing)
 *   flops  host output: the dense-equivalent flops one launch performs
 * NM_ERR_UNSUPPORTED for another kind, NM_ERR_SHAPE for iters out of range.
 */
nm_status nm_mfma_rate_probe(int kind, int64_t iters, float* sink, int64_t* flops, nm_stream stream);

/*
 * The panel layout of a bf16 2:4 form (R rows, K dense columns, R % 4 == 0,
 * K % 256 == 0): the same values and nibbles as the row-major form
 * (values [R][K/2], meta [R][K/8]), in another order, with the same total sizes:
 *   values: the 64 bytes of row r for the 64-column step s (its 32 kept values,
 *           in column order) at byte ((r / 2) * (K / 64) + s) * 128 + (r % 2) * 64;
 *   meta:   the 32 bytes of row r for the 256-column chunk c (its 64 nibbles,
 *           group 0 in bits 0..3) at byte ((r / 4) * (K / 256) + c) * 128 + (r % 4) * 32.
 * Every 64-column step of a 256-row tile is then whole 128-byte lines of each
 * operand, which the four-wave SpMM below needs to load two steps ahead.
 */

/*
 * nm_to_panels -- the panel layout of a bf16 2:4 form given row-major.
 *   values [R][K/2], meta [R][K/8] in; values_p, meta_p (same sizes) out.
 * R % 4 == 0 and K % 256 == 0 (NM_ERR_SHAPE), all four pointers 16-byte aligned
 * (NM_ERR_ALIGN), bf16 only (NM_ERR_UNSUPPORTED).  No output may overlap an input.
 */
nm_status nm_to_panels(nm_dtype dt, const void* values, const uint8_t* meta, int64_t R, int64_t K,
                       void* values_p, uint8_t* meta_p, nm_stream stream);

/*
 * nm_reprune_t_transpose_panels -- nm_reprune_t_transpose with the re-pruned
 * transposed weight written in the panel layout (a K x R form compressed along
 * R): the double-pruned backward's operand (NSF PAR award 2340011, SLOPE
 * abstract) for spmm_nm_t_panels.  Xt as for nm_reprune_t_transpose.
 * bf16 only; R % 256 == 0 and K % 128 == 0 (NM_ERR_SHAPE); values and values_t
 * 16-byte, meta and meta_t 2-byte aligned (NM_ERR_ALIGN).  Outputs equal
 * nm_to_panels of nm_reprune_t's, byte for byte.
 */
nm_status nm_reprune_t_transpose_panels(nm_dtype dt, const void* values, const uint8_t* meta,
                                        int64_t R, int64_t K, void* values_t, uint8_t* meta_t,
                                        const void* X, int64_t ldx, int64_t RX, int64_t CX,
                                        void* Xt, int64_t ldxt, nm_stream stream);

/*
 * spmm_nm_t_panels -- spmm_nm_t of a weight given in the panel layout
 * ("Success story: ESPLAG", Research Topic: the SpMM of a 2:4 layer; the
 * backward's product with the re-pruned transposed weight, SLOPE abstract):
 * C[r][n] = sum_k decompress(values, meta)[r][k] * Bt[n][k].
 *   values, meta: panel layout of the R x K form; Bt [Nc][ldbt]; C [R][ldc] fp32.
 * bf16 only; R % 256 == 0, K % 256 == 0, ldbt >= K, ldbt % 8 == 0, ldc >= Nc
 * (NM_ERR_SHAPE); values, meta and Bt 16-byte, C 4-byte aligned (NM_ERR_ALIGN);
 * NM_ERR_TOO_LARGE when values or Bt reach 4 GiB.  The products are added in the
 * order of spmm_nm_t's pipelined kernel, so C equals spmm_nm_t's bit for bit.
 */
nm_status spmm_nm_t_panels(nm_dtype dt, const void* values, const uint8_t* meta, int64_t R,
                           int64_t K, const void* Bt, int64_t ldbt, int64_t Nc, float* C,
                           int64_t ldc, nm_stream stream);

/*
 * sddmm_nm -- the weight gradient of a 2:4 layer, sampled at the weight's
 * survivors ("Success story: ESPLAG", Research Topic: kernels for the full
 * sparse training step):
 *   values_out[r][2g+s] = sum_t D[r][t] * X[4g + p_s(r, g)][t]
 * with p_s from meta (the 2:4 metadata of the R x Kc weight).
 *   D [R][ldd] (the output gradient), X [Kc][ldx] (the layer input, one row
 *   per input feature), dtype dt; values_out [R][Kc/2] fp32.
 * Kc must be a multiple of 4.
 */
nm_status sddmm_nm(nm_dtype dt, const void* D, int64_t ldd, const void* X, int64_t ldx, int64_t R,
                   int64_t Kc, int64_t T, const uint8_t* meta, float* values_out, nm_stream stream);

/*
 * sddmm_nm_dt -- sddmm_nm that also writes the transpose of the output
 * gradient, Dt[t][r] = D[r][t], which the input gradient's product then reads
 * K-contiguous (spmm_nm_t of the re-pruned transposed weight; "Success story:
 * ESPLAG", Research Topic: the kernels of the sparse training step).  The
 * SDDMM stages every tile of D through LDS, so the transpose costs no extra
 * read of D.
 *   D, X, meta, values_out as for sddmm_nm; Dt [T][lddt] bf16 output
 *   (lddt >= R), not overlapping any input.
 * bf16 only (NM_ERR_UNSUPPORTED otherwise).  Outputs are those of sddmm_nm and
 * nm_transpose(D); without the pipelined SDDMM's conditions the call runs the
 * two.  Errors as for the two calls.
 */
nm_status sddmm_nm_dt(nm_dtype dt, const void* D, int64_t ldd, const void* X, int64_t ldx, int64_t R,
                      int64_t Kc, int64_t T, const uint8_t* meta, float* values_out, void* Dt,
                      int64_t lddt, nm_stream stream);

/*
 * nm_sizes -- host-only helper: element count of values, bytes of meta and of
 * colsel for an R x K matrix in N:M form (V > 0: V:N:M form with N = 2, where
 * N is ignored).  NULL outputs are skipped.
 */
void nm_sizes(int64_t R, int64_t K, int N, int M, int V, int64_t* n_values, int64_t* meta_bytes,
              int64_t* colsel_bytes);

/* Static description of a status code. */
const char* nm_status_str(nm_status status);

/* The HIP error string behind the last NM_ERR_HIP on this thread ("" if none). */
const char* nm_last_hip_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int nm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NMSPARSE_H */
