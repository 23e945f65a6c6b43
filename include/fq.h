/*
 * fq.h — C ABI of the FibQuant KV-cache codec for AMD MI355X (gfx950).
 *
 * Method: "FibQuant: universal vector quantisation for random-access KV-cache
 * compression", technical summary on gist.science (paper 2605.11478, Korean and
 * Dutch pages with the same section numbers).
 *
 *   encode (§2.3): store the norm nu = ||x||_2, rotate the unit vector Pi x / nu
 *                  with one shared Haar rotation, split it into d/k blocks of k
 *                  consecutive coordinates and store, for every block, the index
 *                  of its nearest codeword in one shared codebook of N words.
 *   decode (§2.3): gather the codewords, concatenate the blocks, apply the
 *                  inverse rotation and scale by the norm.
 *   rate   (§2.3, §3.3): b = log2(N)/k bits per coordinate.
 *   store  (§1):   fixed-rate codes at fixed addresses, so every vector decodes
 *                  alone by address arithmetic.
 *   attention (§5): the fixed addresses let decompression be fused into
 *                  attention: q.k_j = nu_j (Pi q).c_j straight from the codes.
 *
 * Conventions shared by every call
 *   - d = 64.  k divides d (1, 2, 4, 8, 16, 32 or 64).  N is a power of two,
 *     2 <= N <= 65536.  Every codeword coordinate must be exactly representable
 *     as an fp16 normal number or zero (the offline construction rounds to that
 *     grid), so matrix units can use the codewords exactly.
 *   - Rotation: row-major d x d fp32 matrix Pi with y = Pi x.
 *   - Code store: B = (d/k) * log2(N) bits per vector; vector i starts at bit
 *     i*B, its block j at bit i*B + j*log2(N); bits are LSB-first inside
 *     little-endian bytes; the store holds ceil(n*B/8) bytes and pad bits are 0.
 *   - Nearest codeword: the minimum of sum_i (y_i - c_i)^2 with y the exactly
 *     rotated unit vector; among exactly equal distances the lowest index.  The
 *     device search runs in fp32 and certifies every result against a rigorous
 *     fp32 error bound; blocks it cannot certify are searched again in fp64.
 *   - Norms: nu is accumulated in fp64 and stored round-to-nearest-even in the
 *     norm dtype directly from fp64 (fp16 overflow stores +inf).  nu = 0 gives
 *     the all-smallest-norm codes and decodes to exactly 0.
 *   - Memory: every bulk pointer is caller-owned device memory on the device
 *     that was current at fq_codebook_load, 16-byte aligned (the int64 slot
 *     and int32 length arrays: 8- and 4-byte aligned).  Inputs are only
 *     read, outputs only written.  Nothing here allocates except
 *     fq_codebook_load.
 *   - Asynchrony: fq_encode, fq_encode_scatter, fq_decode, fq_attn_decode,
 *     fq_attn_decode_varlen and fq_attn_prefill only enqueue work on `stream`
 *     (a hipStream_t; NULL is the default stream) and return; they never
 *     synchronise and never read results back (fq_codebook_train is the
 *     exception and says so).
 *   - Errors: arguments are checked on the host before any launch and return
 *     FQ_ERR_ARG / FQ_ERR_UNSUPPORTED / FQ_ERR_WORKSPACE with nothing enqueued;
 *     a failed launch returns FQ_ERR_HIP.  No call aborts or throws.  n = 0 (or
 *     T = 0 keys) is a no-op that returns FQ_OK.  NaN or Inf inputs give
 *     unspecified codes.
 */
#ifndef FQ_H
#define FQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct fq_codebook fq_codebook; /* opaque; immutable after load */

typedef enum fq_status {
  FQ_OK = 0,
  FQ_ERR_ARG = 1,         /* null pointer, bad size, misaligned pointer, wrong device, bad codebook values */
  FQ_ERR_UNSUPPORTED = 2, /* valid request outside what the kernels implement */
  FQ_ERR_WORKSPACE = 3,   /* attention workspace missing or too small */
  FQ_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} fq_status;

typedef enum fq_dtype { FQ_F32 = 0, FQ_F16 = 1 } fq_dtype;

/* Load a codebook and the shared rotation (FibQuant summary §2.1 shared
 * rotation, §2.2 shared offline codebook) onto the current HIP device.
 *   codewords: host fp32 [N][k], fp16-representable values (see above).
 *   rotation:  host fp32 [d][d] row-major, y = Pi x.
 *   out:       receives the handle; free it with fq_codebook_free.
 * Synchronous.  Allocates device memory that the handle owns: copies of the
 * codebook in the kernels' layouts (about 7 N k bytes; for k = d about 800 N
 * bytes, with the table of decoded unit vectors Pi^T c_n that the decoder
 * gathers) plus about 200 KiB of rotation operands.
 * Returns FQ_ERR_ARG for bad sizes or values, FQ_ERR_UNSUPPORTED for d != 64,
 * FQ_ERR_HIP if an allocation or copy fails (nothing is leaked). */
fq_status fq_codebook_load(int d, int k, int N, const float* codewords, const float* rotation,
                           fq_codebook** out);

/* Release a handle from fq_codebook_load (NULL is ignored).  The caller must
 * make sure no enqueued work still uses it. */
void fq_codebook_free(fq_codebook* cb);

/* Bytes of the fixed-address code store for n vectors: ceil(n * B / 8)
 * (FibQuant summary §1, §2.3).  Returns -1 for a NULL handle or n < 0. */
int64_t fq_code_bytes(const fq_codebook* cb, int64_t n);

/* Encode n vectors (FibQuant summary §2.3 encoder).
 *   x:      device [n][d] in x_dtype (FQ_F32 or FQ_F16), row-major.
 *   codes:  device, fq_code_bytes(cb, n) bytes, written completely (pad bits 0).
 *   norms:  device [n] in norm_dtype.
 * Codes equal the exact nearest codeword (lowest index on exact ties) for
 * every block; see the conventions above for how that is guaranteed. */
fq_status fq_encode(const fq_codebook* cb, const void* x, fq_dtype x_dtype, int64_t n, uint8_t* codes,
                    void* norms, fq_dtype norm_dtype, void* stream);

/* Name of the encoder kernel fq_encode (and fq_encode_scatter) launches for n
 * vectors of dtype x_dtype with this codebook: "encode_wave" (batches of at most
 * 2048 vectors), "encode_h16" (fp16 input, k = 4 or 8), "encode_full" (fp16
 * input, k = 16, 32 or d), "encode_mfma" (k = 4 or 8) or "encode_valu" (every
 * shape).  The
 * environment variable FQ_ENCODE_KERNEL, read by fq_codebook_load, forces one of
 * them (small, h16, full, mfma, valu) wherever it covers the call.  A diagnostic:
 * static string, NULL for a NULL handle, n < 0 or an invalid dtype. */
const char* fq_encode_kernel(const fq_codebook* cb, fq_dtype x_dtype, int64_t n);

/* Encode n vectors into chosen records of an existing code store: the append
 * step of a growing cache (FibQuant summary §1 and §5: every record has a fixed
 * size and address, so one record is rewritten without touching the others).
 * Vector i is encoded exactly as fq_encode would encode it; its record is
 * written to record slots[i] of a store of `capacity` records and its norm to
 * norms[slots[i]].
 *   x:        device [n][d] in x_dtype, row-major.
 *   slots:    device int64 [n], 8-byte aligned.  A slot outside [0, capacity)
 *             skips that vector (nothing is written for it), e.g. a finished
 *             sequence.  Slots within one call must be distinct; two equal
 *             slots leave an unspecified mix of the two records.
 *   codes:    device, fq_code_bytes(cb, capacity) bytes; records not named in
 *             slots are left untouched.
 *   norms:    device [capacity] in norm_dtype.
 * Records must be whole bytes (bits per vector a multiple of 8, so no byte is
 * shared by two records); otherwise FQ_ERR_UNSUPPORTED. */
fq_status fq_encode_scatter(const fq_codebook* cb, const void* x, fq_dtype x_dtype, int64_t n,
                            const int64_t* slots, int64_t capacity, uint8_t* codes, void* norms,
                            fq_dtype norm_dtype, void* stream);

/* Decode n vectors (FibQuant summary §2.3 decoder): x_out = nu * Pi^T concat(c).
 *   codes:  device, fq_code_bytes(cb, n) bytes.  norms: device [n] in norm_dtype.
 *   x_out:  device [n][d] in out_dtype, each value rounded once (RNE) from an
 *           fp32 accumulation. */
fq_status fq_decode(const fq_codebook* cb, const uint8_t* codes, const void* norms, fq_dtype norm_dtype,
                    int64_t n, void* x_out, fq_dtype out_dtype, void* stream);

/* Workspace bytes fq_attn_decode needs for these sizes (0 when T = 0;
 * 0 as well for a NULL handle or invalid sizes). */
size_t fq_attn_workspace_bytes(const fq_codebook* cb, int B, int Hq, int Hkv, int64_t T);

/* Decode-step attention over a compressed cache (FibQuant summary §5: fixed
 * addresses allow decompression fused into attention).  For every batch b and
 * query head h, with KV head g = h / (Hq/Hkv):
 *     out[b][h] = sum_j softmax_j(scale * q[b][h] . k_j) v_j
 * where k_j, v_j are the decoded keys / values of (b, g), computed straight
 * from the codes as nu_j Pi^T c_j without materialising them.
 *   q:        device fp16 [B][Hq][d].
 *   k_codes, v_codes: device code stores of B*Hkv*T vectors in [B][Hkv][T] order
 *             (exactly what fq_encode writes for a [B][Hkv][T][d] tensor).
 *   k_norms, v_norms: device fp16 [B][Hkv][T].
 *   out:      device fp32 [B][Hq][d].
 *   workspace: device, at least fq_attn_workspace_bytes(...) bytes.
 * Hq must be a multiple of Hkv with Hq/Hkv <= 16 (else FQ_ERR_UNSUPPORTED, and
 * fq_attn_workspace_bytes returns 0).  Every codebook is served: k = 4 with 8-bit
 * codes and Hq/Hkv <= 8 by the fast kernel; the full-vector code (k = d) with
 * Hq/Hkv >= 4, N <= 4096 and T >= 4 N through per-head lookup tables of the N
 * scores (Pi q).c_n and LDS histograms of the value weights; every other case by
 * the general kernel, which gathers codewords from an LDS copy of the fp16
 * codebook when 2 N k bytes plus its own 20,992 fit one workgroup's LDS
 * (N*k <= 65536 on gfx950, 160 KiB) and from the codebook in global memory
 * otherwise.  The lookup-table path adds its float atomics in no fixed order, so
 * its repeated calls may differ in the last bits; FQ_ATTN_KERNEL=lut at
 * fq_codebook_load selects it wherever its LDS holds the tables (k = d with
 * N <= 16384, and k = 4), FQ_ATTN_KERNEL=gather the general kernel for k = d.
 * There is no mask: the single query attends to all T keys. */
fq_status fq_attn_decode(const fq_codebook* cb, const void* q, const uint8_t* k_codes, const void* k_norms,
                         const uint8_t* v_codes, const void* v_norms, int B, int Hq, int Hkv, int64_t T,
                         float scale, float* out, void* workspace, size_t workspace_bytes, void* stream);

/* fq_attn_decode over a growing cache (FibQuant summary §5): each slab holds
 * room for T keys (the capacity; all layouts and the workspace as above, sized
 * by T) and batch b attends only to its first L_b = min(max(lens[b], 0), T)
 * keys, the ones written so far:
 *     out[b][h] = sum_{j < L_b} softmax_j(scale * q[b][h] . k_j) v_j,
 * and out[b][h] = 0 when L_b = 0.  Keys at or past L_b are never used, so
 * their codes and norms may hold anything.
 *   lens: device int32 [B], 4-byte aligned (read on the device; the host never
 *         waits for it).
 * T = 0 (or B = 0) is a no-op, as for fq_attn_decode. */
fq_status fq_attn_decode_varlen(const fq_codebook* cb, const void* q, const uint8_t* k_codes, const void* k_norms,
                                const uint8_t* v_codes, const void* v_norms, const int32_t* lens, int B, int Hq,
                                int Hkv, int64_t T, float scale, float* out, void* workspace,
                                size_t workspace_bytes, void* stream);

/* fq_attn_decode / fq_attn_decode_varlen for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same kernels and results, with the partial-record
 * workspace held in the library's own fixed device buffer instead of a caller's
 * (fq_attn_noalloc_max_workspace_bytes() bytes, 16 MiB, one per device, held
 * until the process ends; its device address is looked up once per device when
 * the first codebook is loaded there).  The call allocates nothing.
 *   lens: NULL (every batch attends to all T keys, as fq_attn_decode) or device
 *         int32 [B], 4-byte aligned (as fq_attn_decode_varlen).
 *   other arguments as for fq_attn_decode.
 * Returns FQ_ERR_WORKSPACE when fq_attn_workspace_bytes(cb, B, Hq, Hkv, T)
 * exceeds the buffer.  Every call on one device shares that device's buffer and
 * nothing in it needs clearing between calls: calls that overlap on one device
 * (different streams, or graphs replayed concurrently) race and give undefined
 * results. */
size_t fq_attn_noalloc_max_workspace_bytes(void);
fq_status fq_attn_decode_noalloc(const fq_codebook* cb, const void* q, const uint8_t* k_codes, const void* k_norms,
                                 const uint8_t* v_codes, const void* v_norms, const int32_t* lens, int B, int Hq,
                                 int Hkv, int64_t T, float scale, float* out, void* stream);

/* Workspace bytes fq_attn_prefill needs (0 for invalid sizes, T = 0, B = 0 or Sq = 0). */
size_t fq_attn_prefill_workspace_bytes(const fq_codebook* cb, int B, int Hq, int Hkv, int Sq, int64_t T);

/* Multi-query (prefill) attention over a compressed cache (FibQuant summary §5):
 * Sq queries per query head, each scored as in fq_attn_decode:
 *     out[b][h][i] = sum_{j in K_i} softmax_j(scale * q[b][h][i] . k_j) v_j,
 * K_i = all T keys, or with causal = 1 the keys 0 .. T - Sq + i (the queries
 * are the last Sq positions of the cache; a query that sees no key gets 0).
 *   q:   device fp16 [B][Hq][Sq][d].  out: device fp32 [B][Hq][Sq][d].
 *   cache, grouping, workspace rules as for fq_attn_decode.
 * Every codebook the library loads (codebooks of more than 32 KiB in fp16 are
 * read from global memory).  FQ_PREFILL_KERNEL=wide at fq_codebook_load selects
 * a faster kernel for k = 4 with 8-bit codes whose worst rows can exceed 1e-3
 * relative error on some inputs; the default kernel holds that bound.
 * B * Hq * Sq < 2^31 and B * Hkv <= 65535. */
fq_status fq_attn_prefill(const fq_codebook* cb, const void* q, const uint8_t* k_codes, const void* k_norms,
                          const uint8_t* v_codes, const void* v_norms, int B, int Hq, int Hkv, int Sq, int64_t T,
                          int causal, float scale, float* out, void* workspace, size_t workspace_bytes,
                          void* stream);

/* ---- Codebook construction on the GPU (FibQuant summary §2.2: the codebook is
 * built offline by Lloyd-Max iterations on samples of the canonical block source
 * of §2.1 / §3.1, i.e. k-blocks of points uniform on the unit sphere S^{d-1}).
 *
 * Generalised Lloyd in fp64 from each of `restarts` starting codebooks:
 *   assignment: every training block y goes to the codeword minimising
 *     ||c||^2 - 2 y.c (lowest index on equal values); its error ||y - c||^2;
 *   update: every codeword becomes the mean of its cell; empty cells, in
 *     increasing index order, are re-seeded at the training blocks with the
 *     largest errors (decreasing error, lowest index on equal errors);
 *   stop: no assignment changed, or the training MSE fell by no more than
 *     rel_tol of itself, or max_iter updates were made.
 * The refined codebook with the lowest validation MSE is kept (the first on
 * equal values) and rounded to the fp16 grid (round to nearest even straight
 * from fp64; |v| < 2^-14 becomes 0), which makes it loadable by
 * fq_codebook_load.  Cell sums are accumulated in 64-bit fixed point, so a
 * build is bit-reproducible on one device.
 *   k:         block length, a power of two <= 64.  N: 1 <= N <= 65536.
 *   train:     device fp64 [m_train][k]; valid: device fp64 [m_valid][k]
 *              (coordinates in [-1, 1]; both < 2^31 rows).
 *   starts:    device fp64 [restarts][N][k] starting codebooks.
 *   codewords: device fp32 [N][k] out (fp16-exact values), 16-byte aligned.
 *   codewords64: device fp64 [N][k] out, the kept codebook before rounding
 *              (may be NULL).
 *   restart_valid_mse: host [restarts] out, validation MSE per block of each
 *              refined codebook before rounding (may be NULL);
 *   valid_mse: host out, validation MSE of the rounded codebook (may be NULL);
 *   history:   host [max_iter + 1] out, training MSE of the kept run after
 *              every assignment (may be NULL); history_len: host out (may be
 *              NULL).
 *   workspace: device, fq_codebook_train_workspace_bytes(...) bytes.
 * fp64 arrays are 8-byte aligned.  Unlike the codec calls this one blocks: it
 * synchronises `stream` after every assignment to decide whether to stop, and
 * returns when the build is done. */
size_t fq_codebook_train_workspace_bytes(int k, int N, int64_t m_train, int64_t m_valid);
fq_status fq_codebook_train(int k, int N, const double* train, int64_t m_train, const double* valid,
                            int64_t m_valid, const double* starts, int restarts, int max_iter, double rel_tol,
                            float* codewords, double* codewords64, double* restart_valid_mse, double* valid_mse,
                            double* history, int* history_len, void* workspace, size_t workspace_bytes,
                            void* stream);

/* Static description of a status code (never NULL). */
const char* fq_status_string(fq_status st);

#ifdef __cplusplus
}
#endif

#endif /* FQ_H */
