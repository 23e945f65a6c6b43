// Internal declarations shared by the host API and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fq.h"

// Device-resident state behind an fq_codebook handle.  Immutable after load.
struct fq_codebook {
  int d, k, N;
  int bits;   // log2 N
  int nblk;   // d / k
  int B;      // bits per vector = nblk * bits
  int device; // HIP device the buffers live on
  float* cw;        // [N][k] fp32 codewords (fp16-exact values)
  _Float16* cw16;   // [N][k] the same values as fp16
  float* cn2;       // [N] fp32 ||c_n||^2, rounded to nearest from an fp64 sum
  double* pi64t;    // [d][d] Pi transposed, fp64: pi64t[j*d + i] = Pi[i][j]
  float* pi32;      // [d][d] Pi row-major, fp32
  _Float16* rotp;   // [2 row tiles][4 k steps][hi, mid][64 lanes][8]: 1024 Pi as the A operand of
                    // mfma_f32_32x32x16_f16 for the wide prefill's query rotation; row 8 i + 4 hh + j
                    // of tile t is coordinate 32 t + 16 (i / 2) + 8 hh + 4 (i % 2) + j, k is input
                    // 16 s + 8 (lane / 32) + jj
  float cmax;       // max_n ||c_n||, rounded up
  float c2max;      // max_n ||c_n||^2, rounded up
  // Operands of the matrix-core encoder (k = 4 or 8, N a multiple of 32; else null):
  _Float16* amfma;  // [N/32][64 lanes][8]: codeword tile t as the A operand of
                    // mfma_f32_32x32x16_f16 (row = codeword, k = [c | c] for the
                    // hi / lo parts of the scaled query; zeros where unused)
  float* cinit;     // [N/32][2][16]: 256 ||c||^2 of the 16 rows a lane half holds
  float* cn2s;      // [N] 256 ||c_n||^2 (fp32)
  double* pi64m;    // [4 row tiles][16 k steps][64 lanes]: Pi as the A operand of mfma_f64_16x16x4
  double* pi64;     // [d][d] Pi row-major, fp64
  _Float16* dec_a;  // [2 row tiles][4 k steps][hi, lo][64 lanes][8]: Pi^T as the A operand of
                    // mfma_f32_32x32x16_f16 for the decoder (row = output dim, k = input dim)
  // Operands of the fp16-input matrix-core encoder (k = 4 or 8, N a multiple of 32; else null):
  _Float16* rot16;  // [2 k steps][4 row tiles][hi, mid, lo][64 lanes][8]: 1024 Pi split into three
                    // fp16 parts, as the A operand of mfma_f32_16x16x32_f16; row rho of tile r is
                    // coordinate 16 (rho / 4) + 4 r + rho % 4, k is input 32 s + 8 (lane / 16) + j
  _Float16* crec;   // [N][8]: codeword records, k = 4: c0..c3, hi, lo of 256 ||c||^2, 0, 0; k = 8: c0..c7
  // Operands of the k = 16, 32, 64 matrix-core encoder (N a multiple of 32; else null):
  _Float16* rot32;  // [2 row tiles][4 k steps][hi, mid, lo][64 lanes][8]: 1024 Pi as the A operand of
                    // mfma_f32_32x32x16_f16; row 8 a + 4 hh + b of tile r is coordinate 32 hh + 16 r + 4 a + b
  uint8_t* frec;    // [N / 32 tiles][32 rows][2 k + 16 bytes], zero-padded to whole chunks of 8 tiles:
                    // k fp16 coordinates, then a norm slot: for k = d row 4 g's holds fp32
                    // 256 ||c||^2 of rows 4 g .. 4 g + 3 (the others are zero), for k = 16, 32
                    // each row's holds its 256 ||c||^2 as fp16 hi, lo and six zero halves
  float* dec_full;  // k = d only: [N][d] Pi^T c_n in fp32 (rounded once from fp64), the decoded unit
                    // vector of code n, so a full-vector decode is a row gather scaled by the norm
  float h16_eabs, h16_erel;  // its certificate: scores are within h16_eabs + h16_erel |y_b| of exact
  float full_eabs;           // the same for the k = 16, 32, 64 encoder (its longer rotation sums)
  size_t max_lds;   // bytes of LDS one workgroup may use on the device
  int force_encoder;  // FQ_ENCODE_KERNEL at load time (an fq::EncodeKernel): that encoder wherever it covers
                      // the call (valu: every call), else the automatic choice
  bool force_valu_decode;  // FQ_DECODE_KERNEL=valu at load time: the one-lane-per-vector decoder
  bool force_attn_lut;  // FQ_ATTN_KERNEL=lut at load time: the lookup-table attention for k = 4 codebooks too
  bool force_attn_gather;  // FQ_ATTN_KERNEL=gather: the split kernel (global codebook beyond LDS) for k = d too
  bool prefill_wide;  // FQ_PREFILL_KERNEL=wide: the wide prefill kernel for k = 4 / 8-bit codes (faster; rows past the
                     // 1e-3 bar on some inputs, so not the default)
  bool force_cache_codebook;  // FQ_DECODE_KERNEL=cached: the matrix-core decoders read codebooks of more
                              // than 32 KiB from L1 / L2 (the path of devices with less LDS)
};

namespace fq {

constexpr int kD = 64;

// The encoders.  Auto (0) = the automatic choice: Small for batches of at most
// SMALL_ENCODE_MAX vectors, then H16, Full, Mfma, Valu, the first that covers the call.
enum EncodeKernel { ENC_AUTO = 0, ENC_SMALL, ENC_H16, ENC_FULL, ENC_MFMA, ENC_VALU };
// The encoder fq_encode / fq_encode_scatter launch for n vectors of dtype x_dtype.
EncodeKernel encode_kernel(const fq_codebook* cb, fq_dtype x_dtype, int64_t n);
const char* encode_kernel_name(EncodeKernel e);
bool encode_mfma_supported(const fq_codebook* cb);

// Encoder launchers.  With slots == null vector v goes to record v of the code store;
// otherwise to record slots[v] of a store of `cap` records (slots outside [0, cap) are
// skipped), which needs whole-byte records.
// Matrix-core encoder; returns hipErrorNotSupported when the codebook shape is not covered.
hipError_t launch_encode_mfma(const fq_codebook* cb, const void* x, fq_dtype x_dtype, int64_t n, uint8_t* codes,
                              void* norms, fq_dtype norm_dtype, const int64_t* slots, int64_t cap, hipStream_t s);
// Matrix-core encoder for fp16 input (fp16-split rotation); see encode_h16_supported.
bool encode_h16_supported(const fq_codebook* cb);
hipError_t launch_encode_h16(const fq_codebook* cb, const void* x, int64_t n, uint8_t* codes, void* norms,
                             fq_dtype norm_dtype, const int64_t* slots, int64_t cap, hipStream_t s);
// Matrix-core encoder for k = 16, 32 and d = 64 with fp16 input; see encode_full_supported.
bool encode_full_supported(const fq_codebook* cb);
hipError_t launch_encode_full(const fq_codebook* cb, const void* x, int64_t n, uint8_t* codes, void* norms,
                              fq_dtype norm_dtype, const int64_t* slots, int64_t cap, hipStream_t s);
// Small-batch encoder (one wave per vector, fp64 search) for at most SMALL_ENCODE_MAX
// vectors; see encode_small_supported.
constexpr int64_t SMALL_ENCODE_MAX = 2048;
bool encode_small_supported(const fq_codebook* cb);
hipError_t launch_encode_small(const fq_codebook* cb, const void* x, fq_dtype x_dtype, int64_t n, uint8_t* codes,
                               void* norms, fq_dtype norm_dtype, const int64_t* slots, int64_t cap, hipStream_t s);
hipError_t launch_encode(const fq_codebook* cb, const void* x, fq_dtype x_dtype, int64_t n, uint8_t* codes,
                         void* norms, fq_dtype norm_dtype, const int64_t* slots, int64_t cap, hipStream_t s);
hipError_t launch_decode_mfma(const fq_codebook* cb, const uint8_t* codes, const void* norms, fq_dtype norm_dtype,
                              int64_t n, void* x_out, fq_dtype out_dtype, hipStream_t s);
// k = d decoder: gathers rows of dec_full (null dec_full: hipErrorNotSupported).
hipError_t launch_decode_full(const fq_codebook* cb, const uint8_t* codes, const void* norms, fq_dtype norm_dtype,
                              int64_t n, void* x_out, fq_dtype out_dtype, hipStream_t s);
hipError_t launch_decode(const fq_codebook* cb, const uint8_t* codes, const void* norms, fq_dtype norm_dtype,
                         int64_t n, void* x_out, fq_dtype out_dtype, hipStream_t s);

// Split-K plan of the decode attention: partial records per (batch, query head) and
// tokens per record; on the fast path also the 512-token chunks per slab and the
// chunks one workgroup covers.
struct AttnPlan {
  int nchunks;
  int64_t chunk_tokens;
  int fast_chunks;
  int cpw;
  bool fast;
  int lut_heads;  // > 0: the lookup-table kernel with this many query heads per workgroup
};
bool attn_fast_path(const fq_codebook* cb, int Hq, int Hkv, int64_t T);
// Decode attention covers this codebook (its kernel's LDS fits one workgroup).
bool attn_supported(const fq_codebook* cb);
AttnPlan attn_plan(const fq_codebook* cb, int B, int Hq, int Hkv, int64_t T);
size_t attn_workspace_bytes(int B, int Hq, int Hkv, int nchunks);
// Partial records per (batch, query head) the workspace must hold for this plan.
int attn_record_stride(const AttnPlan& p);
// Workspace bytes of a plan: partial records (+ the lookup tables on that path).
size_t attn_plan_workspace_bytes(const fq_codebook* cb, const AttnPlan& p, int B, int Hq, int Hkv);
// The plan's grid fits the launch limits.
bool attn_plan_launchable(const AttnPlan& p, int B, int Hq, int Hkv);

// Lookup-table decode attention (k = d; k = 4 when forced at load time).
bool attn_lut_supported(const fq_codebook* cb);
int attn_lut_heads(const fq_codebook* cb, int G);
size_t attn_lut_table_bytes(const fq_codebook* cb, int B, int Hq);
hipError_t launch_attn_lut(const fq_codebook* cb, const void* q, const uint8_t* k_codes, const void* k_norms,
                           const uint8_t* v_codes, const void* v_norms, const int32_t* lens, int B, int Hq, int Hkv,
                           int64_t T, float scale, const AttnPlan& p, float* out, void* workspace, hipStream_t s);

// Workgroups of `kernel` (block threads, lds bytes of dynamic LDS) resident at once on
// `device`: per-CU occupancy times the CU count, at least 1.  Cached per (kernel, block,
// lds, device) so that launches do not pay for the occupancy query.
hipError_t resident_workgroups(const void* kernel, int block, size_t lds, int device, int64_t* out);
// lens == null: every batch attends to all T keys; else batch b to its first
// min(max(lens[b], 0), T) keys.
hipError_t launch_attn(const fq_codebook* cb, const void* q, const uint8_t* k_codes, const void* k_norms,
                       const uint8_t* v_codes, const void* v_norms, const int32_t* lens, int B, int Hq, int Hkv,
                       int64_t T, float scale, float* out, void* workspace, hipStream_t s);

// Log-sum-exp merge of `rows` rows of nchunks partial records each (m, l, acc[64] in the
// rotated domain) and the inverse rotation: out[row][64].
hipError_t launch_attn_combine(const float* ws, const float* pi32, int64_t rows, int nchunks, float* out,
                               hipStream_t s);

// Multi-query (prefill) attention.  Split over keys into nchunks ranges of chunk_tokens
// keys, 128 (k = 4 with 8-bit codes) or 64 query rows per workgroup.
struct PrefillPlan {
  int nchunks;
  int64_t chunk_tokens;
  int rblocks;
};
PrefillPlan prefill_plan(const fq_codebook* cb, int B, int Hq, int Hkv, int Sq, int64_t T);
bool prefill_supported(const fq_codebook* cb);
hipError_t launch_prefill(const fq_codebook* cb, const void* q, const uint8_t* k_codes, const void* k_norms,
                          const uint8_t* v_codes, const void* v_norms, int B, int Hq, int Hkv, int Sq, int64_t T,
                          int causal, float scale, float* out, void* workspace, hipStream_t s);

// Codebook construction (generalised Lloyd over fp64 training blocks, several starts,
// validation selection, fp16 grid); blocking: synchronises `s` every iteration.
size_t train_workspace_bytes(int k, int N, int64_t m_train, int64_t m_valid);
hipError_t train_codebook(int k, int N, const double* train, int64_t mt, const double* valid, int64_t mv,
                          const double* starts, int restarts, int max_iter, double rel_tol, float* out, double* out64,
                          double* restart_mse, double* valid_mse, double* history, int* history_len, void* ws,
                          hipStream_t s);

}  // namespace fq
