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
  float cmax;       // max_n ||c_n||, rounded up
  float c2max;      // max_n ||c_n||^2, rounded up
};

namespace fq {

constexpr int kD = 64;

hipError_t launch_encode(const fq_codebook* cb, const void* x, fq_dtype x_dtype, int64_t n, uint8_t* codes,
                         void* norms, fq_dtype norm_dtype, hipStream_t s);
hipError_t launch_decode(const fq_codebook* cb, const uint8_t* codes, const void* norms, fq_dtype norm_dtype,
                         int64_t n, void* x_out, fq_dtype out_dtype, hipStream_t s);

// Split-K plan of the decode attention: number of chunks and tokens per chunk.
struct AttnPlan {
  int nchunks;
  int64_t chunk_tokens;
};
AttnPlan attn_plan(int B, int Hkv, int64_t T);
size_t attn_workspace_bytes(int B, int Hq, int nchunks);
hipError_t launch_attn(const fq_codebook* cb, const void* q, const uint8_t* k_codes, const void* k_norms,
                       const uint8_t* v_codes, const void* v_norms, int B, int Hq, int Hkv, int64_t T, float scale,
                       float* out, void* workspace, hipStream_t s);

}  // namespace fq
