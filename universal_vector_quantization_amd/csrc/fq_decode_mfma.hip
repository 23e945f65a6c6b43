// Matrix-core FibQuant decoder (FibQuant summary §2.3: gather the codewords,
// concatenate the blocks, inverse rotation, scale by the norm; §1: every
// vector decodes alone from its fixed-address record).
//
// A wave decodes 32 vectors per step: x^T[64 x 32] = Pi^T[64 x 64] yhat^T[64 x 32]
// with mfma_f32_32x32x16_f16.  yhat holds fp16-exact codewords, so it is an
// exact fp16 operand; Pi^T is split into fp16 hi + lo (22 bits), accumulation
// is fp32.  Lane l owns vector l % 32 and, per 16-dim k-step, 8 consecutive
// input dims (whole codewords for k <= 8), which it gathers from the codebook
// (LDS copy when it fits, else the fp16 copy in global memory).  The result
// rows a lane holds are 4 runs of 4 consecutive output dims per 32-dim tile,
// written as 8-byte (fp16) or 16-byte (fp32) stores.
#include "fq_device.h"
#include "fq_internal.h"

namespace fq {
namespace {

constexpr int D = kD;
constexpr int WAVES = 4;
constexpr int LDS_CB_HALFS = 16384;  // 32 KiB: codebooks up to N*k = 16384 live in LDS

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Input dims [d0, d0 + 8) of the vector whose record starts at bit `rec`.
template <int K>
__device__ inline half8 gather8(const _Float16* __restrict__ cb, const uint8_t* __restrict__ codes, int64_t rec,
                                int d0, int bits) {
  half8 r;
  if constexpr (K >= 8) {
    const uint32_t code = load_code(codes, rec + (int64_t)(d0 / K) * bits, bits);
    r = *reinterpret_cast<const half8*>(cb + (size_t)code * K + (d0 % K));
  } else {
#pragma unroll
    for (int p = 0; p < 8 / K; p++) {
      const uint32_t code = load_code(codes, rec + (int64_t)(d0 / K + p) * bits, bits);
#pragma unroll
      for (int t = 0; t < K; t++) r[p * K + t] = cb[(size_t)code * K + t];
    }
  }
  return r;
}

template <int K, bool NF16, bool OF16>
__global__ __launch_bounds__(WAVES * 64) void decode_mfma(const uint8_t* __restrict__ codes,
                                                          const void* __restrict__ norms, int64_t n,
                                                          const _Float16* __restrict__ cw16,
                                                          const half8* __restrict__ dec_a, int N, int bits,
                                                          void* __restrict__ out) {
  __shared__ __align__(16) _Float16 cbL[LDS_CB_HALFS];
  const int lane = fq_tid() & 63, w = fq_tid() >> 6;
  const int col = lane & 31, h = lane >> 5;
  const bool in_lds = N * K <= LDS_CB_HALFS;
  if (in_lds) {
    for (int i = fq_tid(); i < N * K * 2 / 16; i += WAVES * 64)
      reinterpret_cast<uint4*>(cbL)[i] = reinterpret_cast<const uint4*>(cw16)[i];
    __syncthreads();
  }
  const _Float16* cb = in_lds ? cbL : cw16;
  const int64_t v = ((int64_t)fq_bid_x() * WAVES + w) * 32 + col;
  const bool valid = v < n;
  const int B = (D / K) * bits;

  float nu = 0.f;
  if (valid) {
    if constexpr (NF16)
      nu = (float)reinterpret_cast<const _Float16*>(norms)[v];
    else
      nu = reinterpret_cast<const float*>(norms)[v];
  }
  f32x16 acc[2];
#pragma unroll
  for (int r = 0; r < 2; r++)
#pragma unroll
    for (int e = 0; e < 16; e++) acc[r][e] = 0.f;
#pragma unroll
  for (int s = 0; s < 4; s++) {
    half8 yb = {};
    if (valid) yb = gather8<K>(cb, codes, v * B, 16 * s + 8 * h, bits);
#pragma unroll
    for (int r = 0; r < 2; r++) {
      const half8 ahi = dec_a[((r * 4 + s) * 2 + 0) * 64 + lane];
      const half8 alo = dec_a[((r * 4 + s) * 2 + 1) * 64 + lane];
      acc[r] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi, yb, acc[r], 0, 0, 0);
      acc[r] = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo, yb, acc[r], 0, 0, 0);
    }
  }
  if (!valid) return;
#pragma unroll
  for (int r = 0; r < 2; r++) {
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int o = 32 * r + 8 * q + 4 * h;  // rows 8q + 4h + i of tile r
      if constexpr (OF16) {
        half4 hv;
#pragma unroll
        for (int i = 0; i < 4; i++) hv[i] = (_Float16)(acc[r][4 * q + i] * nu);
        *reinterpret_cast<half4*>(reinterpret_cast<_Float16*>(out) + v * D + o) = hv;
      } else {
        float4 fv = make_float4(acc[r][4 * q] * nu, acc[r][4 * q + 1] * nu, acc[r][4 * q + 2] * nu,
                                acc[r][4 * q + 3] * nu);
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + v * D + o) = fv;
      }
    }
  }
}

template <int K>
hipError_t launch_k(const fq_codebook* cb, const uint8_t* codes, const void* norms, fq_dtype nd, int64_t n,
                    void* out, fq_dtype od, hipStream_t s) {
  const dim3 grid((unsigned)((n + WAVES * 32 - 1) / (WAVES * 32))), block(WAVES * 64);
  const half8* da = reinterpret_cast<const half8*>(cb->dec_a);
#define FQ_DM(NF, OF)                                                                                      \
  hipLaunchKernelGGL((decode_mfma<K, NF, OF>), grid, block, 0, s, codes, norms, n, cb->cw16, da, cb->N,   \
                     cb->bits, out)
  if (nd == FQ_F16 && od == FQ_F16)
    FQ_DM(true, true);
  else if (nd == FQ_F16)
    FQ_DM(true, false);
  else if (od == FQ_F16)
    FQ_DM(false, true);
  else
    FQ_DM(false, false);
#undef FQ_DM
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_mfma(const fq_codebook* cb, const uint8_t* codes, const void* norms, fq_dtype norm_dtype,
                              int64_t n, void* x_out, fq_dtype out_dtype, hipStream_t s) {
  switch (cb->k) {
    case 1: return launch_k<1>(cb, codes, norms, norm_dtype, n, x_out, out_dtype, s);
    case 2: return launch_k<2>(cb, codes, norms, norm_dtype, n, x_out, out_dtype, s);
    case 4: return launch_k<4>(cb, codes, norms, norm_dtype, n, x_out, out_dtype, s);
    case 8: return launch_k<8>(cb, codes, norms, norm_dtype, n, x_out, out_dtype, s);
    case 16: return launch_k<16>(cb, codes, norms, norm_dtype, n, x_out, out_dtype, s);
    case 32: return launch_k<32>(cb, codes, norms, norm_dtype, n, x_out, out_dtype, s);
    case 64: return launch_k<64>(cb, codes, norms, norm_dtype, n, x_out, out_dtype, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fq
