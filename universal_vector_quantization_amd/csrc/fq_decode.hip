// FibQuant decoder (FibQuant summary §2.3): gather the codewords of every block
// from the fixed-address store (§1), concatenate them, apply the inverse
// rotation Pi^T and scale by the stored norm.  One lane owns one vector; the
// 64x64 inverse rotation runs as fp32 FMAs with Pi read through the scalar
// cache (every lane of a wave uses the same Pi entry at the same time).
#include "fq_device.h"
#include "fq_internal.h"

namespace fq {
namespace {

constexpr int D = kD;
constexpr int WG = 256;

template <int K, bool NF16, bool OF16>
__global__ __launch_bounds__(WG) void decode_valu(const uint8_t* __restrict__ codes, const void* __restrict__ norms,
                                                  int64_t n, const float* __restrict__ cw,
                                                  const float* __restrict__ pi32, int bits, void* __restrict__ out) {
  constexpr int NB = D / K;
  const int64_t i = (int64_t)fq_bid_x() * WG + fq_tid();
  if (i >= n) return;
  const int B = NB * bits;

  float nu;
  if constexpr (NF16)
    nu = (float)reinterpret_cast<const _Float16*>(norms)[i];
  else
    nu = reinterpret_cast<const float*>(norms)[i];

  float yh[D];
#pragma unroll
  for (int b = 0; b < NB; b++) {
    const uint32_t code = load_code(codes, i * B + (int64_t)b * bits, bits);
#pragma unroll
    for (int t = 0; t < K; t++) yh[b * K + t] = cw[code * K + t];
  }

  float acc[D];
#pragma unroll
  for (int r = 0; r < D; r++) acc[r] = 0.f;
#pragma unroll
  for (int j = 0; j < D; j++) {
#pragma unroll
    for (int r = 0; r < D; r++) acc[r] = fmaf(pi32[j * D + r], yh[j], acc[r]);
  }

  if constexpr (OF16) {
    uint4* o = reinterpret_cast<uint4*>(reinterpret_cast<_Float16*>(out) + i * D);
#pragma unroll
    for (int q = 0; q < D / 8; q++) {
      uint32_t w[4];
#pragma unroll
      for (int h = 0; h < 4; h++) {
        const uint32_t lo = __builtin_bit_cast(uint16_t, (_Float16)(acc[8 * q + 2 * h] * nu));
        const uint32_t hi = __builtin_bit_cast(uint16_t, (_Float16)(acc[8 * q + 2 * h + 1] * nu));
        w[h] = lo | (hi << 16);
      }
      o[q] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  } else {
    float4* o = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + i * D);
#pragma unroll
    for (int q = 0; q < D / 4; q++)
      o[q] = make_float4(acc[4 * q] * nu, acc[4 * q + 1] * nu, acc[4 * q + 2] * nu, acc[4 * q + 3] * nu);
  }
}

}  // namespace

// Launcher for one block size, instantiated per K in its own translation unit.
template <int K>
hipError_t launch_decode_k(const fq_codebook* cb, const uint8_t* codes, const void* norms, fq_dtype nd, int64_t n,
                           void* out, fq_dtype od, hipStream_t s) {
  const dim3 grid((unsigned)((n + WG - 1) / WG)), block(WG);
#define FQ_DEC(NF, OF) \
  hipLaunchKernelGGL((decode_valu<K, NF, OF>), grid, block, 0, s, codes, norms, n, cb->cw, cb->pi32, cb->bits, out)
  if (nd == FQ_F16 && od == FQ_F16)
    FQ_DEC(true, true);
  else if (nd == FQ_F16)
    FQ_DEC(true, false);
  else if (od == FQ_F16)
    FQ_DEC(false, true);
  else
    FQ_DEC(false, false);
#undef FQ_DEC
  return hipGetLastError();
}

#ifdef FQ_ONLY_K
template hipError_t launch_decode_k<FQ_ONLY_K>(const fq_codebook*, const uint8_t*, const void*, fq_dtype, int64_t,
                                               void*, fq_dtype, hipStream_t);
#else
extern template hipError_t launch_decode_k<1>(const fq_codebook*, const uint8_t*, const void*, fq_dtype,
                                                 int64_t, void*, fq_dtype, hipStream_t);
extern template hipError_t launch_decode_k<2>(const fq_codebook*, const uint8_t*, const void*, fq_dtype,
                                                 int64_t, void*, fq_dtype, hipStream_t);
extern template hipError_t launch_decode_k<4>(const fq_codebook*, const uint8_t*, const void*, fq_dtype,
                                                 int64_t, void*, fq_dtype, hipStream_t);
extern template hipError_t launch_decode_k<8>(const fq_codebook*, const uint8_t*, const void*, fq_dtype,
                                                 int64_t, void*, fq_dtype, hipStream_t);
extern template hipError_t launch_decode_k<16>(const fq_codebook*, const uint8_t*, const void*, fq_dtype,
                                                 int64_t, void*, fq_dtype, hipStream_t);
extern template hipError_t launch_decode_k<32>(const fq_codebook*, const uint8_t*, const void*, fq_dtype,
                                                 int64_t, void*, fq_dtype, hipStream_t);
extern template hipError_t launch_decode_k<64>(const fq_codebook*, const uint8_t*, const void*, fq_dtype,
                                                 int64_t, void*, fq_dtype, hipStream_t);

hipError_t launch_decode(const fq_codebook* cb, const uint8_t* codes, const void* norms, fq_dtype norm_dtype,
                         int64_t n, void* x_out, fq_dtype out_dtype, hipStream_t s) {
  if (!cb->force_valu_decode && cb->dec_full)
    return launch_decode_full(cb, codes, norms, norm_dtype, n, x_out, out_dtype, s);
  if (!cb->force_valu_decode && cb->dec_a)
    return launch_decode_mfma(cb, codes, norms, norm_dtype, n, x_out, out_dtype, s);
  switch (cb->k) {
    case 1: return launch_decode_k<1>(cb, codes, norms, norm_dtype, n, x_out, out_dtype, s);
    case 2: return launch_decode_k<2>(cb, codes, norms, norm_dtype, n, x_out, out_dtype, s);
    case 4: return launch_decode_k<4>(cb, codes, norms, norm_dtype, n, x_out, out_dtype, s);
    case 8: return launch_decode_k<8>(cb, codes, norms, norm_dtype, n, x_out, out_dtype, s);
    case 16: return launch_decode_k<16>(cb, codes, norms, norm_dtype, n, x_out, out_dtype, s);
    case 32: return launch_decode_k<32>(cb, codes, norms, norm_dtype, n, x_out, out_dtype, s);
    case 64: return launch_decode_k<64>(cb, codes, norms, norm_dtype, n, x_out, out_dtype, s);
    default: return hipErrorInvalidValue;
  }
}

#endif

}  // namespace fq
