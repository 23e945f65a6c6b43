// FibQuant encoder (FibQuant summary §2.3): norm, rotation, d/k blocks of k
// consecutive coordinates, nearest codeword per block, fixed-address packing
// (§1).  For k <= 16 a workgroup of 4 waves owns 64 vectors and wave q the
// coordinates 16 q .. 16 q + 15 of every one (lane = vector), so Pi and the
// codebook are read with wave-uniform addresses and a lane holds a quarter of
// a vector's state; for k = 32, 64 one lane owns one vector.
//
// Precision plan (the codes must be the exact nearest codewords):
//   * nu and y = Pi x / nu are computed in fp64 (products of fp32 Pi entries and
//     fp16/fp32 inputs are exact in fp64), then y is rounded to fp32.
//   * Search: score_n = ||c_n||^2 - 2 y_b . c_n with an fp32 FMA chain; each lane
//     keeps the best and second-best score and the best index per block.
//   * Certificate: every fp32 score is within E_b of the exact score, with
//       E_b = 1.01 (k+2) 2^-24 (max||c||^2 + 2 ||y_b|| max||c||)
//     (k FMA roundings, the rounding of ||c||^2 and of y, first order).  If
//     second - best > 2 E_b the fp32 winner is the exact unique minimiser.
//   * Otherwise the block is searched again in fp64 with the direct distance
//     sum_t (y_t - c_t)^2, lowest index on exact ties.
#include <type_traits>

#include "fq_device.h"
#include "fq_internal.h"

namespace fq {
namespace {

constexpr int D = kD;
constexpr int WG = 256;

template <bool F16>
__device__ inline void load_row(const void* __restrict__ xv, int64_t i, float (&xf)[D]) {
  if constexpr (F16) {
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const _Float16*>(xv) + i * D);
#pragma unroll
    for (int q = 0; q < D / 8; q++) {
      uint4 w = p[q];
      uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int h = 0; h < 4; h++) {
        xf[8 * q + 2 * h] = (float)__builtin_bit_cast(_Float16, (uint16_t)(ws[h] & 0xffffu));
        xf[8 * q + 2 * h + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(ws[h] >> 16));
      }
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(xv) + i * D);
#pragma unroll
    for (int q = 0; q < D / 4; q++) {
      float4 w = p[q];
      xf[4 * q] = w.x;
      xf[4 * q + 1] = w.y;
      xf[4 * q + 2] = w.z;
      xf[4 * q + 3] = w.w;
    }
  }
}

// Inputs j0 .. j0 + 7 of a row (fp16 or fp32), zeros for a vector past the end.
template <bool F16>
using row_t = typename std::conditional<F16, const _Float16*, const float*>::type;
template <bool F16>
__device__ inline void load_piece(row_t<F16> row, int j0, bool valid, float (&v)[8]) {
  if (!valid) {
#pragma unroll
    for (int j = 0; j < 8; j++) v[j] = 0.f;
    return;
  }
  if constexpr (F16) {
    const uint4 w = *reinterpret_cast<const uint4*>(row + j0);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int h = 0; h < 4; h++) {
      v[2 * h] = (float)__builtin_bit_cast(_Float16, (uint16_t)(ws[h] & 0xffffu));
      v[2 * h + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(ws[h] >> 16));
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(row + j0), b = *reinterpret_cast<const float4*>(row + j0 + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <int K, bool XF16, bool NF16>
__global__ __launch_bounds__(WG) void encode_valu(const void* __restrict__ xv, int64_t n,
                                                  const float* __restrict__ cw, const float* __restrict__ cn2,
                                                  const double* __restrict__ pi64t, int N, int bits, float cmax,
                                                  float c2max, uint8_t* __restrict__ codes, void* __restrict__ norms,
                                                  const int64_t* __restrict__ slots, int64_t cap) {
  constexpr int NB = D / K;
  constexpr int PK_WORDS = 2 * NB * 16;  // 64 lanes * B bits / 32, for bits <= 16
  __shared__ uint32_t pk[WG / 64][PK_WORDS];

  const int lane = fq_tid() & 63;
  const int wave = fq_tid() >> 6;
  const int64_t i = (int64_t)fq_bid_x() * WG + fq_tid();
  const bool valid = i < n;
  const int B = NB * bits;

  // ---- norm and fp64 rotation
  float xf[D];
  if (valid) {
    load_row<XF16>(xv, i, xf);
  } else {
#pragma unroll
    for (int j = 0; j < D; j++) xf[j] = 0.f;
  }
  double nu2 = 0.0;
#pragma unroll
  for (int j = 0; j < D; j++) nu2 = fma((double)xf[j], (double)xf[j], nu2);
  const double nu = sqrt(nu2);
  const double inv = nu > 0.0 ? 1.0 / nu : 0.0;

  float m2y[D];  // -2 y in fp32 (exact doubling of the rounded y)
#pragma unroll
  for (int p = 0; p < 2; p++) {
    double acc[D / 2];
#pragma unroll
    for (int r = 0; r < D / 2; r++) acc[r] = 0.0;
#pragma unroll
    for (int j = 0; j < D; j++) {
      const double xj = (double)xf[j];
#pragma unroll
      for (int r = 0; r < D / 2; r++) acc[r] = fma(pi64t[j * D + p * (D / 2) + r], xj, acc[r]);
    }
#pragma unroll
    for (int r = 0; r < D / 2; r++) m2y[p * (D / 2) + r] = -2.0f * (float)(acc[r] * inv);
  }

  // ---- fp32 search with best / second-best per block
  float m1[NB], m2[NB];
  int ix[NB];
#pragma unroll
  for (int b = 0; b < NB; b++) {
    m1[b] = __builtin_huge_valf();
    m2[b] = __builtin_huge_valf();
    ix[b] = 0;
  }
  for (int nn = 0; nn < N; nn++) {
    float c[K];
#pragma unroll
    for (int t = 0; t < K; t++) c[t] = cw[nn * K + t];
    const float cn = cn2[nn];
#pragma unroll
    for (int b = 0; b < NB; b++) {
      float s = cn;
#pragma unroll
      for (int t = 0; t < K; t++) s = fmaf(m2y[b * K + t], c[t], s);
      m2[b] = __builtin_amdgcn_fmed3f(m1[b], m2[b], s);
      const bool lt = s < m1[b];
      ix[b] = lt ? nn : ix[b];
      m1[b] = lt ? s : m1[b];
    }
  }

  // ---- certificate: blocks whose fp32 winner is not provably exact
  const double u = 5.9604644775390625e-08;  // 2^-24
  uint64_t unsure = 0;
#pragma unroll
  for (int b = 0; b < NB; b++) {
    float yn2 = 0.f;
#pragma unroll
    for (int t = 0; t < K; t++) yn2 = fmaf(m2y[b * K + t], m2y[b * K + t], yn2);
    const double yn = 0.5 * sqrt((double)yn2) * 1.01;  // ||y_b||, rounded up
    const double E = 1.01 * (K + 2) * u * ((double)c2max + 2.0 * yn * (double)cmax);
    if (!(((double)m2[b] - (double)m1[b]) > 2.0 * E)) unsure |= 1ull << b;
  }
  if (!valid) unsure = 0;

  // ---- norm store (fp64 -> storage dtype, one rounding)
  const int64_t slot = valid ? out_slot(slots, cap, i) : -1;
  if (slot >= 0) {
    if constexpr (NF16)
      reinterpret_cast<uint16_t*>(norms)[slot] = f64_to_f16_bits(nu);
    else
      reinterpret_cast<float*>(norms)[slot] = (float)nu;
  }

  // ---- pack this wave's 64 records (64*B bits, dword aligned) through LDS
  for (int w = lane; w < 2 * B; w += 64) pk[wave][w] = 0u;
  __syncthreads();
  const uint32_t cmask = (1u << bits) - 1u;
  if (valid) {
#pragma unroll
    for (int b = 0; b < NB; b++) {
      const uint32_t code = (uint32_t)ix[b];
      const int bo = lane * B + b * bits;
      const int sh = bo & 31;
      atomicOr(&pk[wave][bo >> 5], code << sh);
      if (sh + bits > 32) atomicOr(&pk[wave][(bo >> 5) + 1], code >> (32 - sh));
    }
  }

  // ---- fp64 direct-distance search of the uncertified blocks; patch their bits
  if (unsure) {
    float xr[D];
    load_row<XF16>(xv, i, xr);
    while (unsure) {
      const int b = __builtin_ctzll(unsure);
      unsure &= unsure - 1;
      double yb[K];
#pragma unroll
      for (int t = 0; t < K; t++) {
        double a = 0.0;
#pragma unroll
        for (int j = 0; j < D; j++) a = fma(pi64t[j * D + b * K + t], (double)xr[j], a);
        yb[t] = a * inv;
      }
      double best = __builtin_huge_val();
      uint32_t bi = 0;
      for (int nn = 0; nn < N; nn++) {
        double dd = 0.0;
#pragma unroll
        for (int t = 0; t < K; t++) {
          const double df = yb[t] - (double)cw[nn * K + t];
          dd = fma(df, df, dd);
        }
        if (dd < best) {
          best = dd;
          bi = (uint32_t)nn;
        }
      }
      const int bo = lane * B + b * bits;
      const int sh = bo & 31;
      atomicAnd(&pk[wave][bo >> 5], ~(cmask << sh));
      atomicOr(&pk[wave][bo >> 5], bi << sh);
      if (sh + bits > 32) {
        atomicAnd(&pk[wave][(bo >> 5) + 1], ~(cmask >> (32 - sh)));
        atomicOr(&pk[wave][(bo >> 5) + 1], bi >> (32 - sh));
      }
    }
  }
  __syncthreads();
  const int64_t v0 = i - lane;
  if (slots) {
    if (v0 < n) scatter_records(pk[wave], (n - v0) < 64 ? (int)(n - v0) : 64, B / 8, slots, cap, v0, codes, lane);
  } else if (v0 < n) {
    const int64_t nv = (n - v0) < 64 ? (n - v0) : 64;
    const int64_t nbytes = (nv * B + 7) / 8;
    uint8_t* dst = codes + (v0 / 64) * (int64_t)(8 * B);
    const int nfull = (int)(nbytes / 4);
    for (int w = lane; w < nfull; w += 64) reinterpret_cast<uint32_t*>(dst)[w] = pk[wave][w];
    const int rem = (int)(nbytes - 4 * (int64_t)nfull);
    if (lane < rem) dst[4 * nfull + lane] = (uint8_t)((pk[wave][nfull] >> (8 * lane)) & 0xffu);
  }
}

// k <= 16: wave q of the workgroup takes coordinates 16 q .. 16 q + 15 (blocks
// 16 q / k ..) of the workgroup's 64 vectors; records are assembled in LDS by all
// four waves and stored by the workgroup.
template <int K, bool XF16, bool NF16>
__global__ __launch_bounds__(WG) void encode_valu_q(const void* __restrict__ xv, int64_t n,
                                                    const float* __restrict__ cw, const float* __restrict__ cn2,
                                                    const double* __restrict__ pi64t, int N, int bits, float cmax,
                                                    float c2max, uint8_t* __restrict__ codes, void* __restrict__ norms,
                                                    const int64_t* __restrict__ slots, int64_t cap) {
  static_assert(K <= 16, "a quarter of a vector holds whole blocks");
  constexpr int QC = 16;       // coordinates per wave
  constexpr int NBQ = QC / K;  // blocks per lane
  constexpr int NB = D / K;
  __shared__ uint32_t pk[2 * NB * 16];  // 64 records of B = NB bits <= 16 bits each

  const int lane = fq_tid() & 63;
  const int q = __builtin_amdgcn_readfirstlane(fq_tid() >> 6);
  const int64_t v0 = (int64_t)fq_bid_x() * 64;
  const int64_t i = v0 + lane;
  const bool valid = i < n;
  const int B = NB * bits;

  // ---- norm and fp64 rotation of this quarter in one pass over the row, 8 inputs at
  //      a time (a row held whole in registers would cost 64 of them through the search)
  const double* piq = pi64t + QC * q;  // pi64t[j D + 16 q + t] = Pi[16 q + t][j], wave-uniform
  // this lane's input row (only read when the vector exists)
  const row_t<XF16> xrow = reinterpret_cast<row_t<XF16>>(xv) + (valid ? i : 0) * D;
  double acc[QC];
#pragma unroll
  for (int t = 0; t < QC; t++) acc[t] = 0.0;
  double nu2 = 0.0;
#pragma unroll 1
  for (int j0 = 0; j0 < D; j0 += 8) {
    float xp[8];
    load_piece<XF16>(xrow, j0, valid, xp);
#pragma unroll
    for (int jj = 0; jj < 8; jj++) {
      const double xj = (double)xp[jj];
      nu2 = fma(xj, xj, nu2);
#pragma unroll
      for (int t = 0; t < QC; t++) acc[t] = fma(piq[(j0 + jj) * D + t], xj, acc[t]);
    }
  }
  const double nu = sqrt(nu2);
  const double inv = nu > 0.0 ? 1.0 / nu : 0.0;
  float m2y[QC];  // -2 y in fp32 (exact doubling of the rounded y)
#pragma unroll
  for (int t = 0; t < QC; t++) m2y[t] = -2.0f * (float)(acc[t] * inv);

  // ---- fp32 search with best / second-best per block
  float m1[NBQ], m2[NBQ];
  int ix[NBQ];
#pragma unroll
  for (int b = 0; b < NBQ; b++) {
    m1[b] = __builtin_huge_valf();
    m2[b] = __builtin_huge_valf();
    ix[b] = 0;
  }
  for (int nn = 0; nn < N; nn++) {
    float c[K];
#pragma unroll
    for (int t = 0; t < K; t++) c[t] = cw[nn * K + t];
    const float cn = cn2[nn];
#pragma unroll
    for (int b = 0; b < NBQ; b++) {
      float sc = cn;
#pragma unroll
      for (int t = 0; t < K; t++) sc = fmaf(m2y[b * K + t], c[t], sc);
      m2[b] = __builtin_amdgcn_fmed3f(m1[b], m2[b], sc);
      const bool lt = sc < m1[b];
      ix[b] = lt ? nn : ix[b];
      m1[b] = lt ? sc : m1[b];
    }
  }

  // ---- certificate (as in encode_valu)
  const double u = 5.9604644775390625e-08;  // 2^-24
  uint32_t unsure = 0;
#pragma unroll
  for (int b = 0; b < NBQ; b++) {
    float yn2 = 0.f;
#pragma unroll
    for (int t = 0; t < K; t++) yn2 = fmaf(m2y[b * K + t], m2y[b * K + t], yn2);
    const double yn = 0.5 * sqrt((double)yn2) * 1.01;  // ||y_b||, rounded up
    const double E = 1.01 * (K + 2) * u * ((double)c2max + 2.0 * yn * (double)cmax);
    if (!(((double)m2[b] - (double)m1[b]) > 2.0 * E)) unsure |= 1u << b;
  }
  if (!valid) unsure = 0;

  // ---- norm store (fp64 -> storage dtype, one rounding), by the first wave
  const int64_t slot = valid ? out_slot(slots, cap, i) : -1;
  if (q == 0 && slot >= 0) {
    if constexpr (NF16)
      reinterpret_cast<uint16_t*>(norms)[slot] = f64_to_f16_bits(nu);
    else
      reinterpret_cast<float*>(norms)[slot] = (float)nu;
  }

  // ---- pack the 64 records (64 B bits, dword aligned) through LDS
  for (int w = fq_tid(); w < 2 * B; w += WG) pk[w] = 0u;
  __syncthreads();
  const uint32_t cmask = (1u << bits) - 1u;
  if (valid) {
#pragma unroll
    for (int b = 0; b < NBQ; b++) {
      const uint32_t code = (uint32_t)ix[b];
      const int bo = lane * B + (q * NBQ + b) * bits;
      const int sh = bo & 31;
      atomicOr(&pk[bo >> 5], code << sh);
      if (sh + bits > 32) atomicOr(&pk[(bo >> 5) + 1], code >> (32 - sh));
    }
  }

  // ---- fp64 direct-distance search of the uncertified blocks (y_b from the input row
  //      again, 8 inputs at a time); patch their bits
  while (unsure) {
    const int b = __builtin_ctz(unsure);
    unsure &= unsure - 1;
    double yb[K];
#pragma unroll
    for (int t = 0; t < K; t++) yb[t] = 0.0;
#pragma unroll 1
    for (int j0 = 0; j0 < D; j0 += 8) {
      float xp[8];
      load_piece<XF16>(xrow, j0, true, xp);
#pragma unroll
      for (int jj = 0; jj < 8; jj++)
#pragma unroll
        for (int t = 0; t < K; t++) yb[t] = fma(piq[(j0 + jj) * D + b * K + t], (double)xp[jj], yb[t]);
    }
#pragma unroll
    for (int t = 0; t < K; t++) yb[t] *= inv;
    double best = __builtin_huge_val();
    uint32_t bi = 0;
    for (int nn = 0; nn < N; nn++) {
      double dd = 0.0;
#pragma unroll
      for (int t = 0; t < K; t++) {
        const double df = yb[t] - (double)cw[nn * K + t];
        dd = fma(df, df, dd);
      }
      if (dd < best) {
        best = dd;
        bi = (uint32_t)nn;
      }
    }
    const int bo = lane * B + (q * NBQ + b) * bits;
    const int sh = bo & 31;
    atomicAnd(&pk[bo >> 5], ~(cmask << sh));
    atomicOr(&pk[bo >> 5], bi << sh);
    if (sh + bits > 32) {
      atomicAnd(&pk[(bo >> 5) + 1], ~(cmask >> (32 - sh)));
      atomicOr(&pk[(bo >> 5) + 1], bi >> (32 - sh));
    }
  }
  __syncthreads();
  if (v0 >= n) return;
  const int nv = (n - v0) < 64 ? (int)(n - v0) : 64;
  if (slots) {
    if (q == 0) scatter_records(pk, nv, B / 8, slots, cap, v0, codes, lane);
  } else {
    const int64_t nbytes = ((int64_t)nv * B + 7) / 8;
    uint8_t* dst = codes + (v0 / 64) * (int64_t)(8 * B);
    const int nfull = (int)(nbytes / 4);
    for (int w = fq_tid(); w < nfull; w += WG) reinterpret_cast<uint32_t*>(dst)[w] = pk[w];
    const int rem = (int)(nbytes - 4 * (int64_t)nfull);
    if (fq_tid() < rem) dst[4 * nfull + fq_tid()] = (uint8_t)((pk[nfull] >> (8 * fq_tid())) & 0xffu);
  }
}

}  // namespace

namespace {
template <int K, bool XF, bool NF>
void launch_valu(const fq_codebook* cb, const void* x, int64_t n, uint8_t* codes, void* norms, const int64_t* slots,
                 int64_t cap, hipStream_t s) {
  if constexpr (K <= 16) {  // a workgroup per 64 vectors, a wave per quarter
    hipLaunchKernelGGL((encode_valu_q<K, XF, NF>), dim3((unsigned)((n + 63) / 64)), dim3(WG), 0, s, x, n, cb->cw,
                       cb->cn2, cb->pi64t, cb->N, cb->bits, cb->cmax, cb->c2max, codes, norms, slots, cap);
  } else {  // a lane per vector
    hipLaunchKernelGGL((encode_valu<K, XF, NF>), dim3((unsigned)((n + WG - 1) / WG)), dim3(WG), 0, s, x, n, cb->cw,
                       cb->cn2, cb->pi64t, cb->N, cb->bits, cb->cmax, cb->c2max, codes, norms, slots, cap);
  }
}
}  // namespace

// Launcher for one block size; each K is instantiated in its own translation
// unit (compiled with -DFQ_ONLY_K=K) so the build can run in parallel.
template <int K>
hipError_t launch_encode_k(const fq_codebook* cb, const void* x, fq_dtype xd, int64_t n, uint8_t* codes,
                           void* norms, fq_dtype nd, const int64_t* slots, int64_t cap, hipStream_t s) {
  const bool xf16 = xd == FQ_F16, nf16 = nd == FQ_F16;
  if (xf16 && nf16)
    launch_valu<K, true, true>(cb, x, n, codes, norms, slots, cap, s);
  else if (xf16)
    launch_valu<K, true, false>(cb, x, n, codes, norms, slots, cap, s);
  else if (nf16)
    launch_valu<K, false, true>(cb, x, n, codes, norms, slots, cap, s);
  else
    launch_valu<K, false, false>(cb, x, n, codes, norms, slots, cap, s);
  return hipGetLastError();
}

#ifdef FQ_ONLY_K
template hipError_t launch_encode_k<FQ_ONLY_K>(const fq_codebook*, const void*, fq_dtype, int64_t, uint8_t*, void*,
                                               fq_dtype, const int64_t*, int64_t, hipStream_t);
#else
extern template hipError_t launch_encode_k<1>(const fq_codebook*, const void*, fq_dtype, int64_t, uint8_t*,
                                                 void*, fq_dtype, const int64_t*, int64_t, hipStream_t);
extern template hipError_t launch_encode_k<2>(const fq_codebook*, const void*, fq_dtype, int64_t, uint8_t*,
                                                 void*, fq_dtype, const int64_t*, int64_t, hipStream_t);
extern template hipError_t launch_encode_k<4>(const fq_codebook*, const void*, fq_dtype, int64_t, uint8_t*,
                                                 void*, fq_dtype, const int64_t*, int64_t, hipStream_t);
extern template hipError_t launch_encode_k<8>(const fq_codebook*, const void*, fq_dtype, int64_t, uint8_t*,
                                                 void*, fq_dtype, const int64_t*, int64_t, hipStream_t);
extern template hipError_t launch_encode_k<16>(const fq_codebook*, const void*, fq_dtype, int64_t, uint8_t*,
                                                 void*, fq_dtype, const int64_t*, int64_t, hipStream_t);
extern template hipError_t launch_encode_k<32>(const fq_codebook*, const void*, fq_dtype, int64_t, uint8_t*,
                                                 void*, fq_dtype, const int64_t*, int64_t, hipStream_t);
extern template hipError_t launch_encode_k<64>(const fq_codebook*, const void*, fq_dtype, int64_t, uint8_t*,
                                                 void*, fq_dtype, const int64_t*, int64_t, hipStream_t);

namespace {
bool covers(const fq_codebook* cb, EncodeKernel e, fq_dtype x_dtype, int64_t n) {
  switch (e) {
    case ENC_SMALL: return n <= SMALL_ENCODE_MAX && encode_small_supported(cb);
    case ENC_H16: return x_dtype == FQ_F16 && encode_h16_supported(cb);
    case ENC_FULL: return x_dtype == FQ_F16 && encode_full_supported(cb);
    case ENC_MFMA: return encode_mfma_supported(cb);
    case ENC_VALU: return true;
    default: return false;
  }
}
}  // namespace

EncodeKernel encode_kernel(const fq_codebook* cb, fq_dtype x_dtype, int64_t n) {
  const EncodeKernel forced = (EncodeKernel)cb->force_encoder;
  if (forced != ENC_AUTO && covers(cb, forced, x_dtype, n)) return forced;
  // a few vectors (the decode loop's append): latency of one launch is what counts
  for (EncodeKernel e : {ENC_SMALL, ENC_H16, ENC_FULL, ENC_MFMA})
    if (covers(cb, e, x_dtype, n)) return e;
  return ENC_VALU;
}

const char* encode_kernel_name(EncodeKernel e) {
  switch (e) {
    case ENC_SMALL: return "encode_wave";
    case ENC_H16: return "encode_h16";
    case ENC_FULL: return "encode_full";
    case ENC_MFMA: return "encode_mfma";
    case ENC_VALU: return "encode_valu";
    default: return "none";
  }
}

hipError_t launch_encode(const fq_codebook* cb, const void* x, fq_dtype x_dtype, int64_t n, uint8_t* codes,
                         void* norms, fq_dtype norm_dtype, const int64_t* slots, int64_t cap, hipStream_t s) {
  switch (encode_kernel(cb, x_dtype, n)) {
    case ENC_SMALL: return launch_encode_small(cb, x, x_dtype, n, codes, norms, norm_dtype, slots, cap, s);
    case ENC_H16: return launch_encode_h16(cb, x, n, codes, norms, norm_dtype, slots, cap, s);
    case ENC_FULL: return launch_encode_full(cb, x, n, codes, norms, norm_dtype, slots, cap, s);
    case ENC_MFMA: return launch_encode_mfma(cb, x, x_dtype, n, codes, norms, norm_dtype, slots, cap, s);
    default: break;
  }
  switch (cb->k) {
    case 1: return launch_encode_k<1>(cb, x, x_dtype, n, codes, norms, norm_dtype, slots, cap, s);
    case 2: return launch_encode_k<2>(cb, x, x_dtype, n, codes, norms, norm_dtype, slots, cap, s);
    case 4: return launch_encode_k<4>(cb, x, x_dtype, n, codes, norms, norm_dtype, slots, cap, s);
    case 8: return launch_encode_k<8>(cb, x, x_dtype, n, codes, norms, norm_dtype, slots, cap, s);
    case 16: return launch_encode_k<16>(cb, x, x_dtype, n, codes, norms, norm_dtype, slots, cap, s);
    case 32: return launch_encode_k<32>(cb, x, x_dtype, n, codes, norms, norm_dtype, slots, cap, s);
    case 64: return launch_encode_k<64>(cb, x, x_dtype, n, codes, norms, norm_dtype, slots, cap, s);
    default: return hipErrorInvalidValue;
  }
}

#endif

}  // namespace fq
