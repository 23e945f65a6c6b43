// Matrix-core FibQuant encoder for block sizes k = 4 and 8 (FibQuant summary
// §2.3: norm, Haar rotation of the unit vector, d/k blocks of k consecutive
// coordinates, nearest codeword; §1: fixed-address codes).
//
// A wave owns a "group" of 256 blocks (16 vectors for k = 4, 32 for k = 8) at a
// time and loops over groups (persistent grid).  Per group:
//   1. x -> LDS; nu in fp64 (one lane per vector).
//   2. y = Pi x with mfma_f64_16x16x4 (fp64: products of fp32 Pi and fp16/fp32 x
//      are exact, sums carry ~1e-16 error), scaled by 1/nu, stored to LDS as fp32.
//   3. Scores 256 (||c||^2 - 2 y.c) for 32 codewords x 32 blocks per
//      mfma_f32_32x32x16_f16: A = codeword tile (fp16-exact), B = -512 y split
//      into fp16 hi + lo, C = 256 ||c||^2.  A lane holds 16 codeword rows of one
//      block column; it keeps only the minimum of those 16 (v_min3 chains),
//      the best and second-best such tile minimum and the best tile's index:
//      about 0.75 VALU operations per score instead of a compare-select each.
//   4. Recovery: the lane recomputes its best tile's 16 scores in fp32 FMAs and
//      finds the index; the two lanes sharing a column merge.
//   5. Certificate: every computed score (matrix core or VALU) is within
//      E = 1.01 (4k+4) 2^-24 (256 max||c||^2 + 513 max||c|| ||y_b||) of the exact
//      scaled score (2k+1 exact products and the accumulator per matrix op with
//      a 2-ulp-per-operation model, the fp32 FMA chain, and the roundings of y).
//      If second - best > 2E the winner is the exact unique minimiser.
//   6. Uncertified blocks are searched again by the whole wave in fp64 with the
//      direct distance sum_t (y_t - c_t)^2 (lowest index on exact ties).
//   7. Codes are assembled in LDS and written as whole dwords.
#include "fq_device.h"
#include "fq_internal.h"

namespace fq {
namespace {

constexpr int D = kD;
constexpr int WAVES = 4;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef double f64x4 __attribute__((ext_vector_type(4)));

// LDS ordering inside one wave: wait for this wave's LDS operations, keep the
// compiler from moving LDS accesses across.
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
}

// Minimum of 16 values as a chain of 7 three-input minima and one two-input minimum.
__device__ inline float min16(const f32x16& v) {
  float m = fminf(fminf(v[0], v[1]), v[2]);
#pragma unroll
  for (int i = 3; i < 15; i += 2) m = fminf(fminf(m, v[i]), v[i + 1]);
  return fminf(m, v[15]);
}

__device__ inline double shfl_xor_f64(double v, int m) {
  const int2 w = __builtin_bit_cast(int2, v);
  int2 r;
  r.x = __shfl_xor(w.x, m);
  r.y = __shfl_xor(w.y, m);
  return __builtin_bit_cast(double, r);
}

template <int K, bool XF16, bool NF16>
__global__ __launch_bounds__(WAVES * 64) void encode_mfma(
    const void* __restrict__ xv, int64_t n, int64_t ngroups, const half8* __restrict__ amfma,
    const float* __restrict__ cinit, const float* __restrict__ cn2s, const float* __restrict__ cw,
    const _Float16* __restrict__ cw16,
    const double* __restrict__ pi64m, const double* __restrict__ pi64, int N, int bits, float cmax, float c2max,
    uint8_t* __restrict__ codes, void* __restrict__ norms, const int64_t* __restrict__ slots, int64_t cap, int nwg) {
  constexpr int NB = D / K;        // blocks per vector
  constexpr int VG = 256 / NB;     // vectors per group
  constexpr int NSUB = VG / 16;    // 16-vector rotation sub-groups
  constexpr int XB = XF16 ? 2 : 4; // input bytes per coordinate
  // Row strides are padded so that the 16 rows a rotation sub-group touches in
  // one instruction fall into different LDS banks.
  constexpr int YS = D + 4;             // y rows: fp32, 272 B
  constexpr int XS = XF16 ? D + 8 : D + 4;  // x rows: 144 B (fp16) or 272 B (fp32)
  __shared__ __align__(16) float ytile[WAVES][VG * YS];
  __shared__ __align__(16) char xtile[WAVES][VG * XS * XB];
  __shared__ double sinv[WAVES][VG];
  __shared__ uint32_t spk[WAVES][8 * 16];  // 256 codes x bits <= 4096 bits
  constexpr int CBL = K == 4 ? 1024 : 1;   // k = 4 keeps the codebook (N <= 1024) in LDS
  __shared__ __align__(16) _Float16 cwL[CBL * 4];
  __shared__ __align__(16) float cn2L[CBL];
  if constexpr (K == 4) {
    for (int i = fq_tid(); i < N; i += WAVES * 64) {
      cn2L[i] = cn2s[i];
      *reinterpret_cast<uint2*>(cwL + 4 * i) = *reinterpret_cast<const uint2*>(cw16 + 4 * i);
    }
    __syncthreads();
  }

  const int lane = fq_tid() & 63, w = fq_tid() >> 6;
  const int c = lane & 31, h = lane >> 5;
  const int NT = N / 32;
  const int B = NB * bits;
  float* yt = ytile[w];
  char* xs = xtile[w];
  const double u = 5.9604644775390625e-08;

  for (int64_t g = (int64_t)fq_bid_x() * WAVES + w; g < ngroups; g += (int64_t)nwg * WAVES) {
    const int64_t v0 = g * VG;
    const int nv = (int)((n - v0) < VG ? (n - v0) : VG);

    // ---- 1. x tile to LDS (rows past n are zero); nu in fp64 from register partials.
    // Lane l loads bytes [l * LB, (l + 1) * LB) of the tile; 64 / VG lanes share a vector.
    {
      constexpr int LB = VG * D * XB / 64;  // bytes per lane (32 or 64 for fp16 input)
      constexpr int LPV = 64 / VG;           // lanes per vector
      const char* xg = reinterpret_cast<const char*>(xv) + v0 * (D * XB);
      double s = 0.0;
#pragma unroll
      for (int q = 0; q < LB / 16; q++) {
        const int o = lane * LB + q * 16;
        uint4 val = make_uint4(0u, 0u, 0u, 0u);
        if (o < nv * D * XB) val = *reinterpret_cast<const uint4*>(xg + o);
        *reinterpret_cast<uint4*>(xs + (o / (D * XB)) * (XS * XB) + o % (D * XB)) = val;
        const uint32_t wv[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
        for (int t = 0; t < 4; t++) {
          if constexpr (XF16) {
            const double a = (double)__builtin_bit_cast(_Float16, (uint16_t)(wv[t] & 0xffffu));
            const double b = (double)__builtin_bit_cast(_Float16, (uint16_t)(wv[t] >> 16));
            s = fma(a, a, s);
            s = fma(b, b, s);
          } else {
            const double a = (double)__builtin_bit_cast(float, wv[t]);
            s = fma(a, a, s);
          }
        }
      }
#pragma unroll
      for (int m = 1; m < LPV; m <<= 1) s += shfl_xor_f64(s, m);
      if (lane % LPV == 0) {
        const int vl = lane / LPV;
        const double nu = sqrt(s);
        sinv[w][vl] = nu > 0.0 ? 1.0 / nu : 0.0;
        const int64_t sv = vl < nv ? out_slot(slots, cap, v0 + vl) : -1;
        if (sv >= 0) {
          if constexpr (NF16)
            reinterpret_cast<uint16_t*>(norms)[sv] = f64_to_f16_bits(nu);
          else
            reinterpret_cast<float*>(norms)[sv] = (float)nu;
        }
      }
    }
    wave_lds_sync();

    // ---- 2. rotation on the fp64 matrix core, one 16-vector sub-group at a time:
    //         D[coord][vector] in 16 x 16 tiles, then y = D / nu -> LDS (fp32)
#pragma unroll 1
    for (int sg = 0; sg < NSUB; sg++) {
      f64x4 acc[4];
#pragma unroll
      for (int r = 0; r < 4; r++) acc[r] = f64x4{0.0, 0.0, 0.0, 0.0};
      const int vec = 16 * sg + (lane & 15);
#pragma unroll 4
      for (int ks = 0; ks < 16; ks++) {
        const int co = 4 * ks + (lane >> 4);
        double xb;
        if constexpr (XF16)
          xb = (double)reinterpret_cast<const _Float16*>(xs)[vec * XS + co];
        else
          xb = (double)reinterpret_cast<const float*>(xs)[vec * XS + co];
#pragma unroll
        for (int r = 0; r < 4; r++)
          acc[r] = __builtin_amdgcn_mfma_f64_16x16x4f64(pi64m[(r * 16 + ks) * 64 + lane], xb, acc[r], 0, 0, 0);
      }
      const double inv = sinv[w][vec];
#pragma unroll
      for (int r = 0; r < 4; r++)
#pragma unroll
        for (int e = 0; e < 4; e++) yt[vec * YS + 16 * r + (lane >> 4) + 4 * e] = (float)(acc[r][e] * inv);
    }
    wave_lds_sync();

    // ---- 3. B operands: column c of B tile tb is block 32 tb + c of the group
    half8 bop[8];
#pragma unroll
    for (int tb = 0; tb < 8; tb++) {
      const int gb = 32 * tb + c;
      const float* yp = yt + (gb / NB) * YS + (gb % NB) * K;  // block gb of the group
      half8 b = {};
      if constexpr (K == 4) {
        if (h == 0) {
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const float v = -512.0f * yp[i];
            const _Float16 hv = (_Float16)v;
            b[i] = hv;
            b[4 + i] = (_Float16)(v - (float)hv);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; i++) {
          const float v = -512.0f * yp[i];
          const _Float16 hv = (_Float16)v;
          b[i] = h == 0 ? hv : (_Float16)(v - (float)hv);
        }
      }
      bop[tb] = b;
    }

    // ---- 3b. matrix-core search with per-lane tile minima
    float m1[8], m2[8];
    int tid[8];
#pragma unroll
    for (int tb = 0; tb < 8; tb++) {
      m1[tb] = __builtin_huge_valf();
      m2[tb] = __builtin_huge_valf();
      tid[tb] = 0;
    }
    const f32x16* cin = reinterpret_cast<const f32x16*>(cinit);
    half8 A = amfma[lane];
    f32x16 C = cin[h];
    for (int t = 0; t < NT; t++) {
      half8 An = A;
      f32x16 Cn = C;
      if (t + 1 < NT) {
        An = amfma[(t + 1) * 64 + lane];
        Cn = cin[(t + 1) * 2 + h];
      }
#pragma unroll
      for (int tb = 0; tb < 8; tb++) {
        const f32x16 Dv = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, bop[tb], C, 0, 0, 0);
        const float tm = min16(Dv);
        m2[tb] = __builtin_amdgcn_fmed3f(m1[tb], m2[tb], tm);
        const bool lt = tm < m1[tb];
        tid[tb] = lt ? t : tid[tb];
        m1[tb] = fminf(m1[tb], tm);
      }
      A = An;
      C = Cn;
    }

    // ---- 4-6. recovery, certificate, cooperative fp64 re-search
    uint32_t code[8];
#pragma unroll
    for (int tb = 0; tb < 8; tb++) {
      const int gb = 32 * tb + c;
      const float* yp = yt + (gb / NB) * YS + (gb % NB) * K;
      float my[K];
      float yn2 = 0.f;
#pragma unroll
      for (int i = 0; i < K; i++) {
        my[i] = -512.0f * yp[i];
        yn2 = fmaf(yp[i], yp[i], yn2);
      }
      const int t0 = tid[tb];
      float r1 = __builtin_huge_valf(), r2 = __builtin_huge_valf();
      int ri = 0;
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int n0 = 32 * t0 + 8 * q + 4 * h;  // rows n0 .. n0 + 3 of this lane
        float4 c2;
        _Float16 cv[4][K];
        if constexpr (K == 4) {
          c2 = *reinterpret_cast<const float4*>(cn2L + n0);
          const uint4 u0 = *reinterpret_cast<const uint4*>(cwL + n0 * 4);
          const uint4 u1 = *reinterpret_cast<const uint4*>(cwL + n0 * 4 + 8);
          const uint32_t uw[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
          for (int e = 0; e < 4; e++)
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
              cv[e][i] = __builtin_bit_cast(_Float16, (uint16_t)(uw[(e * 4 + i) / 2] & 0xffffu));
              cv[e][i + 1] = __builtin_bit_cast(_Float16, (uint16_t)(uw[(e * 4 + i) / 2] >> 16));
            }
        } else {
          c2 = *reinterpret_cast<const float4*>(cn2s + n0);
#pragma unroll
          for (int e = 0; e < 4; e++) {
            const uint4 u = *reinterpret_cast<const uint4*>(cw16 + (n0 + e) * 8);
            const uint32_t uw[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
              cv[e][i] = __builtin_bit_cast(_Float16, (uint16_t)(uw[i / 2] & 0xffffu));
              cv[e][i + 1] = __builtin_bit_cast(_Float16, (uint16_t)(uw[i / 2] >> 16));
            }
          }
        }
        const float c2a[4] = {c2.x, c2.y, c2.z, c2.w};
#pragma unroll
        for (int e = 0; e < 4; e++) {
          float sc = c2a[e];
#pragma unroll
          // the fp32 operand first (else a wait state between every two mixed FMAs)
          for (int i = 0; i < K; i++) sc = fmaf(my[i], (float)cv[e][i], sc);
          r2 = __builtin_amdgcn_fmed3f(r1, r2, sc);
          const bool lt = sc < r1;
          ri = lt ? (n0 + e) : ri;
          r1 = fminf(r1, sc);
        }
      }
      const float o1 = __shfl_xor(r1, 32), o2 = __shfl_xor(r2, 32), om = __shfl_xor(m2[tb], 32);
      const int oi = __shfl_xor(ri, 32);
      const bool other = (o1 < r1) || (o1 == r1 && oi < ri);
      const float best = other ? o1 : r1;
      const float second = fminf(fminf(fmaxf(r1, o1), fminf(r2, o2)), fminf(m2[tb], om));
      code[tb] = (uint32_t)(other ? oi : ri);
      const double yn = sqrt((double)yn2) * 1.01;
      const double E = 1.01 * (4 * K + 4) * u * (256.0 * (double)c2max + 513.0 * (double)cmax * yn);
      const bool sure = ((double)second - (double)best) > 2.0 * E;
      uint64_t todo = __ballot(h == 0 && !sure && gb / NB < nv);
      while (todo) {
        const int cc = __builtin_ctzll(todo);
        todo &= todo - 1;
        const int fb = 32 * tb + cc;  // block of the group
        const int vec = fb / NB, blk = fb % NB;
        // exact y_b: every lane contributes coordinate j = lane of x
        double xj;
        if constexpr (XF16)
          xj = (double)reinterpret_cast<const _Float16*>(xv)[(v0 + vec) * D + lane];
        else
          xj = (double)reinterpret_cast<const float*>(xv)[(v0 + vec) * D + lane];
        const double inv = sinv[w][vec];
        double yb[K];
#pragma unroll
        for (int i = 0; i < K; i++) {
          double p = pi64[(blk * K + i) * D + lane] * xj;
#pragma unroll
          for (int m = 32; m >= 1; m >>= 1) p += shfl_xor_f64(p, m);
          yb[i] = p * inv;
        }
        double bd = __builtin_huge_val();
        int bn = 0x7fffffff;
        for (int nn = lane; nn < N; nn += 64) {
          double dd = 0.0;
#pragma unroll
          for (int i = 0; i < K; i++) {
            const double df = yb[i] - (double)cw[nn * K + i];
            dd = fma(df, df, dd);
          }
          if (dd < bd) {
            bd = dd;
            bn = nn;
          }
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
          const double od = shfl_xor_f64(bd, m);
          const int on = __shfl_xor(bn, m);
          if (od < bd || (od == bd && on < bn)) {
            bd = od;
            bn = on;
          }
        }
        if (c == cc) code[tb] = (uint32_t)bn;
      }
    }

    // ---- 7. pack the group's 256 codes (bit offset = block index * bits)
    const int words = 8 * bits;
    for (int i = lane; i < words; i += 64) spk[w][i] = 0u;
    wave_lds_sync();
    if (h == 0) {
#pragma unroll
      for (int tb = 0; tb < 8; tb++) {
        const int gb = 32 * tb + c;
        if (gb / NB < nv) {
          const int bo = gb * bits, sh = bo & 31;
          atomicOr(&spk[w][bo >> 5], code[tb] << sh);
          if (sh + bits > 32) atomicOr(&spk[w][(bo >> 5) + 1], code[tb] >> (32 - sh));
        }
      }
    }
    wave_lds_sync();
    if (slots) {
      scatter_records(spk[w], nv, B / 8, slots, cap, v0, codes, lane);
    } else {
      const int64_t nbytes = ((int64_t)nv * B + 7) / 8;
      uint8_t* dst = codes + g * (int64_t)(32 * bits);  // group g starts at bit g * 256 * bits
      const int nfull = (int)(nbytes / 4);
      for (int i = lane; i < nfull; i += 64) reinterpret_cast<uint32_t*>(dst)[i] = spk[w][i];
      const int rem = (int)(nbytes - 4 * (int64_t)nfull);
      if (lane < rem) dst[4 * nfull + lane] = (uint8_t)((spk[w][nfull] >> (8 * lane)) & 0xffu);
    }
    wave_lds_sync();
  }
}

}  // namespace

bool encode_mfma_supported(const fq_codebook* cb) {
  return cb->amfma && (cb->k == 4 || cb->k == 8) && cb->N % 32 == 0 && !(cb->k == 4 && cb->N > 1024);
}

hipError_t launch_encode_mfma(const fq_codebook* cb, const void* x, fq_dtype x_dtype, int64_t n, uint8_t* codes,
                              void* norms, fq_dtype norm_dtype, const int64_t* slots, int64_t cap,
                              hipStream_t s) {
  if (!encode_mfma_supported(cb)) return hipErrorNotSupported;
  const int VG = 256 / (kD / cb->k);
  const int64_t ngroups = (n + VG - 1) / VG;
  int64_t wgs = (ngroups + WAVES - 1) / WAVES;
  if (wgs > 2048) wgs = 2048;
  const dim3 grid((unsigned)wgs), block(WAVES * 64);
  const bool xf = x_dtype == FQ_F16, nf = norm_dtype == FQ_F16;
#define FQ_EM(KK, XF, NF)                                                                                        \
  hipLaunchKernelGGL((encode_mfma<KK, XF, NF>), grid, block, 0, s, x, n, ngroups,                               \
                     reinterpret_cast<const half8*>(cb->amfma), cb->cinit, cb->cn2s, cb->cw, cb->cw16, cb->pi64m,  \
                     cb->pi64,                                                                                 \
                     cb->N, cb->bits, cb->cmax, cb->c2max, codes, norms, slots, cap, (int)wgs)
#define FQ_EM_K(KK)            \
  if (xf && nf)                \
    FQ_EM(KK, true, true);     \
  else if (xf)                 \
    FQ_EM(KK, true, false);    \
  else if (nf)                 \
    FQ_EM(KK, false, true);    \
  else                         \
    FQ_EM(KK, false, false)
  if (cb->k == 4) {
    FQ_EM_K(4);
  } else {
    FQ_EM_K(8);
  }
#undef FQ_EM_K
#undef FQ_EM
  return hipGetLastError();
}

}  // namespace fq
