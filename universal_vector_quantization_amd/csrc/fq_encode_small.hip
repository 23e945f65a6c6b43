// Encoder for small batches (FibQuant summary §2.3 encoder; §5: the decode loop
// appends one token per sequence per step, so the batches are small and the
// latency of one launch is what counts).
//
// One wave per vector.  Lane l holds coordinate l: the norm is a wave sum in
// fp64, the rotated unit vector y = Pi (x / nu) is computed in fp64 with lane l
// producing y_l, and the nearest-codeword search runs directly in fp64 (the
// squared distance of the definition, no certificate needed): lane l scores the
// codewords l, l + 64, ... of every block, then the lanes' winners are merged in
// LDS (lowest distance, lowest index on equal distances).  The codewords a lane
// scores stay in its registers for all blocks, which bounds the shapes to
// ceil(N / 64) * k <= 64 values per lane.  Records must be whole bytes: each wave
// writes its own record with plain stores.
#include "fq_internal.h"
#include "fq_device.h"

namespace fq {
namespace {

constexpr int D = kD;

__device__ inline double shfl_xor_f64(double v, int m) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)u, m), hi = (uint32_t)__shfl_xor((int)(uint32_t)(u >> 32), m);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Value of v in lane l (l the same in every lane).
__device__ inline double readlane_f64(double v, int l) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)u, l);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(u >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

template <int K, int NPL>
__global__ __launch_bounds__(64) void encode_wave(const void* __restrict__ x, int xf16, const double* __restrict__ pi64t,
                                                  const float* __restrict__ cw, int N, int bits,
                                                  uint8_t* __restrict__ codes, void* __restrict__ norms, int nf16,
                                                  const int64_t* __restrict__ slots, int64_t cap) {
  constexpr int NB = D / K;  // blocks per vector
  constexpr int R = K;       // reducer lanes per block: 64 / NB
  __shared__ double sd[NB][64];
  __shared__ int sn[NB][64];
  __shared__ uint32_t rec[32];  // one record: at most 64 codes of 16 bits
  const int lane = fq_tid();
  const int64_t v = fq_bid_x();

  // the lane's codewords (fp16-exact values, exact in fp64); indices past N (N < 64)
  // load codeword N - 1 so that every load is unconditional and all are in flight at
  // once, and are never chosen
  double c[NPL][K];
#pragma unroll
  for (int j = 0; j < NPL; j++) {
    const int nn = lane + 64 * j < N ? lane + 64 * j : N - 1;
#pragma unroll
    for (int i = 0; i < K; i++) c[j][i] = (double)cw[nn * K + i];
  }
  double pr[D];  // row l of Pi (pi64t[j][l] = Pi[l][j]), loaded while the input arrives
#pragma unroll
  for (int j = 0; j < D; j++) pr[j] = pi64t[j * D + lane];
  const double xl = xf16 ? (double)reinterpret_cast<const _Float16*>(x)[v * D + lane]
                         : (double)reinterpret_cast<const float*>(x)[v * D + lane];
  double s = xl * xl;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s += shfl_xor_f64(s, m);
  const double nu = sqrt(s);
  const double ul = nu > 0.0 ? xl / nu : 0.0;  // nu = 0: y = 0, every block takes its smallest codeword
  double ya[4] = {0.0, 0.0, 0.0, 0.0};  // four independent chains: a quarter of the latency
#pragma unroll
  for (int j = 0; j < D; j++) ya[j & 3] = fma(pr[j], readlane_f64(ul, j), ya[j & 3]);
  const double y = (ya[0] + ya[1]) + (ya[2] + ya[3]);

  // ---- per block: the lane's best codeword, then the lanes' winners in LDS
#pragma unroll 2
  for (int b = 0; b < NB; b++) {
    double yb[K];
#pragma unroll
    for (int i = 0; i < K; i++) yb[i] = readlane_f64(y, b * K + i);
    double bd = __builtin_huge_val();
    int bn = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < NPL; j++) {
      double d = 0.0;
#pragma unroll
      for (int i = 0; i < K; i++) {
        const double t = yb[i] - c[j][i];
        d = fma(t, t, d);
      }
      if (lane + 64 * j < N && d < bd) {  // j ascending: the lowest index wins equal distances
        bd = d;
        bn = lane + 64 * j;
      }
    }
    sd[b][lane] = bd;
    sn[b][lane] = bn;
  }
  __syncthreads();
  const int blk = lane / R, r = lane % R;
  double bd = __builtin_huge_val();
  int bn = 0x7fffffff;
#pragma unroll 8
  for (int e = 0; e < NB; e++) {
    const double d = sd[blk][r * NB + e];
    const int nn = sn[blk][r * NB + e];
    if (d < bd || (d == bd && nn < bn)) {
      bd = d;
      bn = nn;
    }
  }
#pragma unroll
  for (int m = 1; m < R; m <<= 1) {
    const double od = shfl_xor_f64(bd, m);
    const int on = __shfl_xor(bn, m);
    if (od < bd || (od == bd && on < bn)) {
      bd = od;
      bn = on;
    }
  }

  // ---- pack the record (block b at bit b * bits) and store it at its slot
  if (lane < 32) rec[lane] = 0u;
  __syncthreads();
  if (r == 0) {
    const int bo = blk * bits, sh = bo & 31;
    atomicOr(&rec[bo >> 5], (uint32_t)bn << sh);
    if (sh + bits > 32) atomicOr(&rec[(bo >> 5) + 1], (uint32_t)bn >> (32 - sh));
  }
  __syncthreads();
  const int64_t slot = out_slot(slots, cap, v);
  if (slot < 0) return;
  const int rb = NB * bits / 8;  // record bytes (whole bytes)
  if ((rb & 3) == 0) {
    for (int t = lane; t < rb / 4; t += 64) reinterpret_cast<uint32_t*>(codes)[slot * (rb / 4) + t] = rec[t];
  } else {
    for (int t = lane; t < rb; t += 64) codes[slot * rb + t] = reinterpret_cast<const uint8_t*>(rec)[t];
  }
  if (lane == 0) {
    if (nf16)
      reinterpret_cast<uint16_t*>(norms)[slot] = f64_to_f16_bits(nu);
    else
      reinterpret_cast<float*>(norms)[slot] = (float)nu;
  }
}

template <int K, int NPL>
hipError_t launch_wave(const fq_codebook* cb, const void* x, fq_dtype xd, int64_t n, uint8_t* codes, void* norms,
                       fq_dtype nd, const int64_t* slots, int64_t cap, hipStream_t s) {
  hipLaunchKernelGGL((encode_wave<K, NPL>), dim3((unsigned)n), dim3(64), 0, s, x, xd == FQ_F16 ? 1 : 0, cb->pi64t,
                     cb->cw, cb->N, cb->bits, codes, norms, nd == FQ_F16 ? 1 : 0, slots, cap);
  return hipGetLastError();
}

}  // namespace

bool encode_small_supported(const fq_codebook* cb) {
  const int npl = (cb->N + 63) / 64;
  return cb->d == D && cb->B % 8 == 0 && npl * cb->k <= 64;
}

hipError_t launch_encode_small(const fq_codebook* cb, const void* x, fq_dtype x_dtype, int64_t n, uint8_t* codes,
                               void* norms, fq_dtype norm_dtype, const int64_t* slots, int64_t cap, hipStream_t s) {
  if (!encode_small_supported(cb) || n > SMALL_ENCODE_MAX) return hipErrorNotSupported;
  const int npl = (cb->N + 63) / 64;
#define FQ_W(KK, NP) \
  if (cb->k == KK && npl == NP) return launch_wave<KK, NP>(cb, x, x_dtype, n, codes, norms, norm_dtype, slots, cap, s)
  FQ_W(1, 1); FQ_W(1, 2); FQ_W(1, 4); FQ_W(1, 8); FQ_W(1, 16); FQ_W(1, 32); FQ_W(1, 64);
  FQ_W(2, 1); FQ_W(2, 2); FQ_W(2, 4); FQ_W(2, 8); FQ_W(2, 16); FQ_W(2, 32);
  FQ_W(4, 1); FQ_W(4, 2); FQ_W(4, 4); FQ_W(4, 8); FQ_W(4, 16);
  FQ_W(8, 1); FQ_W(8, 2); FQ_W(8, 4); FQ_W(8, 8);
  FQ_W(16, 1); FQ_W(16, 2); FQ_W(16, 4);
  FQ_W(32, 1); FQ_W(32, 2);
  FQ_W(64, 1);
#undef FQ_W
  return hipErrorNotSupported;
}

}  // namespace fq
