// Codebook construction on the GPU (FibQuant summary §2.2: the codebook is
// refined offline by Lloyd-Max iterations on samples of the canonical block
// source; §3.1: that source is the same for every input law).
//
// Generalised Lloyd over m training blocks of k coordinates (fp64):
//   assignment  every sample goes to the codeword with the smallest
//               ||c||^2 - 2 y.c (fp64; the lowest index on equal scores), and
//               its squared error to that codeword is measured directly;
//   update      every codeword becomes the mean of its cell; an empty cell is
//               re-seeded at the worst-served sample (largest error; the lowest
//               index on equal errors), empty cells in increasing order taking
//               the samples in decreasing error;
//   stop        when no assignment changes, when the training MSE falls by no
//               more than rel_tol of itself, or after max_iter updates.
// Several starting codebooks are refined; the one with the lowest MSE on an
// independent validation set is kept (the first on equal MSE) and rounded to the
// fp16 grid (round to nearest even, |v| < 2^-14 flushed to 0).
//
// Assignment: one thread per S samples (held in registers), every codeword
// visited in increasing index order.  For k <= 8 codeword tiles are staged in LDS
// and each broadcast LDS read feeds S samples; for k >= 16 a codeword's values
// are read with wave-uniform addresses (scalar cache, scalar registers), since
// with one or two samples per thread an LDS read per FMA would saturate LDS.
//
// The assignment pass also accumulates the cell sums and counts for the next
// update: sample coordinates are added as 64-bit fixed-point integers (scale
// 2^s with m * 2^s < 2^62), so the sums do not depend on the order of the
// atomic additions and a build is bit-reproducible.  Errors are summed per
// workgroup in a fixed order and then added in fixed point as well.
#include <algorithm>
#include <cmath>
#include <vector>

#include "fq_internal.h"
#include "fq_device.h"

namespace fq {
namespace {

constexpr int TW = 256;  // threads per workgroup

template <int K>
struct TrainShape {
  static constexpr int S = K <= 8 ? 4 : (K <= 32 ? 2 : 1);  // samples per thread
  static constexpr int TILE = 128;                          // codewords per LDS tile (k <= 8)
};

// Assignment of samples [0, m) against codebook c [N][K] (fp64) with ||c||^2 in cn2.
// idx / err: per-sample code and squared error; with prev_changed != null, a sample
// whose code differs from the one idx held before sets *prev_changed = 1.  With sums
// != null the sample is added to its cell (fixed point, scale `scale`).  esum gets
// the workgroup error sums (fixed point, scale `escale`).
template <int K>
__global__ __launch_bounds__(TW) void lloyd_assign(const double* __restrict__ y, int64_t m,
                                                   const double* __restrict__ c, const double* __restrict__ cn2, int N,
                                                   int* __restrict__ idx, double* __restrict__ err,
                                                   int* __restrict__ changed, unsigned long long* __restrict__ sums,
                                                   unsigned int* __restrict__ counts, double scale,
                                                   unsigned long long* __restrict__ esum, double escale) {
  typedef TrainShape<K> Sh;
  constexpr int S = Sh::S;
  constexpr int TILE = Sh::TILE;
  __shared__ double tc[K <= 8 ? TILE * K : 1];
  __shared__ double tn[K <= 8 ? TILE : 1];
  __shared__ double red[TW];
  const int tid = fq_tid();
  const int64_t base = (int64_t)fq_bid_x() * (TW * S);
  double ys[S][K];
  bool ok[S];
#pragma unroll
  for (int s = 0; s < S; s++) {
    const int64_t i = base + s * TW + tid;
    ok[s] = i < m;
    const int64_t ic = ok[s] ? i : m - 1;
#pragma unroll
    for (int j = 0; j < K; j++) ys[s][j] = y[ic * K + j];
  }
  double best[S];
  int bi[S];
#pragma unroll
  for (int s = 0; s < S; s++) {
    best[s] = __builtin_huge_val();
    bi[s] = 0;
  }
  if constexpr (K <= 8) {
    // short codewords: tiles staged in LDS, every LDS read (the same address in
    // every lane: a broadcast) feeding S samples
    for (int t0 = 0; t0 < N; t0 += TILE) {
      const int nt = N - t0 < TILE ? N - t0 : TILE;
      __syncthreads();
      for (int e = tid; e < nt * K; e += TW) tc[e] = c[(int64_t)t0 * K + e];
      for (int e = tid; e < nt; e += TW) tn[e] = cn2[t0 + e];
      __syncthreads();
      for (int r = 0; r < nt; r++) {
        double dot[S];
#pragma unroll
        for (int s = 0; s < S; s++) dot[s] = 0.0;
#pragma unroll
        for (int j = 0; j < K; j++) {
          const double cv = tc[r * K + j];
#pragma unroll
          for (int s = 0; s < S; s++) dot[s] = fma(ys[s][j], cv, dot[s]);
        }
        const double cn = tn[r];
#pragma unroll
        for (int s = 0; s < S; s++) {
          const double sc = fma(-2.0, dot[s], cn);
          if (sc < best[s]) {  // codewords in increasing order: the lowest index wins equal scores
            best[s] = sc;
            bi[s] = t0 + r;
          }
        }
      }
    }
  } else {
    // The codeword is the same for every lane: its values are read with uniform
    // addresses, so they arrive through the scalar cache into scalar registers and
    // feed the FMAs directly (no LDS traffic per FMA).
    for (int n = 0; n < N; n++) {
      const double* __restrict__ cr = c + (int64_t)n * K;
      // P partial sums per sample: long dot products would otherwise be one chain of
      // dependent FMAs
      constexpr int P = 4;
      double dot[S][P];
#pragma unroll
      for (int s = 0; s < S; s++)
#pragma unroll
        for (int q = 0; q < P; q++) dot[s][q] = 0.0;
#pragma unroll
      for (int j = 0; j < K; j++) {
        const double cv = cr[j];
#pragma unroll
        for (int s = 0; s < S; s++) dot[s][j % P] = fma(ys[s][j], cv, dot[s][j % P]);
      }
      const double cn = cn2[n];
#pragma unroll
      for (int s = 0; s < S; s++) {
        const double dt = (dot[s][0] + dot[s][1]) + (dot[s][2] + dot[s][3]);
        const double sc = fma(-2.0, dt, cn);
        if (sc < best[s]) {  // codewords in increasing order: the lowest index wins equal scores
          best[s] = sc;
          bi[s] = n;
        }
      }
    }
  }
  double esum_t = 0.0;
#pragma unroll
  for (int s = 0; s < S; s++) {
    if (!ok[s]) continue;
    const int64_t i = base + s * TW + tid;
    const int n = bi[s];
    double e = 0.0;
#pragma unroll
    for (int j = 0; j < K; j++) {
      const double df = ys[s][j] - c[(int64_t)n * K + j];
      e = fma(df, df, e);
    }
    err[i] = e;
    esum_t += e;
    if (changed && idx[i] != n) changed[0] = 1;
    idx[i] = n;
    if (sums) {
#pragma unroll
      for (int j = 0; j < K; j++)
        atomicAdd(&sums[(int64_t)n * K + j], (unsigned long long)(long long)rint(ys[s][j] * scale));
      atomicAdd(&counts[n], 1u);
    }
  }
  // workgroup error sum in a fixed order, then one fixed-point addition
  red[tid] = esum_t;
  __syncthreads();
  for (int w = TW / 2; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  if (tid == 0) atomicAdd(esum, (unsigned long long)(long long)rint(red[0] * escale));
}

// ||c_n||^2 for every codeword.
__global__ __launch_bounds__(TW) void lloyd_norms(const double* __restrict__ c, int N, int K, double* __restrict__ cn2) {
  const int n = fq_bid_x() * TW + fq_tid();
  if (n >= N) return;
  double s = 0.0;
  for (int j = 0; j < K; j++) s = fma(c[(int64_t)n * K + j], c[(int64_t)n * K + j], s);
  cn2[n] = s;
}

// Cell means from the accumulated sums (a cell without samples keeps its codeword
// and is listed in `empty`); clears the sums and counts for the next pass.
__global__ __launch_bounds__(TW) void lloyd_update(double* __restrict__ c, int N, int K,
                                                   unsigned long long* __restrict__ sums,
                                                   unsigned int* __restrict__ counts, double scale,
                                                   int* __restrict__ nempty, int* __restrict__ empty) {
  const int n = fq_bid_x() * TW + fq_tid();
  if (n >= N) return;
  const unsigned int cnt = counts[n];
  if (cnt > 0) {
    for (int j = 0; j < K; j++) c[(int64_t)n * K + j] = ((double)(long long)sums[(int64_t)n * K + j] / scale) / cnt;
  } else {
    empty[atomicAdd(nempty, 1)] = n;
  }
  for (int j = 0; j < K; j++) sums[(int64_t)n * K + j] = 0ull;
  counts[n] = 0u;
}

// Largest error and the lowest sample index holding it: per-workgroup partials,
// then one workgroup over the partials.
__global__ __launch_bounds__(TW) void argmax_partial(const double* __restrict__ err, int64_t m,
                                                     double* __restrict__ pv, int64_t* __restrict__ pi) {
  __shared__ double sv[TW];
  __shared__ int64_t si[TW];
  const int tid = fq_tid();
  double bv = -__builtin_huge_val();
  int64_t bi = INT64_MAX;
  for (int64_t i = (int64_t)fq_bid_x() * TW + tid; i < m; i += (int64_t)TW * 1024) {
    const double v = err[i];
    if (v > bv || (v == bv && i < bi)) {
      bv = v;
      bi = i;
    }
  }
  sv[tid] = bv;
  si[tid] = bi;
  __syncthreads();
  for (int w = TW / 2; w > 0; w >>= 1) {
    if (tid < w) {
      const double v = sv[tid + w];
      const int64_t i = si[tid + w];
      if (v > sv[tid] || (v == sv[tid] && i < si[tid])) {
        sv[tid] = v;
        si[tid] = i;
      }
    }
    __syncthreads();
  }
  if (tid == 0) {
    pv[fq_bid_x()] = sv[0];
    pi[fq_bid_x()] = si[0];
  }
}

// Re-seeds codeword `dst` at the sample named by the partials' winner and takes
// that sample out of later picks.
__global__ __launch_bounds__(TW) void reseed_pick(const double* __restrict__ pv, const int64_t* __restrict__ pi,
                                                  int np, const double* __restrict__ y, double* __restrict__ err,
                                                  double* __restrict__ c, int K, int dst) {
  __shared__ double sv[TW];
  __shared__ int64_t si[TW];
  const int tid = fq_tid();
  double bv = -__builtin_huge_val();
  int64_t bi = INT64_MAX;
  for (int e = tid; e < np; e += TW) {
    if (pv[e] > bv || (pv[e] == bv && pi[e] < bi)) {
      bv = pv[e];
      bi = pi[e];
    }
  }
  sv[tid] = bv;
  si[tid] = bi;
  __syncthreads();
  for (int w = TW / 2; w > 0; w >>= 1) {
    if (tid < w) {
      const double v = sv[tid + w];
      const int64_t i = si[tid + w];
      if (v > sv[tid] || (v == sv[tid] && i < si[tid])) {
        sv[tid] = v;
        si[tid] = i;
      }
    }
    __syncthreads();
  }
  const int64_t pick = si[0];
  if (tid < K) c[(int64_t)dst * K + tid] = y[pick * K + tid];
  __syncthreads();
  if (tid == 0) err[pick] = -__builtin_huge_val();
}

// Rounds the codebook to the fp16 grid (RNE straight from fp64, |v| < 2^-14 -> 0),
// into fp32 and (for the rounded codebook's validation) back into fp64.
__global__ __launch_bounds__(TW) void round_fp16_grid(const double* __restrict__ c, int64_t n,
                                                      float* __restrict__ out, double* __restrict__ back) {
  const int64_t e = (int64_t)fq_bid_x() * TW + fq_tid();
  if (e >= n) return;
  const uint16_t hb = f64_to_f16_bits(c[e]);
  float v = (float)__builtin_bit_cast(_Float16, hb);
  if (fabsf(v) < 0x1p-14f) v = 0.0f;
  out[e] = v;
  back[e] = (double)v;
}

// Device state of one build.
struct TrainBufs {
  double* c;            // [N][K] working codebook
  double* cbest;        // [N][K] kept restart
  double* cn2;          // [N]
  unsigned long long* sums;  // [N][K]
  unsigned int* counts;      // [N]
  int* idx;             // [m_train]
  double* err;          // [max(m_train, m_valid)]
  int* vidx;            // [m_valid]
  unsigned long long* esum;  // [1]
  int* flags;           // [0] changed, [1] number of empty cells
  int* empty;           // [N]
  double* pv;           // [1024]
  int64_t* pi;          // [1024]
};

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t carve(void* ws, int K, int N, int64_t mt, int64_t mv, TrainBufs* b) {
  char* p = reinterpret_cast<char*>(ws);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    void* r = p ? p + off : nullptr;
    off += align256(bytes);
    return r;
  };
  const size_t nk = (size_t)N * K;
  TrainBufs t;
  t.c = (double*)take(nk * 8);
  t.cbest = (double*)take(nk * 8);
  t.cn2 = (double*)take((size_t)N * 8);
  t.sums = (unsigned long long*)take(nk * 8);
  t.counts = (unsigned int*)take((size_t)N * 4);
  t.idx = (int*)take((size_t)mt * 4);
  t.err = (double*)take((size_t)std::max(mt, mv) * 8);
  t.vidx = (int*)take((size_t)mv * 4);
  t.esum = (unsigned long long*)take(8);
  t.flags = (int*)take(8);
  t.empty = (int*)take((size_t)N * 4);
  t.pv = (double*)take(1024 * 8);
  t.pi = (int64_t*)take(1024 * 8);
  if (b) *b = t;
  return off;
}

// 2^s with m * 2^s * bound < 2^62 (bound: the largest magnitude added per sample)
double fixed_scale(int64_t m, double bound) {
  int e = 0;
  while (std::ldexp((double)m * bound, e + 1) < 0x1p62) e++;
  while (e > -60 && std::ldexp((double)m * bound, e) >= 0x1p62) e--;
  return std::ldexp(1.0, e);
}

template <int K>
hipError_t assign_pass(const double* y, int64_t m, const TrainBufs& b, int N, int* idx, bool accumulate,
                       bool track_changes, double scale, double escale, hipStream_t s, double* mse) {
  typedef TrainShape<K> Sh;
  const int64_t wgs = (m + TW * Sh::S - 1) / (TW * Sh::S);
  hipError_t e = hipMemsetAsync(b.esum, 0, 8, s);
  if (e == hipSuccess && track_changes) e = hipMemsetAsync(b.flags, 0, 4, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lloyd_norms, dim3((unsigned)((N + TW - 1) / TW)), dim3(TW), 0, s, b.c, N, K, b.cn2);
  hipLaunchKernelGGL((lloyd_assign<K>), dim3((unsigned)wgs), dim3(TW), 0, s, y, m, b.c, b.cn2, N, idx, b.err,
                     track_changes ? b.flags : nullptr, accumulate ? b.sums : nullptr,
                     accumulate ? b.counts : nullptr, scale, b.esum, escale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  unsigned long long es = 0;
  e = hipMemcpyAsync(&es, b.esum, 8, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return e;
  *mse = ((double)(long long)es / escale) / (double)m;
  return hipSuccess;
}

template <int K>
hipError_t train_k(int N, const double* train, int64_t mt, const double* valid, int64_t mv, const double* starts,
                   int restarts, int max_iter, double rel_tol, float* out, double* out64, double* restart_mse,
                   double* valid_mse, double* history, int* history_len, void* ws, hipStream_t s) {
  TrainBufs b;
  carve(ws, K, N, mt, mv, &b);
  const size_t nk = (size_t)N * K;
  const int ublocks = (N + TW - 1) / TW;
  const double scale_t = fixed_scale(mt, 1.0);   // |y_j| <= 1 on the canonical source
  const double escale_t = fixed_scale(mt, 4.0);  // squared errors inside the unit ball are <= 4
  const double escale_v = fixed_scale(mv, 4.0);
  hipError_t e = hipMemsetAsync(b.sums, 0, nk * 8, s);
  if (e == hipSuccess) e = hipMemsetAsync(b.counts, 0, (size_t)N * 4, s);
  if (e != hipSuccess) return e;
  std::vector<double> best_hist;
  double best_v = 0.0;
  int best_r = -1;
  for (int r = 0; r < restarts; r++) {
    e = hipMemcpyAsync(b.c, starts + (size_t)r * nk, nk * 8, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return e;
    std::vector<double> hist;
    double mse = 0.0;
    e = assign_pass<K>(train, mt, b, N, b.idx, true, false, scale_t, escale_t, s, &mse);
    if (e != hipSuccess) return e;
    hist.push_back(mse);
    for (int it = 0; it < max_iter; it++) {
      // update: means, then empty cells from the current assignment's worst samples
      e = hipMemsetAsync(b.flags + 1, 0, 4, s);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(lloyd_update, dim3((unsigned)ublocks), dim3(TW), 0, s, b.c, N, K, b.sums, b.counts, scale_t,
                         b.flags + 1, b.empty);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      int nempty = 0;
      e = hipMemcpyAsync(&nempty, b.flags + 1, 4, hipMemcpyDeviceToHost, s);
      if (e == hipSuccess) e = hipStreamSynchronize(s);
      if (e != hipSuccess) return e;
      if (nempty > 0) {
        std::vector<int> em((size_t)nempty);
        e = hipMemcpyAsync(em.data(), b.empty, (size_t)nempty * 4, hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) return e;
        std::sort(em.begin(), em.end());
        const int np = (int)std::min<int64_t>(1024, (mt + TW - 1) / TW);
        for (int q : em) {
          hipLaunchKernelGGL(argmax_partial, dim3((unsigned)np), dim3(TW), 0, s, b.err, mt, b.pv, b.pi);
          hipLaunchKernelGGL(reseed_pick, dim3(1), dim3(TW), 0, s, b.pv, b.pi, np, train, b.err, b.c, K, q);
          if ((e = hipGetLastError()) != hipSuccess) return e;
        }
      }
      e = assign_pass<K>(train, mt, b, N, b.idx, true, true, scale_t, escale_t, s, &mse);
      if (e != hipSuccess) return e;
      hist.push_back(mse);
      int changed = 0;
      e = hipMemcpyAsync(&changed, b.flags, 4, hipMemcpyDeviceToHost, s);
      if (e == hipSuccess) e = hipStreamSynchronize(s);
      if (e != hipSuccess) return e;
      if (!changed) break;
      const size_t h = hist.size();
      if (hist[h - 2] - hist[h - 1] <= rel_tol * hist[h - 1]) break;
    }
    // the last assignment pass accumulated sums that no update consumes
    e = hipMemsetAsync(b.sums, 0, nk * 8, s);
    if (e == hipSuccess) e = hipMemsetAsync(b.counts, 0, (size_t)N * 4, s);
    if (e != hipSuccess) return e;
    double v = 0.0;
    e = assign_pass<K>(valid, mv, b, N, b.vidx, false, false, 1.0, escale_v, s, &v);
    if (e != hipSuccess) return e;
    if (restart_mse) restart_mse[r] = v;
    if (best_r < 0 || v < best_v) {
      best_v = v;
      best_r = r;
      best_hist = hist;
      e = hipMemcpyAsync(b.cbest, b.c, nk * 8, hipMemcpyDeviceToDevice, s);
      if (e != hipSuccess) return e;
    }
  }
  if (out64) {
    e = hipMemcpyAsync(out64, b.cbest, nk * 8, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(round_fp16_grid, dim3((unsigned)((nk + TW - 1) / TW)), dim3(TW), 0, s, b.cbest, (int64_t)nk, out,
                     b.c);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  double vr = 0.0;
  e = assign_pass<K>(valid, mv, b, N, b.vidx, false, false, 1.0, escale_v, s, &vr);
  if (e != hipSuccess) return e;
  if (valid_mse) *valid_mse = vr;
  if (history_len) *history_len = (int)best_hist.size();
  if (history)
    for (size_t i = 0; i < best_hist.size(); i++) history[i] = best_hist[i];
  return hipSuccess;
}

}  // namespace

size_t train_workspace_bytes(int k, int N, int64_t m_train, int64_t m_valid) {
  return carve(nullptr, k, N, m_train, m_valid, nullptr);
}

hipError_t train_codebook(int k, int N, const double* train, int64_t mt, const double* valid, int64_t mv,
                          const double* starts, int restarts, int max_iter, double rel_tol, float* out, double* out64,
                          double* restart_mse, double* valid_mse, double* history, int* history_len, void* ws,
                          hipStream_t s) {
#define FQ_T(KK)                                                                                                  \
  case KK:                                                                                                        \
    return train_k<KK>(N, train, mt, valid, mv, starts, restarts, max_iter, rel_tol, out, out64, restart_mse,     \
                       valid_mse, history, history_len, ws, s)
  switch (k) {
    FQ_T(1);
    FQ_T(2);
    FQ_T(4);
    FQ_T(8);
    FQ_T(16);
    FQ_T(32);
    FQ_T(64);
    default: return hipErrorInvalidValue;
  }
#undef FQ_T
}

}  // namespace fq
