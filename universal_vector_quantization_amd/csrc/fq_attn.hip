// Decode attention fused with FibQuant decompression (FibQuant summary §5:
// fixed addresses let decompression live inside the attention kernel; §2.3:
// k_j = nu_j Pi^T concat(c), so q . k_j = nu_j (Pi q) . concat(c)).
//
// Split-K over the context.  One workgroup = one (batch, KV head, chunk of
// tokens); its 4 waves take interleaved 32-token tiles and keep an online
// softmax (running max m, running sum l, accumulator in the rotated domain).
// Per 32-token tile and wave, with the MFMA f32_16x16x32_f16 shape:
//   QK  : S^T[16 tok x 16 heads] = Khat[16 tok x 64] . Qrot^T[64 x 16 heads].
//         Khat rows are gathered straight from the fp16 codebook in LDS, or in
//         global memory for codebooks beyond the LDS (a lane holds one token and
//         8 consecutive dims of its codewords), Qrot is split hi + lo fp16 so the
//         product keeps fp32-class accuracy.
//   softmax: a lane owns one head and 8 tokens; the tile max needs 2 lane swaps.
//   V transpose: Vhat . I (I a 0/1 selector) turns the token-major gather into
//         the dim-major operand PV needs, exactly (products with 1 and 0).
//   PV  : O^T[64 dims x 16 heads] += Vhat^T[64 x 32 tok] . P'^T[32 tok x 16 heads]
//         with P' = p * nu_v split hi + lo fp16.  Token order inside the tile is
//         permuted identically on both operands, so P' comes straight from the
//         QK result registers.
// Heads of one KV group occupy the 16 MFMA columns (groups of up to 16).  A
// second kernel merges the chunks (log-sum-exp) and applies Pi^T once.
#include "fq_device.h"
#include "fq_internal.h"

namespace fq {
namespace {

constexpr int D = kD;
constexpr int AW = 4;     // waves per workgroup
constexpr int TILE = 32;  // tokens per wave step
constexpr int GMAX = 16;  // query heads per KV head held in the MFMA columns
constexpr int REC = 2 + D;  // partial record: m, l, acc[64]

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2_ __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ inline f32x4 mfma16(half8 a, half8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Keys batch b attends to: all T, or its valid length clamped to [0, T].
__device__ inline int64_t valid_keys(const int32_t* __restrict__ lens, int b, int64_t T) {
  if (!lens) return T;
  const int64_t L = lens[b];
  return L < 0 ? 0 : (L < T ? L : T);
}

// Balanced split of the fast kernel's workgroups under per-batch lengths.  Batch b's
// slabs (one per KV head) hold u_b = ceil(L_b / 64) units of 64 keys (a wave's unit).
// Of the W workgroups of the launch, every non-empty slab gets
//     n_b = min(u_b, cap, 1 + floor(u_b W' / U))   (U = Hkv sum_b u_b, W' = W - Hkv #{b : u_b > 0})
// pieces (cap: the records a (batch, head) has room for), so sum n <= W; piece p covers
// units [p u_b / n_b, (p + 1) u_b / n_b).  The largest share is then within one unit of
// the mean, whatever the lengths; a split over the slab capacity would leave the
// workgroups of long slabs with all the work.  Every quantity is wave-uniform; each
// wave computes it from lens on its own.
constexpr int BAL_UNIT = 64;
struct VarlenTotals {
  int64_t U, Wp, cap;
};

__device__ inline int64_t bal_units(const int32_t* __restrict__ lens, int b, int64_t T) {
  return (valid_keys(lens, b, T) + BAL_UNIT - 1) / BAL_UNIT;
}

__device__ inline int64_t bal_pieces(int64_t ub, const VarlenTotals& t) {
  if (ub == 0) return 0;
  int64_t n = 1 + ub * t.Wp / t.U;  // U >= ub > 0
  n = n < ub ? n : ub;
  return n < t.cap ? n : t.cap;
}

__device__ inline VarlenTotals varlen_totals(const int32_t* __restrict__ lens, int B, int Hkv, int64_t T, int64_t W,
                                             int64_t cap, int lane) {
  long long u = 0, e = 0;
  for (int b = lane; b < B; b += 64) {
    const int64_t ub = bal_units(lens, b, T);
    u += ub;
    e += ub > 0 ? 1 : 0;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    u += __shfl_xor(u, m);
    e += __shfl_xor(e, m);
  }
  return VarlenTotals{(int64_t)Hkv * u, W - (int64_t)Hkv * e, cap};
}

// The piece of workgroup `wid`: batch, KV head, piece index, pieces and units of its
// slab.  False when the workgroup has no piece.
__device__ inline bool varlen_piece(const int32_t* __restrict__ lens, int B, int Hkv, int64_t T,
                                    const VarlenTotals& t, int64_t wid, int lane, int& b, int& g, int& p, int64_t& n,
                                    int64_t& u) {
  int64_t base = 0;
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int bb = b0 + lane;
    const int64_t ub = bb < B ? bal_units(lens, bb, T) : 0;
    const int64_t nb = bal_pieces(ub, t);
    const long long c = (long long)Hkv * nb;
    long long incl = c;  // inclusive scan over the lanes
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const long long o = __shfl_up(incl, d);
      if (lane >= d) incl += o;
    }
    const int64_t tot = __shfl(incl, 63);
    if (wid < base + tot) {
      const uint64_t hit = __ballot(base + incl > wid);
      const int L = (int)__builtin_ctzll(hit);
      const int64_t start = base + __shfl(incl - c, L);
      n = __shfl((long long)nb, L);
      u = __shfl((long long)ub, L);
      const int64_t r = wid - start;
      b = b0 + L;
      g = (int)(r / n);
      p = (int)(r - (int64_t)g * n);
      return true;
    }
    base += tot;
  }
  return false;
}

// Dims [dim0, dim0+8) of the concatenated codewords of vector `vec`.
template <int K>
__device__ inline half8 gather8(const _Float16* __restrict__ cbL, const uint8_t* __restrict__ codes, int64_t vec,
                                int dim0, int B, int bits) {
  half8 r;
  if constexpr (K >= 8) {
    const uint32_t code = bits == 8 ? (uint32_t)codes[vec * (B >> 3) + dim0 / K]
                                    : load_code(codes, vec * B + (int64_t)(dim0 / K) * bits, bits);
    r = *reinterpret_cast<const half8*>(cbL + code * K + (dim0 % K));
  } else {
#pragma unroll
    for (int p = 0; p < 8 / K; p++) {
      const int blk = dim0 / K + p;
      const uint32_t code =
          bits == 8 ? (uint32_t)codes[vec * (B >> 3) + blk] : load_code(codes, vec * B + (int64_t)blk * bits, bits);
      if constexpr (K == 4) {
        const half4 c = *reinterpret_cast<const half4*>(cbL + code * 4);
#pragma unroll
        for (int t = 0; t < 4; t++) r[p * 4 + t] = c[t];
      } else if constexpr (K == 2) {
        const half2_ c = *reinterpret_cast<const half2_*>(cbL + code * 2);
        r[p * 2] = c[0];
        r[p * 2 + 1] = c[1];
      } else {
        r[p] = cbL[code];
      }
    }
  }
  return r;
}

// CBG: the codewords are gathered from the fp16 codebook in global memory (through
// L1 / L2) instead of an LDS copy, for codebooks beyond the LDS.
template <int K, bool CBG>
__global__ __launch_bounds__(AW * 64) void attn_split(
    const _Float16* __restrict__ q, const uint8_t* __restrict__ kc, const _Float16* __restrict__ kn,
    const uint8_t* __restrict__ vc, const _Float16* __restrict__ vn, const _Float16* __restrict__ cw16,
    const float* __restrict__ pi32, int N, int bits, int Hq, int Hkv, int64_t T, const int32_t* __restrict__ lens,
    int64_t Tc, int nchunks, float qscale, float* __restrict__ ws) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int cbBytes = CBG ? 0 : (N * K * 2 + 15) & ~15;
  const _Float16* cbL = CBG ? cw16 : reinterpret_cast<const _Float16*>(smem);
  float* qt = reinterpret_cast<float*>(smem + cbBytes);  // [GMAX][64] rotated, scaled queries
  float* sm = qt + GMAX * D;                             // [AW][GMAX]
  float* sl = sm + AW * GMAX;                            // [AW][GMAX]
  float* so = sl + AW * GMAX;                            // [AW][GMAX][64]

  const int tid = fq_tid(), lane = tid & 63, wave = tid >> 6;
  const int chunk = fq_bid_x(), g = fq_bid_y(), b = fq_bid_z();
  const int G = Hq / Hkv;
  const int B = (D / K) * bits;

  if constexpr (!CBG)
    for (int w = tid; w < cbBytes / 16; w += AW * 64)
      reinterpret_cast<uint4*>(smem)[w] = reinterpret_cast<const uint4*>(cw16)[w];
  {
    const int h = tid >> 4, r0 = (tid & 15) * 4;
#pragma unroll
    for (int rr = 0; rr < 4; rr++) {
      float a = 0.f;
      if (h < G) {
        const _Float16* qh = q + ((int64_t)b * Hq + (int64_t)g * G + h) * D;
        for (int j = 0; j < D; j++) a = fmaf(pi32[(r0 + rr) * D + j], (float)qh[j], a);
      }
      qt[h * D + r0 + rr] = a * qscale;
    }
  }
  __syncthreads();

  const int col = lane & 15, grp = lane >> 4;
  half8 qhi[2], qlo[2], isel[2];
#pragma unroll
  for (int s = 0; s < 2; s++) {
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const float v = qt[col * D + 32 * s + 8 * grp + j];
      const _Float16 hv = (_Float16)v;
      qhi[s][j] = hv;
      qlo[s][j] = (_Float16)(v - (float)hv);
      isel[s][j] = (_Float16)((8 * grp + j == 16 * s + col) ? 1.0f : 0.0f);
    }
  }

  const int64_t Tb = valid_keys(lens, b, T);
  const int64_t c0 = (int64_t)chunk * Tc;
  const int64_t c1 = (c0 + Tc) < Tb ? (c0 + Tc) : Tb;
  const int64_t base = ((int64_t)b * Hkv + g) * T;
  const float NEG = -__builtin_huge_valf();
  float m = NEG, l = 0.f;
  f32x4 o[4];
#pragma unroll
  for (int c = 0; c < 4; c++) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One 32-token tile of a wave: kr / vr the gathered key and value rows (lane: token
  // t0 + 16 a + col, dims 32 s + 8 grp .. + 7), nk / nv the norms of the lane's score
  // tokens t0 + 16 a + 4 grp + i.
  auto tile = [&](int64_t t0, const half8 (&kr)[2][2], const half8 (&vr)[2][2], const float (&nk)[2][4],
                  const float (&nv)[2][4]) {
    // ---- scores for tokens t0 + 16a + 4grp + i (a = 0, 1; i = 0..3), head = col
    float L[2][4];
#pragma unroll
    for (int a = 0; a < 2; a++) {
      f32x4 S = {0.f, 0.f, 0.f, 0.f};
      S = mfma16(kr[a][0], qhi[0], S);
      S = mfma16(kr[a][0], qlo[0], S);
      S = mfma16(kr[a][1], qhi[1], S);
      S = mfma16(kr[a][1], qlo[1], S);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int64_t tk = t0 + 16 * a + 4 * grp + i;
        L[a][i] = tk < c1 ? S[i] * nk[a][i] : NEG;
      }
    }
    // ---- online softmax (base 2: the log2(e) factor is folded into Qrot)
    float mx = NEG;
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
      for (int i = 0; i < 4; i++) mx = fmaxf(mx, L[a][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mn = fmaxf(m, mx);  // finite: the tile holds at least one token
    const float alpha = exp2f(m - mn);
    l *= alpha;
#pragma unroll
    for (int c = 0; c < 4; c++) o[c] *= alpha;
    half8 phi, plo;
#pragma unroll
    for (int a = 0; a < 2; a++) {
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int64_t tk = t0 + 16 * a + 4 * grp + i;
        const float p = exp2f(L[a][i] - mn);
        l += p;
        const float pv = tk < c1 ? p * nv[a][i] : 0.f;
        const _Float16 hv = (_Float16)pv;
        phi[4 * a + i] = hv;
        plo[4 * a + i] = (_Float16)(pv - (float)hv);
      }
    }
    // ---- gathered values, transposed to dim-major through the selector MFMA
    half8 av[4];
#pragma unroll
    for (int a = 0; a < 2; a++) {
#pragma unroll
      for (int c = 0; c < 4; c++) {
        const f32x4 X = mfma16(vr[a][c >> 1], isel[c & 1], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int i = 0; i < 4; i++) av[c][4 * a + i] = (_Float16)X[i];
      }
    }
    // ---- accumulate in the rotated domain
#pragma unroll
    for (int c = 0; c < 4; c++) {
      o[c] = mfma16(av[c], phi, o[c]);
      o[c] = mfma16(av[c], plo, o[c]);
    }
    m = mn;
  };
  // norms of the lane's score tokens of the tile at t0 (0 past the chunk)
  auto norms_at = [&](int64_t t0, float (&nk)[2][4], float (&nv)[2][4]) {
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int64_t tk = t0 + 16 * a + 4 * grp + i;
        nk[a][i] = tk < c1 ? (float)kn[base + tk] : 0.f;
        nv[a][i] = tk < c1 ? (float)vn[base + tk] : 0.f;
      }
  };

  if constexpr (CBG && K >= 8) {
    // Codebooks beyond the LDS, gathered from global memory: a tile's rows are one L2
    // round trip after its codes, so the codes run two tiles ahead and the rows one
    // tile ahead of the tile being computed (tokens past the chunk take code 0, whose
    // row is read and never weighted).  A lane's 8 dimensions lie in one block.
    const int64_t step = (int64_t)AW * TILE;
    auto codes_at = [&](int64_t t0, uint32_t (&ck)[2][2], uint32_t (&cv)[2][2]) {
#pragma unroll
      for (int a = 0; a < 2; a++) {
        const int64_t tr = t0 + 16 * a + col;
#pragma unroll
        for (int sx = 0; sx < 2; sx++) {
          const int64_t off = (base + tr) * B + (int64_t)((32 * sx + 8 * grp) / K) * bits;
          ck[a][sx] = tr < c1 ? load_code(kc, off, bits) : 0u;
          cv[a][sx] = tr < c1 ? load_code(vc, off, bits) : 0u;
        }
      }
    };
    auto rows_at = [&](const uint32_t (&ck)[2][2], const uint32_t (&cv)[2][2], half8 (&kr)[2][2],
                       half8 (&vr)[2][2]) {
#pragma unroll
      for (int a = 0; a < 2; a++)
#pragma unroll
        for (int sx = 0; sx < 2; sx++) {
          const int dim = (32 * sx + 8 * grp) % K;
          kr[a][sx] = *reinterpret_cast<const half8*>(cbL + (size_t)ck[a][sx] * K + dim);
          vr[a][sx] = *reinterpret_cast<const half8*>(cbL + (size_t)cv[a][sx] * K + dim);
        }
    };
    int64_t t0 = c0 + (int64_t)wave * TILE;
    uint32_t ck[2][2], cv[2][2];
    half8 kr[2][2], vr[2][2];
    float nk[2][4], nv[2][4];
    codes_at(t0, ck, cv);
    rows_at(ck, cv, kr, vr);
    norms_at(t0, nk, nv);
    codes_at(t0 + step, ck, cv);
    for (; t0 < c1; t0 += step) {
      half8 kr2[2][2], vr2[2][2];
      float nk2[2][4], nv2[2][4];
      rows_at(ck, cv, kr2, vr2);
      norms_at(t0 + step, nk2, nv2);
      codes_at(t0 + 2 * step, ck, cv);
      tile(t0, kr, vr, nk, nv);
#pragma unroll
      for (int a = 0; a < 2; a++)
#pragma unroll
        for (int sx = 0; sx < 2; sx++) {
          kr[a][sx] = kr2[a][sx];
          vr[a][sx] = vr2[a][sx];
        }
#pragma unroll
      for (int a = 0; a < 2; a++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          nk[a][i] = nk2[a][i];
          nv[a][i] = nv2[a][i];
        }
    }
  } else {
    for (int64_t t0 = c0 + (int64_t)wave * TILE; t0 < c1; t0 += AW * TILE) {
      // ---- scores for tokens t0 + 16a + 4grp + i (a = 0, 1; i = 0..3), head = col
      float L[2][4];
  #pragma unroll
      for (int a = 0; a < 2; a++) {
        const int64_t tr = t0 + 16 * a + col;
        half8 k0 = {}, k1 = {};
        if (tr < c1) {
          k0 = gather8<K>(cbL, kc, base + tr, 8 * grp, B, bits);
          k1 = gather8<K>(cbL, kc, base + tr, 32 + 8 * grp, B, bits);
        }
        f32x4 S = {0.f, 0.f, 0.f, 0.f};
        S = mfma16(k0, qhi[0], S);
        S = mfma16(k0, qlo[0], S);
        S = mfma16(k1, qhi[1], S);
        S = mfma16(k1, qlo[1], S);
  #pragma unroll
        for (int i = 0; i < 4; i++) {
          const int64_t tk = t0 + 16 * a + 4 * grp + i;
          L[a][i] = tk < c1 ? S[i] * (float)kn[base + tk] : NEG;
        }
      }
      // ---- online softmax (base 2: the log2(e) factor is folded into Qrot)
      float mx = NEG;
  #pragma unroll
      for (int a = 0; a < 2; a++)
  #pragma unroll
        for (int i = 0; i < 4; i++) mx = fmaxf(mx, L[a][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mn = fmaxf(m, mx);  // finite: the tile holds at least one token
      const float alpha = exp2f(m - mn);
      l *= alpha;
  #pragma unroll
      for (int c = 0; c < 4; c++) o[c] *= alpha;
      half8 phi, plo;
  #pragma unroll
      for (int a = 0; a < 2; a++) {
  #pragma unroll
        for (int i = 0; i < 4; i++) {
          const int64_t tk = t0 + 16 * a + 4 * grp + i;
          const float p = exp2f(L[a][i] - mn);
          l += p;
          const float pv = tk < c1 ? p * (float)vn[base + tk] : 0.f;
          const _Float16 hv = (_Float16)pv;
          phi[4 * a + i] = hv;
          plo[4 * a + i] = (_Float16)(pv - (float)hv);
        }
      }
      // ---- gathered values, transposed to dim-major through the selector MFMA
      half8 av[4];
  #pragma unroll
      for (int a = 0; a < 2; a++) {
        const int64_t tr = t0 + 16 * a + col;
        half8 v0 = {}, v1 = {};
        if (tr < c1) {
          v0 = gather8<K>(cbL, vc, base + tr, 8 * grp, B, bits);
          v1 = gather8<K>(cbL, vc, base + tr, 32 + 8 * grp, B, bits);
        }
  #pragma unroll
        for (int c = 0; c < 4; c++) {
          const f32x4 X = mfma16(c < 2 ? v0 : v1, isel[c & 1], f32x4{0.f, 0.f, 0.f, 0.f});
  #pragma unroll
          for (int i = 0; i < 4; i++) av[c][4 * a + i] = (_Float16)X[i];
        }
      }
      // ---- accumulate in the rotated domain
  #pragma unroll
      for (int c = 0; c < 4; c++) {
        o[c] = mfma16(av[c], phi, o[c]);
        o[c] = mfma16(av[c], plo, o[c]);
      }
      m = mn;
    }
  }

  // ---- merge the 4 waves, write this chunk's partial record per query head
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (grp == 0) {
    sm[wave * GMAX + col] = m;
    sl[wave * GMAX + col] = l;
  }
#pragma unroll
  for (int c = 0; c < 4; c++)
#pragma unroll
    for (int i = 0; i < 4; i++) so[(wave * GMAX + col) * D + 16 * c + 4 * grp + i] = o[c][i];
  __syncthreads();
  {
    const int h = tid >> 4, d0 = (tid & 15) * 4;
    if (h < G) {
      float M = NEG;
#pragma unroll
      for (int w = 0; w < AW; w++) M = fmaxf(M, sm[w * GMAX + h]);
      float wt[AW], Ls = 0.f;
#pragma unroll
      for (int w = 0; w < AW; w++) {
        wt[w] = sm[w * GMAX + h] == NEG ? 0.f : exp2f(sm[w * GMAX + h] - M);  // a wave with no keys adds nothing
        Ls += sl[w * GMAX + h] * wt[w];
      }
      float* rec = ws + (((int64_t)b * Hq + (int64_t)g * G + h) * nchunks + chunk) * REC;
      if (d0 == 0) {
        rec[0] = M;
        rec[1] = Ls;
      }
#pragma unroll
      for (int e = 0; e < 4; e++) {
        float A = 0.f;
#pragma unroll
        for (int w = 0; w < AW; w++) A += so[(w * GMAX + h) * D + d0 + e] * wt[w];
        rec[2 + d0 + e] = A;
      }
    }
  }
}

// Log-sum-exp merge of the chunk partials and the single inverse rotation.
// Lanes take the chunks' statistics in parallel (max, weights, weighted sum); the
// weights go to LDS; then every lane (one dimension) sums the chunks'
// accumulators with the loads of 8 chunks in flight.
constexpr int COMB_W = 1024;  // chunks whose weights are kept in LDS
// stride: records per (batch, query head); with nbh (the fast kernel's balanced split
// under per-batch lengths) only the first nbh[batch] of them exist, else all `stride`.
__global__ __launch_bounds__(64) void attn_combine(const float* __restrict__ ws, const float* __restrict__ pi32,
                                                   int stride, float* __restrict__ out,
                                                   const int32_t* __restrict__ nbh, int Hq) {
  constexpr int PRE = 16;  // accumulators of the first chunks, loaded before anything waits
  __shared__ float ot[D];
  __shared__ float wsh[COMB_W];
  const int64_t bh = fq_bid_x();
  const int lane = fq_tid();
  const float NEG = -__builtin_huge_valf();
  const float* rec = ws + bh * stride * REC;
  // The first records' loads go out together with the record count's; records past
  // the count may hold anything and are dropped by selects below.
  float v[PRE];
#pragma unroll
  for (int e = 0; e < PRE; e++) v[e] = e < stride ? rec[(int64_t)e * REC + 2 + lane] : 0.f;
  // max and sum of chunk `lane` (the common case has at most 64 chunks: one round trip)
  float m0 = lane < stride ? rec[(int64_t)lane * REC] : NEG;
  float l0 = lane < stride ? rec[(int64_t)lane * REC + 1] : 0.f;
  float pc[D];  // column `lane` of Pi
#pragma unroll
  for (int j = 0; j < D; j++) pc[j] = pi32[j * D + lane];
  int nchunks = stride;
  if (nbh) {
    nchunks = nbh[bh / Hq];
#pragma unroll
    for (int e = 0; e < PRE; e++) v[e] = e < nchunks ? v[e] : 0.f;
    m0 = lane < nchunks ? m0 : NEG;
    l0 = lane < nchunks ? l0 : 0.f;
  }
  float M = m0;
  for (int c = lane + 64; c < nchunks; c += 64) M = fmaxf(M, rec[(int64_t)c * REC]);
#pragma unroll
  for (int s2 = 32; s2 >= 1; s2 >>= 1) M = fmaxf(M, __shfl_xor(M, s2));
  float Ls;
  {
    const float wgt = m0 == NEG ? 0.f : __builtin_amdgcn_exp2f(m0 - M);
    if (lane < COMB_W) wsh[lane] = wgt;
    Ls = l0 * wgt;
  }
  for (int c = lane + 64; c < nchunks; c += 64) {
    const float mc = rec[(int64_t)c * REC];
    const float wgt = mc == NEG ? 0.f : __builtin_amdgcn_exp2f(mc - M);
    if (c < COMB_W) wsh[c] = wgt;
    Ls = fmaf(rec[(int64_t)c * REC + 1], wgt, Ls);
  }
#pragma unroll
  for (int s2 = 32; s2 >= 1; s2 >>= 1) Ls += __shfl_xor(Ls, s2);
  __syncthreads();
  auto weight = [&](int c) {
    if (c < COMB_W) return wsh[c];
    const float mc = rec[(int64_t)c * REC];
    return mc == NEG ? 0.f : __builtin_amdgcn_exp2f(mc - M);
  };
  float A = 0.f;
#pragma unroll
  for (int e = 0; e < PRE; e++)
    if (e < nchunks) A = fmaf(v[e], weight(e), A);
  int c = PRE;
  for (; c + 8 <= nchunks; c += 8) {
    float t[8];
#pragma unroll
    for (int e = 0; e < 8; e++) t[e] = rec[(int64_t)(c + e) * REC + 2 + lane];
#pragma unroll
    for (int e = 0; e < 8; e++) A = fmaf(t[e], weight(c + e), A);
  }
  for (; c < nchunks; c++) A = fmaf(rec[(int64_t)c * REC + 2 + lane], weight(c), A);
  ot[lane] = Ls > 0.f ? A / Ls : 0.f;  // no keys at all (a zero valid length): output 0
  __syncthreads();
  float o = 0.f;
#pragma unroll
  for (int j = 0; j < D; j++) o = fmaf(pc[j], ot[j], o);
  out[bh * D + lane] = o;
}

// Fast path: k = 4 with 8-bit codes (N = 256), up to 8 query heads per KV head,
// T a multiple of 8 (the attention workload's shape).  Differences from
// attn_split:
//   * Query hi and lo parts sit in different MFMA columns (heads in 0..7, their
//     lo parts in 8..15) of QK; partner lanes (col, col ^ 8) hold the two parts
//     of both 16-token tiles: one add with the partner's value as a DPP operand
//     per tile and a select give each lane whole scores of its own tile, so every
//     score and every exponential is computed once.  Scores are kept relative to
//     the running softmax offset, which rides in the norm product's FMA.
//   * PV puts P' hi in rows 0..7 and lo in rows 8..15 (summed once at the end)
//     and reads the value operand transposed straight from the LDS codebook
//     with ds_read_tr16_b64: lane 4a + b of a 16-lane group receives element b
//     of the 8-byte rows addressed by lanes a, a+4, a+8, a+12, so lanes
//     address (token, block) rows and receive 4 tokens of one dimension.
//     The K order inside a 32-token tile is permuted (k = 8 grp + 4 a + i is
//     token 16 a + 4 grp + i) so P' comes straight from the QK registers.
//   * Every wave streams its own 64-token units (codes and norms, 2.25 KiB)
//     through 4 private LDS buffers filled by direct global-to-LDS loads issued
//     3 units ahead; it waits only for its own loads.
//   * Software pipeline: iteration h computes the scores and the running max of
//     unit h + 1 while it exponentiates unit h and accumulates its PV, so the
//     two dependency chains (LDS gathers -> QK -> cross-lane max, and
//     exp -> hi/lo split -> DPP exchange -> PV) overlap inside one wave.
//   * The workgroup merges its waves into one partial record per query head;
//     attn_combine merges the records.  (Merging inside the kernel would need a
//     device-scope fence per workgroup, which on this multi-die part writes back
//     and invalidates the die's L2 and costs far more than a second launch.)
constexpr int UT = 64;  // tokens per wave unit
constexpr int NBUF = 4;  // unit buffers per wave
constexpr int GF = 8;    // query heads per KV head on the fast path
constexpr int U_KC = 0, U_VC = UT * 16, U_KN = 2 * UT * 16, U_VN = 2 * UT * 16 + UT * 2;
constexpr int U_BYTES = 2 * UT * 16 + 4 * UT;  // 2304
constexpr int WG_TOKENS_UNIT = 2 * AW * UT;    // 512: workgroup token ranges are multiples of this

typedef short short4_ __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_ lds_s4;
typedef __attribute__((address_space(3))) void lds_void;

// two codewords at LDS byte offsets o0, o1 (8 bytes each) as one operand
__device__ inline half8 gather2(const _Float16* __restrict__ cbL, uint32_t o0, uint32_t o1) {
  const half4 a = *reinterpret_cast<const half4*>(reinterpret_cast<const char*>(cbL) + o0);
  const half4 b = *reinterpret_cast<const half4*>(reinterpret_cast<const char*>(cbL) + o1);
  return half8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

__device__ inline _Float16 hlo(uint32_t w) { return __builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)); }
__device__ inline _Float16 hhi(uint32_t w) { return __builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }
// LDS byte offset of the codeword whose code is byte 0 of a record dword: one shift with
// a byte operand select, as the code generator forms for bytes 1 to 3 by itself (for byte
// 0 it emits a shift and a mask)
__device__ inline uint32_t off_byte0(uint32_t w) {
  uint32_t r;
  __asm__("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0"
          : "=v"(r)
          : "v"(3u), "v"(w));
  return r;
}

// A value that is the same in every lane, declared so (scalar registers).
__device__ inline int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// value of lane (l ^ 8) within its 16-lane row
__device__ inline float swap8(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xf, 0xf, true));
}
// Lanes 8..15 of each row take lane l - 8's `src`, lanes 0..7 keep `keep`.
__device__ inline uint32_t from_lo_partner(uint32_t keep, uint32_t src) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)keep, (int)src, 0x128, 0xf, 0xc, false);
}
// Lanes 0..7 of each row take lane l + 8's `src`, lanes 8..15 keep `keep`.
__device__ inline uint32_t from_hi_partner(uint32_t keep, uint32_t src) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)keep, (int)src, 0x128, 0xf, 0x3, false);
}

// Codes and norms of the nt tokens starting at slab token tok0 into a unit
// buffer: always 3 load instructions (token indices past nt are clamped to the
// last valid token, whose bytes land in slots whose scores are masked), so a
// wave waits for an older unit with vmcnt(3 x younger units).  Norms move in
// pairs: an odd nt also brings the norm of token nt, which lies inside the slab
// (slab lengths are even) but past the valid keys, so its scores are masked and
// its value weight is forced to 0.
__device__ inline void attn_unit_load(const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc,
                                      const _Float16* __restrict__ kn, const _Float16* __restrict__ vn, int64_t tok0,
                                      int nt, char* dst, int lane) {
  const int t = lane < nt ? lane : nt - 1;
  lds_dma16(kc + (tok0 + t) * 16, dst + U_KC);
  lds_dma16(vc + (tok0 + t) * 16, dst + U_VC);
  // lanes 0..31: key norms of tokens 2 l, 2 l + 1; lanes 32..63: value norms
  const int nl = (nt + 1) & ~1;
  const int l2 = 2 * (lane & 31), t2 = l2 < nl ? l2 : nl - 2;
  lds_dma4(lane < 32 ? kn + tok0 + t2 : vn + tok0 + t2, dst + U_KN);
}

// Scores of one unit (stage A).  Layouts inside a 32-token group starting at
// tb = 32 u (lane = 16 grp + col):
//   QK tile a (tokens tb + 16 a + 0..15): A row col = token tb + 16 a + col; its
//   k = 8 grp + j is dimension 16 grp + 8 s + j for matrix op s, i.e. codes
//   4 grp + 2 s and 4 grp + 2 s + 1 = bytes 2 s, 2 s + 1 of the token's record
//   dword grp.  Output column col = head col & 7, query hi part (col < 8) or lo
//   part, rows 4 grp + i.  After the recombination the lane holds whole scores
//   of head col & 7 for tokens tb + own_tok + i (own_tok = 16 ah + 4 grp, ah =
//   0 in lanes col < 8 and 1 in lanes col >= 8).
// L = score - mref, the lane's head's current softmax offset folded into the norm
// product (one rounding).  Returns the maximum of the lane's own 8 values; MASK:
// tokens at or past nt give -inf.
template <bool MASK>
__device__ inline float attn_scores(const char* __restrict__ cur, const _Float16* __restrict__ cbL,
                                    const half8 (&qb)[2], int nt, int col, int grp, bool hi_col, int own_tok,
                                    float mref, float (&L)[2][4]) {
  const float NEG = -__builtin_huge_valf();
#pragma unroll
  for (int u = 0; u < 2; u++) {
    const int tb = 32 * u;
    f32x4 S[2];
#pragma unroll
    for (int a = 0; a < 2; a++) {
      const uint32_t w = reinterpret_cast<const uint32_t*>(cur + U_KC + (tb + 16 * a + col) * 16)[grp];
      const half8 k0 = gather2(cbL, off_byte0(w), ((w >> 8) & 0xffu) * 8u);
      const half8 k1 = gather2(cbL, ((w >> 16) & 0xffu) * 8u, (w >> 24) * 8u);
      S[a] = mfma16(k0, qb[0], f32x4{0.f, 0.f, 0.f, 0.f});
      S[a] = mfma16(k1, qb[1], S[a]);
    }
    const uint2 nw = *reinterpret_cast<const uint2*>(cur + U_KN + 2 * (tb + own_tok));
    const _Float16 kv[4] = {hlo(nw.x), hhi(nw.x), hlo(nw.y), hhi(nw.y)};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      // lanes col and col ^ 8 hold the hi and lo parts of both tiles' scores: each sum
      // is one add with the partner's value as a DPP operand; hi lanes keep tile 0's
      const float s0 = S[0][i] + swap8(S[0][i]);
      const float s1 = S[1][i] + swap8(S[1][i]);
      const float st = hi_col ? s0 : s1;
      L[u][i] = __builtin_fmaf(st, (float)kv[i], -mref);
      if constexpr (MASK) L[u][i] = (tb + own_tok + i) < nt ? L[u][i] : NEG;
      // formed here: sunk past the offset branch that follows, the sums would leave the
      // partner moves behind and lose their fused form
      __asm__ volatile("" : "+v"(L[u][i]));
    }
  }
  return fmaxf(fmaxf(fmaxf(L[0][0], L[0][1]), fmaxf(L[0][2], L[0][3])),
               fmaxf(fmaxf(L[1][0], L[1][1]), fmaxf(L[1][2], L[1][3])));
}

// Maximum over the lanes of one head (col & 7): partner lanes and the 4 row groups.
__device__ inline float head_max(float v) {
  v = fmaxf(v, swap8(v));
  v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
}

// Stage B of one unit: p = 2^L (L is already relative to the offset), l += p,
// P' = p nu_v split hi + lo and
// exchanged with the partner lane, O += V^T P'.  Masked tokens have p = 0; with
// MASK their value weight is set to 0 outright (their norm may be any bits).  Value operand dt,
// lane c = 4 a' + b: the lane addresses token tb + 16 a + 4 grp + c / 4 and the
// block whose code is byte dt of record dword c % 4 (block 4 (c % 4) + dt), and
// receives dimension 16 a' + 4 dt + b of 4 tokens; output column c of
// accumulator dt is dimension 16 (c / 4) + 4 dt + c % 4.
template <bool MASK>
__device__ inline void attn_pv(const char* __restrict__ cur, const _Float16* __restrict__ cbL, int col, int grp,
                               int own_tok, int nt, const float (&L)[2][4], float one, float& l_run,
                               f32x4 (&O)[4]) {
#pragma unroll
  for (int u = 0; u < 2; u++) {
    const int tb = 32 * u;
    const uint2 nw = *reinterpret_cast<const uint2*>(cur + U_VN + 2 * (tb + own_tok));
    const _Float16 vv[4] = {hlo(nw.x), hhi(nw.x), hlo(nw.y), hhi(nw.y)};
    float pv[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const float p = __builtin_amdgcn_exp2f(L[u][i]);
      l_run += p;
      pv[i] = __builtin_fmaf(p, (float)vv[i], 0.0f);
      if constexpr (MASK) pv[i] = (tb + own_tok + i) < nt ? pv[i] : 0.f;
    }
    // hi rounds toward zero (any rounding works: lo takes the exact remainder, formed by
    // one mixed-precision FMA from the packed hi half; `one` is 1.0 in a register the
    // compiler cannot see through, or it would turn the FMA into a convert and a subtract)
    uint32_t hw[2], lw[2];
#pragma unroll
    for (int e = 0; e < 2; e++) {
      hw[e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(pv[2 * e], pv[2 * e + 1]));
      const float ra = __builtin_fmaf(-(float)hlo(hw[e]), one, pv[2 * e]);
      const float rb = __builtin_fmaf(-(float)hhi(hw[e]), one, pv[2 * e + 1]);
      lw[e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(ra, rb));
    }
    // rows < 8 (hi lanes): hi parts of tile 0 (own) and tile 1 (from lane col + 8);
    // rows >= 8 (lo lanes): lo parts of tile 0 (from lane col - 8) and tile 1 (own)
    const uint32_t P0 = from_lo_partner(hw[0], lw[0]), P1 = from_lo_partner(hw[1], lw[1]);
    const uint32_t P2 = from_hi_partner(lw[0], hw[0]), P3 = from_hi_partner(lw[1], hw[1]);
    const half8 P = __builtin_bit_cast(half8, uint4{P0, P1, P2, P3});
    short4_ vt[2][4];
#pragma unroll
    for (int a = 0; a < 2; a++) {
      const uint32_t w =
          reinterpret_cast<const uint32_t*>(cur + U_VC + (tb + 16 * a + 4 * grp + (col >> 2)) * 16)[col & 3];
#pragma unroll
      for (int dt = 0; dt < 4; dt++)
        vt[a][dt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s4*)(reinterpret_cast<const char*>(cbL) + (dt == 0 ? off_byte0(w) : ((w >> (8 * dt)) & 0xffu) * 8u)));
    }
#pragma unroll
    for (int dt = 0; dt < 4; dt++) {
      const short4_ v0 = vt[0][dt], v1 = vt[1][dt];
      const half8 V = __builtin_bit_cast(half8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      O[dt] = mfma16(P, V, O[dt]);
    }
  }
}

__global__ __launch_bounds__(AW * 64, 4) void attn_k4b8(const _Float16* __restrict__ q,
                                                        const uint4* __restrict__ rot16, float qscale,
                                                        const uint8_t* __restrict__ kc,
                                                        const _Float16* __restrict__ kn, const uint8_t* __restrict__ vc,
                                                        const _Float16* __restrict__ vn,
                                                        const _Float16* __restrict__ cw16, int B, int Hq, int Hkv,
                                                        int64_t T, const int32_t* __restrict__ lens, int64_t wg_tokens,
                                                        int nrec, int gx, float* __restrict__ ws,
                                                        int32_t* __restrict__ nbh) {
  __shared__ __align__(16) char wbuf[AW * NBUF * U_BYTES];
  __shared__ __align__(16) _Float16 cbL[256 * 4];
  __shared__ float sm[AW * GF], sl[AW * GF];
  const int tid = fq_tid(), lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int rx = fq_bid_x(), g = fq_bid_y(), b = fq_bid_z();
  const int G = Hq / Hkv;
  int64_t t_begin, t_end;
  if (lens) {
    // balanced split over the valid keys (record index = piece index, stride nrec)
    const int64_t W = (int64_t)gx * Hkv * B;
    const VarlenTotals tt = varlen_totals(lens, B, Hkv, T, W, nrec, lane);
    int64_t pn = 0, pu = 0;
    const int64_t wid = ((int64_t)b * Hkv + g) * gx + rx;
    // records per head of every batch, for the combine (workgroup i < B writes batch i's,
    // empty batches included)
    if (tid == 0 && wid < B) nbh[wid] = (int32_t)bal_pieces(bal_units(lens, (int)wid, T), tt);
    if (!varlen_piece(lens, B, Hkv, T, tt, wid, lane, b, g, rx, pn, pu)) return;
    const int64_t Lb = valid_keys(lens, b, T);
    t_begin = BAL_UNIT * (rx * pu / pn);
    t_end = BAL_UNIT * ((rx + 1) * pu / pn);
    t_end = t_end < Lb ? t_end : Lb;
  } else {
    t_begin = (int64_t)rx * wg_tokens;
    t_end = (t_begin + wg_tokens) < T ? (t_begin + wg_tokens) : T;
  }
  // the slab and range are the same in every lane: keep them (and all unit addresses) in
  // scalar registers
  b = __builtin_amdgcn_readfirstlane(b);
  g = __builtin_amdgcn_readfirstlane(g);
  rx = __builtin_amdgcn_readfirstlane(rx);
  t_begin = uniform64(t_begin);
  t_end = uniform64(t_end);
  const int64_t slab0 = ((int64_t)b * Hkv + g) * T;
  // this wave's units: workgroup units w, w + AW, w + 2 AW, ...
  const int nu_wg = (int)((t_end - t_begin + UT - 1) / UT);
  const int nu = nu_wg > w ? (nu_wg - w + AW - 1) / AW : 0;
  char* mybuf = wbuf + w * NBUF * U_BYTES;
  auto unit_tok0 = [&](int h) { return t_begin + (int64_t)(w + AW * h) * UT; };
  auto unit_nt = [&](int h) {
    const int64_t r = t_end - unit_tok0(h);
    return r < UT ? (int)r : UT;
  };
  // A full unit's loads: codes from wave-uniform bases plus the lane's byte offset, norms
  // from a per-lane pointer that advances by a constant; partial units clamp per lane.
  const uint32_t voff16 = (uint32_t)lane * 16u;
  const char* nptr0 =
      reinterpret_cast<const char*>((lane < 32 ? kn : vn) + slab0 + t_begin + (int64_t)w * UT + 2 * (lane & 31));
  auto load_unit = [&](int h) {
    char* dst = mybuf + (h & (NBUF - 1)) * U_BYTES;
    if (unit_nt(h) == UT) {
      const int64_t tok0 = slab0 + unit_tok0(h);
      lds_dma16_s(kc + tok0 * 16, voff16, dst + U_KC);
      lds_dma16_s(vc + tok0 * 16, voff16, dst + U_VC);
      lds_dma4(nptr0 + (int64_t)h * (AW * UT * 2), dst + U_KN);
    } else {
      attn_unit_load(kc, vc, kn, vn, slab0 + unit_tok0(h), unit_nt(h), dst, lane);
    }
  };

  // The codebook (waves 0 and 1) goes first, through the direct-to-LDS path; the first
  // units follow the query rotation, whose compiler-inserted wait covers every load issued
  // before it: units issued ahead of it made every wave wait for them there, in the
  // start-up burst of all workgroups' loads (no early unit measured about 3 % faster than
  // two).  Every wait in the stream itself is an explicit count.
  if (w < 2)
    lds_dma16(reinterpret_cast<const char*>(cw16) + w * 1024 + lane * 16, reinterpret_cast<char*>(cbL) + w * 1024);
  const int pre = nu < NBUF - 1 ? nu : NBUF - 1;
  const int col = lane & 15, grp = lane >> 4, hd = col & 7;
  const bool hi_col = col < 8;
  const int own_tok = 16 * (hi_col ? 0 : 1) + 4 * grp;
  // Query rotation on the matrix core: wave w computes row tile w of (1024 Pi) q^T for the
  // group's heads with the split rotation operands of the codebook handle (hi + mid parts;
  // the lo part is 2^-22 of them and is left out), B = the raw fp16 queries (exact).  The
  // operand's row permutation leaves coordinates 16 grp + 4 w + i of head col & 7 in lane
  // (col, grp); they go through LDS (wave 2's last buffer, which the stream reaches only
  // after the barriers below) so every lane can build its QK B operand.  These loads are
  // compiler-visible; the compiler's wait for them also covers the codebook load above.
  float* qs = reinterpret_cast<float*>(wbuf + (3 * NBUF - 1) * U_BYTES);  // [GF][D]
  static_assert(GF * D * (int)sizeof(float) <= U_BYTES, "query staging");
  {
    half8 ra[2][2], qin[2];
#pragma unroll
    for (int s = 0; s < 2; s++) {
#pragma unroll
      for (int part = 0; part < 2; part++)
        ra[s][part] = __builtin_bit_cast(half8, rot16[((s * 4 + w) * 3 + part) * 64 + lane]);
      qin[s] = hd < G ? __builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(
                            q + ((int64_t)b * Hq + (int64_t)g * G + hd) * D + 32 * s + 8 * grp))
                      : half8{};
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 2; s++)
#pragma unroll
      for (int part = 0; part < 2; part++) acc = mfma16(ra[s][part], qin[s], acc);
    if (hi_col) {
      const float sc = qscale * (1.0f / 1024.0f);
#pragma unroll
      for (int i = 0; i < 4; i++) qs[hd * D + 16 * grp + 4 * w + i] = acc[i] * sc;
    }
  }
  __syncthreads();  // codebook in place, rotated queries staged
  // B operand of QK: column col = head col & 7, hi part (col < 8) or lo part; k = 8 grp + j
  // is dimension 16 grp + 8 s + j
  half8 qb[2];
#pragma unroll
  for (int s = 0; s < 2; s++)
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const float v = hd < G ? qs[hd * D + 16 * grp + 8 * s + j] : 0.f;
      const _Float16 hv = (_Float16)v;
      qb[s][j] = hi_col ? hv : (_Float16)(v - (float)hv);
    }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __syncthreads();  // the staging buffer is free again
  for (int h = 0; h < pre; h++) load_unit(h);

  // Softmax offset per head, lazily updated: exponentials are taken as 2^(L - m_run)
  // with m_run at least TAU above every score seen when it was last set, and m_run
  // moves only when a score exceeds it, so every weight is at most 1 and the wave
  // rescales its accumulators only when some head's scores rise by more than TAU
  // (after the first unit, rarely).  The decision is wave-uniform (one ballot); the
  // cross-lane maximum is formed only then.
  // Scores are kept relative to the offset (L = score - m_run): the subtraction rides in
  // the norm product, and a unit whose scores arrive before an offset move is shifted
  // once, in the rare moving path.  The first unit sets m_run.
  constexpr float TAU = 4.0f;
  float m_run = 0.f, l_run = 0.f;
  // 1.0 in a scalar register the compiler cannot fold (the P' remainder's FMA)
  float one = 1.0f;
  __asm__ volatile("" : "+s"(one));
  f32x4 O[4];
#pragma unroll
  for (int dt = 0; dt < 4; dt++) O[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto buf = [&](int h) -> const char* { return mybuf + (h & (NBUF - 1)) * U_BYTES; };
  // pipeline state: scores Lc of unit h relative to m_run, and (when pend) the factors
  // that move O and l_run from the previous offset to m_run
  float Lc[2][4], a_own = 0.f, a_row[4] = {0.f, 0.f, 0.f, 0.f};
  bool pend = false;
  // offset update after a unit (not the first) whose scores Lu, relative to m_run, have
  // lane maxima lmx: when some score exceeds the offset, every head's offset moves to TAU
  // above its maximum if that is higher (dm >= 0) and Lu is shifted to the new offset;
  // the factors for the lane's own sum and for the accumulator rows 4 grp + i (head
  // 4 (grp & 1) + i) are 2^-dm
  auto update_offset = [&](float lmx, float (&Lu)[2][4]) {
    pend = __builtin_amdgcn_ballot_w64(lmx > 0.f) != 0;
    if (pend) {
      const float dm = fmaxf(head_max(lmx) + TAU, 0.f);
      a_own = __builtin_amdgcn_exp2f(-dm);
#pragma unroll
      for (int i = 0; i < 4; i++) a_row[i] = __shfl(a_own, 4 * (grp & 1) + i);
      m_run += dm;
#pragma unroll
      for (int u = 0; u < 2; u++)
#pragma unroll
        for (int i = 0; i < 4; i++) Lu[u][i] -= dm;
    }
  };
  if (nu > 0) {
    if (pre == 3)
      __builtin_amdgcn_s_waitcnt(0x3f76);  // vmcnt(6): unit 0 landed
    else if (pre == 2)
      __builtin_amdgcn_s_waitcnt(0x3f73);  // vmcnt(3)
    else
      __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0)
    // the first unit sets the offset (scores relative to 0 until then)
    const float mx = unit_nt(0) == UT
                         ? attn_scores<false>(buf(0), cbL, qb, UT, col, grp, hi_col, own_tok, 0.f, Lc)
                         : attn_scores<true>(buf(0), cbL, qb, unit_nt(0), col, grp, hi_col, own_tok, 0.f, Lc);
    m_run = head_max(mx) + TAU;
#pragma unroll
    for (int u = 0; u < 2; u++)
#pragma unroll
      for (int i = 0; i < 4; i++) Lc[u][i] -= m_run;
  }
  // the pending offset move, applied to what is accumulated before the next PV
  auto apply_factors = [&]() {
    if (pend) {
      l_run *= a_own;
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int dt = 0; dt < 4; dt++) O[dt][i] *= a_row[i];
    }
  };
  // B(h) from scores Lcur at the current offset, then the offset update for unit h + 1
  // (scores Lnxt, lane maxima mxn)
  auto finish_unit = [&](int h, float mxn, const float (&Lcur)[2][4], float (&Lnxt)[2][4]) {
    apply_factors();
    attn_pv<false>(buf(h), cbL, col, grp, own_tok, UT, Lcur, one, l_run, O);
    update_offset(mxn, Lnxt);
  };
  // one steady-state iteration: unit h + 1 is full; its scores (into Lnxt) overlap unit h's PV
  auto step = [&](int h, const float (&Lcur)[2][4], float (&Lnxt)[2][4]) {
    // Waves of different workgroups share a SIMD, and its arbiter favours the oldest:
    // the last workgroups dispatched to a CU lagged by up to 8 us over their loop
    // (per-workgroup timestamps) and finished alone at low occupancy.  A wave lowers its
    // own priority as it gets through its units, so laggards catch up.
    {
      const int lvl = (4 * h) / nu;
      if (lvl == 0)
        __builtin_amdgcn_s_setprio(3);
      else if (lvl == 1)
        __builtin_amdgcn_s_setprio(2);
      else if (lvl == 2)
        __builtin_amdgcn_s_setprio(1);
      else
        __builtin_amdgcn_s_setprio(0);
    }
    if (h + 3 < nu) {
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): reads of unit h - 1's buffer are done
      load_unit(h + 3);
      __builtin_amdgcn_s_waitcnt(0x3f76);  // vmcnt(6): unit h + 1 landed
    } else if (h + 2 < nu) {
      __builtin_amdgcn_s_waitcnt(0x3f73);  // vmcnt(3)
    } else {
      __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0)
    }
    const float mxn = attn_scores<false>(buf(h + 1), cbL, qb, UT, col, grp, hi_col, own_tok, m_run, Lnxt);
    finish_unit(h, mxn, Lcur, Lnxt);
  };
  auto steady = [&](int h) { return h + 1 < nu && unit_nt(h + 1) == UT; };
  int h = 0;
  {
    // unrolled twice so the two score arrays swap roles without copies
    float Lb[2][4];
    bool in_b = false;
    while (true) {
      if (!steady(h)) break;
      step(h, Lc, Lb);
      h++;
      if (!steady(h)) {
        in_b = true;
        break;
      }
      step(h, Lb, Lc);
      h++;
    }
    if (in_b)
#pragma unroll
      for (int u = 0; u < 2; u++)
#pragma unroll
        for (int i = 0; i < 4; i++) Lc[u][i] = Lb[u][i];
  }
  if (h + 1 < nu) {  // unit h + 1 is the wave's last unit and is partial; all its loads were issued
    __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0)
    float Ln[2][4];
    const float mxn = attn_scores<true>(buf(h + 1), cbL, qb, unit_nt(h + 1), col, grp, hi_col, own_tok, m_run, Ln);
    finish_unit(h, mxn, Lc, Ln);
#pragma unroll
    for (int u = 0; u < 2; u++)
#pragma unroll
      for (int i = 0; i < 4; i++) Lc[u][i] = Ln[u][i];
    h++;
  }
  if (nu > 0) {  // the last unit's PV (the only unit that can be partial)
    apply_factors();
    const int ntl = unit_nt(h);
    if (ntl == UT)
      attn_pv<false>(buf(h), cbL, col, grp, own_tok, UT, Lc, one, l_run, O);
    else
      attn_pv<true>(buf(h), cbL, col, grp, own_tok, ntl, Lc, one, l_run, O);
  }

  __builtin_amdgcn_s_setprio(0);
  // ---- merge the waves: rows 4 grp + i (grp < 2) plus their lo rows (lane + 32)
  float l = l_run;  // lanes col and col ^ 8 summed different tokens of the same head
  l += swap8(l);
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  __syncthreads();                            // every wave is done with its buffers
  float* so = reinterpret_cast<float*>(wbuf);  // [AW][GF][D]
#pragma unroll
  for (int dt = 0; dt < 4; dt++)
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const float v = O[dt][i] + __shfl_xor(O[dt][i], 32);
      if (grp < 2) so[(w * GF + 4 * grp + i) * D + 16 * (col >> 2) + 4 * dt + (col & 3)] = v;
    }
  if (grp == 0 && col < GF) {
    sm[w * GF + col] = nu > 0 ? m_run : -__builtin_huge_valf();  // a wave without keys: empty
    sl[w * GF + col] = l;
  }
  __syncthreads();
  const float NEG = -__builtin_huge_valf();
  {
    const int hh = tid >> 5, d0 = (tid & 31) * 2;
    if (hh < G) {
      float M = NEG;
#pragma unroll
      for (int ww = 0; ww < AW; ww++) M = fmaxf(M, sm[ww * GF + hh]);
      float wt[AW], Ls = 0.f;
#pragma unroll
      for (int ww = 0; ww < AW; ww++) {
        wt[ww] = sm[ww * GF + hh] == NEG ? 0.f : __builtin_amdgcn_exp2f(sm[ww * GF + hh] - M);
        Ls += sl[ww * GF + hh] * wt[ww];
      }
      float* rec = ws + (((int64_t)b * Hq + (int64_t)g * G + hh) * nrec + rx) * REC;
      if (d0 == 0) {
        rec[0] = M;
        rec[1] = Ls;
      }
#pragma unroll
      for (int e = 0; e < 2; e++) {
        float A = 0.f;
#pragma unroll
        for (int ww = 0; ww < AW; ww++) A += so[(ww * GF + hh) * D + d0 + e] * wt[ww];
        rec[2 + d0 + e] = A;
      }
    }
  }
}

// LDS of attn_split: the codebook copy (none with the global codebook), then its own buffers
size_t attn_smem_bytes(int N, int K, bool cbg) {
  return (cbg ? (size_t)0 : (size_t)((N * K * 2 + 15) & ~15)) +
         sizeof(float) * (GMAX * D + 2 * AW * GMAX + AW * GMAX * D);
}

}  // namespace

#ifndef FQ_ONLY_K
// k = 4 with 8-bit codes, at most 8 query heads per KV head and T a multiple of 8
// runs attn_k4b8.
bool attn_fast_path(const fq_codebook* cb, int Hq, int Hkv, int64_t T) {
  return cb->k == 4 && cb->bits == 8 && cb->rot16 && Hq / Hkv <= GF && T % 8 == 0 && T < ((int64_t)1 << 40);
}

// Every codebook has a path: the general kernel gathers from an LDS copy of the fp16
// codebook when it fits beside its own buffers, else from the codebook in global
// memory; the lookup-table kernel serves the full-vector code where it is faster.
bool attn_supported(const fq_codebook* cb) {
  (void)cb;
  return true;
}

namespace {
// The lookup tables pay for their construction (N entries per query head) and for the
// final product of the weight histograms with the codebook when many keys share them:
// the full-vector code with at least 4 query heads per KV head, 4 heads' tables and
// histograms in one workgroup's LDS (N <= 4096 here) and T >= 4 N.  Otherwise the
// general kernel's gathers from global memory are faster (encoded caches, evicted:
// B = 12, Hq = Hkv = 12, T = 1024, N = 16384: 45 against 161 us; B = 16, Hq = 32,
// Hkv = 4, T = 32768, N = 16384: 233 against 287 us; at N = 4096 there the tables
// win, 157 against 215 us).
bool attn_use_lut(const fq_codebook* cb, int Hq, int Hkv, int64_t T) {
  if (cb->force_attn_gather) return false;
  if (cb->force_attn_lut) return attn_lut_supported(cb);
  const int G = Hkv > 0 ? Hq / Hkv : 0;
  return cb->k == D && G >= 4 && attn_lut_heads(cb, G) >= 4 && T >= 4 * (int64_t)cb->N;
}
// the split kernel gathers from the global codebook when the LDS copy does not fit
bool attn_split_global(const fq_codebook* cb) { return attn_smem_bytes(cb->N, cb->k, false) > cb->max_lds; }
}  // namespace

AttnPlan attn_plan(const fq_codebook* cb, int B, int Hq, int Hkv, int64_t T) {
  if (attn_use_lut(cb, Hq, Hkv, T)) {
    // one workgroup per CU: about 256 workgroups over (batch, KV head, head set, chunk)
    const int G = Hq / Hkv, gw = attn_lut_heads(cb, G);
    const int64_t sets = (int64_t)B * Hkv * (G / (gw > 0 ? gw : 1));
    int64_t nc = (256 + sets - 1) / sets;
    const int64_t most = (T + 63) / 64;
    if (nc > most) nc = most;
    if (nc < 1) nc = 1;
    int64_t tc = (T + nc - 1) / nc;
    tc = ((tc + 63) / 64) * 64;
    nc = (T + tc - 1) / tc;
    if (nc < 1) nc = 1;
    return AttnPlan{(int)nc, tc, 0, 0, false, gw};
  }
  if (!cb->force_attn_lut && attn_fast_path(cb, Hq, Hkv, T)) {
    // about 1024 workgroups (4 per CU), each over a multiple of 512 consecutive tokens
    const int64_t units = (T + WG_TOKENS_UNIT - 1) / WG_TOKENS_UNIT, slabs = (int64_t)B * Hkv;
    int64_t upw = units * slabs / 1024;
    if (upw < 1) upw = 1;
    if (upw > units) upw = units;
    const int64_t nrec = (units + upw - 1) / upw;
    return AttnPlan{(int)nrec, upw * WG_TOKENS_UNIT, (int)units, (int)upw, true, 0};
  }
  const int64_t per = (int64_t)AW * TILE;
  const int64_t groups = (int64_t)B * Hkv;
  const int64_t want = (2048 + groups - 1) / groups;
  const int64_t most = (T + per - 1) / per;
  int64_t nc = want < most ? want : most;
  if (nc < 1) nc = 1;
  int64_t tc = (T + nc - 1) / nc;
  tc = ((tc + per - 1) / per) * per;
  nc = (T + tc - 1) / tc;
  return AttnPlan{(int)nc, tc, 0, 0, false, 0};
}

hipError_t launch_attn_combine(const float* ws, const float* pi32, int64_t rows, int nchunks, float* out,
                               hipStream_t s) {
  hipLaunchKernelGGL(attn_combine, dim3((unsigned)rows), dim3(64), 0, s, ws, pi32, nchunks, out,
                     static_cast<const int32_t*>(nullptr), 1);
  return hipGetLastError();
}

size_t attn_records_bytes(int B, int Hq, int nchunks) {
  return (((size_t)B * (size_t)Hq * (size_t)nchunks * REC * sizeof(float)) + 255) & ~(size_t)255;
}

size_t attn_workspace_bytes(int B, int Hq, int Hkv, int nchunks) {
  (void)Hkv;
  // partial records, then one record count per batch (balanced split under lengths)
  return attn_records_bytes(B, Hq, nchunks) + (((size_t)B * sizeof(int32_t) + 255) & ~(size_t)255);
}

size_t attn_plan_workspace_bytes(const fq_codebook* cb, const AttnPlan& p, int B, int Hq, int Hkv) {
  return attn_workspace_bytes(B, Hq, Hkv, attn_record_stride(p)) + (p.lut_heads ? attn_lut_table_bytes(cb, B, Hq) : 0);
}

bool attn_plan_launchable(const AttnPlan& p, int B, int Hq, int Hkv) {
  const int64_t gy = p.lut_heads ? (int64_t)Hkv * (Hq / Hkv / p.lut_heads) : Hkv;
  return gy <= 65535 && B <= 65535 && (!p.lut_heads || (int64_t)B * Hkv <= 0x7fffffff);
}

int attn_record_stride(const AttnPlan& p) {
  // the fast path's balanced split under per-batch lengths uses up to one record per
  // 512-key unit of a slab; sized for it in every case so one workspace serves both
  return p.fast ? p.fast_chunks : p.nchunks;
}
#endif

// Launcher of the split kernel for one block size, instantiated per K in its
// own translation unit (compiled with -DFQ_ONLY_K=K).
template <int K>
hipError_t launch_attn_split_k(dim3 grid, bool cbg, hipStream_t s, const _Float16* q, const uint8_t* kc,
                               const _Float16* kn, const uint8_t* vc, const _Float16* vn, const fq_codebook* cb,
                               int Hq, int Hkv, int64_t T, const int32_t* lens, int64_t Tc, int nchunks,
                               float qscale, float* ws) {
  const size_t sh = attn_smem_bytes(cb->N, K, cbg);
  if (cbg) {
    hipLaunchKernelGGL((attn_split<K, true>), grid, dim3(AW * 64), sh, s, q, kc, kn, vc, vn, cb->cw16, cb->pi32,
                       cb->N, cb->bits, Hq, Hkv, T, lens, Tc, nchunks, qscale, ws);
    return hipGetLastError();
  }
  if (sh > 65536) {  // codebooks beyond 32 KiB of fp16 values: raise the dynamic LDS limit
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(attn_split<K, false>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)sh);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((attn_split<K, false>), grid, dim3(AW * 64), sh, s, q, kc, kn, vc, vn, cb->cw16, cb->pi32,
                     cb->N, cb->bits, Hq, Hkv, T, lens, Tc, nchunks, qscale, ws);
  return hipGetLastError();
}

#define FQ_ATT_DECL(KK)                                                                                        \
  template hipError_t launch_attn_split_k<KK>(dim3, bool, hipStream_t, const _Float16*, const uint8_t*,        \
                                              const _Float16*, const uint8_t*, const _Float16*, const fq_codebook*, \
                                              int, int, int64_t, const int32_t*, int64_t, int, float, float*)
#ifdef FQ_ONLY_K
FQ_ATT_DECL(FQ_ONLY_K);
#else
extern FQ_ATT_DECL(1);
extern FQ_ATT_DECL(2);
extern FQ_ATT_DECL(4);
extern FQ_ATT_DECL(8);
extern FQ_ATT_DECL(16);
extern FQ_ATT_DECL(32);
extern FQ_ATT_DECL(64);

hipError_t launch_attn(const fq_codebook* cb, const void* q, const uint8_t* k_codes, const void* k_norms,
                       const uint8_t* v_codes, const void* v_norms, const int32_t* lens, int B, int Hq, int Hkv,
                       int64_t T, float scale, float* out, void* workspace, hipStream_t s) {
  const AttnPlan plan = attn_plan(cb, B, Hq, Hkv, T);
  if (plan.lut_heads)
    return launch_attn_lut(cb, q, k_codes, k_norms, v_codes, v_norms, lens, B, Hq, Hkv, T, scale, plan, out,
                           workspace, s);
  const float qscale = scale * 1.4426950408889634f;  // log2(e)
  const dim3 grid((unsigned)plan.nchunks, (unsigned)Hkv, (unsigned)B);
  const bool cbg = attn_split_global(cb);
  float* ws = reinterpret_cast<float*>(workspace);
  const _Float16* qh = reinterpret_cast<const _Float16*>(q);
  const _Float16* kn = reinterpret_cast<const _Float16*>(k_norms);
  const _Float16* vn = reinterpret_cast<const _Float16*>(v_norms);
  hipError_t e;
  if (plan.fast) {
    // without lengths the records of a (batch, head) are the grid's chunks; with them,
    // the balanced split's pieces at a stride of one per 512-key unit
    const int stride = lens ? plan.fast_chunks : plan.nchunks;
    // batches' record counts after the records (balanced split only)
    int32_t* nbh = lens ? reinterpret_cast<int32_t*>(reinterpret_cast<char*>(workspace) +
                                                     attn_records_bytes(B, Hq, plan.fast_chunks))
                        : nullptr;
    hipLaunchKernelGGL(attn_k4b8, grid, dim3(AW * 64), 0, s, qh, reinterpret_cast<const uint4*>(cb->rot16), qscale,
                       k_codes, kn, v_codes, vn, cb->cw16, B, Hq, Hkv, T, lens, plan.chunk_tokens, stride,
                       plan.nchunks, ws, nbh);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_combine, dim3((unsigned)(B * Hq)), dim3(64), 0, s, ws, cb->pi32, stride, out,
                       static_cast<const int32_t*>(nbh), Hq);
    return hipGetLastError();
  }
#define FQ_ATT(KK)                                                                                                \
  e = launch_attn_split_k<KK>(grid, cbg, s, qh, k_codes, kn, v_codes, vn, cb, Hq, Hkv, T, lens,                  \
                              plan.chunk_tokens, plan.nchunks, qscale, ws)
  switch (cb->k) {
    case 1: FQ_ATT(1); break;
    case 2: FQ_ATT(2); break;
    case 4: FQ_ATT(4); break;
    case 8: FQ_ATT(8); break;
    case 16: FQ_ATT(16); break;
    case 32: FQ_ATT(32); break;
    case 64: FQ_ATT(64); break;
    default: return hipErrorInvalidValue;
  }
#undef FQ_ATT
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine, dim3((unsigned)(B * Hq)), dim3(64), 0, s, ws, cb->pi32, plan.nchunks, out,
                     static_cast<const int32_t*>(nullptr), Hq);
  return hipGetLastError();
}
#endif

}  // namespace fq
