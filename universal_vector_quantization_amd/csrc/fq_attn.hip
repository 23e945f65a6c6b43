// Decode attention fused with FibQuant decompression (FibQuant summary §5:
// fixed addresses let decompression live inside the attention kernel; §2.3:
// k_j = nu_j Pi^T concat(c), so q . k_j = nu_j (Pi q) . concat(c)).
//
// Split-K over the context.  One workgroup = one (batch, KV head, chunk of
// tokens); its 4 waves take interleaved 32-token tiles and keep an online
// softmax (running max m, running sum l, accumulator in the rotated domain).
// Per 32-token tile and wave, with the MFMA f32_16x16x32_f16 shape:
//   QK  : S^T[16 tok x 16 heads] = Khat[16 tok x 64] . Qrot^T[64 x 16 heads].
//         Khat rows are gathered straight from the fp16 codebook in LDS (a lane
//         holds one token and 8 consecutive dims = whole codewords), Qrot is
//         split hi + lo fp16 so the product keeps fp32-class accuracy.
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

template <int K>
__global__ __launch_bounds__(AW * 64) void attn_split(
    const _Float16* __restrict__ q, const uint8_t* __restrict__ kc, const _Float16* __restrict__ kn,
    const uint8_t* __restrict__ vc, const _Float16* __restrict__ vn, const _Float16* __restrict__ cw16,
    const float* __restrict__ pi32, int N, int bits, int Hq, int Hkv, int64_t T, int64_t Tc, int nchunks,
    float qscale, float* __restrict__ ws) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int cbBytes = (N * K * 2 + 15) & ~15;
  _Float16* cbL = reinterpret_cast<_Float16*>(smem);
  float* qt = reinterpret_cast<float*>(smem + cbBytes);  // [GMAX][64] rotated, scaled queries
  float* sm = qt + GMAX * D;                             // [AW][GMAX]
  float* sl = sm + AW * GMAX;                            // [AW][GMAX]
  float* so = sl + AW * GMAX;                            // [AW][GMAX][64]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int chunk = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = Hq / Hkv;
  const int B = (D / K) * bits;

  for (int w = tid; w < cbBytes / 16; w += AW * 64)
    reinterpret_cast<uint4*>(cbL)[w] = reinterpret_cast<const uint4*>(cw16)[w];
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

  const int64_t c0 = (int64_t)chunk * Tc;
  const int64_t c1 = (c0 + Tc) < T ? (c0 + Tc) : T;
  const int64_t base = ((int64_t)b * Hkv + g) * T;
  const float NEG = -__builtin_huge_valf();
  float m = NEG, l = 0.f;
  f32x4 o[4];
#pragma unroll
  for (int c = 0; c < 4; c++) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};

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
        wt[w] = exp2f(sm[w * GMAX + h] - M);
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
// Lane c < nchunks reads chunk c's statistics; the max and the weighted sum are
// wave reductions; every lane then sums its own dim over the chunks.
__global__ __launch_bounds__(64) void attn_combine(const float* __restrict__ ws, const float* __restrict__ pi32,
                                                   int nchunks, float* __restrict__ out) {
  __shared__ float ot[D];
  __shared__ float wsh[256];
  const int64_t bh = blockIdx.x;
  const int lane = threadIdx.x;
  const float* rec = ws + bh * nchunks * REC;
  float M = -__builtin_huge_valf();
  for (int c = lane; c < nchunks; c += 64) M = fmaxf(M, rec[c * REC]);
#pragma unroll
  for (int s2 = 32; s2 >= 1; s2 >>= 1) M = fmaxf(M, __shfl_xor(M, s2));
  float Ls = 0.f;
  for (int c = lane; c < nchunks; c += 64) {
    const float wgt = exp2f(rec[c * REC] - M);
    if (c < 256) wsh[c] = wgt;
    Ls += rec[c * REC + 1] * wgt;
  }
#pragma unroll
  for (int s2 = 32; s2 >= 1; s2 >>= 1) Ls += __shfl_xor(Ls, s2);
  __syncthreads();
  float A = 0.f;
  for (int c = 0; c < nchunks; c++) {
    const float wgt = c < 256 ? wsh[c] : exp2f(rec[c * REC] - M);
    A = fmaf(rec[c * REC + 2 + lane], wgt, A);
  }
  ot[lane] = A / Ls;
  __syncthreads();
  float o = 0.f;
#pragma unroll 8
  for (int j = 0; j < D; j++) o = fmaf(pi32[j * D + lane], ot[j], o);
  out[bh * D + lane] = o;
}

// ---------------------------------------------------------------------------
// Fast path for k = 4 with 8-bit codes (N <= 256), the attention workload's
// codebook.  Differences from attn_split:
//   * MFMA k-slot (lane group q, element j) of k-step s carries dimension
//     16q + 8s + j, i.e. blocks 4q + 2s and 4q + 2s + 1, so a lane's four codes
//     for one token are one aligned dword of the token's 16-byte code record and
//     one load instruction reads 16 consecutive records (256 B, coalesced).
//   * The value transpose selects, for k-step s and half hh, the dims
//     32hh + 16(r/8) + 8s + r%8 (r = 0..15); the accumulator rows follow that
//     order and are put back in place when the partial record is written.
//   * The next tile's codes and norms are loaded before the current tile is
//     processed; token offsets are 32-bit within one (batch, KV head) slab;
//     only the last tile of a chunk carries masks; the rotated queries come
//     precomputed from attn_prep.
__device__ inline half8 gather2(const _Float16* __restrict__ cbL, uint32_t c0, uint32_t c1) {
  const half4 a = *reinterpret_cast<const half4*>(cbL + c0 * 4);
  const half4 b = *reinterpret_cast<const half4*>(cbL + c1 * 4);
  return half8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

__device__ inline float h16lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)); }
__device__ inline float h16hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

struct TileData {
  uint32_t kd[2], vd[2];   // code dwords of tokens t0 + 16a + col (lane group grp)
  float kv[2][4], vv[2][4];  // norms of tokens t0 + 16a + 4grp + i
};

struct AttnState {
  float m, l;
  f32x4 o[4];
};

template <bool MASK>
__device__ inline void process_tile(AttnState& st, const TileData& d, const _Float16* __restrict__ cbL,
                                    const half8 (&qhi)[2], const half8 (&qlo)[2], const half8 (&isel)[2], int t0,
                                    int tend, int grp) {
  const float NEG = -__builtin_huge_valf();
  float L[2][4];
#pragma unroll
  for (int a = 0; a < 2; a++) {
    const uint32_t w = d.kd[a];
    const half8 k0 = gather2(cbL, w & 0xffu, (w >> 8) & 0xffu);
    const half8 k1 = gather2(cbL, (w >> 16) & 0xffu, w >> 24);
    f32x4 S = {0.f, 0.f, 0.f, 0.f};
    S = mfma16(k0, qhi[0], S);
    S = mfma16(k0, qlo[0], S);
    S = mfma16(k1, qhi[1], S);
    S = mfma16(k1, qlo[1], S);
#pragma unroll
    for (int i = 0; i < 4; i++) {
      L[a][i] = S[i] * d.kv[a][i];
      if constexpr (MASK) L[a][i] = (t0 + 16 * a + 4 * grp + i) < tend ? L[a][i] : NEG;
    }
  }
  float mx = fmaxf(fmaxf(fmaxf(L[0][0], L[0][1]), fmaxf(L[0][2], L[0][3])),
                   fmaxf(fmaxf(L[1][0], L[1][1]), fmaxf(L[1][2], L[1][3])));
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float mn = fmaxf(st.m, mx);  // finite: the tile holds at least one token
  const float alpha = __builtin_amdgcn_exp2f(st.m - mn);
  st.l *= alpha;
#pragma unroll
  for (int c = 0; c < 4; c++) st.o[c] *= alpha;
  half8 phi, plo;
#pragma unroll
  for (int a = 0; a < 2; a++) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const float p = __builtin_amdgcn_exp2f(L[a][i] - mn);
      st.l += p;
      const float pv = p * d.vv[a][i];
      const _Float16 hv = (_Float16)pv;
      phi[4 * a + i] = hv;
      plo[4 * a + i] = (_Float16)(pv - (float)hv);
    }
  }
  half8 av[4];
#pragma unroll
  for (int a = 0; a < 2; a++) {
    const uint32_t w = d.vd[a];
    const half8 v0 = gather2(cbL, w & 0xffu, (w >> 8) & 0xffu);
    const half8 v1 = gather2(cbL, (w >> 16) & 0xffu, w >> 24);
#pragma unroll
    for (int c = 0; c < 4; c++) {  // value tile c = (k-step c >> 1, half c & 1)
      const f32x4 X = mfma16((c >> 1) ? v1 : v0, isel[c & 1], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int i = 0; i < 4; i++) av[c][4 * a + i] = (_Float16)X[i];
    }
  }
#pragma unroll
  for (int c = 0; c < 4; c++) {
    st.o[c] = mfma16(av[c], phi, st.o[c]);
    st.o[c] = mfma16(av[c], plo, st.o[c]);
  }
  st.m = mn;
}

// Chunk-resident variant: the workgroup first copies its whole chunk (codes and
// norms of up to FCHUNK tokens, ~34 KB) into LDS with every load in flight at
// once, then the waves run the tile loop from LDS.  With several workgroups
// per CU one loads while another computes.
constexpr int FCHUNK = 512;

template <bool NAL>
__global__ __launch_bounds__(AW * 64) void attn_split_k4b8(
    const float* __restrict__ qrot, const uint32_t* __restrict__ kc, const _Float16* __restrict__ kn,
    const uint32_t* __restrict__ vc, const _Float16* __restrict__ vn, const _Float16* __restrict__ cw16, int N,
    int Hq, int Hkv, int64_t T, int nchunks, float* __restrict__ ws) {
  __shared__ __align__(16) uint32_t kcL[FCHUNK * 4];
  __shared__ __align__(16) uint32_t vcL[FCHUNK * 4];
  __shared__ __align__(16) _Float16 knL[FCHUNK];
  __shared__ __align__(16) _Float16 vnL[FCHUNK];
  __shared__ __align__(16) _Float16 cbL[256 * 4];
  __shared__ float sm[AW * GMAX], sl[AW * GMAX];
  __shared__ float so[AW * GMAX * D];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int chunk = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = Hq / Hkv;
  const int64_t base = ((int64_t)b * Hkv + g) * T + (int64_t)chunk * FCHUNK;
  const int rem = (int)(T - (int64_t)chunk * FCHUNK);
  const int nt = rem < FCHUNK ? rem : FCHUNK;

  // ---- bulk copy: codes (16 B per token), norms, codebook
  {
    const uint4* ks = reinterpret_cast<const uint4*>(kc) + base;
    const uint4* vs = reinterpret_cast<const uint4*>(vc) + base;
    uint4 kr[FCHUNK / (AW * 64)], vr[FCHUNK / (AW * 64)];
#pragma unroll
    for (int i = 0; i < FCHUNK / (AW * 64); i++) {
      const int t = tid + i * AW * 64;
      kr[i] = t < nt ? ks[t] : make_uint4(0u, 0u, 0u, 0u);
      vr[i] = t < nt ? vs[t] : make_uint4(0u, 0u, 0u, 0u);
    }
    uint4 nr = make_uint4(0u, 0u, 0u, 0u);
    const int q = tid & 63;  // 64 threads x 8 norms per array
    const _Float16* nsrc = (tid < 64 ? kn : vn) + base;
    if (tid < 128) {
      if (NAL && 8 * q + 7 < nt) {
        nr = reinterpret_cast<const uint4*>(nsrc)[q];
      } else {
        uint16_t hv[8];
#pragma unroll
        for (int j = 0; j < 8; j++)
          hv[j] = 8 * q + j < nt ? __builtin_bit_cast(uint16_t, nsrc[8 * q + j]) : (uint16_t)0;
        nr = make_uint4(hv[0] | (uint32_t)hv[1] << 16, hv[2] | (uint32_t)hv[3] << 16, hv[4] | (uint32_t)hv[5] << 16,
                        hv[6] | (uint32_t)hv[7] << 16);
      }
    }
    for (int w = tid; w < N * 4 * 2 / 16; w += AW * 64)
      reinterpret_cast<uint4*>(cbL)[w] = reinterpret_cast<const uint4*>(cw16)[w];
#pragma unroll
    for (int i = 0; i < FCHUNK / (AW * 64); i++) {
      const int t = tid + i * AW * 64;
      reinterpret_cast<uint4*>(kcL)[t] = kr[i];
      reinterpret_cast<uint4*>(vcL)[t] = vr[i];
    }
    if (tid < 128) reinterpret_cast<uint4*>(tid < 64 ? knL : vnL)[q] = nr;
  }

  const int col = lane & 15, grp = lane >> 4;
  half8 qhi[2], qlo[2], isel[2];
  {
    const float* qr = qrot + ((int64_t)b * Hq + (int64_t)g * G + (col < G ? col : 0)) * D;
#pragma unroll
    for (int s2 = 0; s2 < 2; s2++) {
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const float v = col < G ? qr[16 * grp + 8 * s2 + j] : 0.f;
        const _Float16 hv = (_Float16)v;
        qhi[s2][j] = hv;
        qlo[s2][j] = (_Float16)(v - (float)hv);
        isel[s2][j] = (_Float16)((grp == 2 * s2 + col / 8 && j == col % 8) ? 1.0f : 0.0f);
      }
    }
  }
  __syncthreads();

  AttnState st;
  st.m = -__builtin_huge_valf();
  st.l = 0.f;
#pragma unroll
  for (int c = 0; c < 4; c++) st.o[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  int t0 = wave * TILE;
  TileData d;
  for (; t0 < nt; t0 += AW * TILE) {
#pragma unroll
    for (int a = 0; a < 2; a++) {
      d.kd[a] = kcL[(t0 + 16 * a + col) * 4 + grp];
      d.vd[a] = vcL[(t0 + 16 * a + col) * 4 + grp];
      const uint2 kw = *reinterpret_cast<const uint2*>(knL + t0 + 16 * a + 4 * grp);
      const uint2 vw = *reinterpret_cast<const uint2*>(vnL + t0 + 16 * a + 4 * grp);
      d.kv[a][0] = h16lo(kw.x);
      d.kv[a][1] = h16hi(kw.x);
      d.kv[a][2] = h16lo(kw.y);
      d.kv[a][3] = h16hi(kw.y);
      d.vv[a][0] = h16lo(vw.x);
      d.vv[a][1] = h16hi(vw.x);
      d.vv[a][2] = h16lo(vw.y);
      d.vv[a][3] = h16hi(vw.y);
    }
    if (t0 + TILE <= nt)
      process_tile<false>(st, d, cbL, qhi, qlo, isel, t0, nt, grp);
    else
      process_tile<true>(st, d, cbL, qhi, qlo, isel, t0, nt, grp);
  }

  float l = st.l;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (grp == 0) {
    sm[wave * GMAX + col] = st.m;
    sl[wave * GMAX + col] = l;
  }
#pragma unroll
  for (int c = 0; c < 4; c++) {
    const int s2 = c >> 1, hh = c & 1;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int r = 4 * grp + i;
      so[(wave * GMAX + col) * D + 32 * hh + 16 * (r >> 3) + 8 * s2 + (r & 7)] = st.o[c][i];
    }
  }
  __syncthreads();
  {
    const float NEG = -__builtin_huge_valf();
    const int h = tid >> 4, d0 = (tid & 15) * 4;
    if (h < G) {
      float M = NEG;
#pragma unroll
      for (int w = 0; w < AW; w++) M = fmaxf(M, sm[w * GMAX + h]);
      float wt[AW], Ls = 0.f;
#pragma unroll
      for (int w = 0; w < AW; w++) {
        wt[w] = sm[w * GMAX + h] == NEG ? 0.f : __builtin_amdgcn_exp2f(sm[w * GMAX + h] - M);
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

// Rotated, scaled queries for the fast path: qrot = (scale log2 e) Pi q, fp32.
__global__ __launch_bounds__(64) void attn_prep(const _Float16* __restrict__ q, const float* __restrict__ pi32,
                                                float qscale, float* __restrict__ qrot) {
  __shared__ float qs[D];
  const int64_t bh = blockIdx.x;
  const int i = threadIdx.x;
  qs[i] = (float)q[bh * D + i];
  __syncthreads();
  float a = 0.f;
#pragma unroll 8
  for (int j = 0; j < D; j++) a = fmaf(pi32[i * D + j], qs[j], a);
  qrot[bh * D + i] = a * qscale;
}

size_t attn_smem_bytes(int N, int K) {
  return (size_t)((N * K * 2 + 15) & ~15) + sizeof(float) * (GMAX * D + 2 * AW * GMAX + AW * GMAX * D);
}

}  // namespace

#ifndef FQ_ONLY_K
// k = 4 with 8-bit codes runs the chunk-resident kernel.
bool attn_fast_path(const fq_codebook* cb, int64_t T) { return cb->k == 4 && cb->bits == 8 && T < ((int64_t)1 << 40); }

AttnPlan attn_plan(const fq_codebook* cb, int B, int Hkv, int64_t T) {
  if (attn_fast_path(cb, T)) return AttnPlan{(int)((T + FCHUNK - 1) / FCHUNK), (int64_t)FCHUNK};
  const int64_t per = (int64_t)AW * TILE;
  const int64_t groups = (int64_t)B * Hkv;
  const int64_t want = (2048 + groups - 1) / groups;
  const int64_t most = (T + per - 1) / per;
  int64_t nc = want < most ? want : most;
  if (nc < 1) nc = 1;
  int64_t tc = (T + nc - 1) / nc;
  tc = ((tc + per - 1) / per) * per;
  nc = (T + tc - 1) / tc;
  return AttnPlan{(int)nc, tc};
}

size_t attn_workspace_bytes(int B, int Hq, int nchunks) {
  // chunk partial records, then the rotated queries of the fast path
  return (size_t)B * (size_t)Hq * ((size_t)nchunks * REC + D) * sizeof(float);
}
#endif

// Launcher of the split kernel for one block size, instantiated per K in its
// own translation unit (compiled with -DFQ_ONLY_K=K).
template <int K>
hipError_t launch_attn_split_k(dim3 grid, size_t sh, hipStream_t s, const _Float16* q, const uint8_t* kc,
                               const _Float16* kn, const uint8_t* vc, const _Float16* vn, const fq_codebook* cb,
                               int Hq, int Hkv, int64_t T, int64_t Tc, int nchunks, float qscale, float* ws) {
  hipLaunchKernelGGL((attn_split<K>), grid, dim3(AW * 64), sh, s, q, kc, kn, vc, vn, cb->cw16, cb->pi32, cb->N,
                     cb->bits, Hq, Hkv, T, Tc, nchunks, qscale, ws);
  return hipGetLastError();
}

#define FQ_ATT_DECL(KK)                                                                                        \
  template hipError_t launch_attn_split_k<KK>(dim3, size_t, hipStream_t, const _Float16*, const uint8_t*,      \
                                              const _Float16*, const uint8_t*, const _Float16*, const fq_codebook*, \
                                              int, int, int64_t, int64_t, int, float, float*)
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
                       const uint8_t* v_codes, const void* v_norms, int B, int Hq, int Hkv, int64_t T, float scale,
                       float* out, void* workspace, hipStream_t s) {
  const AttnPlan plan = attn_plan(cb, B, Hkv, T);
  const float qscale = scale * 1.4426950408889634f;  // log2(e)
  const dim3 grid((unsigned)plan.nchunks, (unsigned)Hkv, (unsigned)B);
  const size_t sh = attn_smem_bytes(cb->N, cb->k);
  float* ws = reinterpret_cast<float*>(workspace);
  const _Float16* qh = reinterpret_cast<const _Float16*>(q);
  const _Float16* kn = reinterpret_cast<const _Float16*>(k_norms);
  const _Float16* vn = reinterpret_cast<const _Float16*>(v_norms);
  hipError_t e;
  if (attn_fast_path(cb, T)) {
    float* qrot = ws + (size_t)B * Hq * plan.nchunks * REC;
    hipLaunchKernelGGL(attn_prep, dim3((unsigned)(B * Hq)), dim3(64), 0, s, qh, cb->pi32, qscale, qrot);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const bool nal = (T % 8) == 0;  // 8 consecutive norms of a chunk are one aligned 16-byte load
#define FQ_FAST(NA)                                                                                           \
  hipLaunchKernelGGL(attn_split_k4b8<NA>, grid, dim3(AW * 64), 0, s, qrot,                                    \
                     reinterpret_cast<const uint32_t*>(k_codes), kn, reinterpret_cast<const uint32_t*>(v_codes), \
                     vn, cb->cw16, cb->N, Hq, Hkv, T, plan.nchunks, ws)
    if (nal)
      FQ_FAST(true);
    else
      FQ_FAST(false);
#undef FQ_FAST
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_combine, dim3((unsigned)(B * Hq)), dim3(64), 0, s, ws, cb->pi32, plan.nchunks, out);
    return hipGetLastError();
  }
#define FQ_ATT(KK)                                                                                                \
  e = launch_attn_split_k<KK>(grid, sh, s, qh, k_codes, kn, v_codes, vn, cb, Hq, Hkv, T, plan.chunk_tokens,       \
                              plan.nchunks, qscale, ws)
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
  hipLaunchKernelGGL(attn_combine, dim3((unsigned)(B * Hq)), dim3(64), 0, s, ws, cb->pi32, plan.nchunks, out);
  return hipGetLastError();
}
#endif

}  // namespace fq
