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
// Lanes take the chunks' statistics in parallel (max, weights, weighted sum); the
// weights go to LDS; then every lane (one dimension) sums the chunks'
// accumulators with the loads of 8 chunks in flight.
constexpr int COMB_W = 1024;  // chunks whose weights are kept in LDS
__global__ __launch_bounds__(64) void attn_combine(const float* __restrict__ ws, const float* __restrict__ pi32,
                                                   int nchunks, float* __restrict__ out) {
  constexpr int PRE = 16;  // accumulators of the first chunks, loaded before anything waits
  __shared__ float ot[D];
  __shared__ float wsh[COMB_W];
  const int64_t bh = blockIdx.x;
  const int lane = threadIdx.x;
  const float NEG = -__builtin_huge_valf();
  const float* rec = ws + bh * nchunks * REC;
  float v[PRE];
#pragma unroll
  for (int e = 0; e < PRE; e++) v[e] = e < nchunks ? rec[(int64_t)e * REC + 2 + lane] : 0.f;
  float pc[D];  // column `lane` of Pi
#pragma unroll
  for (int j = 0; j < D; j++) pc[j] = pi32[j * D + lane];
  float M = NEG;
  for (int c = lane; c < nchunks; c += 64) M = fmaxf(M, rec[(int64_t)c * REC]);
#pragma unroll
  for (int s2 = 32; s2 >= 1; s2 >>= 1) M = fmaxf(M, __shfl_xor(M, s2));
  float Ls = 0.f;
  for (int c = lane; c < nchunks; c += 64) {
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
  ot[lane] = A / Ls;
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
//     lo parts in 8..15), so QK takes 4 matrix ops per 32 tokens; one DPP add
//     (lane col + lane col ^ 8) recombines them.
//   * PV puts P' hi in rows 0..7 and lo in rows 8..15 (summed once at the end)
//     and reads the value operand transposed straight from the LDS codebook
//     with ds_read_tr16_b64: lane 4a + b of a 16-lane group receives element b
//     of the 8-byte rows addressed by lanes a, a+4, a+8, a+12, so lanes
//     address (token a', block) rows and receive 4 tokens of one dimension.
//     The K order inside a 32-token tile is permuted (k = 8 grp + 4 a + i is
//     token 16 a + 4 grp + i) so P' comes straight from the QK registers.
//   * The running max and the rescaling happen once per 64 tokens.
//   * Every wave streams its own 128-token sub-chunks (codes and norms, 4.5 KiB)
//     through a private double buffer filled by direct global-to-LDS loads and
//     waits only for its own loads: no workgroup barrier inside the stream.
//   * The workgroup merges its waves into one partial record per query head;
//     attn_combine merges the records.  (Merging inside the kernel would need a
//     device-scope fence per workgroup, which on this multi-die part writes back
//     and invalidates the die's L2 and costs far more than a second launch.)
constexpr int SC = 128;  // tokens per wave sub-chunk
constexpr int GF = 8;    // query heads per KV head on the fast path
constexpr int SC_KC = 0, SC_VC = SC * 16, SC_KN = 2 * SC * 16, SC_VN = 2 * SC * 16 + SC * 2;
constexpr int SC_BYTES = 2 * SC * 16 + 4 * SC;  // 4608
constexpr int WG_TOKENS_UNIT = AW * SC;         // 512: workgroup token ranges are multiples of this

typedef short short4_ __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_ lds_s4;
typedef __attribute__((address_space(3))) void lds_void;

__device__ inline half8 gather2(const _Float16* __restrict__ cbL, uint32_t c0, uint32_t c1) {
  const half4 a = *reinterpret_cast<const half4*>(cbL + c0 * 4);
  const half4 b = *reinterpret_cast<const half4*>(cbL + c1 * 4);
  return half8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

__device__ inline _Float16 hlo(uint32_t w) { return __builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)); }
__device__ inline _Float16 hhi(uint32_t w) { return __builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// value of lane (l ^ 8) within its 16-lane row
__device__ inline float swap8(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xf, 0xf, true));
}

// Codes and norms of the nt tokens starting at slab token tok0 into the wave's
// buffer: always 6 load instructions (token indices past nt are clamped to the
// last valid token, whose bytes land in slots the compute masks), so a wave can
// wait for exactly the older sub-chunk with vmcnt(6).  nt is a multiple of 8.
__device__ inline void attn_sub_load(const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc,
                                     const _Float16* __restrict__ kn, const _Float16* __restrict__ vn, int64_t tok0,
                                     int nt, char* dst, int lane) {
#pragma unroll
  for (int p = 0; p < 2; p++) {
    const int t = (64 * p + lane) < nt ? (64 * p + lane) : nt - 1;
    lds_dma16(kc + (tok0 + t) * 16, dst + SC_KC + p * 1024);
    lds_dma16(vc + (tok0 + t) * 16, dst + SC_VC + p * 1024);
  }
  const int t2 = (2 * lane) < nt ? 2 * lane : nt - 2;  // two norms per lane
  lds_dma4(kn + tok0 + t2, dst + SC_KN);
  lds_dma4(vn + tok0 + t2, dst + SC_VN);
}

// Value of lane l ^ 8 (row_ror:8 within each 16-lane row).
__device__ inline uint32_t ror8u(uint32_t v) { return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xf, 0xf, true); }
// Lanes 8..15 of each row take lane l - 8's `src`, lanes 0..7 keep `keep`.
__device__ inline uint32_t from_lo_partner(uint32_t keep, uint32_t src) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)keep, (int)src, 0x128, 0xf, 0xc, false);
}
// Lanes 0..7 of each row take lane l + 8's `src`, lanes 8..15 keep `keep`.
__device__ inline uint32_t from_hi_partner(uint32_t keep, uint32_t src) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)keep, (int)src, 0x128, 0xf, 0x3, false);
}

// One wave's sub-chunk (tokens 0 .. 127 of `cur`, nt valid) as two halves of
// 64 tokens: scores first, then one max / rescale, then the exponentials and
// PV.  MASK: tokens at or past `nt` are excluded.
//
// Layouts inside a 32-token group starting at tb (lane = 16 grp + col):
//   QK tile a (tokens tb + 16 a + 0..15): A row col = token tb + 16 a + col; its
//   k = 8 grp + j is dimension 16 grp + 8 s + j for matrix op s, i.e. codes
//   4 grp + 2 s and 4 grp + 2 s + 1 = bytes 2 s, 2 s + 1 of the token's record
//   dword grp.  Output column col = head col & 7, query hi part (col < 8) or lo
//   part, rows 4 grp + i.
//   After the hi + lo recombination a lane holds whole scores of head col & 7
//   for tokens tb + 16 ah + 4 grp + i, ah = 0 in lanes col < 8 (tile 0) and 1
//   in lanes col >= 8 (tile 1): every score is computed once.
//   PV: k = 8 grp + 4 a + i is token tb + 16 a + 4 grp + i; P' rows 0..7 are
//   the hi parts of heads 0..7, rows 8..15 the lo parts.  Value operand dt,
//   lane c = 4 a' + b: the lane addresses token tb + 16 a + 4 grp + c / 4 and
//   the block whose code is byte dt of record dword c % 4 (block 4 (c % 4) + dt),
//   and receives dimension 16 a' + 4 dt + b of 4 tokens; output column c of
//   accumulator dt is dimension 16 (c / 4) + 4 dt + c % 4.
template <bool MASK>
__device__ inline void attn_sub(const char* __restrict__ cur, const _Float16* __restrict__ cbL, const half8 (&qb)[2],
                                int nt, int col, int grp, bool hi_col, float& m_run, float& l_run, f32x4 (&O)[4]) {
  const float NEG = -__builtin_huge_valf();
  const int ah = hi_col ? 0 : 1;
  const int own_tok = 16 * ah + 4 * grp;  // first of the lane's 4 tokens in a 32-token group
#pragma unroll 1
  for (int hf = 0; hf < 2; hf++) {
    // ---- scores: L[u][i] is token 64 hf + 32 u + own_tok + i, head col & 7
    float L[2][4];
#pragma unroll
    for (int u = 0; u < 2; u++) {
      const int tb = 64 * hf + 32 * u;
      f32x4 S[2];
#pragma unroll
      for (int a = 0; a < 2; a++) {
        const uint32_t w = reinterpret_cast<const uint32_t*>(cur + SC_KC + (tb + 16 * a + col) * 16)[grp];
        const half8 k0 = gather2(cbL, w & 0xffu, (w >> 8) & 0xffu);
        const half8 k1 = gather2(cbL, (w >> 16) & 0xffu, w >> 24);
        S[a] = mfma16(k0, qb[0], f32x4{0.f, 0.f, 0.f, 0.f});
        S[a] = mfma16(k1, qb[1], S[a]);
      }
      const uint2 nw = *reinterpret_cast<const uint2*>(cur + SC_KN + 2 * (tb + own_tok));
      const _Float16 kv[4] = {hlo(nw.x), hhi(nw.x), hlo(nw.y), hhi(nw.y)};
#pragma unroll
      for (int i = 0; i < 4; i++) {
        // own part: tile 0 in hi lanes, tile 1 in lo lanes; the partner lane (col ^ 8)
        // sends the other part of the same score
        const float mine = hi_col ? S[0][i] : S[1][i];
        const float send = hi_col ? S[1][i] : S[0][i];
        const float st = mine + __builtin_bit_cast(float, ror8u(__builtin_bit_cast(uint32_t, send)));
        L[u][i] = __builtin_fmaf(st, (float)kv[i], 0.0f);
        if constexpr (MASK) L[u][i] = (tb + own_tok + i) < nt ? L[u][i] : NEG;
      }
    }
    // ---- max per head over these 64 tokens and rescaling of the running state
    float mx = fmaxf(fmaxf(fmaxf(L[0][0], L[0][1]), fmaxf(L[0][2], L[0][3])),
                     fmaxf(fmaxf(L[1][0], L[1][1]), fmaxf(L[1][2], L[1][3])));
    mx = fmaxf(mx, swap8(mx));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (MASK && mx == NEG) continue;  // no valid tokens here (uniform)
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 while m_run is -inf
    l_run *= alpha;
    // accumulator rows 4 grp + i belong to head 4 (grp & 1) + i
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const float ai = __shfl(alpha, 4 * (grp & 1) + i);
#pragma unroll
      for (int dt = 0; dt < 4; dt++) O[dt][i] *= ai;
    }
    m_run = m_new;

    // ---- P' = p nu_v split hi + lo, exchanged with the partner lane, and PV
#pragma unroll
    for (int u = 0; u < 2; u++) {
      const int tb = 64 * hf + 32 * u;
      const uint2 nw = *reinterpret_cast<const uint2*>(cur + SC_VN + 2 * (tb + own_tok));
      const _Float16 vv[4] = {hlo(nw.x), hhi(nw.x), hlo(nw.y), hhi(nw.y)};
      float pv[4];
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const float p = __builtin_amdgcn_exp2f(L[u][i] - m_new);  // 0 for masked tokens
        l_run += p;
        pv[i] = __builtin_fmaf(p, (float)vv[i], 0.0f);
        if constexpr (MASK) pv[i] = (tb + own_tok + i) < nt ? pv[i] : 0.f;
      }
      // hi rounds toward zero (any rounding works: lo takes the exact remainder)
      uint32_t hw[2], lw[2];
#pragma unroll
      for (int e = 0; e < 2; e++) {
        hw[e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(pv[2 * e], pv[2 * e + 1]));
        const float ra = __builtin_fmaf((float)hlo(hw[e]), -1.0f, pv[2 * e]);
        const float rb = __builtin_fmaf((float)hhi(hw[e]), -1.0f, pv[2 * e + 1]);
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
            reinterpret_cast<const uint32_t*>(cur + SC_VC + (tb + 16 * a + 4 * grp + (col >> 2)) * 16)[col & 3];
#pragma unroll
        for (int dt = 0; dt < 4; dt++)
          vt[a][dt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(cbL + ((w >> (8 * dt)) & 0xffu) * 4));
      }
#pragma unroll
      for (int dt = 0; dt < 4; dt++) {
        const short4_ v0 = vt[0][dt], v1 = vt[1][dt];
        const half8 V = __builtin_bit_cast(half8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
        O[dt] = mfma16(P, V, O[dt]);
      }
    }
  }
}

__global__ __launch_bounds__(AW * 64, 4) void attn_k4b8(const _Float16* __restrict__ q, const float* __restrict__ pit32,
                                                        float qscale, const uint8_t* __restrict__ kc,
                                                        const _Float16* __restrict__ kn, const uint8_t* __restrict__ vc,
                                                        const _Float16* __restrict__ vn,
                                                        const _Float16* __restrict__ cw16, int Hq, int Hkv, int64_t T,
                                                        int64_t wg_tokens, int nrec, float* __restrict__ ws) {
  __shared__ __align__(16) char wbuf[AW * 2 * SC_BYTES];
  __shared__ __align__(16) _Float16 cbL[256 * 4];
  __shared__ float sm[AW * GF], sl[AW * GF];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rx = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = Hq / Hkv;
  const int64_t slab0 = ((int64_t)b * Hkv + g) * T;
  const int64_t t_begin = (int64_t)rx * wg_tokens;
  const int64_t t_end = (t_begin + wg_tokens) < T ? (t_begin + wg_tokens) : T;
  const int nsub = (int)((t_end - t_begin + SC - 1) / SC);
  char* mybuf = wbuf + w * 2 * SC_BYTES;

  // first sub-chunk of every wave on its way
  if (w < nsub) {
    const int64_t s0 = t_begin + (int64_t)w * SC;
    attn_sub_load(kc, vc, kn, vn, slab0 + s0, (t_end - s0) < SC ? (int)(t_end - s0) : SC, mybuf, lane);
  }
  for (int i = tid; i < 256 * 4 * 2 / 16; i += AW * 64)
    reinterpret_cast<uint4*>(cbL)[i] = reinterpret_cast<const uint4*>(cw16)[i];
  // rotated, scaled queries of the group's heads: qs[h][i] = qscale sum_j Pi[i][j] q[h][j],
  // computed in wave 0's second buffer, which no load touches before the barrier below;
  // lanes run over i, so the transposed rotation is read coalesced
  float* qs = reinterpret_cast<float*>(wbuf + SC_BYTES);
  {
    float* qin = qs + GF * D;  // raw queries
    for (int i = tid; i < G * D; i += AW * 64) qin[i] = (float)q[((int64_t)b * Hq + (int64_t)g * G) * D + i];
    __syncthreads();
    const int i = lane, h0 = w;  // heads h0 and h0 + AW
    float a0 = 0.f, a1 = 0.f;
#pragma unroll 16
    for (int j = 0; j < D; j++) {
      const float p = pit32[j * D + i];
      a0 = fmaf(p, qin[h0 * D + j], a0);
      a1 = fmaf(p, qin[(h0 + AW) * D + j], a1);
    }
    if (h0 < G) qs[h0 * D + i] = a0 * qscale;
    if (h0 + AW < G) qs[(h0 + AW) * D + i] = a1 * qscale;
    __syncthreads();
  }
  const int col = lane & 15, grp = lane >> 4, hd = col & 7;
  const bool hi_col = col < 8;
  // B operand of QK: column col = head hd, hi part (col < 8) or lo part; k = 8 grp + j is
  // dimension 16 grp + 8 s + j.
  half8 qb[2];
  {
    const float* qr = qs + (hd < G ? hd : 0) * D;
#pragma unroll
    for (int s = 0; s < 2; s++)
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const float v = hd < G ? qr[16 * grp + 8 * s + j] : 0.f;
        const _Float16 hv = (_Float16)v;
        qb[s][j] = hi_col ? hv : (_Float16)(v - (float)hv);
      }
  }
  __syncthreads();  // qs is read; wave 0 may now load into its second buffer

  float m_run = -__builtin_huge_valf(), l_run = 0.f;
  f32x4 O[4];
#pragma unroll
  for (int dt = 0; dt < 4; dt++) O[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  int k = 0;
  for (int j = w; j < nsub; j += AW, k++) {
    const int64_t s0 = t_begin + (int64_t)j * SC;
    const int nt = (t_end - s0) < SC ? (int)(t_end - s0) : SC;
    const int jn = j + AW;
    if (jn < nsub) {
      const int64_t s1 = t_begin + (int64_t)jn * SC;
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): reads of the buffer being refilled are done
      attn_sub_load(kc, vc, kn, vn, slab0 + s1, (t_end - s1) < SC ? (int)(t_end - s1) : SC,
                    mybuf + ((k + 1) & 1) * SC_BYTES, lane);
      __builtin_amdgcn_s_waitcnt(0x3f76);  // vmcnt(6): everything but the 6 loads just issued
    } else {
      __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0)
    }
    const char* cur = mybuf + (k & 1) * SC_BYTES;
    if (nt == SC)
      attn_sub<false>(cur, cbL, qb, nt, col, grp, hi_col, m_run, l_run, O);
    else
      attn_sub<true>(cur, cbL, qb, nt, col, grp, hi_col, m_run, l_run, O);
  }

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
    sm[w * GF + col] = m_run;
    sl[w * GF + col] = l;
  }
  __syncthreads();
  const float NEG = -__builtin_huge_valf();
  {
    const int h = tid >> 5, d0 = (tid & 31) * 2;
    if (h < G) {
      float M = NEG;
#pragma unroll
      for (int ww = 0; ww < AW; ww++) M = fmaxf(M, sm[ww * GF + h]);
      float wt[AW], Ls = 0.f;
#pragma unroll
      for (int ww = 0; ww < AW; ww++) {
        wt[ww] = sm[ww * GF + h] == NEG ? 0.f : __builtin_amdgcn_exp2f(sm[ww * GF + h] - M);
        Ls += sl[ww * GF + h] * wt[ww];
      }
      float* rec = ws + (((int64_t)b * Hq + (int64_t)g * G + h) * nrec + rx) * REC;
      if (d0 == 0) {
        rec[0] = M;
        rec[1] = Ls;
      }
#pragma unroll
      for (int e = 0; e < 2; e++) {
        float A = 0.f;
#pragma unroll
        for (int ww = 0; ww < AW; ww++) A += so[(ww * GF + h) * D + d0 + e] * wt[ww];
        rec[2 + d0 + e] = A;
      }
    }
  }
}


size_t attn_smem_bytes(int N, int K) {
  return (size_t)((N * K * 2 + 15) & ~15) + sizeof(float) * (GMAX * D + 2 * AW * GMAX + AW * GMAX * D);
}

}  // namespace

#ifndef FQ_ONLY_K
// k = 4 with 8-bit codes, at most 8 query heads per KV head and T a multiple of 8
// runs attn_k4b8.
bool attn_fast_path(const fq_codebook* cb, int Hq, int Hkv, int64_t T) {
  return cb->k == 4 && cb->bits == 8 && Hq / Hkv <= GF && T % 8 == 0 && T < ((int64_t)1 << 40);
}

AttnPlan attn_plan(const fq_codebook* cb, int B, int Hq, int Hkv, int64_t T) {
  if (attn_fast_path(cb, Hq, Hkv, T)) {
    // about 1024 workgroups (4 per CU), each over a multiple of 512 consecutive tokens
    const int64_t units = (T + WG_TOKENS_UNIT - 1) / WG_TOKENS_UNIT, slabs = (int64_t)B * Hkv;
    int64_t upw = units * slabs / 1024;
    if (upw < 1) upw = 1;
    if (upw > units) upw = units;
    const int64_t nrec = (units + upw - 1) / upw;
    return AttnPlan{(int)nrec, upw * WG_TOKENS_UNIT, (int)units, (int)upw, true};
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
  return AttnPlan{(int)nc, tc, 0, 0, false};
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
  const AttnPlan plan = attn_plan(cb, B, Hq, Hkv, T);
  const float qscale = scale * 1.4426950408889634f;  // log2(e)
  const dim3 grid((unsigned)plan.nchunks, (unsigned)Hkv, (unsigned)B);
  const size_t sh = attn_smem_bytes(cb->N, cb->k);
  float* ws = reinterpret_cast<float*>(workspace);
  const _Float16* qh = reinterpret_cast<const _Float16*>(q);
  const _Float16* kn = reinterpret_cast<const _Float16*>(k_norms);
  const _Float16* vn = reinterpret_cast<const _Float16*>(v_norms);
  hipError_t e;
  if (plan.fast) {
    hipLaunchKernelGGL(attn_k4b8, grid, dim3(AW * 64), 0, s, qh, cb->pit32, qscale, k_codes, kn, v_codes, vn,
                       cb->cw16, Hq, Hkv, T, plan.chunk_tokens, plan.nchunks, ws);
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
