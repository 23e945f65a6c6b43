// Decode attention through per-head lookup tables (FibQuant summary §5: fixed
// addresses let decompression be fused into attention; §2.3: k_j = nu_j Pi^T
// concat(c), so q . k_j = nu_j (Pi q) . concat(c)).
//
// For one (batch, query head) the table L[blk][n] = (Pi q)_blk . c_n * scale *
// log2 e holds the score per unit of norm of codeword n in block blk, so the
// score of key j is nu_j sum_blk L[blk][code_j,blk]: d/k table reads per key and
// head.  For the full-vector code (k = d) that is one read, and the table is N
// floats per head.  The tables pay off where many keys share them (grouped query
// heads, long contexts, N <= 4096); elsewhere the library sends k = d to the
// general kernel, which gathers the codewords from global memory.
// Values: sum_j p_j nu_j concat(c_j) taken block by block equals
// sum_n W[blk][n] c_n, where W[blk][n] sums p_j nu_j over the keys whose block
// blk holds code n.  Keys add their weights into W (LDS float atomics); one
// product of W with the codebook at the end gives the accumulator in the
// rotated domain.
//
// attn_lut_prep: the tables of every (batch, query head), into the workspace.
// attn_lut: one workgroup = one (batch, KV head, set of GW query heads, chunk of
//   keys); lane = key.
//   prologue: the GW tables into LDS, W = 0.
//   pass 1:   the exact maximum of the chunk's scores per head.
//   pass 2:   p = 2^(s - max), l += p, W[h][blk][vcode] += p nu_v.
//   epilogue: acc_h = per block sum_n W c_n; one record (max, l, acc) per head
//             for attn_combine (log-sum-exp over chunks, then Pi^T).
// Weights never exceed 1 (the maximum is exact), so no rescaling is needed.
// The atomic additions make the low bits of the result depend on their order.
#include "fq_device.h"
#include "fq_internal.h"

namespace fq {
namespace {

constexpr int D = kD;
constexpr int LW = 16;      // waves per workgroup of attn_lut
constexpr int REC = 2 + D;  // partial record: m, l, acc[64]

template <int K, int GW>
__host__ __device__ constexpr size_t lut_lds_bytes(int N) {
  // tables, W, per-wave partial accumulators, per-wave maxima / sums
  return (size_t)2 * GW * (D / K) * N * 4 + (size_t)LW * GW * D * 4 + (size_t)LW * GW * 4;
}

// Tables of all (batch, query head): block (x = batch * Hkv + KV head, y) computes
// the entries of codewords [PT y, PT y + PT) for the G heads of that KV group.
// The rotation (transposed) and the codeword tile (dim-major) are staged in LDS so
// every global read is coalesced and every LDS access is conflict-free or a
// broadcast (the tile's rows are padded by two values).  Query rotation in fp32 (64 products of exact fp16 query values).
constexpr int PT = 256;  // codewords per prep block (one per thread)
template <int K>
__global__ __launch_bounds__(PT) void attn_lut_prep(const _Float16* __restrict__ q, const float* __restrict__ pi32,
                                                    const _Float16* __restrict__ cw16, int N, int Hq, int Hkv,
                                                    float qscale, float* __restrict__ lut) {
  constexpr int NB = D / K;
  __shared__ float piT[D * (D + 1)];    // piT[j (D + 1) + r] = Pi[r][j]
  __shared__ float qv[8 * D];           // raw queries of the group, then rotated + scaled
  __shared__ _Float16 cT[K * (PT + 2)];  // cT[i (PT + 2) + nl] = coordinate i of codeword n0 + nl
  const int tid = fq_tid();
  const int bg = fq_bid_x(), b = bg / Hkv, g = bg % Hkv;
  const int G = Hq / Hkv;
  const int n0 = fq_bid_y() * PT;
  const int nt = (N - n0) < PT ? (N - n0) : PT;
  for (int i = tid; i < D * D; i += PT) piT[(i % D) * (D + 1) + i / D] = pi32[i];
  for (int i = tid; i < nt * K; i += PT) cT[(i % K) * (PT + 2) + i / K] = cw16[(int64_t)n0 * K + i];
  float c[K];
  for (int hb = 0; hb < G; hb += 8) {  // heads in batches of 8 (the qv buffer)
    const int hn = (G - hb) < 8 ? (G - hb) : 8;
    __syncthreads();
    for (int i = tid; i < hn * D; i += PT)
      qv[i] = (float)q[((int64_t)b * Hq + (int64_t)g * G + hb) * D + i];
    __syncthreads();
    float rq[4];  // rotated coordinates this thread computes (hn * D <= 512 = 2 per thread)
#pragma unroll
    for (int u = 0; u < 2; u++) {
      const int e = tid + u * PT;
      float a = 0.f;
      if (e < hn * D) {
        const int h = e / D, r = e % D;
        for (int j = 0; j < D; j++) a = fmaf(piT[j * (D + 1) + r], qv[h * D + j], a);
      }
      rq[u] = a * qscale;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 2; u++)
      if (tid + u * PT < hn * D) qv[tid + u * PT] = rq[u];
    __syncthreads();
    if (tid < nt) {
#pragma unroll
      for (int i = 0; i < K; i++) c[i] = (float)cT[i * (PT + 2) + tid];
      for (int h = 0; h < hn; h++)
#pragma unroll
        for (int blk = 0; blk < NB; blk++) {
          float a = 0.f;
#pragma unroll
          for (int i = 0; i < K; i++) a = fmaf(qv[h * D + blk * K + i], c[i], a);
          lut[(((int64_t)b * Hq + (int64_t)g * G + hb + h) * NB + blk) * N + n0 + tid] = a;
        }
    }
  }
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

template <int K, int GW>
__global__ __launch_bounds__(LW * 64) void attn_lut(const float* __restrict__ lut, const uint8_t* __restrict__ kc,
                                                    const _Float16* __restrict__ kn, const uint8_t* __restrict__ vc,
                                                    const _Float16* __restrict__ vn, const _Float16* __restrict__ cw16,
                                                    int N, int bits, int Hq, int Hkv, int64_t T,
                                                    const int32_t* __restrict__ lens, int64_t Tc, int nchunks,
                                                    float* __restrict__ ws) {
  constexpr int NB = D / K;
  extern __shared__ __align__(16) unsigned char smem[];
  const int TE = NB * N;  // table entries per head
  float* lutL = reinterpret_cast<float*>(smem);        // [GW][NB][N]
  float* wL = lutL + GW * TE;                          // [GW][NB][N]
  float* part = wL + GW * TE;                          // [LW][GW][D]
  float* red = part + LW * GW * D;                     // [LW][GW]

  const int tid = fq_tid(), lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int chunk = fq_bid_x(), b = fq_bid_z();
  const int G = Hq / Hkv, nsets = G / GW;
  const int g = fq_bid_y() / nsets, hs = fq_bid_y() % nsets;
  const int h0 = g * G + hs * GW;  // first query head of the set
  const int B = NB * bits;          // bits per record

  // ---- prologue: tables of the set's heads, W = 0
  {
    const float* src = lut + ((int64_t)b * Hq + h0) * TE;
    if ((TE & 3) == 0) {  // 16-byte aligned rows (the table region itself is 256-byte aligned)
      const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int i = tid; i < GW * TE / 4; i += LW * 64) {
        reinterpret_cast<float4*>(lutL)[i] = reinterpret_cast<const float4*>(src)[i];
        reinterpret_cast<float4*>(wL)[i] = z;
      }
    } else {
      for (int i = tid; i < GW * TE; i += LW * 64) {
        lutL[i] = src[i];
        wL[i] = 0.f;
      }
    }
  }
  const int64_t Tb = [&] {
    if (!lens) return T;
    const int64_t L = lens[b];
    return L < 0 ? (int64_t)0 : (L < T ? L : T);
  }();
  const int64_t c0 = (int64_t)chunk * Tc;
  const int64_t c1 = (c0 + Tc) < Tb ? (c0 + Tc) : Tb;
  const int64_t base = ((int64_t)b * Hkv + g) * T;
  const float NEG = -__builtin_huge_valf();
  __syncthreads();

  // A wave takes U consecutive 64-key runs per iteration, lane = key; the codes and
  // norms of all U keys are loaded before any is used.
  constexpr int U = K == D ? 4 : 1;
  constexpr int64_t STEP = (int64_t)LW * 64 * U;
  const int64_t tw = c0 + (int64_t)w * 64 * U + lane;
  auto load_keys = [&](const uint8_t* __restrict__ cs, const _Float16* __restrict__ ns, int64_t t0,
                       int (&code)[U][NB], float (&nu)[U]) {
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int64_t t = t0 + 64 * u;
      const bool ok = t < c1;
      const int64_t rec = (base + (ok ? t : c0)) * B;
#pragma unroll
      for (int blk = 0; blk < NB; blk++) code[u][blk] = (int)load_code(cs, rec + (int64_t)blk * bits, bits);
      nu[u] = (float)ns[base + (ok ? t : c0)];
    }
  };
  auto scores = [&](const int (&code)[NB], float nu, float* s) {
    float acc[GW];
#pragma unroll
    for (int h = 0; h < GW; h++) acc[h] = 0.f;
#pragma unroll
    for (int blk = 0; blk < NB; blk++)
#pragma unroll
      for (int h = 0; h < GW; h++) acc[h] += lutL[h * TE + blk * N + code[blk]];
#pragma unroll
    for (int h = 0; h < GW; h++) s[h] = nu * acc[h];
  };

  // ---- pass 1: exact maximum per head
  float mx[GW];
#pragma unroll
  for (int h = 0; h < GW; h++) mx[h] = NEG;
  for (int64_t t0 = tw; t0 < c1; t0 += STEP) {
    int kcode[U][NB];
    float knu[U];
    load_keys(kc, kn, t0, kcode, knu);
#pragma unroll
    for (int u = 0; u < U; u++) {
      if (t0 + 64 * u < c1) {
        float s[GW];
        scores(kcode[u], knu[u], s);
#pragma unroll
        for (int h = 0; h < GW; h++) mx[h] = fmaxf(mx[h], s[h]);
      }
    }
  }
#pragma unroll
  for (int h = 0; h < GW; h++) {
    const float m = wave_max(mx[h]);
    if (lane == 0) red[w * GW + h] = m;
  }
  __syncthreads();
  float M[GW];
#pragma unroll
  for (int h = 0; h < GW; h++) {
    M[h] = NEG;
#pragma unroll
    for (int ww = 0; ww < LW; ww++) M[h] = fmaxf(M[h], red[ww * GW + h]);
  }
  float* recs = ws + (((int64_t)b * Hq + h0) * nchunks + chunk) * REC;
  if (c0 >= c1) {  // no key in this chunk (uniform): empty records
    for (int i = tid; i < GW * REC; i += LW * 64) {
      const int h = i / REC, e = i % REC;
      recs[(int64_t)h * nchunks * REC + e] = e == 0 ? NEG : 0.f;
    }
    return;
  }
  __syncthreads();  // every wave has read `red` before it is reused below

  // ---- pass 2: weights into W
  float l[GW];
#pragma unroll
  for (int h = 0; h < GW; h++) l[h] = 0.f;
  for (int64_t t0 = tw; t0 < c1; t0 += STEP) {
    int kcode[U][NB], vcode[U][NB];
    float knu[U], vnu[U];
    load_keys(kc, kn, t0, kcode, knu);
    load_keys(vc, vn, t0, vcode, vnu);
#pragma unroll
    for (int u = 0; u < U; u++) {
      if (t0 + 64 * u < c1) {
        float s[GW];
        scores(kcode[u], knu[u], s);
        float pv[GW];
#pragma unroll
        for (int h = 0; h < GW; h++) {
          const float p = __builtin_amdgcn_exp2f(s[h] - M[h]);
          l[h] += p;
          pv[h] = p * vnu[u];
        }
#pragma unroll
        for (int blk = 0; blk < NB; blk++)
#pragma unroll
          for (int h = 0; h < GW; h++) atomicAdd(&wL[h * TE + blk * N + vcode[u][blk]], pv[h]);
      }
    }
  }
#pragma unroll
  for (int h = 0; h < GW; h++) {
    const float s = wave_sum(l[h]);
    if (lane == 0) red[w * GW + h] = s;
  }
  __syncthreads();

  // ---- epilogue: acc_h[d] = sum_n W[h][d / K][n] c_n[d % K]
  if constexpr (K == D) {
    // lane = (codeword n % 8, dims 8 seg .. 8 seg + 7): one 16-byte load per lane, a
    // wave covers 8 codewords per load, four loads in flight; the 8 lanes of a dim
    // segment are summed at the end
    const int seg = lane & 7, no = lane >> 3;
    float a[GW][8];
#pragma unroll
    for (int h = 0; h < GW; h++)
#pragma unroll
      for (int j = 0; j < 8; j++) a[h][j] = 0.f;
    constexpr int UE = 4;
    for (int nb = 8 * w; nb < N; nb += 8 * LW * UE) {
      uint4 cv[UE];
      float wv[UE][GW];
#pragma unroll
      for (int ue = 0; ue < UE; ue++) {
        const int n = nb + 8 * LW * ue + no;
        cv[ue] = n < N ? *reinterpret_cast<const uint4*>(cw16 + (int64_t)n * D + 8 * seg) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int h = 0; h < GW; h++) wv[ue][h] = n < N ? wL[h * TE + n] : 0.f;
      }
#pragma unroll
      for (int ue = 0; ue < UE; ue++) {
        const uint32_t cw4[4] = {cv[ue].x, cv[ue].y, cv[ue].z, cv[ue].w};
#pragma unroll
        for (int j = 0; j < 8; j++) {
          const float cj = (float)__builtin_bit_cast(_Float16, (uint16_t)(j & 1 ? cw4[j / 2] >> 16 : cw4[j / 2] & 0xffffu));
#pragma unroll
          for (int h = 0; h < GW; h++) a[h][j] = fmaf(wv[ue][h], cj, a[h][j]);
        }
      }
    }
#pragma unroll
    for (int h = 0; h < GW; h++)
#pragma unroll
      for (int j = 0; j < 8; j++) {
        float v = a[h][j];
        v += __shfl_xor(v, 8);
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        a[h][j] = v;
      }
    if (lane < 8) {
#pragma unroll
      for (int h = 0; h < GW; h++)
#pragma unroll
        for (int j = 0; j < 8; j++) part[(w * GW + h) * D + 8 * seg + j] = a[h][j];
    }
  } else {
    // lane = output dim; wave w takes n = w, w + LW, ...
    const int blk = lane / K, i = lane % K;
    float a[GW];
#pragma unroll
    for (int h = 0; h < GW; h++) a[h] = 0.f;
    for (int n = w; n < N; n += LW) {
      const float c = (float)cw16[(int64_t)n * K + i];
#pragma unroll
      for (int h = 0; h < GW; h++) a[h] = fmaf(wL[h * TE + blk * N + n], c, a[h]);
    }
#pragma unroll
    for (int h = 0; h < GW; h++) part[(w * GW + h) * D + lane] = a[h];
  }
  __syncthreads();
  for (int i = tid; i < GW * D; i += LW * 64) {
    const int h = i / D, d = i % D;
    float a = 0.f, ls = 0.f;
#pragma unroll
    for (int ww = 0; ww < LW; ww++) {
      a += part[(ww * GW + h) * D + d];
      ls += red[ww * GW + h];
    }
    float* rec = recs + (int64_t)h * nchunks * REC;
    if (d == 0) {
      float mh = NEG;
#pragma unroll
      for (int hh = 0; hh < GW; hh++)
        if (hh == h) mh = M[hh];
      rec[0] = mh;
      rec[1] = ls;
    }
    rec[2 + d] = a;
  }
}

// Largest head-set size (dividing the group) whose LDS fits the device.
// (At most 4 heads: more would spill registers of the 16-wave workgroup, and at
// k = 4, N = 256 the 16 tables per head leave no LDS for more.)
template <int K>
int lut_heads(const fq_codebook* cb, int G) {
  for (int gw : {4, 2, 1}) {
    if (G % gw) continue;
    size_t bytes = 0;
    switch (gw) {
      case 4: bytes = lut_lds_bytes<K, 4>(cb->N); break;
      case 2: bytes = lut_lds_bytes<K, 2>(cb->N); break;
      default: bytes = lut_lds_bytes<K, 1>(cb->N); break;
    }
    if (bytes <= cb->max_lds) return gw;
  }
  return 0;
}

template <int K, int GW>
hipError_t launch_gw(const fq_codebook* cb, const void* q, const uint8_t* k_codes, const void* k_norms,
                     const uint8_t* v_codes, const void* v_norms, const int32_t* lens, int B, int Hq, int Hkv,
                     int64_t T, float qscale, const AttnPlan& p, float* out, void* workspace, hipStream_t s) {
  float* ws = reinterpret_cast<float*>(workspace);
  float* lut = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + attn_workspace_bytes(B, Hq, Hkv, p.nchunks));
  const int G = Hq / Hkv;
  hipLaunchKernelGGL((attn_lut_prep<K>), dim3((unsigned)(B * Hkv), (unsigned)((cb->N + PT - 1) / PT)), dim3(PT), 0,
                     s, reinterpret_cast<const _Float16*>(q), cb->pi32, cb->cw16, cb->N, Hq, Hkv, qscale, lut);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = lut_lds_bytes<K, GW>(cb->N);
  if (lds > 65536) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(attn_lut<K, GW>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((attn_lut<K, GW>), dim3((unsigned)p.nchunks, (unsigned)(Hkv * (G / GW)), (unsigned)B),
                     dim3(LW * 64), lds, s, lut, k_codes, reinterpret_cast<const _Float16*>(k_norms), v_codes,
                     reinterpret_cast<const _Float16*>(v_norms), cb->cw16, cb->N, cb->bits, Hq, Hkv, T, lens,
                     p.chunk_tokens, p.nchunks, ws);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_attn_combine(ws, cb->pi32, (int64_t)B * Hq, p.nchunks, out, s);
}

template <int K>
hipError_t launch_k(const fq_codebook* cb, const void* q, const uint8_t* k_codes, const void* k_norms,
                    const uint8_t* v_codes, const void* v_norms, const int32_t* lens, int B, int Hq, int Hkv,
                    int64_t T, float qscale, const AttnPlan& p, float* out, void* workspace, hipStream_t s) {
  switch (p.lut_heads) {
#define FQ_GW(X)                                                                                                   \
  case X:                                                                                                          \
    return launch_gw<K, X>(cb, q, k_codes, k_norms, v_codes, v_norms, lens, B, Hq, Hkv, T, qscale, p, out, workspace, \
                           s);
    FQ_GW(1)
    FQ_GW(2)
    FQ_GW(4)
#undef FQ_GW
    default: break;
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool attn_lut_supported(const fq_codebook* cb) {
  if (cb->k == D) return lut_heads<64>(cb, 1) > 0;
  if (cb->k == 4 && cb->force_attn_lut) return lut_heads<4>(cb, 1) > 0;
  return false;
}

int attn_lut_heads(const fq_codebook* cb, int G) {
  if (cb->k == D) return lut_heads<64>(cb, G);
  if (cb->k == 4) return lut_heads<4>(cb, G);
  return 0;
}

size_t attn_lut_table_bytes(const fq_codebook* cb, int B, int Hq) {
  return (((size_t)B * Hq * (D / cb->k) * cb->N * sizeof(float)) + 255) & ~(size_t)255;
}

hipError_t launch_attn_lut(const fq_codebook* cb, const void* q, const uint8_t* k_codes, const void* k_norms,
                           const uint8_t* v_codes, const void* v_norms, const int32_t* lens, int B, int Hq, int Hkv,
                           int64_t T, float scale, const AttnPlan& p, float* out, void* workspace, hipStream_t s) {
  const float qscale = scale * 1.4426950408889634f;  // log2(e)
  if (cb->k == D)
    return launch_k<64>(cb, q, k_codes, k_norms, v_codes, v_norms, lens, B, Hq, Hkv, T, qscale, p, out, workspace, s);
  if (cb->k == 4)
    return launch_k<4>(cb, q, k_codes, k_norms, v_codes, v_norms, lens, B, Hq, Hkv, T, qscale, p, out, workspace, s);
  return hipErrorNotSupported;
}

}  // namespace fq
