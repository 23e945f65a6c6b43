// Multi-query (prefill) attention over a FibQuant-compressed cache (FibQuant
// summary §5: fixed-address codes let decompression be fused into attention;
// §2.3: k_j = nu_j Pi^T concat(c_j), so q . k_j = nu_j (Pi q) . concat(c_j)).
//
// Sq queries per query head attend to the T keys of their KV head's slab; with
// the causal flag the queries are the slab's last Sq positions, so query i sees
// keys 0 .. T - Sq + i.  Many query rows share every key, so the products run on
// the matrix core (mfma_f32_16x16x32_f16) over codeword tiles decoded into LDS:
//   * a workgroup takes 64 query rows of one (batch, KV head) slab (row r = head
//     r / Sq of the group, query r % Sq) and a range of its keys; each of its 4
//     waves owns 16 rows (the MFMA columns);
//   * per 64-key unit the threads decode the keys' records into LDS: K as
//     [key][dim] fp16 (the A operand of S^T = K Qrot^T), V transposed as
//     [dim][key] (the A operand of O^T += V^T P^T), norms as fp32.  For k = 4
//     with 8-bit codes every thread takes one quarter record, loaded a unit ahead
//     into registers; for other codebooks a thread takes pieces of min(k, 16)
//     dimensions of a key (the code read at its fixed bit address), copied from
//     an LDS copy of the codebook when that is at most 32 KiB, else from the
//     fp16 codebook in global memory (L2-resident: 512 KiB for k = d, N = 4096);
//   * the rotated, scaled query is split fp16 hi + lo (two products per K step:
//     scores carry ~22 bits); P' = p * nu_v enters as one fp16 operand (relative
//     rounding 2^-12 of each weight);
//   * the key order inside a 32-key PV step is chosen so that the score
//     registers of a lane are exactly its P^T operand (no shuffles): operand k
//     index 8 h + j is key 4 h + j (j < 4) or 16 + 4 h + j - 4 of the step;
//   * online softmax in base 2 per query column; the workgroup writes one
//     partial record (m, l, acc[64], rotated domain) per row and key range, and
//     the decode combine kernel merges the records and applies Pi^T.
#include "fq_internal.h"
#include "fq_device.h"

namespace fq {
namespace {

constexpr int D = kD;
constexpr int PW = 4;       // waves per workgroup
constexpr int PU = 64;      // keys per unit
constexpr int PROWS = 16 * PW;  // query rows per workgroup
constexpr int REC_F = 2 + D;
// LDS row strides (halves): 128-byte rows would put the 16 rows one MFMA operand read
// touches on the same banks; 144- and 136-byte rows spread them over all 64 banks
constexpr int KS = D + 8;   // K tile [key][KS]
constexpr int VS = PU + 4;  // V tile [dim][VS]
constexpr int QSCR = 17;    // floats per lane of the query rotation's scratch (odd: no bank conflicts)
// How a workgroup gets codewords: the k = 4, 8-bit path (registers a unit ahead, LDS
// codebook), or pieces read from an LDS copy of the codebook, or from global memory.
enum CbMode { CB_K4B8 = 0, CB_LDS = 1, CB_GLOBAL = 2 };
constexpr size_t CB_LDS_MAX = 32768;  // bytes of fp16 codebook held in LDS
// the query rotation's scratch shares the LDS of the K and V tiles (used before them)
constexpr int TILE_BYTES = (PU * KS + D * VS) * 2;
static_assert(PW * 64 * QSCR * 4 <= TILE_BYTES, "query scratch must fit the tile space");

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ inline f32x4 mfma16(half8 a, half8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Per-thread registers of one unit's records: threads 0..127 decode K, 128..255 V;
// thread t of a half takes keys 2 (t / 4) and 2 (t / 4) + 1, record dword t % 4 of each,
// and (threads < 64) the two norms of key `tid`.
struct UnitRegs {
  uint32_t w0, w1;
  _Float16 kn, vn;
};

// Copy one piece of KW fp16 codeword coordinates (KW-aligned) from src into registers.
template <int KW>
__device__ inline void load_piece(const _Float16* src, _Float16 (&v)[KW]) {
  if constexpr (KW >= 8) {
#pragma unroll
    for (int c = 0; c < KW / 8; c++) {
      const half8 h = *reinterpret_cast<const half8*>(src + 8 * c);
#pragma unroll
      for (int j = 0; j < 8; j++) v[8 * c + j] = h[j];
    }
  } else if constexpr (KW == 4) {
    const half4 h = *reinterpret_cast<const half4*>(src);
#pragma unroll
    for (int j = 0; j < 4; j++) v[j] = h[j];
  } else if constexpr (KW == 2) {
    const half2_t h = *reinterpret_cast<const half2_t*>(src);
    v[0] = h[0];
    v[1] = h[1];
  } else {
    v[0] = src[0];
  }
}

// Store a piece to KW consecutive fp16 slots (KW-aligned, 16-byte aligned for KW >= 8).
template <int KW>
__device__ inline void store_piece(_Float16* dst, const _Float16 (&v)[KW]) {
  if constexpr (KW >= 8) {
#pragma unroll
    for (int c = 0; c < KW / 8; c++) {
      half8 h;
#pragma unroll
      for (int j = 0; j < 8; j++) h[j] = v[8 * c + j];
      *reinterpret_cast<half8*>(dst + 8 * c) = h;
    }
  } else if constexpr (KW == 4) {
    *reinterpret_cast<half4*>(dst) = half4{v[0], v[1], v[2], v[3]};
  } else if constexpr (KW == 2) {
    *reinterpret_cast<half2_t*>(dst) = half2_t{v[0], v[1]};
  } else {
    dst[0] = v[0];
  }
}

// KW = min(k, 16) dimensions per decode piece (CB_K4B8: 4); CM: a CbMode.
template <int KW, int CM>
__global__ __launch_bounds__(PW * 64, 4) void attn_prefill(
    const _Float16* __restrict__ q, float qscale, const float* __restrict__ pi32, const uint8_t* __restrict__ kc,
    const _Float16* __restrict__ kn, const uint8_t* __restrict__ vc, const _Float16* __restrict__ vn,
    const _Float16* __restrict__ cw16, int k, int bits, int N, int Hq, int Hkv, int64_t T, int Sq, int causal,
    int64_t chunk_tokens, int nchunks, float* __restrict__ ws) {
  extern __shared__ __align__(16) _Float16 cbL[];  // the codebook [N][k] (CB_K4B8, CB_LDS)
  __shared__ __align__(16) unsigned char tiles[TILE_BYTES];
  _Float16* const Kt = reinterpret_cast<_Float16*>(tiles);  // [key][KS]
  _Float16* const Vt = Kt + PU * KS;                        // [dim][VS]
  float* const qscr = reinterpret_cast<float*>(tiles);      // per-lane scratch of the query rotation
  __shared__ float knL[PU], vnL[PU];
  const int tid = fq_tid(), lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int chunk = fq_bid_x(), rb = fq_bid_y(), slab = fq_bid_z();
  const int b = slab / Hkv, g = slab - b * Hkv;
  const int G = Hq / Hkv, rows = G * Sq;
  const int64_t slab0 = (int64_t)slab * T;
  const int col = lane & 15, hq = lane >> 4;
  // this lane's query row (an MFMA column)
  const int r = rb * PROWS + 16 * w + col;
  const bool row_ok = r < rows;
  const int hl = row_ok ? r / Sq : 0, qi = row_ok ? r - hl * Sq : 0;
  const int64_t lim = causal ? T - Sq + qi : T - 1;  // last key this row sees
  // key range of the workgroup (causal: no row of the block sees past its last row's limit)
  const int64_t t_begin = (int64_t)chunk * chunk_tokens;
  int64_t t_end = t_begin + chunk_tokens < T ? t_begin + chunk_tokens : T;
  if (causal) {
    const int rlast = rb * PROWS + PROWS - 1 < rows - 1 ? rb * PROWS + PROWS - 1 : rows - 1;
    // the largest query index among the block's rows
    int imax = 0;
    for (int rr = rb * PROWS; rr <= rlast && imax < Sq - 1; rr++) {
      const int ii = rr % Sq;
      imax = ii > imax ? ii : imax;
    }
    const int64_t kmax = T - Sq + imax + 1;
    t_end = t_end < kmax ? t_end : kmax;
  }

  // codebook
  if constexpr (CM != CB_GLOBAL) {
    const int nh = N * k;  // a power of two
    if (nh % 8 == 0) {
      for (int e = tid; e < nh / 8; e += PW * 64)
        reinterpret_cast<uint4*>(cbL)[e] = reinterpret_cast<const uint4*>(cw16)[e];
    } else {
      for (int e = tid; e < nh; e += PW * 64) cbL[e] = cw16[e];
    }
  }

  // B operands of QK: column col = query row r, k = 8 hq + j is dimension 32 s + 8 hq + j
  // of the rotated query (Pi q) * scale * log2(e), split fp16 hi + lo
  half8 qhi[2], qlo[2];
  {
    float qv[D];
    // hl = qi = 0 for a row past the block's end: the address stays inside q
    const uint4* qr = reinterpret_cast<const uint4*>(q + ((((int64_t)b * Hq + (int64_t)g * G + hl) * Sq) + qi) * D);
#pragma unroll
    for (int e8 = 0; e8 < D / 8; e8++) {
      const half8 h8 = __builtin_bit_cast(half8, qr[e8]);
#pragma unroll
      for (int j = 0; j < 8; j++) qv[8 * e8 + j] = row_ok ? (float)h8[j] : 0.0f;
    }
    // one rotated dimension per iteration (not unrolled: all 16 rows of Pi at once
    // would not fit in registers); each lane parks its 16 values in its own LDS slots
#pragma unroll 1
    for (int jj = 0; jj < 16; jj++) {
      const int d = 32 * (jj >> 3) + 8 * hq + (jj & 7);
      float a = 0.0f;
#pragma unroll
      for (int e = 0; e < D; e++) a = __builtin_fmaf(pi32[d * D + e], qv[e], a);
      qscr[tid * QSCR + jj] = a * qscale;
    }
#pragma unroll
    for (int s = 0; s < 2; s++)
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const float a = qscr[tid * QSCR + 8 * s + j];
        const _Float16 h = (_Float16)a;
        qhi[s][j] = h;
        qlo[s][j] = (_Float16)(a - (float)h);
      }
  }

  const float NEG = -__builtin_huge_valf();
  float m_run = NEG, l_run = 0.0f;
  f32x4 O[4];
#pragma unroll
  for (int dt = 0; dt < 4; dt++) O[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // unit loads (registers), one unit ahead
  const bool vhalf = tid >= 128;  // wave-uniform: waves 2, 3 decode V
  const int kp = (tid & 127) >> 2, lp = tid & 3;
  const uint8_t* __restrict__ store = vhalf ? vc : kc;
  auto load_unit = [&](int64_t t0, UnitRegs& u) {
    const int64_t nt = t_end - t0;
    const int64_t key0 = slab0 + t0 + (2 * kp < nt ? 2 * kp : nt - 1);
    const int64_t key1 = slab0 + t0 + (2 * kp + 1 < nt ? 2 * kp + 1 : nt - 1);
    u.w0 = reinterpret_cast<const uint32_t*>(store + key0 * 16)[lp];
    u.w1 = reinterpret_cast<const uint32_t*>(store + key1 * 16)[lp];
    if (tid < PU) {
      const int64_t kk = slab0 + t0 + (tid < nt ? tid : nt - 1);
      u.kn = kn[kk];
      u.vn = vn[kk];
    }
  };
  UnitRegs cur{}, nxt{};
  if (CM == CB_K4B8 && t_begin < t_end) load_unit(t_begin, cur);
  __syncthreads();  // codebook in place

  const int lk = __builtin_ctz((unsigned)k);
  const int64_t vbits = (int64_t)(D / k) * bits;  // bits of one vector's record
  for (int64_t t0 = t_begin; t0 < t_end; t0 += PU) {
    // ---- decode the unit into LDS
    __syncthreads();  // the previous unit's tiles (or the query scratch) are no longer read
    if constexpr (CM != CB_K4B8) {
      // item it: piece p = it % P of key (it / P) % PU, of V when it >= PU P (wave-uniform)
      constexpr int P = D / KW;
      const int64_t nt = t_end - t0;
#pragma unroll 2
      for (int it = tid; it < 2 * PU * P; it += PW * 64) {
        const int p = it % P, key = (it / P) % PU;
        const bool isv = it >= PU * P;
        const int dim0 = p * KW, blk = dim0 >> lk, off = dim0 & (k - 1);
        const int64_t kk = slab0 + t0 + (key < nt ? key : nt - 1);
        const uint32_t code = load_code(isv ? vc : kc, kk * vbits + (int64_t)blk * bits, bits);
        const _Float16* src = (CM == CB_LDS ? cbL : cw16) + (size_t)code * k + off;
        _Float16 v[KW];
        load_piece<KW>(src, v);
        if (isv) {
#pragma unroll
          for (int e = 0; e < KW; e++) Vt[(dim0 + e) * VS + key] = v[e];
        } else {
          store_piece<KW>(Kt + key * KS + dim0, v);
        }
      }
      if (tid < PU) {
        const int64_t kk = slab0 + t0 + (tid < nt ? tid : nt - 1);
        knL[tid] = (float)kn[kk];
        vnL[tid] = (float)vn[kk];
      }
    } else {
      const uint32_t w0 = cur.w0, w1 = cur.w1;
#pragma unroll
      for (int c = 0; c < 4; c++) {
        const half4 c0 = *reinterpret_cast<const half4*>(cbL + ((w0 >> (8 * c)) & 0xffu) * 4);
        const half4 c1 = *reinterpret_cast<const half4*>(cbL + ((w1 >> (8 * c)) & 0xffu) * 4);
        const int d0 = 16 * lp + 4 * c;  // block 4 lp + c covers dims d0 .. d0 + 3
        if (vhalf) {
          // the two keys' values of one dimension are neighbours in the transposed tile
#pragma unroll
          for (int e = 0; e < 4; e++) {
            const half2_t pair = {c0[e], c1[e]};
            *reinterpret_cast<half2_t*>(Vt + (d0 + e) * VS + 2 * kp) = pair;
          }
        } else {
          *reinterpret_cast<half4*>(Kt + (2 * kp) * KS + d0) = c0;
          *reinterpret_cast<half4*>(Kt + (2 * kp + 1) * KS + d0) = c1;
        }
      }
      if (tid < PU) {
        knL[tid] = (float)cur.kn;
        vnL[tid] = (float)cur.vn;
      }
    }
    if (CM == CB_K4B8 && t0 + PU < t_end) load_unit(t0 + PU, nxt);
    __syncthreads();

    // keys of this unit the lane's row may see: kk <= bound (32-bit; -1 = none)
    const int64_t nt = t_end - t0;
    const bool need_mask = nt < PU || (causal && t0 + PU - 1 > T - Sq) || !row_ok;
    int bound = PU - 1;
    if (need_mask) {
      const int64_t bl = lim - t0, bn = nt - 1;
      int64_t bb = bl < bn ? bl : bn;
      bb = bb < -1 ? -1 : (bb > PU - 1 ? PU - 1 : bb);
      bound = row_ok ? (int)bb : -1;
    }
    // ---- S^T = K Qrot^T: tile a covers keys 16 a .. 16 a + 15; the lane holds keys
    // 16 a + 4 hq + i of query column col
    float sc[4][4];
#pragma unroll
    for (int a = 0; a < 4; a++) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 2; s++) {
        const half8 A = *reinterpret_cast<const half8*>(Kt + (16 * a + col) * KS + 32 * s + 8 * hq);
        acc = mfma16(A, qhi[s], acc);
        acc = mfma16(A, qlo[s], acc);
      }
#pragma unroll
      for (int i = 0; i < 4; i++) sc[a][i] = acc[i] * knL[16 * a + 4 * hq + i];
    }
    if (need_mask) {  // uniform: the last units of a range, the causal diagonal, short blocks
#pragma unroll
      for (int a = 0; a < 4; a++)
#pragma unroll
        for (int i = 0; i < 4; i++) sc[a][i] = 16 * a + 4 * hq + i <= bound ? sc[a][i] : NEG;
    }
    float mx = NEG;
#pragma unroll
    for (int a = 0; a < 4; a++)
#pragma unroll
      for (int i = 0; i < 4; i++) mx = fmaxf(mx, sc[a][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == NEG ? 0.0f : m_new;  // a column with no key yet: nothing to scale
    if (__ballot(m_new > m_run)) {  // some column's max moved (rare after the first units)
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; dt++) O[dt] *= alpha;
    }
    m_run = m_new;
    // ---- O^T += V^T P'^T over two 32-key steps
#pragma unroll
    for (int st = 0; st < 2; st++) {
      half8 P;
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const int a = 2 * st + (j >> 2), i = j & 3;
        const float p = __builtin_amdgcn_exp2f(sc[a][i] - m_use);
        l_run += p;
        P[j] = (_Float16)(p * vnL[16 * a + 4 * hq + i]);
      }
#pragma unroll
      for (int dt = 0; dt < 4; dt++) {
        const _Float16* vrow = Vt + (16 * dt + col) * VS + 32 * st + 4 * hq;
        const half4 lo4 = *reinterpret_cast<const half4*>(vrow);
        const half4 hi4 = *reinterpret_cast<const half4*>(vrow + 16);
        const half8 A = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        O[dt] = mfma16(A, P, O[dt]);
      }
    }
    cur = nxt;
  }

  // ---- this row's partial record: O^T rows 16 dt + 4 hq + i of column col
  float l = l_run;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  // the row's indices again, from the lane index the shuffles use (mbcnt): carried
  // across the loop from the prologue (where the query load forms the same offset)
  // they were spilled
  const int ln = __lane_id();
  const int ecol = ln & 15, ehq = ln >> 4;
  const int er = rb * PROWS + 16 * w + ecol;
  if (er >= rows) return;
  const int ehl = er / Sq, eqi = er - ehl * Sq;
  const int64_t bh = ((int64_t)b * Hq + (int64_t)g * G + ehl) * Sq + eqi;
  float* rec = ws + (bh * nchunks + chunk) * REC_F;
  if (ehq == 0) {
    rec[0] = m_run;
    rec[1] = l;
  }
#pragma unroll
  for (int dt = 0; dt < 4; dt++)
#pragma unroll
    for (int i = 0; i < 4; i++) rec[2 + 16 * dt + 4 * ehq + i] = O[dt][i];
}

}  // namespace

PrefillPlan prefill_plan(int B, int Hq, int Hkv, int Sq, int64_t T) {
  const int rows = (Hq / Hkv) * Sq;
  const int rblocks = (rows + PROWS - 1) / PROWS;
  const int64_t wgs = (int64_t)rblocks * B * Hkv;
  int64_t nc = (1024 + wgs - 1) / wgs;
  const int64_t most = (T + 511) / 512;
  if (nc > most) nc = most;
  if (nc < 1) nc = 1;
  int64_t ct = (T + nc - 1) / nc;
  ct = (ct + PU - 1) / PU * PU;
  nc = (T + ct - 1) / ct;
  return PrefillPlan{(int)nc, ct, rblocks};
}

bool prefill_supported(const fq_codebook* cb) { return cb->k >= 1 && cb->k <= D && D % cb->k == 0; }

namespace {
CbMode prefill_cb_mode(const fq_codebook* cb) {
  if (cb->k == 4 && cb->bits == 8) return CB_K4B8;
  return (size_t)cb->N * cb->k * 2 <= CB_LDS_MAX ? CB_LDS : CB_GLOBAL;
}

struct PrefillArgs {
  const _Float16* q;
  float qscale;
  const uint8_t *kc, *vc;
  const _Float16 *kn, *vn;
  int Hq, Hkv, Sq, causal;
  int64_t T;
  PrefillPlan p;
  dim3 grid;
  float* ws;
};

template <int KW, int CM>
hipError_t launch_variant(const fq_codebook* cb, const PrefillArgs& a, hipStream_t s) {
  const size_t lds = CM == CB_GLOBAL ? 0 : (size_t)cb->N * cb->k * sizeof(_Float16);
  hipLaunchKernelGGL((attn_prefill<KW, CM>), a.grid, dim3(PW * 64), lds, s, a.q, a.qscale, cb->pi32, a.kc, a.kn,
                     a.vc, a.vn, cb->cw16, cb->k, cb->bits, cb->N, a.Hq, a.Hkv, a.T, a.Sq, a.causal,
                     a.p.chunk_tokens, a.p.nchunks, a.ws);
  return hipGetLastError();
}

template <int KW>
hipError_t launch_generic(const fq_codebook* cb, CbMode m, const PrefillArgs& a, hipStream_t s) {
  return m == CB_LDS ? launch_variant<KW, CB_LDS>(cb, a, s) : launch_variant<KW, CB_GLOBAL>(cb, a, s);
}
}  // namespace

hipError_t launch_prefill(const fq_codebook* cb, const void* q, const uint8_t* k_codes, const void* k_norms,
                          const uint8_t* v_codes, const void* v_norms, int B, int Hq, int Hkv, int Sq, int64_t T,
                          int causal, float scale, float* out, void* workspace, hipStream_t s) {
  const PrefillPlan p = prefill_plan(B, Hq, Hkv, Sq, T);
  PrefillArgs a;
  a.q = reinterpret_cast<const _Float16*>(q);
  a.qscale = scale * 1.4426950408889634f;  // log2(e)
  a.kc = k_codes;
  a.vc = v_codes;
  a.kn = reinterpret_cast<const _Float16*>(k_norms);
  a.vn = reinterpret_cast<const _Float16*>(v_norms);
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Sq = Sq;
  a.causal = causal;
  a.T = T;
  a.p = p;
  a.grid = dim3((unsigned)p.nchunks, (unsigned)p.rblocks, (unsigned)(B * Hkv));
  a.ws = reinterpret_cast<float*>(workspace);
  const CbMode m = prefill_cb_mode(cb);
  hipError_t e;
  if (m == CB_K4B8) {
    e = launch_variant<4, CB_K4B8>(cb, a, s);
  } else {
    switch (cb->k < 16 ? cb->k : 16) {
      case 1: e = launch_generic<1>(cb, m, a, s); break;
      case 2: e = launch_generic<2>(cb, m, a, s); break;
      case 4: e = launch_generic<4>(cb, m, a, s); break;
      case 8: e = launch_generic<8>(cb, m, a, s); break;
      default: e = launch_generic<16>(cb, m, a, s); break;
    }
  }
  if (e != hipSuccess) return e;
  return launch_attn_combine(reinterpret_cast<const float*>(workspace), cb->pi32, (int64_t)B * Hq * Sq, p.nchunks,
                             out, s);
}

}  // namespace fq
