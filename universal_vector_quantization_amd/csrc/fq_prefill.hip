// Multi-query (prefill) attention over a FibQuant-compressed cache (FibQuant
// summary §5: fixed-address codes let decompression be fused into attention;
// §2.3: k_j = nu_j Pi^T concat(c_j), so q . k_j = nu_j (Pi q) . concat(c_j)).
//
// Sq queries per query head attend to the T keys of their KV head's slab; with
// the causal flag the queries are the slab's last Sq positions, so query i sees
// keys 0 .. T - Sq + i.  Many query rows share every key, so the products run on
// the matrix core over codeword tiles decoded into LDS:
//   * a workgroup takes a block of query rows of one (batch, KV head) slab (row r =
//     head r / Sq of the group, query r % Sq) and a range of its keys; each of its 4
//     waves owns the MFMA columns of 32 rows (k = 4 with 8-bit codes, the wide kernel,
//     mfma_f32_32x32x16_f16) or 16 rows (every other codebook, mfma_f32_16x16x32_f16);
//   * per 64-key unit the threads decode the keys' records into LDS: K as
//     [key][dim] fp16 (the A operand of S^T = K Qrot^T), V transposed as
//     [dim][key] (the A operand of O^T += V^T P^T), norms as fp32.  For k = 4
//     with 8-bit codes every thread takes one quarter record, loaded a unit ahead
//     into registers; for other codebooks a thread takes pieces of min(k, 16)
//     dimensions of a key (the code read at its fixed bit address), copied from
//     an LDS copy of the codebook when that is at most 32 KiB, else from the
//     fp16 codebook in global memory (L2-resident: 512 KiB for k = d, N = 4096).
//     Units are double-buffered: unit h + 1 is decoded before unit h is computed,
//     one barrier per unit;
//   * the rotated, scaled query is split fp16 hi + lo (two products per K step:
//     scores carry ~22 bits); P' = p * nu_v enters as one fp16 operand (relative
//     rounding 2^-12 of each weight);
//   * the key order inside a PV step is chosen so that the score registers of a
//     lane are exactly its P^T operand (no shuffles);
//   * online softmax in base 2 per query row; the workgroup writes one partial
//     record (m, l, acc[64], rotated domain) per row and key range, and the decode
//     combine kernel merges the records and applies Pi^T.
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
// How a workgroup gets codewords: the k = 4, 8-bit path (the wide kernel: registers a
// unit ahead, LDS codebook), or pieces read from an LDS copy of the codebook, or from
// global memory.
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

// General kernel (every codebook but k = 4 with 8-bit codes): KW = min(k, 16) dimensions
// per decode piece; CM: CB_LDS or CB_GLOBAL.
template <int KW, int CM>
__global__ __launch_bounds__(PW * 64, 4) void attn_prefill(
    const _Float16* __restrict__ q, float qscale, const float* __restrict__ pi32, const uint8_t* __restrict__ kc,
    const _Float16* __restrict__ kn, const uint8_t* __restrict__ vc, const _Float16* __restrict__ vn,
    const _Float16* __restrict__ cw16, int k, int bits, int N, int Hq, int Hkv, int64_t T, int Sq, int causal,
    int64_t chunk_tokens, int nchunks, float* __restrict__ ws) {
  extern __shared__ __align__(16) _Float16 cbL[];  // the codebook [N][k] (CB_LDS)
  // two unit buffers, each K [key][KS] then V [dim][VS]; the query rotation's per-lane
  // scratch uses buffer 1 before any unit reaches it
  __shared__ __align__(16) unsigned char tiles[2][TILE_BYTES];
  float* const qscr = reinterpret_cast<float*>(tiles[1]);
  __shared__ float knL[2][PU], vnL[2][PU];
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

  const int lk = __builtin_ctz((unsigned)k);
  const int64_t vbits = (int64_t)(D / k) * bits;  // bits of one vector's record
  // decode the unit at t0 into buffer bf: K as [key][dim], V transposed, norms as fp32
  auto decode_unit = [&](int64_t t0, int bf) {
    _Float16* const Kt = reinterpret_cast<_Float16*>(tiles[bf]);
    _Float16* const Vt = Kt + PU * KS;
    {
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
        knL[bf][tid] = (float)kn[kk];
        vnL[bf][tid] = (float)vn[kk];
      }
    }
  };

  // Units are double-buffered: unit h + 1 is decoded into the other buffer before unit h
  // is computed, so one barrier per unit both publishes the next unit and retires the
  // buffer the one after it overwrites; different waves overlap decoding and matrix work.
  if (t_begin < t_end) {
    __syncthreads();  // codebook in place; every lane is done with its query scratch
    decode_unit(t_begin, 0);
    __syncthreads();  // unit 0 in buffer 0
  }
  int bf = 0;
  for (int64_t t0 = t_begin; t0 < t_end; t0 += PU, bf ^= 1) {
    if (t0 + PU < t_end) decode_unit(t0 + PU, bf ^ 1);
    const _Float16* const Kt = reinterpret_cast<const _Float16*>(tiles[bf]);
    const _Float16* const Vt = Kt + PU * KS;
    const float* const knU = knL[bf];
    const float* const vnU = vnL[bf];

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
      for (int i = 0; i < 4; i++) sc[a][i] = acc[i] * knU[16 * a + 4 * hq + i];
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
        P[j] = (_Float16)(p * vnU[16 * a + 4 * hq + i]);
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
    __syncthreads();  // unit h + 1 is in its buffer; this unit's buffer is free again
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


// Wide variant for k = 4 with 8-bit codes (the prefill workload's codebook): a wave owns
// 32 query rows and works with mfma_f32_32x32x16_f16, so every K or V operand it reads
// from LDS feeds 32 queries instead of 16.  The first version (16 rows a wave) spent most
// of its time in LDS (four waves each reading the whole unit's K and V tiles; 82 % of the
// cycles LDS-active, half of that bank conflicts), not on the matrix core.
//   * QK: A = K tile rows (keys 32 kt + 0..31) x 16 dimensions per K-step, B = the
//     rotated query, fp16 hi and lo (lane col + 32 h holds dimensions 16 s + 8 h + 0..7
//     of query row col); output rows (keys) 8 i + 4 h + j of query col in acc[4 i + j].
//   * PV over 16-key steps: operand k index 8 h + 4 a + j is key 16 ks + 8 a + 4 h + j,
//     so a lane's P' operand is 8 of its own scores and the V^T operand is two 8-byte
//     reads per lane; O^T tile dtt holds dimensions 32 dtt + 8 i + 4 h + j of query col.
constexpr int WROWS = 32 * PW;  // query rows per workgroup

typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ inline f32x16 mfma32(half8 a, half8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Value of lane l ^ 32 (the other half of the wave), by one permute from the lane index
// (no width handling, which kept a per-lane bound alive across the loop).
__device__ inline float xor32(float v) {
  const int src = (int)(__lane_id() ^ 32u) << 2;
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, v)));
}

__global__ __launch_bounds__(PW * 64, 3) void attn_prefill_w(
    const _Float16* __restrict__ q, float qscale, const half8* __restrict__ rotp, const uint8_t* __restrict__ kc,
    const _Float16* __restrict__ kn, const uint8_t* __restrict__ vc, const _Float16* __restrict__ vn,
    const _Float16* __restrict__ cw16, int Hq, int Hkv, int64_t T, int Sq, int causal, int64_t chunk_tokens,
    int nchunks, float* __restrict__ ws) {
  __shared__ __align__(16) _Float16 cbL[256 * 4];
  __shared__ __align__(16) unsigned char tiles[2][TILE_BYTES];
  __shared__ float knL[2][PU], vnL[2][PU];
  const int tid = fq_tid(), lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int chunk = fq_bid_x(), rb = fq_bid_y(), slab = fq_bid_z();
  const int b = slab / Hkv, g = slab - b * Hkv;
  const int G = Hq / Hkv, rows = G * Sq;
  const int64_t slab0 = (int64_t)slab * T;
  const int col = lane & 31, h = lane >> 5;
  const int r = rb * WROWS + 32 * w + col;  // this lane's query row (an MFMA column)
  const bool row_ok = r < rows;
  const int hl = row_ok ? r / Sq : 0, qi = row_ok ? r - hl * Sq : 0;
  const int64_t lim = causal ? T - Sq + qi : T - 1;  // last key this row sees
  const int64_t t_begin = (int64_t)chunk * chunk_tokens;
  int64_t t_end = t_begin + chunk_tokens < T ? t_begin + chunk_tokens : T;
  if (causal) {
    const int rlast = rb * WROWS + WROWS - 1 < rows - 1 ? rb * WROWS + WROWS - 1 : rows - 1;
    int imax = 0;  // the largest query index among the block's rows
    for (int rr = rb * WROWS; rr <= rlast && imax < Sq - 1; rr++) {
      const int ii = rr % Sq;
      imax = ii > imax ? ii : imax;
    }
    const int64_t kmax = T - Sq + imax + 1;
    t_end = t_end < kmax ? t_end : kmax;
  }
  if (tid < 128) reinterpret_cast<uint4*>(cbL)[tid] = reinterpret_cast<const uint4*>(cw16)[tid];

  // B operands of QK: dimensions 16 s + 8 h + j of the rotated query (Pi q) * scale *
  // log2(e) of row r, split fp16 hi + lo.  The rotation runs on the matrix core: A = 1024 Pi
  // as fp16 hi + mid with rows permuted so that output row 8 i + 4 h + j of tile t is
  // dimension 16 (2 t + i / 2) + 8 h + 4 (i % 2) + j, i.e. exactly the lane's own operand
  // coordinates; B = the raw fp16 query (exact products, fp32 sums).
  half8 qhi[4], qlo[4];
  {
    half8 qb[4];
    const half8* qr = reinterpret_cast<const half8*>(q + ((((int64_t)b * Hq + (int64_t)g * G + hl) * Sq) + qi) * D);
#pragma unroll
    for (int s = 0; s < 4; s++) qb[s] = row_ok ? qr[2 * s + h] : half8{};
    f32x16 ah[2], am[2];
#pragma unroll
    for (int t = 0; t < 2; t++)
#pragma unroll
      for (int e = 0; e < 16; e++) ah[t][e] = am[t][e] = 0.f;
#pragma unroll
    for (int t = 0; t < 2; t++)
#pragma unroll
      for (int s = 0; s < 4; s++) {
        ah[t] = mfma32(rotp[((t * 4 + s) * 2 + 0) * 64 + lane], qb[s], ah[t]);
        am[t] = mfma32(rotp[((t * 4 + s) * 2 + 1) * 64 + lane], qb[s], am[t]);
      }
    const float sc = qscale * (1.0f / 1024.0f);
#pragma unroll
    for (int t = 0; t < 2; t++)
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const float a = (ah[t][4 * i + j] + am[t][4 * i + j]) * sc;
          const _Float16 hv = (_Float16)a;
          qhi[2 * t + i / 2][4 * (i % 2) + j] = hv;
          qlo[2 * t + i / 2][4 * (i % 2) + j] = (_Float16)(a - (float)hv);
        }
  }

  // Softmax offset per row, lazily: scores are kept relative to m_run (the subtraction
  // rides in the norm product's FMA); m_run moves only when a score exceeds it, to TAU above
  // the row's maximum, so weights 2^L stay <= 1 (the fp16 P' cannot overflow) and the
  // rescale is rare after the first units.  `have`: the row has seen a key (until then
  // m_run is 0 and its first finite maximum sets it).
  const float NEG = -__builtin_huge_valf();
  constexpr float TAU = 4.0f;
  float m_run = 0.0f, l_run = 0.0f;
  bool have = false;
  f32x16 O[2];
#pragma unroll
  for (int e = 0; e < 16; e++) O[0][e] = O[1][e] = 0.f;

  // unit records in registers, a unit ahead: threads 0..127 decode K, 128..255 V; thread t
  // of a half takes keys 2 (t / 4) and 2 (t / 4) + 1, record dword t % 4 of each
  const bool vhalf = tid >= 128;
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
  // the four blocks of a record dword are taken in a lane-rotated order, so the lanes of
  // one write instruction spread over all LDS banks (in order, the K writes of a wave hit
  // 16 of the 64 banks and the V writes paired up)
  const int rot = vhalf ? 2 * (lp >> 1) : lp;
  auto decode_unit = [&](int bf, const UnitRegs& u) {
    _Float16* const Kt = reinterpret_cast<_Float16*>(tiles[bf]);
    _Float16* const Vt = Kt + PU * KS;
#pragma unroll
    for (int cr = 0; cr < 4; cr++) {
      const int c = (cr + rot) & 3;
      const half4 c0 = *reinterpret_cast<const half4*>(cbL + __builtin_amdgcn_ubfe(u.w0, 8 * c, 8) * 4);
      const half4 c1 = *reinterpret_cast<const half4*>(cbL + __builtin_amdgcn_ubfe(u.w1, 8 * c, 8) * 4);
      const int d0 = 16 * lp + 4 * c;  // block 4 lp + c covers dims d0 .. d0 + 3
      if (vhalf) {
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
      int t = tid;  // opaque: the norm slots' address is formed per unit, not carried (spilled)
      __asm__ volatile("" : "+v"(t));
      knL[bf][t] = (float)u.kn;
      vnL[bf][t] = (float)u.vn;
    }
  };

  UnitRegs cur{}, nxt{};
  if (t_begin < t_end) {
    load_unit(t_begin, cur);
    __syncthreads();  // codebook in place
    decode_unit(0, cur);
    if (t_begin + PU < t_end) load_unit(t_begin + PU, nxt);
    __syncthreads();  // unit 0 in buffer 0
  }
  int bf = 0;
  for (int64_t t0 = t_begin; t0 < t_end; t0 += PU, bf ^= 1) {
    if (t0 + PU < t_end) {  // the next unit into the other buffer (retired by the last barrier)
      cur = nxt;
      decode_unit(bf ^ 1, cur);
      if (t0 + 2 * PU < t_end) load_unit(t0 + 2 * PU, nxt);
    }
    const _Float16* const Kt = reinterpret_cast<const _Float16*>(tiles[bf]);
    const _Float16* const Vt = Kt + PU * KS;
    const float* const knU = knL[bf];
    const float* const vnU = vnL[bf];
    const int64_t nt = t_end - t0;
    const bool need_mask = nt < PU || (causal && t0 + PU - 1 > T - Sq) || !row_ok;
    int bound = PU - 1;  // keys of this unit the lane's row may see: index <= bound
    if (need_mask) {
      const int64_t bl = lim - t0, bn = nt - 1;
      int64_t bb = bl < bn ? bl : bn;
      bb = bb < -1 ? -1 : (bb > PU - 1 ? PU - 1 : bb);
      bound = row_ok ? (int)bb : -1;
    }
    // ---- per key tile kt (keys 32 kt .. 32 kt + 31): S^T = K Qrot^T, the offset check,
    //      then O^T += V^T P'^T over its two 16-key steps (the lazy offset lets each tile
    //      finish before the next one's scores exist: half the score registers live)
#pragma unroll
    for (int kt = 0; kt < 2; kt++) {
      f32x16 acc;
#pragma unroll
      for (int e = 0; e < 16; e++) acc[e] = 0.f;
#pragma unroll
      for (int s = 0; s < 4; s++) {
        const half8 A = *reinterpret_cast<const half8*>(Kt + (32 * kt + col) * KS + 16 * s + 8 * h);
        acc = mfma32(A, qhi[s], acc);
        acc = mfma32(A, qlo[s], acc);
      }
      float sc[16];
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const float4 kv = *reinterpret_cast<const float4*>(knU + 32 * kt + 8 * i + 4 * h);
        sc[4 * i] = __builtin_fmaf(acc[4 * i], kv.x, -m_run);
        sc[4 * i + 1] = __builtin_fmaf(acc[4 * i + 1], kv.y, -m_run);
        sc[4 * i + 2] = __builtin_fmaf(acc[4 * i + 2], kv.z, -m_run);
        sc[4 * i + 3] = __builtin_fmaf(acc[4 * i + 3], kv.w, -m_run);
      }
      if (need_mask) {  // uniform: the last units of a range, the causal diagonal, short blocks
#pragma unroll
        for (int e = 0; e < 16; e++) sc[e] = 32 * kt + 8 * (e >> 2) + 4 * h + (e & 3) <= bound ? sc[e] : NEG;
      }
      float mx = NEG;
#pragma unroll
      for (int e = 0; e < 16; e++) mx = fmaxf(mx, sc[e]);
      mx = fmaxf(mx, xor32(mx));  // the row's maximum relative to m_run (-inf: no key)
      const bool first = !have && mx != NEG;
      if (__ballot(first || mx > 0.0f)) {  // some row's offset moves (rare after the first units)
        const float dm = mx == NEG ? 0.0f : (have ? fmaxf(mx + TAU, 0.0f) : mx + TAU);
        const float alpha = have ? __builtin_amdgcn_exp2f(-dm) : 0.0f;  // nothing accumulated before
        l_run *= alpha;
#pragma unroll
        for (int e = 0; e < 16; e++) {
          O[0][e] *= alpha;
          O[1][e] *= alpha;
        }
#pragma unroll
        for (int e = 0; e < 16; e++) sc[e] -= dm;
        m_run += dm;
        have = have || mx != NEG;
      }
#pragma unroll
      for (int kh = 0; kh < 2; kh++) {
        const int ks = 2 * kt + kh;
        half8 P;
#pragma unroll
        for (int jj = 0; jj < 8; jj++) {
          const int i = 2 * kh + (jj >> 2), j = jj & 3;
          const float p = __builtin_amdgcn_exp2f(sc[4 * i + j]);
          l_run += p;
          P[jj] = (_Float16)(p * vnU[32 * kt + 8 * i + 4 * h + j]);
        }
#pragma unroll
        for (int dtt = 0; dtt < 2; dtt++) {
          const _Float16* vrow = Vt + (32 * dtt + col) * VS + 16 * ks + 4 * h;
          const half4 a0 = *reinterpret_cast<const half4*>(vrow);
          const half4 a1 = *reinterpret_cast<const half4*>(vrow + 8);
          const half8 A = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
          O[dtt] = mfma32(A, P, O[dtt]);
        }
      }
    }
    __syncthreads();  // unit h + 1 is in its buffer; this unit's buffer is free again
  }

  // ---- this row's partial record: O^T rows 32 dtt + 8 i + 4 h + j of column col
  float l = l_run + xor32(l_run);
  // the row's indices again, from a lane index formed here (one carried across the loop
  // from the prologue was spilled)
  uint32_t all = ~0u;
  __asm__ volatile("" : "+s"(all));
  const int ln = (int)__builtin_amdgcn_mbcnt_hi(all, __builtin_amdgcn_mbcnt_lo(all, 0u));
  const int ecol = ln & 31, eh = ln >> 5;
  const int er = rb * WROWS + 32 * w + ecol;
  if (er >= rows) return;
  const int ehl = er / Sq, eqi = er - ehl * Sq;
  const int64_t bh = ((int64_t)b * Hq + (int64_t)g * G + ehl) * Sq + eqi;
  float* rec = ws + (bh * nchunks + chunk) * REC_F;
  if (eh == 0) {
    rec[0] = have ? m_run : NEG;  // a row without keys in this range: an empty record
    rec[1] = l;
  }
#pragma unroll
  for (int dtt = 0; dtt < 2; dtt++)
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 4; j++) rec[2 + 32 * dtt + 8 * i + 4 * eh + j] = O[dtt][4 * i + j];
}

}  // namespace

PrefillPlan prefill_plan(const fq_codebook* cb, int B, int Hq, int Hkv, int Sq, int64_t T) {
  // the wide k = 4 / 8-bit kernel: 128 rows per workgroup, three workgroups per CU, so the
  // key ranges are cut for one wave of 768 workgroups; the general kernel: 64 rows, 1024
  const bool wide = cb->k == 4 && cb->bits == 8 && cb->prefill_wide;
  const int prows = wide ? WROWS : PROWS;
  const int64_t target = wide ? 768 : 1024;
  const int rows = (Hq / Hkv) * Sq;
  const int rblocks = (rows + prows - 1) / prows;
  const int64_t wgs = (int64_t)rblocks * B * Hkv;
  int64_t nc = (target + wgs - 1) / wgs;
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
  if (cb->k == 4 && cb->bits == 8 && cb->prefill_wide) return CB_K4B8;
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
  const PrefillPlan p = prefill_plan(cb, B, Hq, Hkv, Sq, T);
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
    hipLaunchKernelGGL(attn_prefill_w, a.grid, dim3(PW * 64), 0, s, a.q, a.qscale,
                       reinterpret_cast<const half8*>(cb->rotp), a.kc, a.kn, a.vc, a.vn,
                       cb->cw16, a.Hq, a.Hkv, a.T, a.Sq, a.causal, a.p.chunk_tokens, a.p.nchunks, a.ws);
    e = hipGetLastError();
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
