// Matrix-core FibQuant encoder for k = d = 64 (the whole rotated unit vector is
// one block; FibQuant summary §2.3 with d/k = 1, nearest codeword among N),
// fp16 input.  The search is a dense contraction: scores 256 (||c||^2 - 2 y.c)
// for every (codeword, vector) pair, reduced by a minimum over codewords.
//
// A wave owns 32 vectors (one column tile).  The workgroup streams the codebook
// through LDS in chunks of 8 tiles of 32 codewords (double buffered, loaded
// straight from global memory into LDS), so every codeword read from L2 serves
// all 16 waves.
//
//  1. Rotation on the fp16 matrix core (mfma_f32_32x32x16_f16): 1024 Pi split
//     into fp16 hi + mid + lo, x is fp16, products exact, hi and mid / lo
//     products summed in fp32 separately.  The rows of Pi are permuted so that
//     lane l holds coordinates 32 (l / 32) .. + 31 of vector l % 32.
//  2. -512 y is rounded to fp16 ("hi"); lanes exchange halves so that each holds
//     the B operands of 4 K-steps of 16 coordinates.  A fifth K-step multiplies
//     the record's norm slots (256 ||c||^2 as fp16 hi + lo) by 1, so the
//     accumulator starts at 0 and no per-tile LDS reads seed it.
//  3. Per codeword tile: 5 chained matrix ops; the lane keeps the minimum of its
//     16 rows, the best, second and third tile minima (with the tiles of the
//     first two) and the 16 scores of its best tile.
//  4. Certificate.  The residual r = -512 y - hi is known exactly per vector, and
//     leaving it out moves a score by at most |c| |r|_2, so every score is within
//        E = E0 + 1.0001 cmax |r|_2 + 2^-22 256 c2max 1.01
//     of the exact scaled score, E0 the bound of the k = 4 / 8 encoder
//     (1.01 ((2k+7) u (256 c2max + 512 cmax |y|) + 35840 sqrt(k) cmax u
//     + 2^-25 (1 + sqrt(k) cmax)), |y| <= 1) and the last term the fp16 hi + lo
//     split of 256 ||c||^2.  If second - best > 2E the winner is the exact
//     minimiser.
//  5. Uncertified vectors (about 2 % of the full-vector workload): every codeword
//     whose computed score is within 2E of the best lies in the best or second
//     tile of a half unless a third tile minimum is that close too; those at most
//     4 x 16 rows are scored in fp64 with the direct distance by the owning wave,
//     one row per lane (lowest index on exact ties).  Otherwise the vector is
//     searched again in fp64 over the whole codebook by the whole workgroup: each
//     wave queues its vectors (y in fp64) in LDS, then every wave scores its
//     sixteenth of the codebook (fp16 records read straight from global memory,
//     four lanes per codeword, 16 coordinates each) for up to four queued vectors
//     per pass.
#include "fq_device.h"
#include "fq_internal.h"

namespace fq {
namespace {

constexpr int D = kD;
constexpr int WAVES = 16;
constexpr int CT = 8;                          // codeword tiles per LDS chunk
constexpr int ROWB = 144;                      // bytes per codeword row: 64 fp16, 256 ||c||^2 as fp16 hi, lo, 0 x 6
constexpr int TILEB = 32 * ROWB;               // 4608
constexpr int CHUNKB = CT * TILEB;             // 36864
constexpr int SCR_DW = 2 * 64 * 2 + 16;        // per wave: x and y (fp64) of a re-searched vector + codes
constexpr int QMAX = 16;                       // queued re-searches per workgroup and round
constexpr int QB = 4;                          // queued vectors scored per pass over the codebook
// queue: y (fp64) per entry, owner (wave << 8 | column) per entry, per-wave best
// (distance, index) per entry, and the count
constexpr int UMAX = WAVES * 32;               // list of uncertified vectors: every column of a round fits
constexpr int Q_BYTES = QMAX * 64 * 8 + QMAX * 4 + QMAX * WAVES * 16 + 16 + UMAX * 12 + 16;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

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

__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
}

__device__ inline uint32_t pack_h2(float a, float b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
}
__device__ inline float h_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)); }
__device__ inline float h_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// Copy chunk `ch` of the tile records into LDS buffer `dst`: each wave moves
// 1 KiB pieces (lane i: bytes 16 i .. 16 i + 15 of the piece) straight to LDS.
__device__ inline void load_chunk(const uint8_t* __restrict__ rec, int ch, int nchunk_bytes, char* dst, int w,
                                  int lane) {
  const uint8_t* src = rec + (size_t)ch * CHUNKB;
  for (int p = w; p * 1024 < nchunk_bytes; p += WAVES)
    lds_dma16(src + p * 1024 + lane * 16, dst + p * 1024);
}

// chunk buffers, per-wave scratch, queue and list, Pi^T in fp64 (for the exact y of re-searches)
constexpr size_t full_lds_bytes() {
  return 2 * (size_t)CHUNKB + (size_t)WAVES * SCR_DW * 4 + Q_BYTES + (size_t)D * D * 8;
}

template <bool NF16>
__global__ __launch_bounds__(WAVES * 64, 4) void encode_full(
    const _Float16* __restrict__ x, int64_t n, int64_t ngroups, const uint4* __restrict__ rotA,
    const uint8_t* __restrict__ rec, const float* __restrict__ cw, const double* __restrict__ pi64t, int N, int bits,
    float e_abs, float e_rel, float cmax, float c2max, uint8_t* __restrict__ codes, void* __restrict__ norms,
    const int64_t* __restrict__ slots, int64_t cap, int nwg) {
  extern __shared__ uint4 smem[];
  char* buf0 = reinterpret_cast<char*>(smem);
  const int w = __builtin_amdgcn_readfirstlane((int)(fq_tid() >> 6));
  const int lane = fq_tid() & 63;
  const int c = lane & 31, h = lane >> 5;
  uint32_t* scr = reinterpret_cast<uint32_t*>(buf0 + 2 * CHUNKB) + w * SCR_DW;
  double* xs = reinterpret_cast<double*>(scr);  // 64 fp64
  double* ys = xs + 64;                          // 64 fp64
  uint32_t* spk = scr + 256;                     // 16 words: 32 codes x <= 16 bits
  char* qbase = buf0 + 2 * CHUNKB + WAVES * SCR_DW * 4;
  double* qy = reinterpret_cast<double*>(qbase);                          // [QMAX][64]
  int* qown = reinterpret_cast<int*>(qbase + QMAX * 64 * 8);              // [QMAX]
  double* qbd = reinterpret_cast<double*>(qbase + QMAX * 64 * 8 + QMAX * 4);  // [QMAX][WAVES]
  int* qbi = reinterpret_cast<int*>(qbd + QMAX * WAVES);                  // [QMAX][WAVES]
  int* qcnt = qbi + QMAX * WAVES;
  uint32_t* ulist = reinterpret_cast<uint32_t*>(qcnt + 4);  // [UMAX][3]: owner << 8 | column | few << 16, candidates
  int* ucnt = reinterpret_cast<int*>(ulist + UMAX * 3);
  const int NT = N / 32;
  const int nch = (NT + CT - 1) / CT;
  double* piL = reinterpret_cast<double*>(qbase + Q_BYTES);  // Pi^T: piL[j D + r] = Pi[r][j]
  for (int i = fq_tid(); i < D * D; i += WAVES * 64) piL[i] = pi64t[i];
  // (visible after the first barrier of the stream below)

  for (int64_t base = (int64_t)fq_bid_x() * WAVES; base < ngroups; base += (int64_t)nwg * WAVES) {
    const int64_t g = base + w;
    const int64_t v0 = g * 32;
    const int nv = g < ngroups ? (int)((n - v0) < 32 ? (n - v0) : 32) : 0;
    const bool valid = c < nv;

    // first chunk on its way while the rotation runs
    load_chunk(rec, 0, (NT < CT ? NT : CT) * TILEB, buf0, w, lane);

    // ---- 1. x, nu, rotation.  Lane l: vector l % 32, inputs 16 s + 8 h .. + 7.
    uint4 xin[4];
#pragma unroll
    for (int s = 0; s < 4; s++) xin[s] = make_uint4(0u, 0u, 0u, 0u);
    if (valid) {
      const uint4* xp = reinterpret_cast<const uint4*>(x + (v0 + c) * D);
#pragma unroll
      for (int s = 0; s < 4; s++) xin[s] = xp[2 * s + h];
    }
    double sq = 0.0;
#pragma unroll
    for (int s = 0; s < 4; s++) {
      const uint32_t wv[4] = {xin[s].x, xin[s].y, xin[s].z, xin[s].w};
#pragma unroll
      for (int t = 0; t < 4; t++) {
        const double a = (double)h_lo(wv[t]), b = (double)h_hi(wv[t]);
        sq = fma(a, a, sq);
        sq = fma(b, b, sq);
      }
    }
    sq += shfl_xor_f64(sq, 32);
    const double nu = sqrt(sq);
    if (h == 0 && valid) {
      const int64_t sv = out_slot(slots, cap, v0 + c);
      if (sv >= 0) {
        if constexpr (NF16)
          reinterpret_cast<uint16_t*>(norms)[sv] = f64_to_f16_bits(nu);
        else
          reinterpret_cast<float*>(norms)[sv] = (float)nu;
      }
    }
    const float inv = nu > 0.0 ? (float)(1.0 / (1024.0 * nu)) : 0.0f;

    // An offset the compiler cannot see through: keeps the 24 operand loads inside
    // the loop instead of hoisted into (spilled) registers.
    int rot_off = 0;
    __asm__ volatile("" : "+s"(rot_off));
    uint32_t hi[16];  // coordinates 32 h + 16 r + e of -512 y rounded to fp16, packed in pairs
    float rr = 0.f;   // sum of the squared residuals -512 y - hi of these coordinates
#pragma unroll
    for (int r = 0; r < 2; r++) {
      f32x16 ah, am;
#pragma unroll
      for (int e = 0; e < 16; e++) {
        ah[e] = 0.f;
        am[e] = 0.f;
      }
#pragma unroll
      for (int s = 0; s < 4; s++) {
        const half8 xv = __builtin_bit_cast(half8, xin[s]);
        const uint4* op = rotA + rot_off + ((r * 4 + s) * 3) * 64 + lane;
        ah = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, op[0]), xv, ah, 0, 0, 0);
        am = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, op[64]), xv, am, 0, 0, 0);
        am = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, op[128]), xv, am, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const float va = -512.0f * ((ah[e] + am[e]) * inv);
        const float vb = -512.0f * ((ah[e + 1] + am[e + 1]) * inv);
        const float ha = (float)(_Float16)va, hb = (float)(_Float16)vb;
        hi[8 * r + e / 2] = pack_h2(ha, hb);
        rr = fmaf(va - ha, va - ha, rr);  // the differences are exact in fp32
        rr = fmaf(vb - hb, vb - hb, rr);
      }
    }
    rr += __shfl_xor(rr, 32);
    // error bound of this vector's scores (see 4.)
    const float E = e_abs + e_rel * 1.01f + 1.0001f * cmax * __builtin_sqrtf(rr) * 1.0001f +
                    256.0f * c2max * 2.4e-7f;
    // ---- 2. B operands: step s covers coordinates 16 s .. 16 s + 15, lanes 0-31 the
    //         first 8, lanes 32-63 the last 8.  Lane c holds coordinates 0 .. 31 of
    //         vector c, lane c + 32 coordinates 32 .. 63: one exchange of 8 dwords.
    uint32_t bq[4][4];
    {
      uint32_t recv[8];
#pragma unroll
      for (int d = 0; d < 8; d++) {
        const int src = h == 0 ? (d < 4 ? 4 + d : 8 + d) : (d < 4 ? d : 4 + d);
        recv[d] = (uint32_t)__shfl_xor((int)hi[src], 32);
      }
#pragma unroll
      for (int d = 0; d < 4; d++) {
        bq[0][d] = h == 0 ? hi[d] : recv[d];           // 0 .. 7   | 8 .. 15
        bq[1][d] = h == 0 ? hi[8 + d] : recv[4 + d];   // 16 .. 23 | 24 .. 31
        bq[2][d] = h == 0 ? recv[d] : hi[4 + d];       // 32 .. 39 | 40 .. 47
        bq[3][d] = h == 0 ? recv[4 + d] : hi[12 + d];  // 48 .. 55 | 56 .. 63
      }
    }
#pragma unroll
    for (int s = 0; s < 4; s++)
#pragma unroll
      for (int d = 0; d < 4; d++) __asm__ volatile("" : "+v"(bq[s][d]));
    // step 4: the norm slots (K 0, 1 of lanes 0-31) times 1
    const half8 bnorm = __builtin_bit_cast(half8, make_uint4(h == 0 ? 0x3c003c00u : 0u, 0u, 0u, 0u));

    // ---- 3. stream the codebook
    float m1 = __builtin_huge_valf(), m2 = __builtin_huge_valf(), m3 = __builtin_huge_valf();
    int tid = 0, tid2 = 0;
    f32x16 bestD;
#pragma unroll
    for (int e = 0; e < 16; e++) bestD[e] = __builtin_huge_valf();
    if (w == 0 && lane == 0) {  // read after the barriers below
      *qcnt = 0;
      *ucnt = 0;
    }
    __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): this wave's pieces of chunk 0 are in LDS
    __syncthreads();
    for (int ch = 0; ch < nch; ch++) {
      char* cur = buf0 + (ch & 1) * CHUNKB;
      if (ch + 1 < nch) {
        const int nt = (NT - (ch + 1) * CT) < CT ? (NT - (ch + 1) * CT) : CT;
        load_chunk(rec, ch + 1, nt * TILEB, buf0 + ((ch + 1) & 1) * CHUNKB, w, lane);
      }
      const int nt = (NT - ch * CT) < CT ? (NT - ch * CT) : CT;
      for (int tt = 0; tt < nt; tt++) {
        const char* arow = cur + tt * TILEB + c * ROWB;
        half8 A[4];
#pragma unroll
        for (int s = 0; s < 4; s++) A[s] = *reinterpret_cast<const half8*>(arow + 32 * s + 16 * h);
        // lanes 32-63 read the same finite norm slots against a zero B: no contribution
        const half8 An = *reinterpret_cast<const half8*>(arow + 128);
        f32x16 acc;
#pragma unroll
        for (int e = 0; e < 16; e++) acc[e] = 0.f;
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(An, bnorm, acc, 0, 0, 0);
#pragma unroll
        for (int s = 0; s < 4; s++)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[s], __builtin_bit_cast(half8, bq[s]), acc, 0, 0, 0);
        const float tm = min16(acc);
        const int t = ch * CT + tt;
        const bool c1 = tm < m1, c2 = tm < m2;
        m3 = __builtin_amdgcn_fmed3f(m2, m3, tm);
        tid2 = c1 ? tid : (c2 ? t : tid2);
        m2 = __builtin_amdgcn_fmed3f(m1, m2, tm);
        tid = c1 ? t : tid;
        m1 = fminf(m1, tm);
#pragma unroll
        for (int e = 0; e < 16; e++) bestD[e] = c1 ? acc[e] : bestD[e];
      }
      __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0)
      __syncthreads();
    }

    // ---- 4. best row of the best tile, merge, certificate
    float r1 = __builtin_huge_valf(), r2 = __builtin_huge_valf();
    int ri = 0;
#pragma unroll
    for (int e = 0; e < 16; e++) {
      const float v = bestD[e];
      r2 = __builtin_amdgcn_fmed3f(r1, r2, v);
      ri = v < r1 ? e : ri;  // first (lowest row) minimum: rows grow with e
      r1 = fminf(r1, v);
    }
    ri = 32 * tid + (ri >> 2) * 8 + 4 * h + (ri & 3);
    const float o1 = __shfl_xor(r1, 32), o2 = __shfl_xor(r2, 32), om = __shfl_xor(m2, 32);
    const int oi = __shfl_xor(ri, 32);
    const bool other = (o1 < r1) || (o1 == r1 && oi < ri);
    const float best = other ? o1 : r1;
    const float second = fminf(fminf(fmaxf(r1, o1), fminf(r2, o2)), fminf(m2, om));
    const uint32_t code = (uint32_t)(other ? oi : ri);
    const bool sure = (second - best) > 2.0f * E;
    // candidate tiles of an uncertified column, per half: the best tile always, the
    // second if its minimum is within 2E of the best; a third that close sends the
    // vector to the full search
    const float lim = best + 2.0f * E;
    const uint32_t cand = (uint32_t)(tid & 0xffff) | ((uint32_t)(m2 <= lim ? (tid2 & 0x7fff) | 0x8000 : 0) << 16);
    const bool far3 = m3 > lim;

    const int words = bits;  // 32 codes x bits
    for (int i = lane; i < words; i += 64) spk[i] = 0u;
    wave_lds_sync();
    if (h == 0 && valid && sure) {
      const int bo = c * bits, sh = bo & 31;
      atomicOr(&spk[bo >> 5], code << sh);
      if (sh + bits > 32) atomicOr(&spk[(bo >> 5) + 1], code >> (32 - sh));
    }
    // ---- 5. uncertified vectors: the owner lists them; after a barrier every wave takes
    //      list entries (the exact y of a vector costs a chain of dependent loads, so one
    //      wave per entry; the list holds every column of a round).  A vector whose candidates lie in its listed tiles is scored
    //      over those rows; any other goes to the workgroup's fp64 queue (or, past QMAX
    //      entries, is searched by the wave alone).  Codes go to the owner's packing words.
    auto research = [&](int ow, int cc, bool few, uint32_t cd0, uint32_t cd1) {
      uint32_t* ospk = reinterpret_cast<uint32_t*>(buf0 + 2 * CHUNKB) + ow * SCR_DW + 256;
      auto put = [&](uint32_t cv) {
        const int bo = cc * bits, sh = bo & 31;
        atomicOr(&ospk[bo >> 5], cv << sh);
        if (sh + bits > 32) atomicOr(&ospk[(bo >> 5) + 1], cv >> (32 - sh));
      };
      const double xj = (double)x[((base + ow) * 32 + cc) * D + lane];
      xs[lane] = xj;
      double s2 = xj * xj;
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) s2 += shfl_xor_f64(s2, m);
      const double nuf = sqrt(s2);
      const double iv = nuf > 0.0 ? 1.0 / nuf : 0.0;
      wave_lds_sync();
      double yt = 0.0;  // coordinate `lane` of y, Pi from LDS
#pragma unroll 8
      for (int j = 0; j < D; j++) yt = fma(piL[j * D + lane], xs[j], yt);
      yt *= iv;
      if (few) {
        // lane L scores row L % 16 of candidate (tile, half) L / 16: the best and second
        // tiles of half 0 (lanes 0-31) and of half 1 (lanes 32-63)
        ys[lane] = yt;
        wave_lds_sync();
        const int hh = lane >> 5;
        const uint32_t cd = hh ? cd1 : cd0;
        const bool sec = ((lane >> 4) & 1) != 0;
        const bool use = !sec || (cd & 0x80000000u);
        const int tl = sec ? (int)((cd >> 16) & 0x7fff) : (int)(cd & 0xffff);
        const int j = lane & 15;
        const int nn = 32 * tl + 8 * (j >> 2) + 4 * hh + (j & 3);
        double dd = __builtin_huge_val();
        if (use) {
          const uint4* rowp = reinterpret_cast<const uint4*>(rec + (size_t)nn * ROWB);
          dd = 0.0;
          for (int q0 = 0; q0 < 8; q0 += 4) {
            uint4 rw[4];
#pragma unroll
            for (int q = 0; q < 4; q++) rw[q] = rowp[q0 + q];
#pragma unroll
            for (int q = 0; q < 4; q++) {
              const uint32_t ww[4] = {rw[q].x, rw[q].y, rw[q].z, rw[q].w};
#pragma unroll
              for (int i = 0; i < 4; i++) {
                const double d0 = ys[8 * (q0 + q) + 2 * i] - (double)h_lo(ww[i]);
                const double d1 = ys[8 * (q0 + q) + 2 * i + 1] - (double)h_hi(ww[i]);
                dd = fma(d0, d0, dd);
                dd = fma(d1, d1, dd);
              }
            }
          }
        }
        int bn = use ? nn : 0x7fffffff;
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
          const double od = shfl_xor_f64(dd, m);
          const int on = __shfl_xor(bn, m);
          if (od < dd || (od == dd && on < bn)) {
            dd = od;
            bn = on;
          }
        }
        if (lane == 0) put((uint32_t)bn);
        wave_lds_sync();
        return;
      }
      int slot = 0;
      if (lane == 0) slot = atomicAdd(qcnt, 1);
      slot = __builtin_amdgcn_readfirstlane(__shfl(slot, 0));
      if (slot < QMAX) {
        qy[slot * 64 + lane] = yt;
        if (lane == 0) qown[slot] = (ow << 8) | cc;
        return;
      }
      ys[lane] = yt;
      wave_lds_sync();
      double bd = __builtin_huge_val();
      int bn = 0x7fffffff;
      for (int nn = lane; nn < N; nn += 64) {
        const float* cp = cw + (size_t)nn * D;
        double dd = 0.0;
        for (int t = 0; t < D; t++) {
          const double df = ys[t] - (double)cp[t];
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
      if (lane == 0) put((uint32_t)bn);
      wave_lds_sync();
    };
    const bool far3_col = far3 && __shfl_xor((int)far3, 32);
    uint64_t todo = __ballot(h == 0 && valid && !sure);
    while (todo) {
      const int cc = __builtin_ctzll(todo);
      todo &= todo - 1;
      const bool few = __shfl((int)far3_col, cc) != 0;  // every candidate in the listed tiles
      const uint32_t cd0 = (uint32_t)__shfl((int)cand, cc), cd1 = (uint32_t)__shfl((int)cand, cc + 32);
      if (lane == 0) {
        const int slot = atomicAdd(ucnt, 1);  // < UMAX: at most every column of the round
        ulist[3 * slot] = (uint32_t)((w << 8) | cc | (few ? 0x10000 : 0));
        ulist[3 * slot + 1] = cd0;
        ulist[3 * slot + 2] = cd1;
      }
    }
    __syncthreads();  // the list is complete
    {
      const int nu0 = *ucnt;
      const int nu = __builtin_amdgcn_readfirstlane(nu0 < UMAX ? nu0 : UMAX);
      for (int e = w; e < nu; e += WAVES) {
        const uint32_t ent = __builtin_amdgcn_readfirstlane(ulist[3 * e]);
        const uint32_t cd0 = __builtin_amdgcn_readfirstlane(ulist[3 * e + 1]);
        const uint32_t cd1 = __builtin_amdgcn_readfirstlane(ulist[3 * e + 2]);
        research((int)((ent >> 8) & 0xff), (int)(ent & 0xff), (ent & 0x10000) != 0, cd0, cd1);
      }
    }
    __syncthreads();  // the queue is complete
    const int nq0 = *qcnt;  // the queue is complete: the list's entries were processed above
    const int nq = __builtin_amdgcn_readfirstlane(nq0 < QMAX ? nq0 : QMAX);
    // Workgroup pass(es) over the codebook for the queued vectors, QB at a time: lane l
    // of wave w scores codewords 256 i + 16 w + l / 4 over coordinates 16 (l % 4) .. + 15;
    // the four partial sums are added in a fixed order.
    for (int e0 = 0; e0 < nq; e0 += QB) {
      const int ne = (nq - e0) < QB ? (nq - e0) : QB;
      double bd[QB];
      int bn[QB];
#pragma unroll
      for (int e = 0; e < QB; e++) {
        bd[e] = __builtin_huge_val();
        bn[e] = 0x7fffffff;
      }
      const int cl = 16 * w + (lane >> 2), q4 = lane & 3;
      const int nit = (N + 255) / 256;
      // codeword it * 256 + cl: its 16 coordinates of this lane straight from the fp16
      // records in global memory (four lanes read one row's 128 bytes), four rows in flight
      for (int it0 = 0; it0 < nit; it0 += 4) {
        uint4 rr[4][2];
#pragma unroll
        for (int u = 0; u < 4; u++) {
          const int nn = (it0 + u) * 256 + cl;
          const int nc = nn < N ? nn : N - 1;
          const uint4* rowp = reinterpret_cast<const uint4*>(rec + (size_t)nc * ROWB + 32 * q4);
          rr[u][0] = rowp[0];
          rr[u][1] = rowp[1];
        }
#pragma unroll
        for (int u = 0; u < 4; u++) {
          const int nn = (it0 + u) * 256 + cl;
          const uint32_t cwv[8] = {rr[u][0].x, rr[u][0].y, rr[u][0].z, rr[u][0].w,
                                   rr[u][1].x, rr[u][1].y, rr[u][1].z, rr[u][1].w};
#pragma unroll
          for (int e = 0; e < QB; e++) {
            if (e < ne) {
              const double* yq = qy + (e0 + e) * 64 + 16 * q4;
              double pp = 0.0;
#pragma unroll
              for (int i = 0; i < 8; i++) {
                const double d0 = yq[2 * i] - (double)h_lo(cwv[i]);
                const double d1 = yq[2 * i + 1] - (double)h_hi(cwv[i]);
                pp = fma(d0, d0, pp);
                pp = fma(d1, d1, pp);
              }
              const double p1 = shfl_xor_f64(pp, 1);
              const double lo2 = (q4 & 1) ? p1 + pp : pp + p1;  // (q0 + q1) and (q2 + q3)
              const double p2 = shfl_xor_f64(lo2, 2);
              const double dd = (q4 & 2) ? p2 + lo2 : lo2 + p2;  // (q0 + q1) + (q2 + q3)
              if (nn < N && dd < bd[e]) {
                bd[e] = dd;
                bn[e] = nn;
              }
            }
          }
        }
      }
      // best of the wave (lowest index on equal distances), then of the workgroup
#pragma unroll
      for (int e = 0; e < QB; e++) {
        if (e < ne) {
#pragma unroll
          for (int m = 4; m <= 32; m <<= 1) {
            const double od = shfl_xor_f64(bd[e], m);
            const int on = __shfl_xor(bn[e], m);
            if (od < bd[e] || (od == bd[e] && on < bn[e])) {
              bd[e] = od;
              bn[e] = on;
            }
          }
          if (lane == 0) {
            qbd[(e0 + e) * WAVES + w] = bd[e];
            qbi[(e0 + e) * WAVES + w] = bn[e];
          }
        }
      }
      __syncthreads();
      for (int e = 0; e < ne; e++) {
        const int own = qown[e0 + e];
        if ((own >> 8) == w && lane == 0) {
          double b = qbd[(e0 + e) * WAVES];
          int bi = qbi[(e0 + e) * WAVES];
          for (int ww = 1; ww < WAVES; ww++) {
            const double od = qbd[(e0 + e) * WAVES + ww];
            const int on = qbi[(e0 + e) * WAVES + ww];
            if (od < b || (od == b && on < bi)) {
              b = od;
              bi = on;
            }
          }
          const uint32_t cv = (uint32_t)bi;
          const int bo = (own & 0xff) * bits, sh = bo & 31;
          atomicOr(&spk[bo >> 5], cv << sh);
          if (sh + bits > 32) atomicOr(&spk[(bo >> 5) + 1], cv >> (32 - sh));
        }
      }
      __syncthreads();  // per-wave bests free again
    }
    wave_lds_sync();
    if (slots) {
      scatter_records(spk, nv, bits / 8, slots, cap, v0, codes, lane);
    } else if (nv > 0) {
      const int nbytes = (nv * bits + 7) / 8;
      uint8_t* dst = codes + g * (int64_t)(4 * bits);  // group g starts at bit g * 32 * bits
      const int nfull = nbytes / 4;
      for (int i = lane; i < nfull; i += 64) reinterpret_cast<uint32_t*>(dst)[i] = spk[i];
      const int rem = nbytes - 4 * nfull;
      if (lane < rem) dst[4 * nfull + lane] = (uint8_t)((spk[nfull] >> (8 * lane)) & 0xffu);
    }
    wave_lds_sync();
  }
}

template <bool NF16>
hipError_t launch_full(const fq_codebook* cb, const void* x, int64_t n, uint8_t* codes, void* norms,
                       const int64_t* slots, int64_t cap, hipStream_t s) {
  const size_t lds = full_lds_bytes();
  int64_t resident = 0;
  const hipError_t e =
      resident_workgroups(reinterpret_cast<const void*>(encode_full<NF16>), WAVES * 64, lds, cb->device, &resident);
  if (e != hipSuccess) return e;
  const int64_t ngroups = (n + 31) / 32;
  int64_t wgs = (ngroups + WAVES - 1) / WAVES;
  if (wgs > resident) wgs = resident;
  hipLaunchKernelGGL((encode_full<NF16>), dim3((unsigned)wgs), dim3(WAVES * 64), lds, s,
                     reinterpret_cast<const _Float16*>(x), n, ngroups, reinterpret_cast<const uint4*>(cb->rot32),
                     reinterpret_cast<const uint8_t*>(cb->frec), cb->cw, cb->pi64t, cb->N, cb->bits, cb->h16_eabs,
                     cb->h16_erel, cb->cmax, cb->c2max, codes, norms, slots, cap, (int)wgs);
  return hipGetLastError();
}

}  // namespace

bool encode_full_supported(const fq_codebook* cb) {
  return cb->k == D && cb->rot32 && cb->frec && cb->N % 32 == 0 && cb->N >= 32 && cb->bits <= 16 &&
         full_lds_bytes() <= cb->max_lds;
}

hipError_t launch_encode_full(const fq_codebook* cb, const void* x, int64_t n, uint8_t* codes, void* norms,
                              fq_dtype norm_dtype, const int64_t* slots, int64_t cap, hipStream_t s) {
  if (!encode_full_supported(cb)) return hipErrorNotSupported;
  return norm_dtype == FQ_F16 ? launch_full<true>(cb, x, n, codes, norms, slots, cap, s)
                              : launch_full<false>(cb, x, n, codes, norms, slots, cap, s);
}

}  // namespace fq
