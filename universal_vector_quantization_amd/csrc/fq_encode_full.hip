// Matrix-core FibQuant encoder for fp16 input with blocks of KB = 16, 32 or 64
// coordinates (FibQuant summary §2.3: d/k blocks, nearest codeword among N;
// KB = d = 64 is the full-vector code, the whole rotated unit vector one block).
// The search is a dense contraction: scores 256 (||c||^2 - 2 y.c) for every
// (codeword, block) pair, reduced by a minimum over codewords.
//
// A wave owns 32 vectors, i.e. 64 / KB column tiles of 32 blocks (tile b holds
// block b of the 32 vectors).  The workgroup streams the codebook through LDS in
// chunks of 8 tiles of 32 codewords (double buffered, loaded straight from global
// memory into LDS), so every codeword read from L2 serves all the waves, and every
// codeword tile a wave reads serves all its column tiles.
//
//  1. Rotation on the fp16 matrix core (mfma_f32_32x32x16_f16): 1024 Pi split
//     into fp16 hi + mid + lo, x is fp16, products exact, hi and mid / lo
//     products summed in fp32 separately.  The rows of Pi are permuted so that
//     lane l holds coordinates 32 (l / 32) .. + 31 of vector l % 32.
//  2. -512 y is rounded to fp16 ("hi"); lanes exchange halves so that each holds
//     the B operands of 4 K-steps of 16 coordinates: block b of size KB is the
//     K-steps KB / 16 b .. KB / 16 (b + 1) - 1.  For KB = 64 the accumulators
//     start at the fp32 256 ||c||^2 of the lane's rows, read from the tile's norm
//     slots in LDS (four 16-byte reads per tile, each shared by half the wave); for
//     KB = 16, 32 a further K-step multiplies the record's norm slot (256 ||c||^2 as
//     fp16 hi + lo) by 1, so the accumulator starts at 0 (there each codeword tile
//     serves two column tiles, and the per-tile seed registers measured slower).
//  3. Per codeword tile and column tile: KB / 16 (KB = 64) or KB / 16 + 1 chained
//     matrix ops; the lane
//     takes the minimum of its 16 rows, writes the tile index into its low
//     tagbits = ceil(log2(N / 32)) mantissa bits (one and-or), keeps the best,
//     second and third such tagged minima (so the first two name their tiles)
//     and the 16 scores of its best tile.  A tag moves a minimum by less than
//     2^(tagbits - 23) of itself; every test below that reads a tagged minimum
//     (the runner-up of the certificate, the second and third tiles' distance
//     from the best) allows for that in the safe direction.
//  4. Certificate.  The residual r_b = (-512 y - hi) over block b is known exactly,
//     and leaving it out moves a score by at most |c| |r_b|_2, so every score is
//     within
//        E = E0 + 1.0001 cmax |r_b|_2 + 2^-22 256 c2max 1.01
//     of the exact scaled score, E0 the bound of the k = 4 / 8 encoder for this k
//     (1.01 ((2k+7) u (256 c2max + 512 cmax |y_b|) + 35840 sqrt(k) cmax u
//     + 2^-25 (1 + sqrt(k) cmax)), |y_b| <= 1) and the last term the fp16 hi + lo
//     split of 256 ||c||^2 (KB = 16, 32), which also covers its rounding to fp32
//     (KB = 64).  If second - best > 2E the winner is the exact minimiser.
//  5. Uncertified blocks (about 2 % on the full-vector workload): every codeword
//     whose computed score is within 2E of the best lies in the best or second
//     tile of a half unless a third tile minimum is that close too; those at most
//     4 x 16 rows are scored in fp64 with the direct distance by one wave, one row
//     per lane (lowest index on exact ties).  Otherwise the block is searched
//     again in fp64 over the whole codebook by the whole workgroup: each wave
//     queues its blocks (y in fp64) in LDS, then every wave scores its share of
//     the codebook (fp16 records read straight from global memory, KB / 16 lanes
//     per codeword, 16 coordinates each) for up to four queued blocks per pass.
#include "fq_device.h"
#include "fq_internal.h"

namespace fq {
namespace {

constexpr int D = kD;
constexpr int CT = 8;   // codeword tiles per LDS chunk
constexpr int QMAX = 16;  // queued re-searches per workgroup and round
constexpr int QB = 4;     // queued blocks scored per pass over the codebook

// Waves per workgroup and the waves per SIMD their register budget is set for (one
// workgroup per CU); column tiles searched per pass over the codebook (the statistics
// and best-tile scores of more would not fit in registers).  KB < 64: 168 registers
// (3 waves per SIMD) for two column tiles per pass.
template <int KB>
struct FullShape {
  static constexpr int WAVES = KB == 64 ? 16 : 12;
  static constexpr int OCC = KB == 64 ? 4 : 3;
  static constexpr int CBP = KB == 64 ? 1 : 2;
};
// bytes per codeword row: KB fp16, then a 16-byte norm slot (KB = 64: row 4 g's holds
// the fp32 256 ||c||^2 of rows 4 g .. 4 g + 3, the others are zero; KB = 16, 32: the
// row's 256 ||c||^2 as fp16 hi, lo and six zeros)
__host__ __device__ constexpr int row_bytes(int KB) { return 2 * KB + 16; }
__host__ __device__ constexpr int chunk_bytes(int KB) { return CT * 32 * row_bytes(KB); }
// per wave: x and y (fp64) of a re-searched vector, then the packing words
// (32 vectors x 64 / KB codes x <= 16 bits)
__host__ __device__ constexpr int scr_dwords(int KB) { return 2 * 64 * 2 + 16 * (64 / KB); }
// queue: y (fp64) per entry, owner per entry, per-wave best (distance, index) per entry,
// the count, then the list of uncertified blocks (every column of a round fits)
template <int KB>
__host__ __device__ constexpr int q_bytes() {
  return QMAX * 64 * 8 + QMAX * 4 + QMAX * FullShape<KB>::WAVES * 16 + 16 +
         FullShape<KB>::WAVES * 32 * (64 / KB) * 12 + 16;
}

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
// A piece may run past the chunk's last tile into the record array's zero padding
// (whole chunks of CT tiles, a multiple of 1 KiB).
template <int KB>
__device__ inline void load_chunk(const uint8_t* __restrict__ rec, int ch, int nchunk_bytes, char* dst, int w,
                                  int lane) {
  const uint8_t* src = rec + (size_t)ch * chunk_bytes(KB);
  for (int p = w; p * 1024 < nchunk_bytes; p += FullShape<KB>::WAVES)
    lds_dma16(src + p * 1024 + lane * 16, dst + p * 1024);
}

// chunk buffers, per-wave scratch, queue and list, Pi^T in fp64 (for the exact y of re-searches)
template <int KB>
constexpr size_t full_lds_bytes() {
  return 2 * (size_t)chunk_bytes(KB) + (size_t)FullShape<KB>::WAVES * scr_dwords(KB) * 4 + q_bytes<KB>() +
         (size_t)D * D * 8;
}

template <int KB, bool NF16>
__global__ __launch_bounds__(FullShape<KB>::WAVES * 64, FullShape<KB>::OCC) void encode_full(
    const _Float16* __restrict__ x, int64_t n, int64_t ngroups, const uint4* __restrict__ rotA,
    const uint8_t* __restrict__ rec, const float* __restrict__ cw, const double* __restrict__ pi64t, int N, int bits,
    float e_abs, float e_rel, float cmax, float c2max, uint8_t* __restrict__ codes, void* __restrict__ norms,
    const int64_t* __restrict__ slots, int64_t cap, int nwg) {
  constexpr int WAVES = FullShape<KB>::WAVES;
  constexpr int CB = D / KB;   // column tiles (blocks per vector)
  constexpr int KS = KB / 16;  // K-steps of coordinates per block
  constexpr int ROWB = row_bytes(KB), TILEB = 32 * ROWB, CHUNKB = chunk_bytes(KB);
  constexpr int SCR_DW = scr_dwords(KB), UMAX = WAVES * 32 * CB;
  extern __shared__ uint4 smem[];
  char* buf0 = reinterpret_cast<char*>(smem);
  const int w = __builtin_amdgcn_readfirstlane((int)(fq_tid() >> 6));
  const int lane = fq_tid() & 63;
  const int c = lane & 31, h = lane >> 5;
  uint32_t* scr = reinterpret_cast<uint32_t*>(buf0 + 2 * CHUNKB) + w * SCR_DW;
  double* xs = reinterpret_cast<double*>(scr);  // 64 fp64
  double* ys = xs + 64;                          // 64 fp64
  uint32_t* spk = scr + 256;                     // 32 x CB codes x <= 16 bits
  char* qbase = buf0 + 2 * CHUNKB + WAVES * SCR_DW * 4;
  double* qy = reinterpret_cast<double*>(qbase);                          // [QMAX][64] (a block's KB coordinates)
  int* qown = reinterpret_cast<int*>(qbase + QMAX * 64 * 8);              // [QMAX]: block << 16 | wave << 8 | column
  double* qbd = reinterpret_cast<double*>(qbase + QMAX * 64 * 8 + QMAX * 4);  // [QMAX][WAVES]
  int* qbi = reinterpret_cast<int*>(qbd + QMAX * WAVES);                  // [QMAX][WAVES]
  int* qcnt = qbi + QMAX * WAVES;
  // [UMAX][3]: block << 17 | few << 16 | wave << 8 | column, candidates of the two halves
  uint32_t* ulist = reinterpret_cast<uint32_t*>(qcnt + 4);
  int* ucnt = reinterpret_cast<int*>(ulist + UMAX * 3);
  const int NT = N / 32;
  const int tagbits = NT > 1 ? 32 - __builtin_clz((unsigned)(NT - 1)) : 0;
  const uint32_t tmask = ~((1u << tagbits) - 1u);
  const float tag_rel = (float)(1u << tagbits) * (1.01f / 8388608.0f);
  const int nch = (NT + CT - 1) / CT;
  double* piL = reinterpret_cast<double*>(qbase + q_bytes<KB>());  // Pi^T: piL[j D + r] = Pi[r][j]
  for (int i = fq_tid(); i < D * D; i += WAVES * 64) piL[i] = pi64t[i];
  // (visible after the first barrier of the stream below)

  for (int64_t base = (int64_t)fq_bid_x() * WAVES; base < ngroups; base += (int64_t)nwg * WAVES) {
    const int64_t g = base + w;
    const int64_t v0 = g * 32;
    const int nv = g < ngroups ? (int)((n - v0) < 32 ? (n - v0) : 32) : 0;
    const bool valid = c < nv;

    // first chunk on its way while the rotation runs
    load_chunk<KB>(rec, 0, (NT < CT ? NT : CT) * TILEB, buf0, w, lane);

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
    uint32_t hi[16];   // coordinates 32 h + 16 r + e of -512 y rounded to fp16, packed in pairs
    float rr[2];       // per r: sum of the squared residuals -512 y - hi of those 16 coordinates
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
      // the full-vector code sums all 32 residuals of the lane in one chain
      float acc = KB == D && r == 1 ? rr[0] : 0.f;
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const float va = -512.0f * ((ah[e] + am[e]) * inv);
        const float vb = -512.0f * ((ah[e + 1] + am[e + 1]) * inv);
        const float ha = (float)(_Float16)va, hb = (float)(_Float16)vb;
        hi[8 * r + e / 2] = pack_h2(ha, hb);
        acc = fmaf(va - ha, va - ha, acc);  // the differences are exact in fp32
        acc = fmaf(vb - hb, vb - hb, acc);
      }
      rr[r] = acc;
    }
    // error bound of each block's scores (see 4.): K-step s = 2 h + r of the lane's own
    // coordinates; the partner lane holds the other half
    float E[CB];
    {
      const float o0 = __shfl_xor(rr[0], 32), o1 = __shfl_xor(rr[1], 32);
#pragma unroll
      for (int b = 0; b < CB; b++) {
        float rb;
        if constexpr (KB == D)
          rb = rr[1] + o1;  // rr[1] already holds both of this lane's K-steps
        else if constexpr (KB == 32)
          rb = b == h ? rr[0] + rr[1] : o0 + o1;
        else
          rb = (b >> 1) == h ? ((b & 1) ? rr[1] : rr[0]) : ((b & 1) ? o1 : o0);
        E[b] = e_abs + e_rel * 1.01f + 1.0001f * cmax * __builtin_sqrtf(rb) * 1.0001f + 256.0f * c2max * 2.4e-7f;
      }
    }
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

    // the norm step of KB = 16, 32: the norm slots (K 0, 1 of lanes 0-31) times 1
    const half8 bnorm = __builtin_bit_cast(half8, make_uint4(h == 0 ? 0x3c003c00u : 0u, 0u, 0u, 0u));

    // ---- 3-4. stream the codebook (once per CBP column tiles), then per column tile the
    //      best row of the best tile, merge and certificate
    constexpr int CBP = FullShape<KB>::CBP;
    uint32_t code[CB], cand[CB];
    bool sure[CB], far3[CB];
    if (w == 0 && lane == 0) {  // read after the barriers below
      *qcnt = 0;
      *ucnt = 0;
    }
#pragma unroll
    for (int pb = 0; pb < CB; pb += CBP) {
      if (pb > 0) {  // every wave is past the previous pass's last barrier: buffer 0 is free
        load_chunk<KB>(rec, 0, (NT < CT ? NT : CT) * TILEB, buf0, w, lane);
      }
      float m1[CBP], m2[CBP], m3[CBP];  // tagged tile minima
      f32x16 bestD[CBP];
#pragma unroll
      for (int j = 0; j < CBP; j++) {
        m1[j] = m2[j] = m3[j] = __builtin_huge_valf();
#pragma unroll
        for (int e = 0; e < 16; e++) bestD[j][e] = __builtin_huge_valf();
      }
      __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): this wave's pieces of chunk 0 are in LDS
      __syncthreads();
      for (int ch = 0; ch < nch; ch++) {
        char* cur = buf0 + (ch & 1) * CHUNKB;
        if (ch + 1 < nch) {
          const int nt = (NT - (ch + 1) * CT) < CT ? (NT - (ch + 1) * CT) : CT;
          load_chunk<KB>(rec, ch + 1, nt * TILEB, buf0 + ((ch + 1) & 1) * CHUNKB, w, lane);
        }
        const int nt = (NT - ch * CT) < CT ? (NT - ch * CT) : CT;
        for (int tt = 0; tt < nt; tt++) {
          const char* arow = cur + tt * TILEB + c * ROWB;
          half8 A[KS];
#pragma unroll
          for (int s = 0; s < KS; s++) A[s] = *reinterpret_cast<const half8*>(arow + 32 * s + 16 * h);
          // KB = 64: accumulators start at the fp32 256 ||c||^2 of the lane's rows
          // 8 i + 4 h + 0..3, held in the norm slot of row 8 i + 4 h.  KB = 16, 32: they
          // start at 0 and the norm step multiplies the row's norm slot by 1 (lanes 32-63
          // read the same finite slots against a zero B: no contribution)
          f32x16 seed;
          half8 An;
          if constexpr (KB == 64) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
              const float4 sv =
                  *reinterpret_cast<const float4*>(cur + tt * TILEB + (8 * i + 4 * h) * ROWB + 2 * KB);
              seed[4 * i] = sv.x;
              seed[4 * i + 1] = sv.y;
              seed[4 * i + 2] = sv.z;
              seed[4 * i + 3] = sv.w;
            }
          } else {
            An = *reinterpret_cast<const half8*>(arow + 2 * KB);
          }
          // the tile index in a vector register (one move per tile): the tag's and-or may
          // read only one scalar operand, which the mask takes
          uint32_t tv = (uint32_t)(ch * CT + tt);
          __asm__ volatile("" : "+v"(tv));
#pragma unroll
          for (int j = 0; j < CBP; j++) {
            const int b = pb + j;
            f32x16 acc;
            if constexpr (KB == 64) {
              acc = seed;
            } else {
#pragma unroll
              for (int e = 0; e < 16; e++) acc[e] = 0.f;
              acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(An, bnorm, acc, 0, 0, 0);
            }
#pragma unroll
            for (int s = 0; s < KS; s++)
              acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[s], __builtin_bit_cast(half8, bq[KS * b + s]), acc, 0,
                                                            0, 0);
            const float tm = __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, min16(acc)) & tmask) | tv);
            const bool c1 = tm < m1[j];
            m3[j] = __builtin_amdgcn_fmed3f(m2[j], m3[j], tm);
            m2[j] = __builtin_amdgcn_fmed3f(m1[j], m2[j], tm);
            m1[j] = fminf(m1[j], tm);
            // k = d (128 tiles and more): after the first tiles most tiles improve no lane, so
            // the copy is skipped wave-wide when none does (the smaller codebooks of k = 16 / 32
            // improve some lane at nearly every tile: there the test only costs)
            if (KB != 64 || __ballot(c1)) {
#pragma unroll
              for (int e = 0; e < 16; e++) bestD[j][e] = c1 ? acc[e] : bestD[j][e];
            }
          }
        }
        __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0)
        __syncthreads();
      }

#pragma unroll
      for (int j = 0; j < CBP; j++) {
        const int b = pb + j;
        float r1 = __builtin_huge_valf(), r2 = __builtin_huge_valf();
        int ri = 0;
#pragma unroll
        for (int e = 0; e < 16; e++) {
          const float v = bestD[j][e];
          r2 = __builtin_amdgcn_fmed3f(r1, r2, v);
          ri = v < r1 ? e : ri;  // first (lowest row) minimum: rows grow with e
          r1 = fminf(r1, v);
        }
        const int tid = (int)(__builtin_bit_cast(uint32_t, m1[j]) & ~tmask);
        const int tid2 = (int)(__builtin_bit_cast(uint32_t, m2[j]) & ~tmask);  // read only when m2 is finite
        ri = 32 * tid + (ri >> 2) * 8 + 4 * h + (ri & 3);
        const float o1 = __shfl_xor(r1, 32), o2 = __shfl_xor(r2, 32), om = __shfl_xor(m2[j], 32);
        const int oi = __shfl_xor(ri, 32);
        const bool other = (o1 < r1) || (o1 == r1 && oi < ri);
        const float best = other ? o1 : r1;
        const float second = fminf(fminf(fmaxf(r1, o1), fminf(r2, o2)), fminf(m2[j], om));
        code[b] = (uint32_t)(other ? oi : ri);
        // second may be a tagged minimum: lowered by what its tag can have added
        sure[b] = (second - fabsf(second) * tag_rel - best) > 2.0f * E[b];
        // candidate tiles of an uncertified column, per half: the best tile always, the
        // second if its minimum may be within 2E of the best; a third that may be that
        // close sends the block to the full search (tagged minima lowered by their tags)
        const float lim = best + 2.0f * E[b];
        const bool near2 = m2[j] - fabsf(m2[j]) * tag_rel <= lim;
        cand[b] = (uint32_t)(tid & 0xffff) | ((uint32_t)(near2 ? (tid2 & 0x7fff) | 0x8000 : 0) << 16);
        far3[b] = m3[j] - fabsf(m3[j]) * tag_rel > lim;
      }
    }

    const int words = CB * bits;  // 32 x CB codes x bits
    for (int i = lane; i < words; i += 64) spk[i] = 0u;
    wave_lds_sync();
    if (h == 0 && valid) {
#pragma unroll
      for (int b = 0; b < CB; b++) {
        if (sure[b]) {
          const int bo = (c * CB + b) * bits, sh = bo & 31;
          atomicOr(&spk[bo >> 5], code[b] << sh);
          if (sh + bits > 32) atomicOr(&spk[(bo >> 5) + 1], code[b] >> (32 - sh));
        }
      }
    }
    // ---- 5. uncertified blocks: the owner lists them; after a barrier every wave takes
    //      list entries (the exact y of a vector costs a chain of dependent loads, so one
    //      wave per entry; the list holds every column of a round).  A block whose
    //      candidates lie in its listed tiles is scored over those rows; any other goes
    //      to the workgroup's fp64 queue (or, past QMAX entries, is searched by the wave
    //      alone).  Codes go to the owner's packing words.
    auto research = [&](int ow, int cc, int bb, bool few, uint32_t cd0, uint32_t cd1) {
      uint32_t* ospk = reinterpret_cast<uint32_t*>(buf0 + 2 * CHUNKB) + ow * SCR_DW + 256;
      auto put = [&](uint32_t cv) {
        const int bo = (cc * CB + bb) * bits, sh = bo & 31;
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
      ys[lane] = yt;
      wave_lds_sync();
      const double* yb = ys + KB * bb;  // the block's coordinates
      if (few) {
        // lane L scores row L % 16 of candidate (tile, half) L / 16: the best and second
        // tiles of half 0 (lanes 0-31) and of half 1 (lanes 32-63)
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
          constexpr int NQ = KB / 8;  // 16-byte pieces of the row's coordinates
          for (int q0 = 0; q0 < NQ; q0 += 2) {
            uint4 rw[2];
#pragma unroll
            for (int q = 0; q < 2; q++) rw[q] = rowp[q0 + q];
#pragma unroll
            for (int q = 0; q < 2; q++) {
              const uint32_t ww[4] = {rw[q].x, rw[q].y, rw[q].z, rw[q].w};
#pragma unroll
              for (int i = 0; i < 4; i++) {
                const double d0 = yb[8 * (q0 + q) + 2 * i] - (double)h_lo(ww[i]);
                const double d1 = yb[8 * (q0 + q) + 2 * i + 1] - (double)h_hi(ww[i]);
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
        if (lane < KB) qy[slot * 64 + lane] = yb[lane];
        if (lane == 0) qown[slot] = (bb << 16) | (ow << 8) | cc;
        return;
      }
      double bd = __builtin_huge_val();
      int bn = 0x7fffffff;
      for (int nn = lane; nn < N; nn += 64) {
        const float* cp = cw + (size_t)nn * KB;
        double dd = 0.0;
        for (int t = 0; t < KB; t++) {
          const double df = yb[t] - (double)cp[t];
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
#pragma unroll
    for (int b = 0; b < CB; b++) {
      const bool far3_col = far3[b] && __shfl_xor((int)far3[b], 32);
      uint64_t todo = __ballot(h == 0 && valid && !sure[b]);
      while (todo) {
        const int cc = __builtin_ctzll(todo);
        todo &= todo - 1;
        const bool few = __shfl((int)far3_col, cc) != 0;  // every candidate in the listed tiles
        const uint32_t cd0 = (uint32_t)__shfl((int)cand[b], cc), cd1 = (uint32_t)__shfl((int)cand[b], cc + 32);
        if (lane == 0) {
          const int slot = atomicAdd(ucnt, 1);  // < UMAX: at most every column of the round
          ulist[3 * slot] = (uint32_t)((b << 17) | (few ? 0x10000 : 0) | (w << 8) | cc);
          ulist[3 * slot + 1] = cd0;
          ulist[3 * slot + 2] = cd1;
        }
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
        research((int)((ent >> 8) & 0xff), (int)(ent & 0xff), (int)(ent >> 17), (ent & 0x10000) != 0, cd0, cd1);
      }
    }
    __syncthreads();  // the queue is complete
    const int nq0 = *qcnt;  // the queue is complete: the list's entries were processed above
    const int nq = __builtin_amdgcn_readfirstlane(nq0 < QMAX ? nq0 : QMAX);
    // Workgroup pass(es) over the codebook for the queued blocks, QB at a time: LPC lanes
    // per codeword, lane l of wave w scoring codeword PASS i + (64 / LPC) w + l / LPC over
    // coordinates 16 (l % LPC) .. + 15; the partial sums are added in a fixed order.
    constexpr int LPC = KB / 16;
    constexpr int PASS = WAVES * (64 / LPC);  // codewords per pass of the workgroup
    for (int e0 = 0; e0 < nq; e0 += QB) {
      const int ne = (nq - e0) < QB ? (nq - e0) : QB;
      double bd[QB];
      int bn[QB];
#pragma unroll
      for (int e = 0; e < QB; e++) {
        bd[e] = __builtin_huge_val();
        bn[e] = 0x7fffffff;
      }
      const int cl = (64 / LPC) * w + lane / LPC, q4 = lane % LPC;
      const int nit = (N + PASS - 1) / PASS;
      // codeword it * PASS + cl: its 16 coordinates of this lane straight from the fp16
      // records in global memory (LPC lanes read one row's coordinates), four rows in flight
      for (int it0 = 0; it0 < nit; it0 += 4) {
        uint4 rr4[4][2];
#pragma unroll
        for (int u = 0; u < 4; u++) {
          const int nn = (it0 + u) * PASS + cl;
          const int nc = nn < N ? nn : N - 1;
          const uint4* rowp = reinterpret_cast<const uint4*>(rec + (size_t)nc * ROWB + 32 * q4);
          rr4[u][0] = rowp[0];
          rr4[u][1] = rowp[1];
        }
#pragma unroll
        for (int u = 0; u < 4; u++) {
          const int nn = (it0 + u) * PASS + cl;
          const uint32_t cwv[8] = {rr4[u][0].x, rr4[u][0].y, rr4[u][0].z, rr4[u][0].w,
                                   rr4[u][1].x, rr4[u][1].y, rr4[u][1].z, rr4[u][1].w};
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
              double dd = pp;
              if constexpr (LPC >= 2) {
                const double p1 = shfl_xor_f64(pp, 1);
                dd = (q4 & 1) ? p1 + pp : pp + p1;  // (q0 + q1) [and (q2 + q3)]
              }
              if constexpr (LPC == 4) {
                const double p2 = shfl_xor_f64(dd, 2);
                dd = (q4 & 2) ? p2 + dd : dd + p2;  // (q0 + q1) + (q2 + q3)
              }
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
          for (int m = LPC; m <= 32; m <<= 1) {
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
        if (((own >> 8) & 0xff) == w && lane == 0) {
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
          const int bo = ((own & 0xff) * CB + (own >> 16)) * bits, sh = bo & 31;
          atomicOr(&spk[bo >> 5], cv << sh);
          if (sh + bits > 32) atomicOr(&spk[(bo >> 5) + 1], cv >> (32 - sh));
        }
      }
      __syncthreads();  // per-wave bests free again
    }
    wave_lds_sync();
    if (slots) {
      scatter_records(spk, nv, CB * bits / 8, slots, cap, v0, codes, lane);
    } else if (nv > 0) {
      const int nbytes = (nv * CB * bits + 7) / 8;
      uint8_t* dst = codes + g * (int64_t)(4 * CB * bits);  // group g starts at bit g * 32 * CB * bits
      const int nfull = nbytes / 4;
      for (int i = lane; i < nfull; i += 64) reinterpret_cast<uint32_t*>(dst)[i] = spk[i];
      const int rem = nbytes - 4 * nfull;
      if (lane < rem) dst[4 * nfull + lane] = (uint8_t)((spk[nfull] >> (8 * lane)) & 0xffu);
    }
    wave_lds_sync();
  }
}

template <int KB, bool NF16>
hipError_t launch_full(const fq_codebook* cb, const void* x, int64_t n, uint8_t* codes, void* norms,
                       const int64_t* slots, int64_t cap, hipStream_t s) {
  constexpr int WAVES = FullShape<KB>::WAVES;
  const auto kern = encode_full<KB, NF16>;
  const size_t lds = full_lds_bytes<KB>();
  hipError_t e = hipSuccess;
  if (lds > 65536)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  int64_t resident = 0;
  e = resident_workgroups(reinterpret_cast<const void*>(kern), WAVES * 64, lds, cb->device, &resident);
  if (e != hipSuccess) return e;
  const int64_t ngroups = (n + 31) / 32;
  int64_t wgs = (ngroups + WAVES - 1) / WAVES;
  if (wgs > resident) wgs = resident;
  hipLaunchKernelGGL(kern, dim3((unsigned)wgs), dim3(WAVES * 64), lds, s, reinterpret_cast<const _Float16*>(x), n,
                     ngroups, reinterpret_cast<const uint4*>(cb->rot32), reinterpret_cast<const uint8_t*>(cb->frec),
                     cb->cw, cb->pi64t, cb->N, cb->bits, cb->full_eabs, cb->h16_erel, cb->cmax, cb->c2max, codes, norms,
                     slots, cap, (int)wgs);
  return hipGetLastError();
}

size_t full_lds_for(int k) {
  return k == 16 ? full_lds_bytes<16>() : k == 32 ? full_lds_bytes<32>() : full_lds_bytes<64>();
}

}  // namespace

bool encode_full_supported(const fq_codebook* cb) {
  return (cb->k == 16 || cb->k == 32 || cb->k == D) && cb->rot32 && cb->frec && cb->N % 32 == 0 && cb->N >= 32 &&
         cb->bits <= 16 && full_lds_for(cb->k) <= cb->max_lds;
}

hipError_t launch_encode_full(const fq_codebook* cb, const void* x, int64_t n, uint8_t* codes, void* norms,
                              fq_dtype norm_dtype, const int64_t* slots, int64_t cap, hipStream_t s) {
  if (!encode_full_supported(cb)) return hipErrorNotSupported;
  const bool nf = norm_dtype == FQ_F16;
  switch (cb->k) {
    case 16:
      return nf ? launch_full<16, true>(cb, x, n, codes, norms, slots, cap, s)
                : launch_full<16, false>(cb, x, n, codes, norms, slots, cap, s);
    case 32:
      return nf ? launch_full<32, true>(cb, x, n, codes, norms, slots, cap, s)
                : launch_full<32, false>(cb, x, n, codes, norms, slots, cap, s);
    default:
      return nf ? launch_full<D, true>(cb, x, n, codes, norms, slots, cap, s)
                : launch_full<D, false>(cb, x, n, codes, norms, slots, cap, s);
  }
}

}  // namespace fq
