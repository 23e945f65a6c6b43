// Matrix-core FibQuant encoder for fp16 input and block sizes k = 4 and 8
// (FibQuant summary §2.3: norm, Haar rotation of the unit vector, d/k blocks of
// k consecutive coordinates, nearest codeword; §1: fixed-address codes).
//
// A wave owns a "group" of 256 blocks (16 vectors for k = 4, 32 for k = 8) at a
// time; the workgroup keeps the codebook and the rotation operands in LDS.
//
//  1. Each lane loads 16 of the 64 inputs of one vector straight into the
//     B operand of mfma_f32_16x16x32_f16 (lane l: vector l % 16, inputs
//     32 s + 8 (l / 16) .. + 7); nu is summed in fp64 from those registers.
//  2. Rotation on the fp16 matrix core: 1024 Pi is split exactly enough into
//     fp16 hi + mid + lo (33 bits), x is fp16, so every product is exact; the
//     hi products and the mid / lo products are accumulated in fp32 separately.
//     The rows of Pi are permuted so that lane l ends up holding coordinates
//     16 (l / 16) .. + 15 of its vector: 4 whole blocks (k = 4) or 2 (k = 8).
//  3. Scores 256 (||c||^2 - 2 y.c) for 32 codewords x 32 blocks per
//     mfma_f32_32x32x16_f16: A = codeword record (fp16-exact), B = -512 y split
//     into fp16 hi (lanes 0-31) + lo (lanes 32-63).  For k = 4 the record also
//     carries 256 ||c||^2 as fp16 hi + lo in K slots the block does not use (B
//     holds 1 there), so the accumulator starts at 0; for k = 8 it starts at
//     256 ||c||^2 read from LDS.  A lane takes the minimum of its 16 rows
//     (v_min3 chains), writes the tile index into its low mantissa bits (one
//     and-or) and keeps the best and second-best such tagged minimum (so the
//     best one names its tile); the next tile's matrix op is issued before this
//     one is reduced.
//  4. Recovery: per column, the half whose tile minimum won recomputes that
//     tile's 16 rows in fp32 FMAs from the fp32 256 ||c||^2 (lane c takes
//     column c of one tile of a pair, lane c + 32 the other tile's); the second
//     best is the least of the recomputed runner-up, the winning half's other
//     tiles and the other half's minimum.  The recomputed scores carry their row
//     in the low 4 mantissa bits (one and-or per row instead of a compare and a
//     select), so the best one names its row.
//  5. Certificate: every computed score is within
//        E = 1.01 ((2k+7) u (256 c2max + 512 cmax |y_b|) + 19456 sqrt(k) cmax u
//                  + 2^-25 (1 + sqrt(k) cmax)),   u = 2^-24,
//     of the exact scaled score: (2k+3) roundings of the matrix / FMA sums, the
//     fp16 lo parts of -512 y and of 256 ||c||^2 (2^-22 relative, 2^-25 absolute
//     when subnormal), and the rotation: each coordinate of y is within 38 u of
//     Pi x / nu (the hi products of each K-step summed apart, at most 33
//     roundings each over its share of |Pi_t| |x| <= nu, one to add the two,
//     then the add of the mid / lo sums, 1 / nu and the product; the mid / lo
//     sums are 2^-11 smaller, and one u of slack), which moves a score by at most
//     512 |c| sqrt(k) 38 u.  (With one chain of 64 products it was 70 u; the
//     certificate's width is mostly this term, and the blocks it leaves to the
//     re-search fell with it.)  The host folds E into
//     e_abs + e_rel |y_b| (with 1.02 for the fp32 evaluation here).  If
//     second - best > 2E the winner is the exact unique minimiser; "second"
//     is first lowered and "best" raised by what a tag can have moved them
//     (2^(tagbits - 23) of itself for a tile tag, tagbits = ceil(log2(N / 32)),
//     2^-19 for a row tag), and a tag that picked another tile or row than the
//     true best can only do so within that amount, which the adjusted test then
//     fails.
//  6. Uncertified blocks are listed in LDS and searched again, one at a time by
//     the whole wave, in fp64 with the direct distance sum_t (y_t - c_t)^2
//     (lowest index on exact ties), after an fp32 screen that leaves (nearly
//     always) one fp64 candidate per lane.
//  7. Codes are assembled in LDS and written as whole dwords.
// k = 4 codebooks too large for LDS (beyond 2048 words) are streamed instead (ST): the workgroup's waves take one group each per round and
// the codebook passes through two LDS buffers of CN codewords, loaded straight
// from global memory while the previous chunk is searched; recovery and the
// re-search read their few codewords from global memory.
#include "fq_device.h"
#include "fq_internal.h"

namespace fq {
namespace {

constexpr int D = kD;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int K>
struct Shape;
template <>
struct Shape<4> {
  static constexpr int WAVES = 8;  // 2 workgroups of 8 waves per CU
  static constexpr int NSUB = 1;   // 16-vector rotation sub-groups per group
  static constexpr int OCC = 4;    // waves per SIMD the register budget is set for (128 registers)
};
template <>
struct Shape<8> {
  static constexpr int WAVES = 16;  // the 4096-word codebook fills most of the LDS
  static constexpr int NSUB = 2;
  static constexpr int OCC = 4;
};

constexpr int ROT_OPS = 2 * 4 * 3 * 64;  // [k step][row tile][piece][lane] half8 operands
constexpr int SPK_WORDS = 128;           // 256 codes x 16 bits
// + 256 uint16 entries of uncertified blocks, 32 fp64 inverse norms, fp64 y of a re-searched block
constexpr int WAVE_WORDS = SPK_WORDS + 128 + 64 + 16;

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

// Bytes of dynamic LDS the kernel needs: rotation operands, codeword records,
// 256 ||c||^2 (k = 8), and per wave the code-packing words and the list of
// uncertified blocks.
// Record n sits at slot n + n / 32 and 256 ||c_n||^2 at n + 4 (n / 32): without the
// padding every tile maps to the same LDS banks, and the recovery's per-lane reads
// (each lane in its own best tile) would all collide.
__host__ __device__ constexpr size_t h16_lds_bytes(int K, int N, int waves) {
  return (size_t)ROT_OPS * 16 + (size_t)(N + N / 32) * 16 + (size_t)(N + N / 8) * 4 + (size_t)waves * WAVE_WORDS * 4;
}
constexpr int CN = 1024;  // codewords per streamed chunk
__host__ __device__ constexpr size_t h16s_lds_bytes(int waves) {
  return (size_t)ROT_OPS * 16 + (size_t)2 * CN * 16 + (size_t)2 * CN * 4 + (size_t)waves * WAVE_WORDS * 4;
}
__device__ inline int rslot(int n) { return n + (n >> 5); }
__device__ inline int cslot(int n) { return n + 4 * (n >> 5); }

// SC: records and norms go to the slots given per vector (an instantiation of its own,
// so the contiguous kernel keeps its register allocation).
template <int K, bool NF16, bool SC, bool ST>
__global__ __launch_bounds__(Shape<K>::WAVES * 64, Shape<K>::OCC) void encode_h16(
    const _Float16* __restrict__ x, int64_t n, int64_t ngroups, const uint4* __restrict__ rot16,
    const uint4* __restrict__ crec, const float* __restrict__ cn2s, const double* __restrict__ pi64, int N,
    int bits, float e_abs, float e_rel, float c2max, float cmax, uint8_t* __restrict__ codes,
    void* __restrict__ norms, const int64_t* __restrict__ slots, int64_t cap, int nwg) {
  constexpr int WAVES = Shape<K>::WAVES;
  constexpr int NSUB = Shape<K>::NSUB;
  constexpr int VG = 16 * NSUB;    // vectors per group
  constexpr int DW = K / 2;        // dwords of fp16 hi (or lo) per block
  constexpr int SLOTS = 4 / NSUB;  // block slots a lane fills per sub-group
  extern __shared__ uint4 smem[];
  uint4* rotL = smem;
  uint4* recL = smem + ROT_OPS;  // ST: two chunk buffers of CN records (unpadded)
  float* c2L = reinterpret_cast<float*>(recL + (ST ? 2 * CN : N + N / 32));  // ST: two of CN floats
  const int w = __builtin_amdgcn_readfirstlane((int)(fq_tid() >> 6));
  uint32_t* spk = reinterpret_cast<uint32_t*>(c2L + (ST ? 2 * CN : N + N / 8)) + w * WAVE_WORDS;
  uint16_t* todoL = reinterpret_cast<uint16_t*>(spk + SPK_WORDS);
  double* invL = reinterpret_cast<double*>(spk + SPK_WORDS + 128);  // [VG] 1 / nu (0 for nu = 0)
  double* ysL = invL + 32;                                           // [K] y of a re-searched block
  for (int i = fq_tid(); i < ROT_OPS; i += WAVES * 64) rotL[i] = rot16[i];
  if constexpr (!ST) {
    for (int i = fq_tid(); i < N; i += WAVES * 64) {
      recL[rslot(i)] = crec[i];
      c2L[cslot(i)] = cn2s[i];
    }
  }
  __syncthreads();

  const int lane = fq_tid() & 63;
  const int c = lane & 31, h = lane >> 5, q = lane >> 4, vl = lane & 15;
  const int NT = N / 32;
  // tile tags: the low tagbits bits of a tile minimum hold its tile index, which moves the
  // value by less than 2^(tagbits - 23) of itself (1 % slack)
  const int tagbits = NT > 1 ? 32 - __builtin_clz((unsigned)(NT - 1)) : 0;
  const uint32_t tmask = ~((1u << tagbits) - 1u);
  const float tag_rel = (float)(1u << tagbits) * (1.01f / 8388608.0f);
  const float row_rel = 16.0f * (1.01f / 8388608.0f);  // the recovery's row tags (4 bits)
  const float sec_rel = tag_rel > row_rel ? tag_rel : row_rel;
  // codeword n as 8 halves: in LDS at slot rslot(n), or (ST) in global memory
  const _Float16* cbh = ST ? reinterpret_cast<const _Float16*>(crec) : reinterpret_cast<const _Float16*>(recL);
  auto rec_of = [&](int nn) { return ST ? nn : rslot(nn); };

  // ST: rounds are uniform across the workgroup (every wave meets every barrier); a
  // wave past the last group searches zero inputs and stores nothing
  // Progress-based wave priority: a SIMD's arbiter favours its oldest waves, so without
  // this the youngest waves of the persistent grid lagged and finished their last groups
  // alone at low occupancy; a wave lowers its priority as it gets through its groups.
  const int64_t gstep = (int64_t)nwg * WAVES, gfirst = (int64_t)fq_bid_x() * WAVES;
  const int64_t gtotal = gfirst < ngroups ? (ngroups - gfirst + gstep - 1) / gstep : 1;
  for (int64_t gb = gfirst; gb < ngroups; gb += gstep) {
    const int64_t g = gb + w;
    {
      const int lvl = (int)((4 * ((gb - gfirst) / gstep)) / gtotal);
      if (lvl == 0)
        __builtin_amdgcn_s_setprio(3);
      else if (lvl == 1)
        __builtin_amdgcn_s_setprio(2);
      else if (lvl == 2)
        __builtin_amdgcn_s_setprio(1);
      else
        __builtin_amdgcn_s_setprio(0);
    }
    // (a signed 64-bit compare has no scalar form: as one, ngroups would be held, and
    // spilled, in vector registers)
    const int64_t left = ngroups - g;
    if (!ST && ((int)(left >> 32) < 0 || left == 0)) break;
    const int64_t v0 = g * VG;
    const int nv = g < ngroups ? (int)((n - v0) < VG ? (n - v0) : VG) : 0;

    // ---- 1-3 per 16-vector sub-group: x, nu, rotation, B operands
    // bq[2 sigma + hp]: B operand of the tile whose column c is block slot sigma of lane c + 32 hp.
    uint32_t bq[8][4];
#pragma unroll
    for (int sg = 0; sg < NSUB; sg++) {
      const int vec = 16 * sg + vl;
      uint4 xa = make_uint4(0u, 0u, 0u, 0u), xb = xa;
      if (vec < nv) {
        // a uniform group base plus a 32-bit lane offset the compiler cannot carry from
        // one group to the next (a per-lane 64-bit pointer, or the offset itself, would
        // live across the search)
        int ln = lane;
        __asm__ volatile("" : "+v"(ln));
        const int off = (16 * sg + (ln & 15)) * (D / 8) + (ln >> 4);
        const uint4* xp = reinterpret_cast<const uint4*>(x + v0 * D);
        xa = xp[off];
        xb = xp[off + 4];
      }
      double s = 0.0;
      {
        const uint32_t wv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
        for (int t = 0; t < 8; t++) {
          const double a = (double)h_lo(wv[t]), b = (double)h_hi(wv[t]);
          s = fma(a, a, s);
          s = fma(b, b, s);
        }
      }
      s += shfl_xor_f64(s, 16);
      s += shfl_xor_f64(s, 32);
      const double nu = sqrt(s);
      if (q == 0 && vec < nv) {
        const int64_t sv = SC ? out_slot(slots, cap, v0 + vec) : v0 + vec;
        if (sv >= 0) {
          if constexpr (NF16)
            reinterpret_cast<uint16_t*>(norms)[sv] = f64_to_f16_bits(nu);
          else
            reinterpret_cast<float*>(norms)[sv] = (float)nu;
        }
      }
      const float inv = nu > 0.0 ? (float)(1.0 / (1024.0 * nu)) : 0.0f;
      if (q == 0) invL[vec] = nu > 0.0 ? 1.0 / nu : 0.0;  // for the fp64 re-search

      // hi products of the two K-steps summed separately and added once: each sum of 32
      // products carries at most 33 roundings over its own |terms| (64 + 2 with one chain)
      f32x4 ah[4], am[4];
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const uint4* op0 = rotL + (r * 3) * 64 + lane;
        const uint4* op1 = rotL + ((4 + r) * 3) * 64 + lane;
        const half8 xv0 = __builtin_bit_cast(half8, xa), xv1 = __builtin_bit_cast(half8, xb);
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        const f32x4 h0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, op0[0]), xv0, z, 0, 0, 0);
        const f32x4 h1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, op1[0]), xv1, z, 0, 0, 0);
        ah[r] = h0 + h1;
        f32x4 m = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, op0[64]), xv0, z, 0, 0, 0);
        m = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, op0[128]), xv0, m, 0, 0, 0);
        m = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, op1[64]), xv1, m, 0, 0, 0);
        am[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, op1[128]), xv1, m, 0, 0, 0);
      }
      // v = -512 y for coordinates 16 q + 4 r + i; hi / lo fp16 parts packed two per dword.
      uint32_t hi[8], lo[8];
#pragma unroll
      for (int r = 0; r < 4; r++)
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const float va = -512.0f * ((ah[r][i] + am[r][i]) * inv);
          const float vb = -512.0f * ((ah[r][i + 1] + am[r][i + 1]) * inv);
          const float ha = (float)(_Float16)va, hb = (float)(_Float16)vb;
          hi[2 * r + i / 2] = pack_h2(ha, hb);
          lo[2 * r + i / 2] = pack_h2(va - ha, vb - hb);
        }
      // Block slots of this sub-group: k = 4: slot r = coordinates 16 q + 4 r ..;
      // k = 8: slot 2 sg + s = coordinates 16 q + 8 s ...
#pragma unroll
      for (int sl = 0; sl < SLOTS; sl++) {
        const int sigma = sg * SLOTS + sl;
        uint32_t recv[DW];
#pragma unroll
        for (int d = 0; d < DW; d++) {
          const uint32_t send = h == 0 ? lo[sl * DW + d] : hi[sl * DW + d];
          recv[d] = (uint32_t)__shfl_xor((int)send, 32);
        }
#pragma unroll
        for (int d = 0; d < DW; d++) {
          bq[2 * sigma][d] = h == 0 ? hi[sl * DW + d] : recv[d];
          bq[2 * sigma + 1][d] = h == 0 ? recv[d] : lo[sl * DW + d];
        }
        if constexpr (K == 4) {
          bq[2 * sigma][2] = bq[2 * sigma + 1][2] = h == 0 ? 0x3c003c00u : 0u;  // 1.0, 1.0 against 256 ||c||^2
          bq[2 * sigma][3] = bq[2 * sigma + 1][3] = 0u;
        }
      }
    }

    // The operands are opaque from here on: otherwise the compiler folds the
    // recovery's selects through the ones above and keeps hi / lo alive as well.
#pragma unroll
    for (int tb = 0; tb < 8; tb++)
#pragma unroll
      for (int d = 0; d < 4; d++) __asm__ volatile("" : "+v"(bq[tb][d]));

    // ---- 3b. matrix-core search with per-lane tile minima.  A tile minimum carries its
    //      tile index in its low tagbits mantissa bits (one and-or instead of a compare and
    //      a select per tile and column); the certificate allows for the change of value.
    float m1[8], m2[8];
#pragma unroll
    for (int tb = 0; tb < 8; tb++) {
      m1[tb] = __builtin_huge_valf();
      m2[tb] = __builtin_huge_valf();
    }
    // tile t of the codebook; `tiles` tiles of `buf` (LDS, padded unless ST), first tile t0
    int lh = lane;  // the lane's half for the norm seeds' LDS base, formed per group
    __asm__ volatile("" : "+v"(lh));
    lh >>= 5;
    auto search = [&](const uint4* buf, const float* c2b, int tiles, int t0) {
      const int RS = ST ? 32 : 33, CS = ST ? 32 : 36;  // record / norm slots per tile
      half8 A = __builtin_bit_cast(half8, buf[c]);
      for (int tl = 0; tl < tiles; tl++) {
        const int t = t0 + tl;
        // the tile index in a vector register (one move per tile): the tag's and-or may
        // read only one scalar operand, which the mask takes
        uint32_t tv = (uint32_t)t;
        __asm__ volatile("" : "+v"(tv));
        const half8 An = __builtin_bit_cast(half8, buf[(tl + 1 < tiles ? RS * (tl + 1) : 0) + c]);
        f32x16 C;
        if constexpr (K == 8) {
#pragma unroll
          for (int j = 0; j < 4; j++) {
            const float4 cv = *reinterpret_cast<const float4*>(c2b + CS * tl + 8 * j + 4 * lh);
            C[4 * j] = cv.x;
            C[4 * j + 1] = cv.y;
            C[4 * j + 2] = cv.z;
            C[4 * j + 3] = cv.w;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 16; e++) C[e] = 0.f;
        }
        f32x16 Dc = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, __builtin_bit_cast(half8, bq[0]), C, 0, 0, 0);
#pragma unroll
        for (int tb = 0; tb < 8; tb++) {
          f32x16 Dn;
          if (tb < 7) Dn = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, __builtin_bit_cast(half8, bq[tb + 1]), C, 0, 0, 0);
          const float tm = __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, min16(Dc)) & tmask) | tv);
          m2[tb] = __builtin_amdgcn_fmed3f(m1[tb], m2[tb], tm);
          m1[tb] = fminf(m1[tb], tm);
          if (tb < 7) Dc = Dn;
        }
        A = An;
      }
    };
    if constexpr (!ST) {
      search(recL, c2L, NT, 0);
    } else {
      // chunk ch in buffer ch & 1: CN records (16 KiB, 1 KiB per wave-wide load) and,
      // for k = 8, CN norms (4 KiB)
      auto stage = [&](int ch) {
        const char* src = reinterpret_cast<const char*>(crec + (size_t)ch * CN);
        char* dst = reinterpret_cast<char*>(recL + (ch & 1) * CN);
        for (int pc = w; pc < CN * 16 / 1024; pc += WAVES) lds_dma16(src + pc * 1024 + lane * 16, dst + pc * 1024);
        if constexpr (K == 8) {
          const char* s2 = reinterpret_cast<const char*>(cn2s + (size_t)ch * CN);
          char* d2 = reinterpret_cast<char*>(c2L + (ch & 1) * CN);
          for (int pc = w; pc < CN * 4 / 1024; pc += WAVES) lds_dma16(s2 + pc * 1024 + lane * 16, d2 + pc * 1024);
        }
      };
      const int nchunk = N / CN;
      stage(0);
      __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): this wave's pieces of chunk 0 are in LDS
      __syncthreads();
      for (int ch = 0; ch < nchunk; ch++) {
        if (ch + 1 < nchunk) stage(ch + 1);
        search(recL + (ch & 1) * CN, c2L + (ch & 1) * CN, CN / 32, ch * (CN / 32));
        __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): the next chunk's pieces of this wave
        __syncthreads();                      // every wave is done with this chunk
      }
    }

    // ---- 4-5. recovery and certificate; uncertified blocks go to a list.  Each
    //      column needs one recompute, of the half whose tile minimum won: lane c
    //      takes column c of tile 2p, lane c + 32 column c of tile 2p + 1.
    uint32_t code[4];  // code | block index << 16, or ~0 when there is nothing to pack from this lane
    int ntodo = 0;
#pragma unroll
    for (int p = 0; p < 4; p++) {
      const int tb = 2 * p + h;  // this lane's tile: slot sigma = p, partner offset hp = h
      // statistics of this tile from both halves (the partner sends those of the tile it takes)
      const float mm1 = h == 0 ? m1[2 * p] : m1[2 * p + 1];
      const float mm2 = h == 0 ? m2[2 * p] : m2[2 * p + 1];
      const float pm1 = __shfl_xor(h == 0 ? m1[2 * p + 1] : m1[2 * p], 32);
      const float pm2 = __shfl_xor(h == 0 ? m2[2 * p + 1] : m2[2 * p], 32);
      const bool win = (mm1 < pm1) || (mm1 == pm1 && h == 0);
      const int hw = win ? h : 1 - h;       // half (rows 4 hw + ..) holding the tile minimum
      const int t0 = (int)(__builtin_bit_cast(uint32_t, win ? mm1 : pm1) & ~tmask);  // its tile (the tag)
      const float m2w = win ? mm2 : pm2;    // its other tiles' minimum
      const float m1l = win ? pm1 : mm1;    // minimum over the other half's rows
      // hi and lo of this column's block: this lane's operand half plus the partner's
      float vp[K];
      {
        uint32_t mine[DW], X[DW];
#pragma unroll
        for (int d = 0; d < DW; d++) {
          mine[d] = h == 0 ? bq[2 * p][d] : bq[2 * p + 1][d];
          X[d] = (uint32_t)__shfl_xor((int)(h == 0 ? bq[2 * p + 1][d] : bq[2 * p][d]), 32);
        }
#pragma unroll
        for (int d = 0; d < DW; d++) {
          const uint32_t hw_ = h == 0 ? mine[d] : X[d];
          const uint32_t lw_ = h == 0 ? X[d] : mine[d];
          vp[2 * d] = h_lo(hw_) + h_lo(lw_);  // exact: the value the matrix core multiplied
          vp[2 * d + 1] = h_hi(hw_) + h_hi(lw_);
        }
      }
      float vn2 = 0.f;
#pragma unroll
      for (int i = 0; i < K; i++) vn2 = fmaf(vp[i], vp[i], vn2);
      // best and second row scores, each tagged with its row (4 qq + e) in the low 4
      // mantissa bits (one and-or instead of a compare and a select per row)
      float r1 = __builtin_huge_valf(), r2 = __builtin_huge_valf();
#pragma unroll
      for (int qq = 0; qq < 4; qq++) {
        const int n0 = 32 * t0 + 8 * qq + 4 * hw;  // rows n0 .. n0 + 3 of the winning half
        const float4 c2v = ST ? *reinterpret_cast<const float4*>(cn2s + n0)   // fp32 256 ||c||^2
                              : *reinterpret_cast<const float4*>(c2L + cslot(n0));
        const float c2a[4] = {c2v.x, c2v.y, c2v.z, c2v.w};
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const uint4 rw = ST ? crec[n0 + e] : recL[rslot(n0 + e)];
          const uint32_t ww[4] = {rw.x, rw.y, rw.z, rw.w};
          float sc = c2a[e];
          // the fp32 operand first: with the fp16 one first the code generator puts a wait
          // state between every two mixed-precision FMAs of the chain
#pragma unroll
          for (int i = 0; i < K; i += 2) {
            sc = fmaf(vp[i], h_lo(ww[i / 2]), sc);
            sc = fmaf(vp[i + 1], h_hi(ww[i / 2]), sc);
          }
          const float st = __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, sc) & ~15u) | (uint32_t)(4 * qq + e));
          r2 = __builtin_amdgcn_fmed3f(r1, r2, st);
          r1 = fminf(r1, st);
        }
      }
      const int ri = (int)(__builtin_bit_cast(uint32_t, r1) & 15u);  // row 8 (ri / 4) + 4 hw + ri % 4
      const uint32_t cbest = (uint32_t)(32 * t0 + 8 * (ri >> 2) + 4 * hw + (ri & 3));
      const float second = fminf(r2, fminf(m2w, m1l));
      // block of this column: slot p of lane o = c + 32 h (formed per group from an opaque
      // value: hoisted out of the group loop these constants would be spilled)
      int o = lane;
      __asm__ volatile("" : "+v"(o));
      const int vec = K == 4 ? (o & 15) : 16 * (p >> 1) + (o & 15);
      const int bi = K == 4 ? 4 * (o >> 4) + p : 2 * (o >> 4) + (p & 1);
      const float yn = __builtin_sqrtf(vn2) * (1.01f / 512.0f);
      // second is a tagged tile minimum or row score and r1 a tagged row score: a tag moved
      // each by at most sec_rel (row tags: 2^-19) of itself
      const bool sure = (second - fabsf(second) * sec_rel - (r1 + fabsf(r1) * row_rel)) > 2.0f * (e_abs + e_rel * yn);
      const bool mine_ = vec < nv;
      code[p] = (mine_ && sure) ? (cbest | ((uint32_t)(vec * (D / K) + bi) << 16)) : ~0u;
      const uint64_t um = __ballot(mine_ && !sure);
      if (um) {
        if (mine_ && !sure) {
          const int pos = ntodo + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(um >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)um, 0u));
          todoL[pos] = (uint16_t)((tb << 8) | c);
        }
        ntodo += __builtin_popcountll(um);
      }
    }

    // ---- 6-7. pack the certified codes, search the listed blocks again in fp64, store
    const int words = 8 * bits;
    {
      int li = lane;  // opaque: the lane's packing-word address is formed per group, not carried
      __asm__ volatile("" : "+v"(li));
      for (int i = li; i < words; i += 64) spk[i] = 0u;
    }
    wave_lds_sync();
#pragma unroll
    for (int p = 0; p < 4; p++) {
      if (code[p] != ~0u) {
        const uint32_t cv = code[p] & 0xffffu;
        const int bo = (int)(code[p] >> 16) * bits, sh = bo & 31;
        atomicOr(&spk[bo >> 5], cv << sh);
        if (sh + bits > 32) atomicOr(&spk[(bo >> 5) + 1], cv >> (32 - sh));
      }
    }
    for (int it = 0; it < ntodo; it++) {
      const int ent = __builtin_amdgcn_readfirstlane((int)todoL[it]);
      const int tb = ent >> 8, cc = ent & 255;
      const int sigma = tb >> 1, hp = tb & 1;
      const int oc = cc + 32 * hp;
      const int fvec = K == 4 ? (oc & 15) : 16 * (sigma >> 1) + (oc & 15);
      const int fbi = K == 4 ? 4 * (oc >> 4) + sigma : 2 * (oc >> 4) + (sigma & 1);
      // exact y_b in fp64: D / K lanes per coordinate i of the block, each summing
      // K products of Pi[fbi K + i][j] x_j over its own K inputs j, then a butterfly
      // over those lanes; 1 / nu from the rotation phase (fp64)
      constexpr int LPO = D / K;
      // lane-derived offsets the compiler cannot see through: otherwise it keeps the
      // re-search's addresses (spilled) across the whole search loop
      int ln = lane;
      __asm__ volatile("" : "+v"(ln));
      const int oi = ln / LPO, qq = ln % LPO;
      double part = 0.0;
      {
        const _Float16* xr = x + (v0 + fvec) * D + K * qq;
        const double* pr = pi64 + (fbi * K + oi) * D + K * qq;
        _Float16 xh[K];
        if constexpr (K == 8) {
          const uint4 xv = *reinterpret_cast<const uint4*>(xr);
          __builtin_memcpy(xh, &xv, 16);
        } else {
          const uint2 xv = *reinterpret_cast<const uint2*>(xr);
          __builtin_memcpy(xh, &xv, 8);
        }
#pragma unroll
        for (int j = 0; j < K; j++) part = fma(pr[j], (double)xh[j], part);
      }
#pragma unroll
      for (int m = 1; m < LPO; m <<= 1) part += shfl_xor_f64(part, m);
      if (qq == 0) ysL[oi] = part * invL[fvec];
      wave_lds_sync();
      double yb[K];
#pragma unroll
      for (int i = 0; i < K; i++) yb[i] = ysL[i];
      // Large codebooks (16 or more codewords per lane) are screened in fp32 first
      // (for smaller ones the screen costs more than it saves), with the expanded score
      // s = 256 ||c||^2 - 512 y.c: the stored fp32 256 ||c||^2 plus one mixed-precision
      // FMA per coordinate (fp32 -512 y times the fp16 codeword).  Every screened s is
      // within e = (k + 2) u (256 c2max + 512 cmax |y_b|) of the exact s of the fp64 y
      // (the rounding of y to fp32, of ||c||^2 to fp32, and of each of the k FMAs, whose
      // partial sums stay below 256 c2max + 512 cmax |y_b|), and s is 256 (d - |y_b|^2)
      // for the distance d, so the fp64 minimiser and all its ties lie within 2 e of the
      // smallest screened s (plus the fp64 rounding of the distances, far below the
      // absolute 1e-12).  When no lane holds two such candidates, each lane scores its
      // one candidate in fp64; otherwise every codeword is scored in fp64.  The bound
      // carries 2 % of slack for its own fp32 evaluation.
      double bd = __builtin_huge_val();
      int bn = 0x7fffffff;
      bool full_scan = N < 1024;
      if (!full_scan) {
        float v[K];
        float yn2 = 0.f;
#pragma unroll
        for (int i = 0; i < K; i++) {
          const float yf = (float)yb[i];
          v[i] = -512.0f * yf;  // exact scaling
          yn2 = fmaf(yf, yf, yn2);
        }
        float f1 = __builtin_huge_valf(), f2 = __builtin_huge_valf();
        int fi = 0x7fffffff;
        // lane l scores codewords l + 64 r: their record and norm slots advance by a
        // constant per round (66 and 72 in the padded LDS layout); the lane keeps the round
        // of its minimum (a scalar), its codeword is formed after the loop
        auto screen = [&](const uint4* rp, float c2, int tag) {
          const uint32_t ww[4] = {rp->x, rp->y, rp->z, rp->w};
          float sf = c2;
#pragma unroll
          for (int i = 0; i < K; i += 2) {
            sf = fmaf(v[i], h_lo(ww[i / 2]), sf);
            sf = fmaf(v[i + 1], h_hi(ww[i / 2]), sf);
          }
          f2 = __builtin_amdgcn_fmed3f(f1, f2, sf);
          fi = sf < f1 ? tag : fi;
          f1 = fminf(f1, sf);
        };
        {
          const int RST = ST ? 64 : 66, CST = ST ? 64 : 72;
          const uint4* rp = reinterpret_cast<const uint4*>(cbh) + rec_of(lane);
          const float* cp = ST ? cn2s + lane : c2L + cslot(lane);
          // N is a power of two of at least 1024 here: whole rounds of 64
#pragma unroll 4
          for (int r = 0; r < (N >> 6); r++) screen(rp + RST * r, cp[CST * r], r);
          if (fi != 0x7fffffff) fi = 64 * fi + lane;
        }
        float mf = f1;
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) mf = fminf(mf, __shfl_xor(mf, m));
        const float tol = 2.0f * (1.02f * (float)(K + 2) * 5.9604645e-8f) *
                              (256.0f * c2max + 512.0f * cmax * (__builtin_sqrtf(yn2) * 1.0001f)) +
                          1e-12f;
        const bool cand = f1 <= mf + tol;
        full_scan = __ballot(cand && f2 <= mf + tol) != 0;
        if (!full_scan && cand) {
          double dd = 0.0;
#pragma unroll
          for (int i = 0; i < K; i++) {
            const double df = yb[i] - (double)cbh[8 * rec_of(fi) + i];
            dd = fma(df, df, dd);
          }
          bd = dd;
          bn = fi;
        }
      }
      if (full_scan) {
        for (int nn = lane; nn < N; nn += 64) {
          double dd = 0.0;
#pragma unroll
          for (int i = 0; i < K; i++) {
            const double df = yb[i] - (double)cbh[8 * rec_of(nn) + i];
            dd = fma(df, df, dd);
          }
          if (dd < bd) {
            bd = dd;
            bn = nn;
          }
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
      if (lane == 0) {
        const uint32_t cv = (uint32_t)bn;
        const int bo = (fvec * (D / K) + fbi) * bits, sh = bo & 31;
        atomicOr(&spk[bo >> 5], cv << sh);
        if (sh + bits > 32) atomicOr(&spk[(bo >> 5) + 1], cv >> (32 - sh));
      }
    }
    wave_lds_sync();
    if constexpr (SC) {
      scatter_records(spk, nv, (D / K) * bits / 8, slots, cap, v0, codes, lane);
    } else {
      const int64_t nbytes = ((int64_t)nv * (D / K) * bits + 7) / 8;
      uint8_t* dst = codes + g * (int64_t)(32 * bits);  // group g starts at bit g * 256 * bits
      const int nfull = (int)(nbytes / 4);
      int i0 = lane;  // opaque: no per-lane 64-bit store pointer carried across groups
      __asm__ volatile("" : "+v"(i0));
      for (int i = i0; i < nfull; i += 64) reinterpret_cast<uint32_t*>(dst)[i] = spk[i];
      const int rem = (int)(nbytes - 4 * (int64_t)nfull);
      if (lane < rem) dst[4 * nfull + lane] = (uint8_t)((spk[nfull] >> (8 * lane)) & 0xffu);
    }
    wave_lds_sync();
  }
}

template <int K, bool NF16, bool SC, bool ST>
hipError_t launch_h16(const fq_codebook* cb, const void* x, int64_t n, uint8_t* codes, void* norms,
                      const int64_t* slots, int64_t cap, hipStream_t s) {
  constexpr int WAVES = Shape<K>::WAVES;
  constexpr int VG = 16 * Shape<K>::NSUB;
  const auto kern = encode_h16<K, NF16, SC, ST>;
  const size_t lds = ST ? h16s_lds_bytes(WAVES) : h16_lds_bytes(K, cb->N, WAVES);
  hipError_t e = hipSuccess;
  if (lds > 65536)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  int64_t resident = 0;
  e = resident_workgroups(reinterpret_cast<const void*>(kern), WAVES * 64, lds, cb->device, &resident);
  if (e != hipSuccess) return e;
  const int64_t ngroups = (n + VG - 1) / VG;
  int64_t wgs = (ngroups + WAVES - 1) / WAVES;
  if (wgs > resident) wgs = resident;
  hipLaunchKernelGGL(kern, dim3((unsigned)wgs), dim3(WAVES * 64), lds, s, reinterpret_cast<const _Float16*>(x), n,
                     ngroups, reinterpret_cast<const uint4*>(cb->rot16), reinterpret_cast<const uint4*>(cb->crec),
                     cb->cn2s, cb->pi64, cb->N, cb->bits, cb->h16_eabs, cb->h16_erel, cb->c2max, cb->cmax, codes,
                     norms, slots, cap,
                     (int)wgs);
  return hipGetLastError();
}

// The whole codebook fits in LDS beside the rotation operands and the waves' scratch.
bool h16_in_lds(const fq_codebook* cb) {
  if (!((cb->k == 4 && cb->N <= 2048) || (cb->k == 8 && cb->N <= 4096))) return false;
  const int waves = cb->k == 4 ? Shape<4>::WAVES : Shape<8>::WAVES;
  return h16_lds_bytes(cb->k, cb->N, waves) <= cb->max_lds;
}

}  // namespace

bool encode_h16_supported(const fq_codebook* cb) {
  if (!cb->rot16 || !cb->crec || cb->N % 32 != 0 || cb->N < 32) return false;
  if (cb->k != 4 && cb->k != 8) return false;
  if (h16_in_lds(cb)) return true;
  // streamed: k = 4 only (the k = 8 search's registers leave no room for it)
  return cb->k == 4 && cb->N % CN == 0 && h16s_lds_bytes(Shape<4>::WAVES) <= cb->max_lds;
}

hipError_t launch_encode_h16(const fq_codebook* cb, const void* x, int64_t n, uint8_t* codes, void* norms,
                             fq_dtype norm_dtype, const int64_t* slots, int64_t cap, hipStream_t s) {
  if (!encode_h16_supported(cb)) return hipErrorNotSupported;
  const bool nf = norm_dtype == FQ_F16, st = !h16_in_lds(cb);
#define FQ_H16S(KK, NF, SCC) \
  (st ? launch_h16<KK, NF, SCC, true>(cb, x, n, codes, norms, slots, cap, s) \
      : launch_h16<KK, NF, SCC, false>(cb, x, n, codes, norms, slots, cap, s))
#define FQ_H16(KK, NF) (slots ? FQ_H16S(KK, NF, true) : FQ_H16S(KK, NF, false))
  if (cb->k == 4) return nf ? FQ_H16(4, true) : FQ_H16(4, false);
#define FQ_H16_8(NF) \
  (slots ? launch_h16<8, NF, true, false>(cb, x, n, codes, norms, slots, cap, s) \
         : launch_h16<8, NF, false, false>(cb, x, n, codes, norms, slots, cap, s))
  return nf ? FQ_H16_8(true) : FQ_H16_8(false);
#undef FQ_H16_8
#undef FQ_H16
#undef FQ_H16S
}

}  // namespace fq
