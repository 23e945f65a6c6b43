// Matrix-core FibQuant decoder (FibQuant summary §2.3: gather the codewords,
// concatenate the blocks, inverse rotation, scale by the norm; §1: every
// vector decodes alone from its fixed-address record).
//
// A wave decodes 32 vectors per step: x^T[64 x 32] = Pi^T[64 x 64] yhat^T[64 x 32]
// with mfma_f32_32x32x16_f16.  yhat holds fp16-exact codewords, so it is an
// exact fp16 operand; Pi^T is split into fp16 hi + lo (22 bits), accumulation
// is fp32.  Lane l owns vector l % 32 and, per 16-dim k-step, 8 consecutive
// input dims (whole codewords for k <= 8), which it gathers from the codebook
// (LDS copy when it fits, else the fp16 copy in global memory).
//
// Whole-word records (the stream decoder): one workgroup per CU holds the
// codebook in LDS and splits its waves into one producer and C consumers.  The
// producer only loads: the records and norms of the next rounds (a round = one
// 32-vector group per consumer) go into an LDS ring by direct global-to-LDS
// loads.  The consumers only compute and store: every consumer keeps the 16 Pi^T
// operands in registers, reads its group from the ring, and the result rows it
// holds (scattered over the 32 vectors) pass through a padded LDS tile and leave
// as 16-byte stores that cover 8 (fp16) or 4 (fp32) whole output vectors per
// instruction.  One workgroup barrier per round hands the ring over.  (A wave's
// loads and stores share one completion counter, so a wave that both loads and
// stores waits for its own older stores whenever it waits for a load: loops built
// that way sustained about 4.7 TB/s of mixed traffic on this part, against about
// 5.9 TB/s with the two roles in different waves.)
#include "fq_device.h"
#include "fq_internal.h"

namespace fq {
namespace {

constexpr int D = kD;
constexpr int WAVES = 4;
constexpr int LDS_CB_HALFS = 16384;  // codebooks up to N*k = 16384 (32 KiB) live in LDS
// The stream decoders also hold codebooks of up to 64 KiB (k = 8, N = 4096) in LDS, in
// one workgroup per CU (the producer / consumer decoder: 15 consumers for fp16 output,
// 8 for fp32, 156 / 151 KiB with the ring and staging tiles; the per-wave ring decoder:
// 12 or 8 waves, 136 / 146 KiB): gathered from L1 / L2 instead, every 16-byte codeword
// read fills a whole cache line, and that path ran at a third of the write bandwidth.
constexpr int LDS_CB_HALFS_BIG = 32768;
constexpr int LDS_MAX_BYTES = 160 * 1024;
constexpr int RING = 4;  // rounds in the LDS ring: one read by the consumers, up to three loading
constexpr int PF = 4;    // small launches: groups whose records are in flight ahead of the one decoded
constexpr int waves_ring(bool of16) { return of16 ? 12 : 8; }  // small launches, codebook of 64 KiB
constexpr int MIN_ROUNDS = 4;  // fewer rounds of the producer / consumer decoder: the per-wave ring decoder

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Output staging row of one vector: 64 values plus 4 of padding (bank spread).
template <bool OF16>
constexpr int stage_row_bytes() {
  return OF16 ? 68 * 2 : 68 * 4;
}

// `bits`-wide code starting at bit `bo` (a compile-time offset) of a record held
// in registers.
template <int RW>
__device__ inline uint32_t code_at(const uint32_t (&w)[RW], int bo, int bits) {
  const int wi = bo >> 5, sh = bo & 31;
  uint32_t v = w[wi] >> sh;
  if (sh + bits > 32 && wi + 1 < RW) v |= w[wi + 1] << (32 - sh);
  return v & ((1u << bits) - 1u);
}

// Input dims [d0, d0 + 8) from a codebook copy `cb` (LDS or global), for the
// codes of blocks d0 / K ... (K >= 8: one code; else 8 / K codes).
template <int K>
__device__ inline half8 gather_codes(const _Float16* __restrict__ cb, const uint32_t (&c)[8 / K > 0 ? 8 / K : 1],
                                     int d0) {
  half8 r;
  if constexpr (K >= 8) {
    r = *reinterpret_cast<const half8*>(cb + (size_t)c[0] * K + (d0 % K));
  } else if constexpr (K == 4) {
#pragma unroll
    for (int p = 0; p < 2; p++) {
      const half4 v = *reinterpret_cast<const half4*>(cb + (size_t)c[p] * 4);
#pragma unroll
      for (int t = 0; t < 4; t++) r[4 * p + t] = v[t];
    }
  } else {
#pragma unroll
    for (int p = 0; p < 8 / K; p++)
#pragma unroll
      for (int t = 0; t < K; t++) r[p * K + t] = cb[(size_t)c[p] * K + t];
  }
  return r;
}

// Scale the accumulators by the norm, pass them through the wave's padded staging
// tile and store the first `nv` of the 32 vectors: rows 8 q + 4 h + i of tile r
// are output dims 32 r + 8 q + 4 h + i of vector col, and each 16-byte store
// covers 8 (fp16) or 4 (fp32) consecutive whole output vectors.
template <bool OF16>
__device__ inline void stage_and_store(const f32x16 (&acc)[2], float nu, char* stage, int col, int h, int lane,
                                       char* out_g, int nv) {
  constexpr int ROWB = stage_row_bytes<OF16>();
#pragma unroll
  for (int r = 0; r < 2; r++)
#pragma unroll
    for (int qd = 0; qd < 4; qd++) {
      const int o = 32 * r + 8 * qd + 4 * h;
      if constexpr (OF16) {
        half4 hv;
#pragma unroll
        for (int i = 0; i < 4; i++) hv[i] = (_Float16)(acc[r][4 * qd + i] * nu);
        *reinterpret_cast<half4*>(stage + col * ROWB + o * 2) = hv;
      } else {
        *reinterpret_cast<float4*>(stage + col * ROWB + o * 4) =
            make_float4(acc[r][4 * qd] * nu, acc[r][4 * qd + 1] * nu, acc[r][4 * qd + 2] * nu, acc[r][4 * qd + 3] * nu);
      }
    }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the tile is written (the wave reads it back)
  constexpr int CHUNKS = OF16 ? 8 : 16;  // 16-byte chunks per output vector
  constexpr int VPP = 64 / CHUNKS;       // vectors per pass
#pragma unroll
  for (int ps = 0; ps < 32 / VPP; ps++) {
    const int vl = ps * VPP + lane / CHUNKS, ch = lane % CHUNKS;
    const uint4 val = *reinterpret_cast<const uint4*>(stage + vl * ROWB + ch * 16);
    if (nv == 32 || vl < nv) reinterpret_cast<uint4*>(out_g + vl * (OF16 ? 128 : 256))[ch] = val;
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the tile is read before the next group writes it
}


// s_waitcnt vmcnt(N) that is also a compiler memory barrier.
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __asm__ volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Small launches (a few groups per wave): decode of whole 32-vector groups whose
// records are RW whole words, every wave loading and storing for itself.  Every wave
// keeps the records and norms of its next PF groups in a private LDS ring, filled
// by direct global-to-LDS loads (REC_DMA + 1 per group, always issued, clamped to
// the last group) ahead of use; the output leaves through the staging tile as
// STORES 16-byte stores per group.  With these fixed counts the wait for a slot is
// an exact vmcnt, and no compiler-inserted wait ever covers the ring.
// OPL: the Pi^T operands are staged in LDS once per workgroup (the small-codebook
// configurations; with the 64 KiB codebook the LDS has no room and every wave loads
// them into registers)
template <int K, bool NF16, bool OF16, int RW, bool CBL, int WV, bool OPL>
struct RingShape {
  static constexpr int ROWB = stage_row_bytes<OF16>();
  static constexpr int REC_BYTES = 32 * RW * 4;
  static constexpr int SLOT_BYTES = (REC_BYTES + 32 * (NF16 ? 2 : 4) + 15) & ~15;
  static constexpr int REC_DMA = RW % 4 == 0 ? (8 * RW + 63) / 64 : (32 * RW + 63) / 64;
  static constexpr int LOADS = REC_DMA + 1;
  static constexpr int STORES = OF16 ? 4 : 8;
  static constexpr int WAIT_STEADY = (PF - 1) * LOADS + PF * STORES;
  static constexpr int OP_BYTES = OPL ? 16 * 64 * 16 : 0;  // the staged Pi^T operands
  static size_t lds_bytes(int N) {
    const size_t cb = CBL ? (size_t)((N * K * 2 + 15) & ~15) : 0;
    return cb + (size_t)WV * (32 * ROWB + PF * SLOT_BYTES) + OP_BYTES;
  }
};

template <int K, bool NF16, bool OF16, int RW, bool CBL, int WV, bool OPL>
__global__ __launch_bounds__(WV * 64) void decode_ring(const uint8_t* __restrict__ codes,
                                                            const void* __restrict__ norms, int64_t ngroups,
                                                            const _Float16* __restrict__ cw16,
                                                            const half8* __restrict__ dec_a, int N, int bits,
                                                            void* __restrict__ out, int nwg) {
  typedef RingShape<K, NF16, OF16, RW, CBL, WV, OPL> S;
  constexpr int NC = 8 / K > 0 ? 8 / K : 1;
  constexpr int BITS = RW * K / 2;  // (64 / K) blocks of BITS bits fill RW words
  static_assert((D / K) * BITS == 32 * RW, "whole-word records");
  (void)bits;
  constexpr int ROWB = S::ROWB;
  extern __shared__ uint4 smem[];
  const int tid = fq_tid(), lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, h = lane >> 5;
  const int cb_bytes = CBL ? ((N * K * 2 + 15) & ~15) : 0;
  char* stage = reinterpret_cast<char*>(smem) + cb_bytes + w * 32 * ROWB;
  char* ring = reinterpret_cast<char*>(smem) + cb_bytes + WV * 32 * ROWB + w * PF * S::SLOT_BYTES;
  char* opL = reinterpret_cast<char*>(smem) + cb_bytes + WV * (32 * ROWB + PF * S::SLOT_BYTES);

  // OPL: the Pi^T operands (16 sets of 64 lanes x 16 bytes) and the codebook go to LDS once
  // per workgroup by direct loads, issued ahead of the wave's first ring loads: those first
  // waits then cover them too (one load counter, completed in order), so the operand fetch
  // overlaps the ring's first loads instead of preceding them.  Otherwise every wave loads
  // the operands into registers (16 KiB a wave from L2) before any ring load.
  half8 da[2][4][2];  // Pi^T operands (hi, lo) of both 32-row tiles and all 4 k-steps
  if constexpr (OPL) {
    for (int pc = w; pc < 16; pc += WV)
      lds_dma16(reinterpret_cast<const char*>(dec_a) + pc * 1024 + lane * 16, opL + pc * 1024);
  } else {
#pragma unroll
    for (int r = 0; r < 2; r++)
#pragma unroll
      for (int s = 0; s < 4; s++)
#pragma unroll
        for (int p = 0; p < 2; p++) da[r][s][p] = dec_a[((r * 4 + s) * 2 + p) * 64 + lane];
    __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): the operands are in registers before any ring load
  }
  if constexpr (CBL)
    for (int pc = w; pc * 1024 < cb_bytes; pc += WV)
      if (pc * 1024 + lane * 16 < cb_bytes)
        lds_dma16(reinterpret_cast<const char*>(cw16) + pc * 1024 + lane * 16,
                  reinterpret_cast<char*>(smem) + pc * 1024);
  const _Float16* cb = CBL ? reinterpret_cast<const _Float16*>(smem) : cw16;

  const int64_t step = (int64_t)nwg * WV;
  int64_t g = (int64_t)fq_bid_x() * WV + w;
  if (g >= ngroups) {  // no groups: only its share of the staging, then the barrier
    wait_vmcnt<0>();
    __syncthreads();
    return;
  }
  int64_t left = (ngroups - 1 - g) / step + 1;  // groups of this wave
  const int64_t total = left;

  auto issue = [&](int sl, int64_t gg) {
    gg = gg < ngroups ? gg : ngroups - 1;
    char* dst = ring + sl * S::SLOT_BYTES;
    const char* rsrc = reinterpret_cast<const char*>(codes) + gg * S::REC_BYTES;
    // records: REC_BYTES in 16-byte (RW % 4 == 0) or 4-byte pieces, 64 lanes per instruction,
    // lanes past the end of the group masked off
    constexpr int PIECE = RW % 4 == 0 ? 16 : 4;
#pragma unroll
    for (int p = 0; p < S::REC_DMA; p++) {
      constexpr int TOTAL = S::REC_BYTES / PIECE;
      if (64 * p + lane < TOTAL) {
        if constexpr (PIECE == 16)
          lds_dma16(rsrc + (64 * p + lane) * 16, dst + p * 1024);
        else
          lds_dma4(rsrc + (64 * p + lane) * 4, dst + p * 256);
      }
    }
    // norms: 32 x 2 or 32 x 4 bytes in 4-byte pieces
    constexpr int NPIECES = 32 * (NF16 ? 2 : 4) / 4;
    const char* nsrc = reinterpret_cast<const char*>(norms) + gg * 32 * (NF16 ? 2 : 4);
    if (lane < NPIECES) lds_dma4(nsrc + lane * 4, dst + S::REC_BYTES);
  };
#pragma unroll
  for (int i = 0; i < PF; i++) issue(i, g + i * step);

  // One copy of the loop body (a kernel that runs only a few groups per wave would
  // otherwise execute several cold copies of it from the instruction cache).  Step i
  // reads slot i mod PF; younger operations when it waits: the later prologue groups'
  // loads plus the stores and loads of the steps before it, S::WAIT_STEADY from step PF on.
  constexpr int L = S::LOADS, T = S::STORES;
  static_assert(PF == 4, "one wait case per prologue slot");
  for (int i = 0;; i++) {
    // progress-based priority: the SIMD's arbiter favours the oldest waves, which left the
    // youngest to finish alone; a wave lowers its priority as it gets through its groups
    {
      const int lvl = (int)((4 * (int64_t)i) / total);
      if (lvl == 0)
        __builtin_amdgcn_s_setprio(3);
      else if (lvl == 1)
        __builtin_amdgcn_s_setprio(2);
      else if (lvl == 2)
        __builtin_amdgcn_s_setprio(1);
      else
        __builtin_amdgcn_s_setprio(0);
    }
    switch (i < PF ? i : PF) {
      case 0:
        // this wave's operand and codebook pieces and its first ring slot have landed;
        // after the barrier every wave's pieces have
        wait_vmcnt<(PF - 1) * L>();
        __syncthreads();
        if constexpr (OPL) {
#pragma unroll
          for (int r = 0; r < 2; r++)
#pragma unroll
            for (int s = 0; s < 4; s++)
#pragma unroll
              for (int p = 0; p < 2; p++)
                da[r][s][p] = *reinterpret_cast<const half8*>(opL + ((r * 4 + s) * 2 + p) * 1024 + lane * 16);
        }
        break;
      case 1: wait_vmcnt<(PF - 1) * L + T>(); break;
      case 2: wait_vmcnt<(PF - 1) * L + 2 * T>(); break;
      case 3: wait_vmcnt<(PF - 1) * L + 3 * T>(); break;
      default: wait_vmcnt<S::WAIT_STEADY>(); break;
    }
    const int sl = i & (PF - 1);
    const char* src = ring + sl * S::SLOT_BYTES;
    uint32_t rc[RW];
    {
      const uint32_t* rp = reinterpret_cast<const uint32_t*>(src) + col * RW;
#pragma unroll
      for (int e = 0; e < RW; e++) rc[e] = rp[e];
    }
    float nu;
    if constexpr (NF16)
      nu = (float)reinterpret_cast<const _Float16*>(src + S::REC_BYTES)[col];
    else
      nu = reinterpret_cast<const float*>(src + S::REC_BYTES)[col];
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the slot is read before it is refilled
    issue(sl, g + PF * step);
    f32x16 acc[2];
#pragma unroll
    for (int r = 0; r < 2; r++)
#pragma unroll
      for (int e = 0; e < 16; e++) acc[r][e] = 0.f;
#pragma unroll
    for (int s = 0; s < 4; s++) {
      uint32_t c[NC];  // codes of this lane's input dims 16 s + 8 h .. + 7
#pragma unroll
      for (int p = 0; p < NC; p++) {
        const uint32_t c0 = code_at<RW>(rc, ((16 * s) / K + p) * BITS, BITS);
        const uint32_t c1 = code_at<RW>(rc, ((16 * s + 8) / K + p) * BITS, BITS);
        c[p] = h ? c1 : c0;
      }
      const half8 yb = gather_codes<K>(cb, c, 16 * s + 8 * h);
#pragma unroll
      for (int r = 0; r < 2; r++) {
        acc[r] = __builtin_amdgcn_mfma_f32_32x32x16_f16(da[r][s][0], yb, acc[r], 0, 0, 0);
        acc[r] = __builtin_amdgcn_mfma_f32_32x32x16_f16(da[r][s][1], yb, acc[r], 0, 0, 0);
      }
    }
    stage_and_store<OF16>(acc, nu, stage, col, h, lane, reinterpret_cast<char*>(out) + g * 32 * (OF16 ? 128 : 256),
                          32);
    if (--left == 0) return;
    g += step;
  }
}

// Decode of whole 32-vector groups whose records are RW whole words, C consumer
// waves per workgroup (see the file header).  Round r of workgroup b is groups
// (r nwg + b) C + c, c < C: C consecutive records (C REC_BYTES bytes) and their
// norms, loaded as LOADS 16-byte direct-to-LDS instructions (every one always
// issued, addresses clamped to the last whole group), so the producer's waits are
// exact vmcnt values.
template <int K, bool NF16, bool OF16, int RW, bool CBL, int C>
struct StreamShape {
  static constexpr int ROWB = stage_row_bytes<OF16>();
  static constexpr int REC_BYTES = 32 * RW * 4;
  static constexpr int NORM_BYTES = 32 * (NF16 ? 2 : 4);
  static constexpr int REC_PIECES = C * REC_BYTES / 16;  // 16-byte pieces per round
  static constexpr int NORM_PIECES = C * NORM_BYTES / 16;
  static constexpr int REC_DMA = (REC_PIECES + 63) / 64;
  static constexpr int NORM_DMA = (NORM_PIECES + 63) / 64;
  static constexpr int LOADS = REC_DMA + NORM_DMA;
  static constexpr int ROUND_BYTES = 1024 * LOADS;  // each instruction fills its own 1 KiB
  static constexpr int THREADS = (C + 1) * 64;
  static_assert(2 * LOADS < 64, "vmcnt range");
  static size_t lds_bytes(int N) {
    const size_t cb = CBL ? (size_t)((N * K * 2 + 15) & ~15) : 0;
    return cb + (size_t)RING * ROUND_BYTES + (size_t)C * 32 * ROWB;
  }
};

// Consumers per workgroup: as many as fit next to the codebook (at most 15, the
// 1024-thread limit).
template <int K, bool NF16, bool OF16, int RW, bool CBL>
constexpr int stream_consumers(int cb_bytes) {
  int c = 15;
  while (c > 1 && StreamShape<K, NF16, OF16, RW, CBL, 15>::ROWB * 32 * c + RING * 1024 *
                          ((c * 32 * RW * 4 / 16 + 63) / 64 + (c * 32 * (NF16 ? 2 : 4) / 16 + 63) / 64) +
                          cb_bytes > LDS_MAX_BYTES)
    c--;
  return c;
}


// Workgroup barrier after this wave's LDS operations completed; no wait on its
// global stores (a compiler memory barrier as well).
__device__ inline void ring_barrier() { __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory"); }

template <int K, bool NF16, bool OF16, int RW, bool CBL, int C>
__global__ __launch_bounds__((C + 1) * 64) void decode_stream(const uint8_t* __restrict__ codes,
                                                               const void* __restrict__ norms, int64_t ngroups,
                                                               const _Float16* __restrict__ cw16,
                                                               const half8* __restrict__ dec_a, int N, int bits,
                                                               void* __restrict__ out, int nwg, int rounds) {
  typedef StreamShape<K, NF16, OF16, RW, CBL, C> S;
  constexpr int NC = 8 / K > 0 ? 8 / K : 1;
  constexpr int BITS = RW * K / 2;  // (64 / K) blocks of BITS bits fill RW words
  static_assert((D / K) * BITS == 32 * RW, "whole-word records");
  (void)bits;
  constexpr int ROWB = S::ROWB;
  extern __shared__ uint4 smem[];
  const int tid = fq_tid(), lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = fq_bid_x();
  const int cb_bytes = CBL ? ((N * K * 2 + 15) & ~15) : 0;
  char* const ring = reinterpret_cast<char*>(smem) + cb_bytes;

  if constexpr (CBL)
    for (int i = tid; i < cb_bytes / 16; i += S::THREADS) smem[i] = reinterpret_cast<const uint4*>(cw16)[i];
  half8 da[2][4][2];  // Pi^T operands (hi, lo) of both 32-row tiles and all 4 k-steps (consumers)
  if (w > 0) {
#pragma unroll
    for (int r = 0; r < 2; r++)
#pragma unroll
      for (int s = 0; s < 4; s++)
#pragma unroll
        for (int p = 0; p < 2; p++) da[r][s][p] = dec_a[((r * 4 + s) * 2 + p) * 64 + lane];
  }
  __syncthreads();  // codebook in place; every compiler-visible load has completed

  if (w == 0) {
    // ---- producer
    const int64_t rec_pieces = ngroups * (S::REC_BYTES / 16), norm_pieces = ngroups * (S::NORM_BYTES / 16);
    auto issue = [&](int r) {
      char* dst = ring + (r & (RING - 1)) * S::ROUND_BYTES;
      const int64_t g0 = ((int64_t)r * nwg + b) * C;
#pragma unroll
      for (int i = 0; i < S::REC_DMA; i++) {
        int64_t q = g0 * (S::REC_BYTES / 16) + 64 * i + lane;
        q = q < rec_pieces ? q : rec_pieces - 1;
        lds_dma16(codes + q * 16, dst + 1024 * i);
      }
#pragma unroll
      for (int i = 0; i < S::NORM_DMA; i++) {
        int64_t q = g0 * (S::NORM_BYTES / 16) + 64 * i + lane;
        q = q < norm_pieces ? q : norm_pieces - 1;
        lds_dma16(reinterpret_cast<const char*>(norms) + q * 16, dst + 1024 * (S::REC_DMA + i));
      }
    };
    constexpr int L = S::LOADS;
    for (int r = 0; r < RING - 1 && r < rounds; r++) issue(r);
    if (rounds >= 3)
      wait_vmcnt<2 * L>();
    else if (rounds == 2)
      wait_vmcnt<L>();
    else
      wait_vmcnt<0>();
    ring_barrier();  // round 0 in place
    for (int r = 0; r < rounds; r++) {
      // the slot of round r + 3 was read in round r - 1, which ended at the last barrier
      if (r + 3 < rounds) issue(r + 3);
      // round r + 1 in place; younger: rounds r + 2 and r + 3 where issued
      if (r + 3 < rounds)
        wait_vmcnt<2 * L>();
      else if (r + 2 < rounds)
        wait_vmcnt<L>();
      else
        wait_vmcnt<0>();
      ring_barrier();
    }
    return;
  }

  // ---- consumers: group c of every round
  const int c = w - 1, col = lane & 31, h = lane >> 5;
  char* const stage = ring + RING * S::ROUND_BYTES + c * 32 * ROWB;
  const _Float16* cb = CBL ? reinterpret_cast<const _Float16*>(smem) : cw16;
  ring_barrier();
  for (int r = 0; r < rounds; r++) {
    const char* src = ring + (r & (RING - 1)) * S::ROUND_BYTES;
    uint32_t rc[RW];
    {
      const uint32_t* rp = reinterpret_cast<const uint32_t*>(src + c * S::REC_BYTES) + col * RW;
#pragma unroll
      for (int e = 0; e < RW; e++) rc[e] = rp[e];
    }
    float nu;
    if constexpr (NF16)
      nu = (float)reinterpret_cast<const _Float16*>(src + 1024 * S::REC_DMA + c * S::NORM_BYTES)[col];
    else
      nu = reinterpret_cast<const float*>(src + 1024 * S::REC_DMA + c * S::NORM_BYTES)[col];
    const int64_t g = ((int64_t)r * nwg + b) * C + c;
    if (g < ngroups) {  // wave-uniform
      f32x16 acc[2];
#pragma unroll
      for (int rr = 0; rr < 2; rr++)
#pragma unroll
        for (int e = 0; e < 16; e++) acc[rr][e] = 0.f;
#pragma unroll
      for (int s = 0; s < 4; s++) {
        uint32_t cc[NC];  // codes of this lane's input dims 16 s + 8 h .. + 7
#pragma unroll
        for (int p = 0; p < NC; p++) {
          const uint32_t c0 = code_at<RW>(rc, ((16 * s) / K + p) * BITS, BITS);
          const uint32_t c1 = code_at<RW>(rc, ((16 * s + 8) / K + p) * BITS, BITS);
          cc[p] = h ? c1 : c0;
        }
        const half8 yb = gather_codes<K>(cb, cc, 16 * s + 8 * h);
#pragma unroll
        for (int rr = 0; rr < 2; rr++) {
          acc[rr] = __builtin_amdgcn_mfma_f32_32x32x16_f16(da[rr][s][0], yb, acc[rr], 0, 0, 0);
          acc[rr] = __builtin_amdgcn_mfma_f32_32x32x16_f16(da[rr][s][1], yb, acc[rr], 0, 0, 0);
        }
      }
      stage_and_store<OF16>(acc, nu, stage, col, h, lane,
                            reinterpret_cast<char*>(out) + g * 32 * (OF16 ? 128 : 256), 32);
    }
    ring_barrier();  // this round's slot has been read
  }
}

// Generic decoder: any record length (codes read bit-wise from global memory) and
// partial groups; one group per wave step, no prefetch.  Used for non-word records
// and for the last n mod 32 vectors of the stream decoder's input.
template <int K, bool NF16, bool OF16, bool CBL>
__global__ __launch_bounds__(WAVES * 64) void decode_mfma(const uint8_t* __restrict__ codes,
                                                          const void* __restrict__ norms, int64_t n,
                                                          const _Float16* __restrict__ cw16,
                                                          const half8* __restrict__ dec_a, int N, int bits,
                                                          void* __restrict__ out, int nwg) {
  constexpr int NC = 8 / K > 0 ? 8 / K : 1;
  constexpr int ROWB = stage_row_bytes<OF16>();
  extern __shared__ uint4 smem[];
  const int tid = fq_tid(), lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, h = lane >> 5;
  const int cb_bytes = CBL ? ((N * K * 2 + 15) & ~15) : 0;
  char* stage = reinterpret_cast<char*>(smem) + cb_bytes + w * 32 * ROWB;
  half8 da[2][4][2];
#pragma unroll
  for (int r = 0; r < 2; r++)
#pragma unroll
    for (int s = 0; s < 4; s++)
#pragma unroll
      for (int p = 0; p < 2; p++) da[r][s][p] = dec_a[((r * 4 + s) * 2 + p) * 64 + lane];
  if constexpr (CBL) {
    for (int i = tid; i < cb_bytes / 16; i += WAVES * 64) smem[i] = reinterpret_cast<const uint4*>(cw16)[i];
    __syncthreads();
  }
  const _Float16* cb = CBL ? reinterpret_cast<const _Float16*>(smem) : cw16;
  const int B = (D / K) * bits;
  const int64_t ngroups = (n + 31) / 32;
  const int64_t step = (int64_t)nwg * WAVES;
  for (int64_t g = (int64_t)fq_bid_x() * WAVES + w; g < ngroups; g += step) {
    const int64_t v = g * 32 + col;
    const int64_t vv = v < n ? v : n - 1;  // invalid lanes decode a valid record, never stored
    float nu;
    if constexpr (NF16)
      nu = (float)reinterpret_cast<const _Float16*>(norms)[vv];
    else
      nu = reinterpret_cast<const float*>(norms)[vv];
    f32x16 acc[2];
#pragma unroll
    for (int r = 0; r < 2; r++)
#pragma unroll
      for (int e = 0; e < 16; e++) acc[r][e] = 0.f;
#pragma unroll
    for (int s = 0; s < 4; s++) {
      uint32_t c[NC];
#pragma unroll
      for (int p = 0; p < NC; p++) c[p] = load_code(codes, vv * B + (int64_t)((16 * s + 8 * h) / K + p) * bits, bits);
      const half8 yb = gather_codes<K>(cb, c, 16 * s + 8 * h);
#pragma unroll
      for (int r = 0; r < 2; r++) {
        acc[r] = __builtin_amdgcn_mfma_f32_32x32x16_f16(da[r][s][0], yb, acc[r], 0, 0, 0);
        acc[r] = __builtin_amdgcn_mfma_f32_32x32x16_f16(da[r][s][1], yb, acc[r], 0, 0, 0);
      }
    }
    const int64_t nv = n - g * 32;
    stage_and_store<OF16>(acc, nu, stage, col, h, lane, reinterpret_cast<char*>(out) + g * 32 * (OF16 ? 128 : 256),
                          nv < 32 ? (int)nv : 32);
  }
}

// Full-vector code (k = d): the decoded unit vector of code c is row c of dec_full
// (Pi^T c_n, fp32), so decoding is a gather of that row scaled by the norm, with no
// rotation left to do.  Eight lanes per vector, 8 output dims each (two 16-byte table
// loads; one 16-byte fp16 store or two fp32 ones); a workgroup takes FULL_PASSES x 32
// consecutive vectors per step, every pass's loads issued before its first store, and
// steps through the input at a stride of nwg steps (the launch gives every step its own
// workgroup).
constexpr int FULL_PASSES = 4;
constexpr int FULL_VEC_PER_STEP = 32 * FULL_PASSES;

template <bool NF16, bool OF16>
__global__ __launch_bounds__(256) void decode_full(const uint8_t* __restrict__ codes, const void* __restrict__ norms,
                                                   int64_t n, int bits, const float* __restrict__ tab,
                                                   void* __restrict__ out, int64_t nsteps, int nwg) {
  const int tid = fq_tid();
  const int sub = tid & 7;
  for (int64_t st = fq_bid_x(); st < nsteps; st += nwg) {
    const int64_t v0 = st * FULL_VEC_PER_STEP + (tid >> 3);
    uint32_t c[FULL_PASSES];
    float nu[FULL_PASSES];
#pragma unroll
    for (int p = 0; p < FULL_PASSES; p++) {
      const int64_t v = v0 + 32 * p;
      const int64_t vv = v < n ? v : n - 1;  // lanes past the end read a valid record, store nothing
      c[p] = load_code(codes, vv * bits, bits);
      if constexpr (NF16)
        nu[p] = (float)reinterpret_cast<const _Float16*>(norms)[vv];
      else
        nu[p] = reinterpret_cast<const float*>(norms)[vv];
    }
    float4 a[FULL_PASSES], b[FULL_PASSES];
#pragma unroll
    for (int p = 0; p < FULL_PASSES; p++) {
      const float4* row = reinterpret_cast<const float4*>(tab + (size_t)c[p] * D + 8 * sub);
      a[p] = row[0];
      b[p] = row[1];
    }
#pragma unroll
    for (int p = 0; p < FULL_PASSES; p++) {
      const int64_t v = v0 + 32 * p;
      if (v >= n) continue;
      const float u = nu[p];
      if constexpr (OF16) {
        half8 h;
        h[0] = (_Float16)(a[p].x * u);
        h[1] = (_Float16)(a[p].y * u);
        h[2] = (_Float16)(a[p].z * u);
        h[3] = (_Float16)(a[p].w * u);
        h[4] = (_Float16)(b[p].x * u);
        h[5] = (_Float16)(b[p].y * u);
        h[6] = (_Float16)(b[p].z * u);
        h[7] = (_Float16)(b[p].w * u);
        reinterpret_cast<half8*>(out)[v * (D / 8) + sub] = h;
      } else {
        float4* o = reinterpret_cast<float4*>(out) + v * (D / 4) + 2 * sub;
        o[0] = make_float4(a[p].x * u, a[p].y * u, a[p].z * u, a[p].w * u);
        o[1] = make_float4(b[p].x * u, b[p].y * u, b[p].z * u, b[p].w * u);
      }
    }
  }
}

template <bool OF16>
size_t generic_lds_bytes(int N, int K, bool cbl) {
  const size_t cb = cbl ? (size_t)((N * K * 2 + 15) & ~15) : 0;
  return cb + (size_t)WAVES * 32 * stage_row_bytes<OF16>();
}

// Persistent grid: the workgroups of `block` threads that fit at once, at most one
// per `work` units.
template <typename KernelT>
hipError_t persistent_grid(const fq_codebook* cb, KernelT kernel, int block, size_t lds, int64_t work, int64_t* wgs) {
  int64_t resident = 0;
  const hipError_t e = resident_workgroups(reinterpret_cast<const void*>(kernel), block, lds, cb->device, &resident);
  if (e != hipSuccess) return e;
  *wgs = work < resident ? work : resident;
  if (*wgs < 1) *wgs = 1;
  return hipSuccess;
}

template <int K, bool NF, bool OF, bool CBL>
hipError_t launch_generic(const fq_codebook* cb, const uint8_t* codes, const void* norms, int64_t n, void* out,
                          hipStream_t s) {
  const size_t lds = generic_lds_bytes<OF>(cb->N, K, CBL);
  int64_t wgs = 0;
  hipError_t e =
      persistent_grid(cb, decode_mfma<K, NF, OF, CBL>, WAVES * 64, lds, ((n + 31) / 32 + WAVES - 1) / WAVES, &wgs);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_mfma<K, NF, OF, CBL>), dim3((unsigned)wgs), dim3(WAVES * 64), lds, s, codes, norms, n,
                     cb->cw16, reinterpret_cast<const half8*>(cb->dec_a), cb->N, cb->bits, out, (int)wgs);
  return hipGetLastError();
}

// RW > 0: the whole groups go to decode_stream, the last n mod 32 vectors to the
// generic kernel; RW = 0: everything to the generic kernel.  CBL: both hold the
// codebook in LDS; BIG (with CBL false): the stream decoder holds it in LDS (with
// fewer consumer waves), the generic kernel reads it from global memory.
template <int K, bool NF, bool OF, int RW, bool CBL, bool BIG>
hipError_t launch_one(const fq_codebook* cb, const uint8_t* codes, const void* norms, int64_t n, void* out,
                      hipStream_t s) {
  int64_t done = 0;
  if constexpr (RW > 0) {
    constexpr bool SCBL = CBL || BIG;
    constexpr int CBB = SCBL ? (CBL ? LDS_CB_HALFS * 2 : LDS_CB_HALFS_BIG * 2) : 0;  // largest codebook it holds
    constexpr int C = stream_consumers<K, NF, OF, RW, SCBL>(CBB);
    typedef StreamShape<K, NF, OF, RW, SCBL, C> S;
    const int64_t ngroups = n / 32;
    if (ngroups > 0) {
      const auto kern = decode_stream<K, NF, OF, RW, SCBL, C>;
      const size_t lds = S::lds_bytes(cb->N);
      if constexpr (BIG) {
        // a device with less LDS per workgroup reads the codebook from L1 / L2 instead
        if (lds > cb->max_lds || lds > (size_t)LDS_MAX_BYTES || cb->force_cache_codebook)
          return launch_one<K, NF, OF, RW, false, false>(cb, codes, norms, n, out, s);
      }
      hipError_t e = hipSuccess;
      int64_t wgs = 0, rounds = 0;
      // (a device with less LDS per workgroup than the consumers' staging tiles need runs
      // the per-wave ring decoder)
      if (lds <= cb->max_lds) {
        if (lds > 65536)
          e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)lds);
        if (e != hipSuccess) return e;
        e = persistent_grid(cb, kern, S::THREADS, lds, (ngroups + C - 1) / C, &wgs);
        if (e != hipSuccess) return e;
        rounds = (ngroups + wgs * C - 1) / (wgs * C);
      }
      if (rounds >= MIN_ROUNDS) {
        if (rounds > INT32_MAX) return hipErrorInvalidValue;
        hipLaunchKernelGGL(kern, dim3((unsigned)wgs), dim3(S::THREADS), lds, s, codes, norms, ngroups, cb->cw16,
                           reinterpret_cast<const half8*>(cb->dec_a), cb->N, cb->bits, out, (int)wgs, (int)rounds);
      } else {
        // a few groups per consumer: waves that load and store for themselves start sooner
        constexpr int WV = BIG ? waves_ring(OF) : WAVES;
        typedef RingShape<K, NF, OF, RW, SCBL, WV, !BIG> RS;
        const auto rkern = decode_ring<K, NF, OF, RW, SCBL, WV, !BIG>;
        const size_t rlds = RS::lds_bytes(cb->N);
        if (rlds > 65536)
          e = hipFuncSetAttribute(reinterpret_cast<const void*>(rkern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)rlds);
        if (e != hipSuccess) return e;
        e = persistent_grid(cb, rkern, WV * 64, rlds, (ngroups + WV - 1) / WV, &wgs);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(rkern, dim3((unsigned)wgs), dim3(WV * 64), rlds, s, codes, norms, ngroups, cb->cw16,
                           reinterpret_cast<const half8*>(cb->dec_a), cb->N, cb->bits, out, (int)wgs);
      }
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      done = ngroups * 32;
    }
  }
  if (done == n) return hipSuccess;
  const int B = (D / K) * cb->bits;  // done is a multiple of 32, so done B bits are whole bytes
  return launch_generic<K, NF, OF, CBL>(cb, codes + done * B / 8,
                                        reinterpret_cast<const char*>(norms) + done * (NF ? 2 : 4), n - done,
                                        reinterpret_cast<char*>(out) + done * (OF ? 128 : 256), s);
}

template <int K, int RW, bool CBL, bool BIG>
hipError_t launch_cbl(const fq_codebook* cb, const uint8_t* codes, const void* norms, fq_dtype nd, int64_t n,
                      void* out, fq_dtype od, hipStream_t s) {
  if (nd == FQ_F16 && od == FQ_F16) return launch_one<K, true, true, RW, CBL, BIG>(cb, codes, norms, n, out, s);
  if (nd == FQ_F16) return launch_one<K, true, false, RW, CBL, BIG>(cb, codes, norms, n, out, s);
  if (od == FQ_F16) return launch_one<K, false, true, RW, CBL, BIG>(cb, codes, norms, n, out, s);
  return launch_one<K, false, false, RW, CBL, BIG>(cb, codes, norms, n, out, s);
}

template <int K, int RW>
hipError_t launch_rw(const fq_codebook* cb, const uint8_t* codes, const void* norms, fq_dtype nd, int64_t n,
                     void* out, fq_dtype od, hipStream_t s) {
  if (cb->N * K <= LDS_CB_HALFS) return launch_cbl<K, RW, true, false>(cb, codes, norms, nd, n, out, od, s);
  if constexpr (RW > 0) {
    // (checked against the device's LDS per workgroup at launch: 8 fp32-output waves
    // need 146 KiB)
    if (cb->N * K <= LDS_CB_HALFS_BIG) return launch_cbl<K, RW, false, true>(cb, codes, norms, nd, n, out, od, s);
  }
  return launch_cbl<K, RW, false, false>(cb, codes, norms, nd, n, out, od, s);
}

// Whole-word record lengths are specialised: k = 2, N = 16 and k = 4, N = 256
// (4 words), k = 8, N = 4096 (3 words); everything else reads codes bit-wise.
template <int K>
hipError_t launch_k(const fq_codebook* cb, const uint8_t* codes, const void* norms, fq_dtype nd, int64_t n,
                    void* out, fq_dtype od, hipStream_t s) {
  const int B = (D / K) * cb->bits;
  if constexpr (K == 2 || K == 4) {
    if (B == 128) return launch_rw<K, 4>(cb, codes, norms, nd, n, out, od, s);
  }
  if constexpr (K == 8) {
    if (B == 96) return launch_rw<K, 3>(cb, codes, norms, nd, n, out, od, s);
  }
  return launch_rw<K, 0>(cb, codes, norms, nd, n, out, od, s);
}

template <bool NF, bool OF>
hipError_t launch_full(const fq_codebook* cb, const uint8_t* codes, const void* norms, int64_t n, void* out,
                       hipStream_t s) {
  const int64_t nsteps = (n + FULL_VEC_PER_STEP - 1) / FULL_VEC_PER_STEP;
  // one step per workgroup: a wave that walked several steps waited, at each step's code
  // loads, for its own older stores as well (one completion counter), about 5 % slower
  const int64_t wgs = nsteps < INT32_MAX ? nsteps : INT32_MAX;
  hipLaunchKernelGGL((decode_full<NF, OF>), dim3((unsigned)wgs), dim3(256), 0, s, codes, norms, n, cb->bits,
                     cb->dec_full, out, nsteps, (int)wgs);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_full(const fq_codebook* cb, const uint8_t* codes, const void* norms, fq_dtype norm_dtype,
                              int64_t n, void* x_out, fq_dtype out_dtype, hipStream_t s) {
  if (!cb->dec_full || cb->k != D) return hipErrorNotSupported;
  if (n <= 0) return hipSuccess;
  if (norm_dtype == FQ_F16 && out_dtype == FQ_F16) return launch_full<true, true>(cb, codes, norms, n, x_out, s);
  if (norm_dtype == FQ_F16) return launch_full<true, false>(cb, codes, norms, n, x_out, s);
  if (out_dtype == FQ_F16) return launch_full<false, true>(cb, codes, norms, n, x_out, s);
  return launch_full<false, false>(cb, codes, norms, n, x_out, s);
}

hipError_t launch_decode_mfma(const fq_codebook* cb, const uint8_t* codes, const void* norms, fq_dtype norm_dtype,
                              int64_t n, void* x_out, fq_dtype out_dtype, hipStream_t s) {
  switch (cb->k) {
    case 1: return launch_k<1>(cb, codes, norms, norm_dtype, n, x_out, out_dtype, s);
    case 2: return launch_k<2>(cb, codes, norms, norm_dtype, n, x_out, out_dtype, s);
    case 4: return launch_k<4>(cb, codes, norms, norm_dtype, n, x_out, out_dtype, s);
    case 8: return launch_k<8>(cb, codes, norms, norm_dtype, n, x_out, out_dtype, s);
    case 16: return launch_k<16>(cb, codes, norms, norm_dtype, n, x_out, out_dtype, s);
    case 32: return launch_k<32>(cb, codes, norms, norm_dtype, n, x_out, out_dtype, s);
    case 64: return launch_k<64>(cb, codes, norms, norm_dtype, n, x_out, out_dtype, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fq
