// Device helpers used by several kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fq {

// Work-item and workgroup indices read straight from the hardware registers.  The
// HIP index variables go through library functions that are not inlined into
// kernels built without IEEE mode, which turns every index into an opaque call
// result held in vector registers.  Grid sizes are passed as kernel arguments:
// reading them from the dispatch packet (host memory) in every wave costs
// several microseconds at the start of a kernel.
__device__ inline int fq_tid() { return (int)__builtin_amdgcn_workitem_id_x(); }
__device__ inline int fq_bid_x() { return (int)__builtin_amdgcn_workgroup_id_x(); }
__device__ inline int fq_bid_y() { return (int)__builtin_amdgcn_workgroup_id_y(); }
__device__ inline int fq_bid_z() { return (int)__builtin_amdgcn_workgroup_id_z(); }

// Round a double to the nearest fp16 value, ties to even, in one step (no
// detour through fp32, whose double rounding can differ).  Returns the fp16
// bit pattern; |v| >= 65520 gives +-inf, NaN gives a quiet NaN.
__device__ inline uint16_t f64_to_f16_bits(double v) {
  uint64_t u = __double_as_longlong(v);
  uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
  if ((u & 0x7fffffffffffffffull) > 0x7ff0000000000000ull) return (uint16_t)(sign | 0x7e00u);  // NaN (bit test)
  double a = fabs(v);
  if (a >= 65520.0) return (uint16_t)(sign | 0x7c00u);
  if (a < 6.103515625e-05) {  // below 2^-14: subnormal grid, spacing 2^-24
    double r = rint(a * 16777216.0);  // exact scaling; rint rounds half to even
    return (uint16_t)(sign | (uint16_t)r);  // r == 1024 is the smallest normal
  }
  int e = (int)((u >> 52) & 0x7ff) - 1023;       // a is a normal double here
  double q = ldexp(a, 10 - e);                    // in [1024, 2048), exact
  double r = rint(q);
  if (r >= 2048.0) { r = 1024.0; e += 1; }
  if (e > 15) return (uint16_t)(sign | 0x7c00u);
  return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(r - 1024.0));
}

// Read one `bits`-wide code (bits <= 16) that starts at bit `bitoff` of an
// LSB-first little-endian bitstream.  Touches only the bytes the code spans.
__device__ inline uint32_t load_code(const uint8_t* __restrict__ p, int64_t bitoff, int bits) {
  int64_t byte = bitoff >> 3;
  int sh = (int)(bitoff & 7);
  uint32_t v = p[byte];
  int need = sh + bits;
  if (need > 8) v |= (uint32_t)p[byte + 1] << 8;
  if (need > 16) v |= (uint32_t)p[byte + 2] << 16;
  return (v >> sh) & ((1u << bits) - 1u);
}

// Scattered stores (one new token per sequence appended to a fixed-address cache):
// vector v of a launch goes to record slots[v] of a code store of `cap` records, or to
// record v when slots is null.  A slot outside [0, cap) gives -1: the vector is not stored.
__device__ inline int64_t out_slot(const int64_t* __restrict__ slots, int64_t cap, int64_t v) {
  if (!slots) return v;
  const int64_t s = slots[v];
  return (s >= 0 && s < cap) ? s : -1;
}

// Copies the nv records of a group packed in LDS (record r is bytes [r rb, (r + 1) rb) of
// src, rb = record bytes) to their slots.  Records are whole bytes, so no byte of the
// store is shared between records: plain stores, dwords when rb is a multiple of 4, else
// bytes.  Called by every lane of a wave.
__device__ inline void scatter_records(const uint32_t* src, int nv, int rb, const int64_t* __restrict__ slots,
                                       int64_t cap, int64_t v0, uint8_t* __restrict__ codes, int lane) {
  if ((rb & 3) == 0) {
    const int rw = rb >> 2;
    for (int t = lane; t < nv * rw; t += 64) {
      const int r = t / rw, w = t - r * rw;
      const int64_t s = out_slot(slots, cap, v0 + r);
      if (s >= 0) reinterpret_cast<uint32_t*>(codes)[s * rw + w] = src[r * rw + w];
    }
  } else {
    const uint8_t* sb = reinterpret_cast<const uint8_t*>(src);
    for (int t = lane; t < nv * rb; t += 64) {
      const int r = t / rb, c = t - r * rb;
      const int64_t s = out_slot(slots, cap, v0 + r);
      if (s >= 0) codes[s * rb + c] = sb[r * rb + c];
    }
  }
}

// Direct global-to-LDS loads: lane i moves its 16 (or 4) bytes from `gptr` to
// LDS address lds + 16 i (4 i).  Written as inline assembly on purpose: the
// compiler's wait insertion treats such a load as a write to all of LDS and puts
// a full vmcnt(0) before the next LDS read, which serialises any double buffer.
// Callers wait for these loads explicitly (s_waitcnt vmcnt); nothing else in the
// calling kernels uses M0.  `lds` must be the same in every lane of the wave.
typedef __attribute__((address_space(3))) void fq_lds_void;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ inline void lds_dma16(const void* gptr, char* lds) {
  const uint32_t la = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(fq_lds_void*)lds);
  __asm__ volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(gptr), "s"(la) : "memory", "m0");
}
// Same as lds_dma16 with a wave-uniform base address (scalar registers) and a
// per-lane 32-bit byte offset: no 64-bit address arithmetic per lane.
__device__ inline void lds_dma16_s(const void* sbase, uint32_t voff, char* lds) {
  const uint32_t la = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(fq_lds_void*)lds);
  __asm__ volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "s"(la)
                   : "memory", "m0");
}
__device__ inline void lds_dma4(const void* gptr, char* lds) {
  const uint32_t la = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(fq_lds_void*)lds);
  __asm__ volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" : : "v"(gptr), "s"(la) : "memory", "m0");
}
#pragma clang diagnostic pop

}  // namespace fq
