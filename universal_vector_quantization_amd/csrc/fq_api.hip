// Host side of the C ABI in include/fq.h: argument checks (before any HIP call
// where possible), codebook upload, and dispatch to the kernel launchers.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <new>

#include "fq_internal.h"

#include <map>
#include <mutex>
#include <tuple>

#define FQ_EXPORT extern "C" __attribute__((visibility("default")))

// Device memory of fq_attn_decode_noalloc: its partial-record workspace lives in this
// array instead of a caller's buffer.  Every device the library runs on holds one copy
// until the process ends.  Host code must never use the array's name as an address
// (on the host it is only a stand-in): the device address of the current device's
// copy comes from hipGetSymbolAddress, looked up once per device at codebook load.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace fq {

hipError_t resident_workgroups(const void* kernel, int block, size_t lds, int device, int64_t* out) {
  static std::mutex mu;
  static std::map<std::tuple<const void*, int, size_t, int>, int64_t> cache;
  const auto key = std::make_tuple(kernel, block, lds, device);
  {
    std::lock_guard<std::mutex> lock(mu);
    const auto it = cache.find(key);
    if (it != cache.end()) {
      *out = it->second;
      return hipSuccess;
    }
  }
  int per_cu = 0, cus = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, lds);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess) return e;
  const int64_t r = (int64_t)(per_cu < 1 ? 1 : per_cu) * (cus < 1 ? 1 : cus);
  {
    std::lock_guard<std::mutex> lock(mu);
    cache[key] = r;
  }
  *out = r;
  return hipSuccess;
}

}  // namespace fq

namespace {

bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

int log2i(int v) {
  int b = 0;
  while ((1 << b) < v) b++;
  return b;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_dtype(fq_dtype t) { return t == FQ_F32 || t == FQ_F16; }

// True if v is zero or an fp16 normal number exactly (finite, |v| in [2^-14, 65504]).
bool fp16_exact_normal(float v) {
  if (v == 0.0f) return true;
  if (!isfinite(v)) return false;
  const float a = fabsf(v);
  if (a < 6.103515625e-05f || a > 65504.0f) return false;
  const _Float16 h = (_Float16)v;
  return (float)h == v;
}

// Device the handle lives on must be current.
fq_status check_device(const fq_codebook* cb) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return FQ_ERR_HIP;
  return dev == cb->device ? FQ_OK : FQ_ERR_ARG;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on device `dev`, which must be current: looked up on
// the first call for that device, then cached.
fq_status scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return FQ_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FQ_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FQ_OK;
}

void release(fq_codebook* cb) {
  if (!cb) return;
  (void)hipFree(cb->cw);
  (void)hipFree(cb->cw16);
  (void)hipFree(cb->cn2);
  (void)hipFree(cb->pi64t);
  (void)hipFree(cb->pi32);
  (void)hipFree(cb->rotp);
  (void)hipFree(cb->amfma);
  (void)hipFree(cb->cinit);
  (void)hipFree(cb->cn2s);
  (void)hipFree(cb->pi64m);
  (void)hipFree(cb->pi64);
  (void)hipFree(cb->dec_a);
  (void)hipFree(cb->rot16);
  (void)hipFree(cb->crec);
  (void)hipFree(cb->rot32);
  (void)hipFree(cb->frec);
  (void)hipFree(cb->dec_full);
  delete cb;
}

template <class T>
fq_status upload(T** dst, const T* src, size_t count) {
  if (hipMalloc(dst, count * sizeof(T)) != hipSuccess) return FQ_ERR_HIP;
  return hipMemcpy(*dst, src, count * sizeof(T), hipMemcpyHostToDevice) == hipSuccess ? FQ_OK : FQ_ERR_HIP;
}

// The wide prefill's query rotation: 1024 Pi as fp16 hi + mid (the rest is 2^-22 of it),
// rows permuted so that the output rows a lane holds are exactly the query coordinates
// its QK operand needs (coordinates 16 s + 8 hh + jj for lane half hh).
fq_status upload_prefill_rotation(fq_codebook* cb, const float* rotation) {
  const int d = cb->d;
  _Float16* rp = new (std::nothrow) _Float16[2 * 4 * 2 * 64 * 8];
  if (!rp) return FQ_ERR_HIP;
  for (int t = 0; t < 2; t++)
    for (int s = 0; s < 4; s++)
      for (int l = 0; l < 64; l++)
        for (int jj = 0; jj < 8; jj++) {
          const int m = l % 32, i = m / 8, hh = (m / 4) % 2, j = m % 4;
          const int coord = 32 * t + 16 * (i / 2) + 8 * hh + 4 * (i % 2) + j, in = 16 * s + 8 * (l / 32) + jj;
          const double P = 1024.0 * (double)rotation[coord * d + in];
          const _Float16 hi = (_Float16)P;
          const _Float16 mid = (_Float16)(P - (double)hi);
          rp[((((t * 4 + s) * 2 + 0) * 64) + l) * 8 + jj] = hi;
          rp[((((t * 4 + s) * 2 + 1) * 64) + l) * 8 + jj] = mid;
        }
  const fq_status st = upload(&cb->rotp, rp, (size_t)2 * 4 * 2 * 64 * 8);
  delete[] rp;
  return st;
}

// Operand layouts of the matrix-core encoder, built once per codebook.
// Operands of the k = 16, 32, 64 encoder: the rotation as 32 x 32 x 16 A operands (three
// fp16 parts of 1024 Pi, rows permuted so that a lane ends up with 32 consecutive
// coordinates) and the codeword rows in their LDS layout (k fp16 coordinates, then a
// 16-byte norm slot: for k = d row 4 g's holds the fp32 256 ||c||^2 of rows
// 4 g .. 4 g + 3 and the other rows' are zero; for k = 16, 32 each row's holds its own
// 256 ||c||^2 as fp16 hi + lo and six zeros), zero-padded to whole chunks of 8 tiles.
fq_status upload_full_operands(fq_codebook* cb, const float* codewords, const float* rotation) {
  const int d = cb->d, k = cb->k, N = cb->N;
  const int tiles = N / 32, chunks = (tiles + 7) / 8;
  const int rowb = 2 * k + 16;
  const size_t rec_bytes = (size_t)chunks * 8 * 32 * rowb;
  _Float16* rt = new (std::nothrow) _Float16[2 * 4 * 3 * 64 * 8];
  uint8_t* rc = new (std::nothrow) uint8_t[rec_bytes]();
  if (!rt || !rc) {
    delete[] rt;
    delete[] rc;
    return FQ_ERR_HIP;
  }
  for (int r = 0; r < 2; r++)
    for (int s = 0; s < 4; s++)
      for (int l = 0; l < 64; l++)
        for (int j = 0; j < 8; j++) {
          const int rho = l % 32, a = rho / 8, hh = (rho / 4) % 2, b = rho % 4;
          const int coord = 32 * hh + 16 * r + 4 * a + b, in = 16 * s + 8 * (l / 32) + j;
          const double P = 1024.0 * (double)rotation[coord * d + in];
          const _Float16 hi = (_Float16)P;
          const _Float16 mid = (_Float16)(P - (double)hi);
          const _Float16 lo = (_Float16)(P - (double)hi - (double)mid);
          const _Float16 parts[3] = {hi, mid, lo};
          for (int p = 0; p < 3; p++) rt[((((r * 4 + s) * 3 + p) * 64) + l) * 8 + j] = parts[p];
        }
  for (int n = 0; n < N; n++) {
    uint8_t* row = rc + (size_t)n * rowb;
    double c2 = 0.0;
    for (int t = 0; t < k; t++) {
      const double v = (double)codewords[(size_t)n * k + t];
      const _Float16 hv = (_Float16)v;  // exact: codewords are fp16 values
      memcpy(row + 2 * t, &hv, 2);
      c2 += v * v;
    }
    if (k == d) {
      // 256 ||c||^2 in fp32, in the norm slot of the first row of its group of four
      // (rows 4 g .. 4 g + 3 of a tile are the four accumulator rows a lane starts from)
      const float s2 = (float)(256.0 * c2);
      memcpy(rc + (size_t)(n & ~3) * rowb + 2 * k + 4 * (n & 3), &s2, 4);
    } else {
      // 256 ||c||^2 as fp16 hi + lo (22 bits) in the row's norm slot, then zeros
      const double s2 = 256.0 * c2;
      const _Float16 nh = (_Float16)s2;
      const _Float16 nl = (_Float16)(s2 - (double)nh);
      memcpy(row + 2 * k, &nh, 2);
      memcpy(row + 2 * k + 2, &nl, 2);
    }
  }
  fq_status st = upload(&cb->rot32, rt, (size_t)2 * 4 * 3 * 64 * 8);
  if (st == FQ_OK) st = upload(&cb->frec, rc, rec_bytes);
  delete[] rt;
  delete[] rc;
  return st;
}

fq_status upload_mfma_operands(fq_codebook* cb, const float* codewords, const float* rotation, const float* cn2) {
  const int d = cb->d, k = cb->k, N = cb->N;
  // Pi in fp64, row-major and as the A operand of mfma_f64_16x16x4 (lane l: row l%16, k l/16).
  double* pr = new (std::nothrow) double[(size_t)d * d];
  double* pm = new (std::nothrow) double[(size_t)d * d];
  if (!pr || !pm) {
    delete[] pr;
    delete[] pm;
    return FQ_ERR_HIP;
  }
  for (int i = 0; i < d * d; i++) pr[i] = (double)rotation[i];
  for (int r = 0; r < 4; r++)
    for (int s = 0; s < 16; s++)
      for (int l = 0; l < 64; l++) pm[(r * 16 + s) * 64 + l] = pr[(16 * r + (l % 16)) * d + 4 * s + l / 16];
  fq_status st = upload(&cb->pi64, pr, (size_t)d * d);
  if (st == FQ_OK) st = upload(&cb->pi64m, pm, (size_t)d * d);
  // Decoder operand: A[o][i] = Pi[i][o] split into fp16 hi + lo; lane l of tile (r, s)
  // holds row o = 32 r + l % 32 and k = 8 (l / 32) + j, i.e. input dim 16 s + 8 (l / 32) + j.
  _Float16* da = new (std::nothrow) _Float16[2 * 4 * 2 * 64 * 8];
  if (!da) st = FQ_ERR_HIP;
  if (st == FQ_OK) {
    for (int r = 0; r < 2; r++)
      for (int s = 0; s < 4; s++)
        for (int l = 0; l < 64; l++)
          for (int j = 0; j < 8; j++) {
            const int o = 32 * r + (l % 32), i = 16 * s + 8 * (l / 32) + j;
            const float v = rotation[i * d + o];
            const _Float16 hi = (_Float16)v;
            const _Float16 lo = (_Float16)(v - (float)hi);
            da[(((r * 4 + s) * 2 + 0) * 64 + l) * 8 + j] = hi;
            da[(((r * 4 + s) * 2 + 1) * 64 + l) * 8 + j] = lo;
          }
    st = upload(&cb->dec_a, da, (size_t)2 * 4 * 2 * 64 * 8);
  }
  delete[] da;
  delete[] pr;
  delete[] pm;
  if (st == FQ_OK && (k == 16 || k == 32 || k == 64) && N % 32 == 0) st = upload_full_operands(cb, codewords, rotation);
  if (st == FQ_OK && k == d) {
    // full-vector code: decoded unit vectors Pi^T c_n, summed in fp64 and rounded once to fp32
    float* tab = new (std::nothrow) float[(size_t)N * d];
    if (!tab) return FQ_ERR_HIP;
    for (int n = 0; n < N; n++)
      for (int o = 0; o < d; o++) {
        double acc = 0.0;
        for (int i = 0; i < d; i++) acc += (double)rotation[i * d + o] * (double)codewords[(size_t)n * d + i];
        tab[(size_t)n * d + o] = (float)acc;
      }
    st = upload(&cb->dec_full, tab, (size_t)N * d);
    delete[] tab;
  }
  if (st != FQ_OK || !((k == 4 || k == 8) && N % 32 == 0)) return st;

  const int NT = N / 32;
  _Float16* am = new (std::nothrow) _Float16[(size_t)NT * 64 * 8]();
  float* ci = new (std::nothrow) float[(size_t)NT * 2 * 16];
  float* cs = new (std::nothrow) float[N];
  if (!am || !ci || !cs) {
    delete[] am;
    delete[] ci;
    delete[] cs;
    return FQ_ERR_HIP;
  }
  for (int n = 0; n < N; n++) cs[n] = 256.0f * cn2[n];  // exact power-of-two scaling
  for (int t = 0; t < NT; t++) {
    for (int l = 0; l < 64; l++) {
      const int row = 32 * t + (l % 32), h = l / 32;
      _Float16* a = am + ((size_t)t * 64 + l) * 8;
      for (int j = 0; j < 8; j++) {
        float v = 0.0f;
        if (k == 8) v = codewords[(size_t)row * 8 + j];                 // k = 0..7 and 8..15: c
        else if (h == 0) v = codewords[(size_t)row * 4 + (j & 3)];      // k = 0..3, 4..7: c, c; 8..15: 0
        a[j] = (_Float16)v;
      }
    }
    for (int h = 0; h < 2; h++)
      for (int e = 0; e < 16; e++) ci[((size_t)t * 2 + h) * 16 + e] = cs[32 * t + (e / 4) * 8 + 4 * h + (e % 4)];
  }
  st = upload(&cb->amfma, am, (size_t)NT * 64 * 8);
  if (st == FQ_OK) st = upload(&cb->cinit, ci, (size_t)NT * 2 * 16);
  if (st == FQ_OK) st = upload(&cb->cn2s, cs, (size_t)N);
  delete[] am;
  delete[] ci;
  delete[] cs;
  if (st != FQ_OK) return st;

  // fp16-input encoder.  Rotation: P = 1024 Pi (exact), hi = fp16(P), mid = fp16(P - hi),
  // lo = fp16(P - hi - mid); the differences are exact in fp64.
  _Float16* rt = new (std::nothrow) _Float16[2 * 4 * 3 * 64 * 8];
  _Float16* rc = new (std::nothrow) _Float16[(size_t)N * 8]();
  if (!rt || !rc) {
    delete[] rt;
    delete[] rc;
    return FQ_ERR_HIP;
  }
  for (int s = 0; s < 2; s++)
    for (int r = 0; r < 4; r++)
      for (int l = 0; l < 64; l++)
        for (int j = 0; j < 8; j++) {
          const int rho = l % 16, coord = 16 * (rho / 4) + 4 * r + rho % 4, in = 32 * s + 8 * (l / 16) + j;
          const double P = 1024.0 * (double)rotation[coord * d + in];
          const _Float16 hi = (_Float16)P;
          const _Float16 mid = (_Float16)(P - (double)hi);
          const _Float16 lo = (_Float16)(P - (double)hi - (double)mid);
          const _Float16 parts[3] = {hi, mid, lo};
          for (int p = 0; p < 3; p++) rt[((((s * 4 + r) * 3 + p) * 64) + l) * 8 + j] = parts[p];
        }
  for (int n = 0; n < N; n++) {
    double c2 = 0.0;
    for (int t = 0; t < k; t++) {
      const double v = (double)codewords[(size_t)n * k + t];
      rc[(size_t)n * 8 + t] = (_Float16)v;  // exact: codewords are fp16 values
      c2 += v * v;
    }
    if (k == 4) {  // 256 ||c||^2 as fp16 hi + lo (22 bits)
      const double s2 = 256.0 * c2;
      const _Float16 hi = (_Float16)s2;
      rc[(size_t)n * 8 + 4] = hi;
      rc[(size_t)n * 8 + 5] = (_Float16)(s2 - (double)hi);
    }
  }
  st = upload(&cb->rot16, rt, (size_t)2 * 4 * 3 * 64 * 8);
  if (st == FQ_OK) st = upload(&cb->crec, rc, (size_t)N * 8);
  delete[] rt;
  delete[] rc;
  return st;
}

}  // namespace

FQ_EXPORT const char* fq_status_string(fq_status st) {
  // C callers may pass any int: read its bytes, never the value as the C++ enum type
  int v;
  memcpy(&v, &st, sizeof v);
  switch (v) {
    case FQ_OK: return "ok";
    case FQ_ERR_ARG: return "invalid argument";
    case FQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case FQ_ERR_WORKSPACE: return "workspace missing or too small";
    case FQ_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

FQ_EXPORT fq_status fq_codebook_load(int d, int k, int N, const float* codewords, const float* rotation,
                                     fq_codebook** out) {
  if (!out || !codewords || !rotation) return FQ_ERR_ARG;
  *out = nullptr;
  if (d <= 0 || k <= 0 || N <= 0) return FQ_ERR_ARG;
  if (d != fq::kD) return FQ_ERR_UNSUPPORTED;
  if (d % k != 0 || !is_pow2(k)) return FQ_ERR_ARG;
  if (!is_pow2(N) || N < 2 || N > 65536) return FQ_ERR_ARG;
  const size_t nk = (size_t)N * (size_t)k;
  for (size_t t = 0; t < nk; t++)
    if (!fp16_exact_normal(codewords[t])) return FQ_ERR_ARG;
  for (int t = 0; t < d * d; t++)
    if (!isfinite(rotation[t])) return FQ_ERR_ARG;

  fq_codebook* cb = new (std::nothrow) fq_codebook();
  if (!cb) return FQ_ERR_HIP;
  cb->d = d;
  cb->k = k;
  cb->N = N;
  cb->bits = log2i(N);
  cb->nblk = d / k;
  cb->B = cb->nblk * cb->bits;
  {
    const char* ek = getenv("FQ_ENCODE_KERNEL");
    cb->force_encoder = fq::ENC_AUTO;
    if (ek) {
      if (!strcmp(ek, "valu")) cb->force_encoder = fq::ENC_VALU;
      if (!strcmp(ek, "mfma64") || !strcmp(ek, "mfma")) cb->force_encoder = fq::ENC_MFMA;
      if (!strcmp(ek, "h16")) cb->force_encoder = fq::ENC_H16;
      if (!strcmp(ek, "full")) cb->force_encoder = fq::ENC_FULL;
      if (!strcmp(ek, "small")) cb->force_encoder = fq::ENC_SMALL;
    }
    const char* ak = getenv("FQ_ATTN_KERNEL");
    cb->force_attn_lut = ak && strcmp(ak, "lut") == 0;
    cb->force_attn_gather = ak && strcmp(ak, "gather") == 0;
    const char* dk = getenv("FQ_DECODE_KERNEL");
    cb->force_valu_decode = dk && strcmp(dk, "valu") == 0;
    cb->force_cache_codebook = dk && strcmp(dk, "cached") == 0;
    const char* pk = getenv("FQ_PREFILL_KERNEL");
    cb->prefill_wide = pk && strcmp(pk, "wide") == 0;
  }
  int lds_max = 0;
  if (hipGetDevice(&cb->device) != hipSuccess ||
      hipDeviceGetAttribute(&lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, cb->device) != hipSuccess) {
    delete cb;
    return FQ_ERR_HIP;
  }
  cb->max_lds = (size_t)lds_max;
  {
    // set-up of the no-allocation attention entry point for this device
    void* sp = nullptr;
    const fq_status ss = scratch_address(cb->device, &sp);
    if (ss == FQ_ERR_HIP) {
      delete cb;
      return FQ_ERR_HIP;
    }
  }

  // Host staging: fp16 copy (padded to 16 bytes), ||c||^2, bounds, rotations.
  const size_t cw16_bytes = ((nk * 2 + 15) / 16) * 16;
  _Float16* h16 = new (std::nothrow) _Float16[cw16_bytes / 2]();
  float* hcn2 = new (std::nothrow) float[N];
  double* hpi64t = new (std::nothrow) double[d * d];
  if (!h16 || !hcn2 || !hpi64t) {
    delete[] h16;
    delete[] hcn2;
    delete[] hpi64t;
    delete cb;
    return FQ_ERR_HIP;
  }
  double c2max = 0.0;
  for (int n = 0; n < N; n++) {
    double s = 0.0;
    for (int t = 0; t < k; t++) {
      const double v = codewords[(size_t)n * k + t];
      s += v * v;
      h16[(size_t)n * k + t] = (_Float16)codewords[(size_t)n * k + t];
    }
    hcn2[n] = (float)s;
    if (s > c2max) c2max = s;
  }
  cb->c2max = nextafterf((float)c2max, INFINITY);
  cb->cmax = nextafterf((float)sqrt(c2max), INFINITY);
  {
    // Score error bounds of the fp16-input matrix-core encoders (derivations at the kernels);
    // 1.02 covers the 1.01 slack of the bound and its fp32 evaluation in the kernel.  The
    // rotation term is 512 |c| sqrt(k) times the per-coordinate error of y: 38 u for the
    // k = 4 / 8 encoder (two sums of 32 products added once), 70 u for the k = 16, 32, 64
    // encoder (one chain of 64).
    const double u = 0x1p-24, sk = sqrt((double)k), cm = cb->cmax, c2 = cb->c2max;
    const double rel = 1.02 * (2 * k + 7) * u * 512.0 * cm;
    const double abs_h16 = 1.02 * ((2 * k + 7) * u * 256.0 * c2 + 19456.0 * sk * cm * u + 0x1p-25 * (1.0 + sk * cm));
    const double abs_full = 1.02 * ((2 * k + 7) * u * 256.0 * c2 + 35840.0 * sk * cm * u + 0x1p-25 * (1.0 + sk * cm));
    cb->h16_erel = nextafterf((float)rel, INFINITY);
    cb->h16_eabs = nextafterf((float)abs_h16, INFINITY);
    cb->full_eabs = nextafterf((float)abs_full, INFINITY);
  }
  for (int i = 0; i < d; i++)
    for (int j = 0; j < d; j++) hpi64t[j * d + i] = (double)rotation[i * d + j];

  fq_status st = FQ_OK;
  if (hipMalloc(&cb->cw, nk * sizeof(float)) != hipSuccess || hipMalloc(&cb->cw16, cw16_bytes) != hipSuccess ||
      hipMalloc(&cb->cn2, N * sizeof(float)) != hipSuccess ||
      hipMalloc(&cb->pi64t, (size_t)d * d * sizeof(double)) != hipSuccess ||
      hipMalloc(&cb->pi32, (size_t)d * d * sizeof(float)) != hipSuccess)
    st = FQ_ERR_HIP;
  if (st == FQ_OK &&
      (hipMemcpy(cb->cw, codewords, nk * sizeof(float), hipMemcpyHostToDevice) != hipSuccess ||
       hipMemcpy(cb->cw16, h16, cw16_bytes, hipMemcpyHostToDevice) != hipSuccess ||
       hipMemcpy(cb->cn2, hcn2, N * sizeof(float), hipMemcpyHostToDevice) != hipSuccess ||
       hipMemcpy(cb->pi64t, hpi64t, (size_t)d * d * sizeof(double), hipMemcpyHostToDevice) != hipSuccess ||
       hipMemcpy(cb->pi32, rotation, (size_t)d * d * sizeof(float), hipMemcpyHostToDevice) != hipSuccess))
    st = FQ_ERR_HIP;
  if (st == FQ_OK) st = upload_prefill_rotation(cb, rotation);
  if (st == FQ_OK) st = upload_mfma_operands(cb, codewords, rotation, hcn2);
  delete[] h16;
  delete[] hcn2;
  delete[] hpi64t;
  if (st != FQ_OK) {
    release(cb);
    return st;
  }
  *out = cb;
  return FQ_OK;
}

FQ_EXPORT void fq_codebook_free(fq_codebook* cb) { release(cb); }

FQ_EXPORT int64_t fq_code_bytes(const fq_codebook* cb, int64_t n) {
  if (!cb || n < 0) return -1;
  return (n * (int64_t)cb->B + 7) / 8;
}

FQ_EXPORT fq_status fq_encode(const fq_codebook* cb, const void* x, fq_dtype x_dtype, int64_t n, uint8_t* codes,
                              void* norms, fq_dtype norm_dtype, void* stream) {
  if (!cb || n < 0 || !valid_dtype(x_dtype) || !valid_dtype(norm_dtype)) return FQ_ERR_ARG;
  if (n == 0) return FQ_OK;
  if (!x || !codes || !norms) return FQ_ERR_ARG;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(norms)) return FQ_ERR_ARG;
  if (n > ((int64_t)1 << 40)) return FQ_ERR_UNSUPPORTED;
  const fq_status ds = check_device(cb);
  if (ds != FQ_OK) return ds;
  return fq::launch_encode(cb, x, x_dtype, n, codes, norms, norm_dtype, nullptr, 0, (hipStream_t)stream) ==
                 hipSuccess
             ? FQ_OK
             : FQ_ERR_HIP;
}

FQ_EXPORT const char* fq_encode_kernel(const fq_codebook* cb, fq_dtype x_dtype, int64_t n) {
  if (!cb || n < 0 || !valid_dtype(x_dtype)) return nullptr;
  return fq::encode_kernel_name(fq::encode_kernel(cb, x_dtype, n));
}

FQ_EXPORT fq_status fq_encode_scatter(const fq_codebook* cb, const void* x, fq_dtype x_dtype, int64_t n,
                                      const int64_t* slots, int64_t capacity, uint8_t* codes, void* norms,
                                      fq_dtype norm_dtype, void* stream) {
  if (!cb || n < 0 || capacity < 0 || !valid_dtype(x_dtype) || !valid_dtype(norm_dtype)) return FQ_ERR_ARG;
  if (cb->B % 8 != 0) return FQ_ERR_UNSUPPORTED;  // records must not share bytes
  if (n == 0) return FQ_OK;
  if (!x || !slots || !codes || !norms) return FQ_ERR_ARG;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(norms) || (reinterpret_cast<uintptr_t>(slots) & 7) != 0)
    return FQ_ERR_ARG;
  if (n > ((int64_t)1 << 40) || capacity > ((int64_t)1 << 40)) return FQ_ERR_UNSUPPORTED;
  const fq_status ds = check_device(cb);
  if (ds != FQ_OK) return ds;
  return fq::launch_encode(cb, x, x_dtype, n, codes, norms, norm_dtype, slots, capacity, (hipStream_t)stream) ==
                 hipSuccess
             ? FQ_OK
             : FQ_ERR_HIP;
}

FQ_EXPORT fq_status fq_decode(const fq_codebook* cb, const uint8_t* codes, const void* norms, fq_dtype norm_dtype,
                              int64_t n, void* x_out, fq_dtype out_dtype, void* stream) {
  if (!cb || n < 0 || !valid_dtype(norm_dtype) || !valid_dtype(out_dtype)) return FQ_ERR_ARG;
  if (n == 0) return FQ_OK;
  if (!codes || !norms || !x_out) return FQ_ERR_ARG;
  if (!aligned16(codes) || !aligned16(norms) || !aligned16(x_out)) return FQ_ERR_ARG;
  if (n > ((int64_t)1 << 40)) return FQ_ERR_UNSUPPORTED;
  const fq_status ds = check_device(cb);
  if (ds != FQ_OK) return ds;
  return fq::launch_decode(cb, codes, norms, norm_dtype, n, x_out, out_dtype, (hipStream_t)stream) == hipSuccess
             ? FQ_OK
             : FQ_ERR_HIP;
}

namespace {
// Shapes both attention kernels take; decode attention also needs fq::attn_supported.
fq_status attn_check_shape(const fq_codebook* cb, int B, int Hq, int Hkv, int64_t T) {
  if (!cb || B < 0 || Hq <= 0 || Hkv <= 0 || T < 0) return FQ_ERR_ARG;
  if (Hq % Hkv != 0) return FQ_ERR_ARG;
  if (Hq / Hkv > 16) return FQ_ERR_UNSUPPORTED;
  if (B > 65535 || Hkv > 65535 || (int64_t)B * Hq > ((int64_t)1 << 31) - 1) return FQ_ERR_UNSUPPORTED;
  if (T > ((int64_t)1 << 40)) return FQ_ERR_UNSUPPORTED;
  return FQ_OK;
}

fq_status attn_check_sizes(const fq_codebook* cb, int B, int Hq, int Hkv, int64_t T) {
  const fq_status st = attn_check_shape(cb, B, Hq, Hkv, T);
  if (st != FQ_OK) return st;
  if (!fq::attn_supported(cb)) return FQ_ERR_UNSUPPORTED;
  return FQ_OK;
}
}  // namespace

FQ_EXPORT size_t fq_attn_workspace_bytes(const fq_codebook* cb, int B, int Hq, int Hkv, int64_t T) {
  if (attn_check_sizes(cb, B, Hq, Hkv, T) != FQ_OK || T == 0 || B == 0) return 0;
  const fq::AttnPlan p = fq::attn_plan(cb, B, Hq, Hkv, T);
  if (!fq::attn_plan_launchable(p, B, Hq, Hkv)) return 0;
  return fq::attn_plan_workspace_bytes(cb, p, B, Hq, Hkv);
}

namespace {
// Checks shared by the decode-attention entry points; *launch is false for a no-op.
fq_status attn_validate(const fq_codebook* cb, const void* q, const uint8_t* k_codes, const void* k_norms,
                        const uint8_t* v_codes, const void* v_norms, int B, int Hq, int Hkv, int64_t T, float scale,
                        const float* out, size_t* need, bool* launch) {
  *launch = false;
  const fq_status ss = attn_check_sizes(cb, B, Hq, Hkv, T);
  if (ss != FQ_OK) return ss;
  if (!isfinite(scale)) return FQ_ERR_ARG;
  if (B == 0) return FQ_OK;
  if (!q || !out) return FQ_ERR_ARG;
  if (T == 0) return FQ_OK;  // documented no-op: nothing to attend to
  if (!k_codes || !k_norms || !v_codes || !v_norms) return FQ_ERR_ARG;
  if (!aligned16(q) || !aligned16(k_codes) || !aligned16(k_norms) || !aligned16(v_codes) || !aligned16(v_norms) ||
      !aligned16(out))
    return FQ_ERR_ARG;
  const fq::AttnPlan plan = fq::attn_plan(cb, B, Hq, Hkv, T);
  if (!fq::attn_plan_launchable(plan, B, Hq, Hkv)) return FQ_ERR_UNSUPPORTED;
  *need = fq::attn_plan_workspace_bytes(cb, plan, B, Hq, Hkv);
  *launch = true;
  return FQ_OK;
}

fq_status attn_decode(const fq_codebook* cb, const void* q, const uint8_t* k_codes, const void* k_norms,
                      const uint8_t* v_codes, const void* v_norms, const int32_t* lens, int B, int Hq, int Hkv,
                      int64_t T, float scale, float* out, void* workspace, size_t workspace_bytes, void* stream) {
  size_t need = 0;
  bool launch = false;
  const fq_status vs =
      attn_validate(cb, q, k_codes, k_norms, v_codes, v_norms, B, Hq, Hkv, T, scale, out, &need, &launch);
  if (vs != FQ_OK || !launch) return vs;
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return FQ_ERR_WORKSPACE;
  const fq_status ds = check_device(cb);
  if (ds != FQ_OK) return ds;
  return fq::launch_attn(cb, q, k_codes, k_norms, v_codes, v_norms, lens, B, Hq, Hkv, T, scale, out, workspace,
                         (hipStream_t)stream) == hipSuccess
             ? FQ_OK
             : FQ_ERR_HIP;
}
}  // namespace

FQ_EXPORT size_t fq_attn_noalloc_max_workspace_bytes(void) { return kNoAllocScratchBytes; }

FQ_EXPORT fq_status fq_attn_decode_noalloc(const fq_codebook* cb, const void* q, const uint8_t* k_codes,
                                           const void* k_norms, const uint8_t* v_codes, const void* v_norms,
                                           const int32_t* lens, int B, int Hq, int Hkv, int64_t T, float scale,
                                           float* out, void* stream) {
  if (lens && (reinterpret_cast<uintptr_t>(lens) & 3) != 0) return FQ_ERR_ARG;
  size_t need = 0;
  bool launch = false;
  const fq_status vs =
      attn_validate(cb, q, k_codes, k_norms, v_codes, v_norms, B, Hq, Hkv, T, scale, out, &need, &launch);
  if (vs != FQ_OK || !launch) return vs;
  if (need > kNoAllocScratchBytes) return FQ_ERR_WORKSPACE;
  const fq_status ds = check_device(cb);
  if (ds != FQ_OK) return ds;
  void* ws = nullptr;
  const fq_status ss = scratch_address(cb->device, &ws);
  if (ss != FQ_OK) return ss;
  return fq::launch_attn(cb, q, k_codes, k_norms, v_codes, v_norms, lens, B, Hq, Hkv, T, scale, out, ws,
                         (hipStream_t)stream) == hipSuccess
             ? FQ_OK
             : FQ_ERR_HIP;
}

FQ_EXPORT fq_status fq_attn_decode(const fq_codebook* cb, const void* q, const uint8_t* k_codes, const void* k_norms,
                                   const uint8_t* v_codes, const void* v_norms, int B, int Hq, int Hkv, int64_t T,
                                   float scale, float* out, void* workspace, size_t workspace_bytes, void* stream) {
  return attn_decode(cb, q, k_codes, k_norms, v_codes, v_norms, nullptr, B, Hq, Hkv, T, scale, out, workspace,
                     workspace_bytes, stream);
}

FQ_EXPORT size_t fq_attn_prefill_workspace_bytes(const fq_codebook* cb, int B, int Hq, int Hkv, int Sq, int64_t T) {
  if (attn_check_shape(cb, B, Hq, Hkv, T) != FQ_OK || !fq::prefill_supported(cb) || Sq <= 0 || T == 0 || B == 0)
    return 0;
  if ((int64_t)B * Hq * Sq > ((int64_t)1 << 31) - 1) return 0;
  const fq::PrefillPlan p = fq::prefill_plan(cb, B, Hq, Hkv, Sq, T);
  return ((size_t)B * Hq * Sq * p.nchunks * (2 + fq::kD) * sizeof(float) + 255) & ~(size_t)255;
}

FQ_EXPORT fq_status fq_attn_prefill(const fq_codebook* cb, const void* q, const uint8_t* k_codes, const void* k_norms,
                                    const uint8_t* v_codes, const void* v_norms, int B, int Hq, int Hkv, int Sq,
                                    int64_t T, int causal, float scale, float* out, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  const fq_status ss = attn_check_shape(cb, B, Hq, Hkv, T);
  if (ss != FQ_OK) return ss;
  if (Sq < 0 || (causal != 0 && causal != 1) || !isfinite(scale)) return FQ_ERR_ARG;
  if (!fq::prefill_supported(cb)) return FQ_ERR_UNSUPPORTED;
  if (B == 0 || Sq == 0) return FQ_OK;
  if (!q || !out) return FQ_ERR_ARG;
  if (T == 0) return FQ_OK;  // nothing to attend to
  if ((int64_t)B * Hq * Sq > ((int64_t)1 << 31) - 1 || (int64_t)B * Hkv > 65535) return FQ_ERR_UNSUPPORTED;
  if (fq::prefill_plan(cb, B, Hq, Hkv, Sq, T).rblocks > 65535) return FQ_ERR_UNSUPPORTED;  // grid y
  if (!k_codes || !k_norms || !v_codes || !v_norms) return FQ_ERR_ARG;
  if (!aligned16(q) || !aligned16(k_codes) || !aligned16(k_norms) || !aligned16(v_codes) || !aligned16(v_norms) ||
      !aligned16(out))
    return FQ_ERR_ARG;
  if (!workspace || !aligned16(workspace) ||
      workspace_bytes < fq_attn_prefill_workspace_bytes(cb, B, Hq, Hkv, Sq, T))
    return FQ_ERR_WORKSPACE;
  const fq_status ds = check_device(cb);
  if (ds != FQ_OK) return ds;
  return fq::launch_prefill(cb, q, k_codes, k_norms, v_codes, v_norms, B, Hq, Hkv, Sq, T, causal, scale, out,
                            workspace, (hipStream_t)stream) == hipSuccess
             ? FQ_OK
             : FQ_ERR_HIP;
}

namespace {
bool train_sizes_ok(int k, int N, int64_t m_train, int64_t m_valid) {
  if (k < 1 || k > 64 || (k & (k - 1)) != 0) return false;
  if (N < 1 || N > 65536) return false;
  return m_train >= 1 && m_valid >= 1 && m_train <= INT32_MAX && m_valid <= INT32_MAX;
}
}  // namespace

FQ_EXPORT size_t fq_codebook_train_workspace_bytes(int k, int N, int64_t m_train, int64_t m_valid) {
  if (!train_sizes_ok(k, N, m_train, m_valid)) return 0;
  return fq::train_workspace_bytes(k, N, m_train, m_valid);
}

FQ_EXPORT fq_status fq_codebook_train(int k, int N, const double* train, int64_t m_train, const double* valid,
                                      int64_t m_valid, const double* starts, int restarts, int max_iter,
                                      double rel_tol, float* codewords, double* codewords64,
                                      double* restart_valid_mse, double* valid_mse, double* history,
                                      int* history_len, void* workspace, size_t workspace_bytes, void* stream) {
  if (!train_sizes_ok(k, N, m_train, m_valid)) return FQ_ERR_ARG;
  if (restarts < 1 || max_iter < 0 || !(rel_tol >= 0.0) || !isfinite(rel_tol)) return FQ_ERR_ARG;
  if (!train || !valid || !starts || !codewords) return FQ_ERR_ARG;
  auto al8 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7) == 0; };
  if (!al8(train) || !al8(valid) || !al8(starts) || !aligned16(codewords) || (codewords64 && !al8(codewords64)))
    return FQ_ERR_ARG;
  if (!workspace || !aligned16(workspace) ||
      workspace_bytes < fq::train_workspace_bytes(k, N, m_train, m_valid))
    return FQ_ERR_WORKSPACE;
  return fq::train_codebook(k, N, train, m_train, valid, m_valid, starts, restarts, max_iter, rel_tol, codewords,
                            codewords64, restart_valid_mse, valid_mse, history, history_len, workspace,
                            (hipStream_t)stream) == hipSuccess
             ? FQ_OK
             : FQ_ERR_HIP;
}

FQ_EXPORT fq_status fq_attn_decode_varlen(const fq_codebook* cb, const void* q, const uint8_t* k_codes,
                                          const void* k_norms, const uint8_t* v_codes, const void* v_norms,
                                          const int32_t* lens, int B, int Hq, int Hkv, int64_t T, float scale,
                                          float* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (B > 0 && T > 0 && (!lens || (reinterpret_cast<uintptr_t>(lens) & 3) != 0)) return FQ_ERR_ARG;
  return attn_decode(cb, q, k_codes, k_norms, v_codes, v_norms, lens, B, Hq, Hkv, T, scale, out, workspace,
                     workspace_bytes, stream);
}
