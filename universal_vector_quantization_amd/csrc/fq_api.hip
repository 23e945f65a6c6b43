// Host side of the C ABI in include/fq.h: argument checks (before any HIP call
// where possible), codebook upload, and dispatch to the kernel launchers.
#include <math.h>
#include <string.h>

#include <new>

#include "fq_internal.h"

#define FQ_EXPORT extern "C" __attribute__((visibility("default")))

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

void release(fq_codebook* cb) {
  if (!cb) return;
  (void)hipFree(cb->cw);
  (void)hipFree(cb->cw16);
  (void)hipFree(cb->cn2);
  (void)hipFree(cb->pi64t);
  (void)hipFree(cb->pi32);
  delete cb;
}

}  // namespace

FQ_EXPORT const char* fq_status_string(fq_status st) {
  switch (st) {
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
  if (hipGetDevice(&cb->device) != hipSuccess) {
    delete cb;
    return FQ_ERR_HIP;
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
  return fq::launch_encode(cb, x, x_dtype, n, codes, norms, norm_dtype, (hipStream_t)stream) == hipSuccess
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
fq_status attn_check_sizes(const fq_codebook* cb, int B, int Hq, int Hkv, int64_t T) {
  if (!cb || B < 0 || Hq <= 0 || Hkv <= 0 || T < 0) return FQ_ERR_ARG;
  if (Hq % Hkv != 0) return FQ_ERR_ARG;
  if (Hq / Hkv > 16) return FQ_ERR_UNSUPPORTED;
  if ((int64_t)cb->N * cb->k > 16384) return FQ_ERR_UNSUPPORTED;
  if (B > 65535 || Hkv > 65535 || (int64_t)B * Hq > ((int64_t)1 << 31) - 1) return FQ_ERR_UNSUPPORTED;
  if (T > ((int64_t)1 << 40)) return FQ_ERR_UNSUPPORTED;
  return FQ_OK;
}
}  // namespace

FQ_EXPORT size_t fq_attn_workspace_bytes(const fq_codebook* cb, int B, int Hq, int Hkv, int64_t T) {
  if (attn_check_sizes(cb, B, Hq, Hkv, T) != FQ_OK || T == 0 || B == 0) return 0;
  return fq::attn_workspace_bytes(B, Hq, fq::attn_plan(B, Hkv, T).nchunks);
}

FQ_EXPORT fq_status fq_attn_decode(const fq_codebook* cb, const void* q, const uint8_t* k_codes, const void* k_norms,
                                   const uint8_t* v_codes, const void* v_norms, int B, int Hq, int Hkv, int64_t T,
                                   float scale, float* out, void* workspace, size_t workspace_bytes, void* stream) {
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
  const size_t need = fq::attn_workspace_bytes(B, Hq, fq::attn_plan(B, Hkv, T).nchunks);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return FQ_ERR_WORKSPACE;
  const fq_status ds = check_device(cb);
  if (ds != FQ_OK) return ds;
  return fq::launch_attn(cb, q, k_codes, k_norms, v_codes, v_norms, B, Hq, Hkv, T, scale, out, workspace,
                         (hipStream_t)stream) == hipSuccess
             ? FQ_OK
             : FQ_ERR_HIP;
}
