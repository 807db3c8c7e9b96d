// C ABI of libsbl: argument validation, workspace sizing and kernel launches
// on the caller's stream.  Every check runs on the host before any launch, so
// an error return means nothing was enqueued.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>

#include <cmath>
#include <mutex>

#include "sbl_internal.h"

namespace sbl {

static thread_local char g_last_error[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
}

int hip_fail(hipError_t e, const char* what) {
  set_error("%s: %s (%s)", what, hipGetErrorString(e), hipGetErrorName(e));
  return SBL_ERR_HIP;
}

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

#define SBL_REQUIRE(cond, code, ...)   \
  do {                                 \
    if (!(cond)) {                     \
      set_error(__VA_ARGS__);          \
      return (code);                   \
    }                                  \
  } while (0)

static int check_dims(int64_t d_out, int64_t d_in) {
  SBL_REQUIRE(d_in >= 8 && d_in % 8 == 0, SBL_ERR_SHAPE, "d_in=%lld must be a positive multiple of 8",
              (long long)d_in);
  SBL_REQUIRE(d_out >= 1, SBL_ERR_SHAPE, "d_out=%lld must be >= 1", (long long)d_out);
  SBL_REQUIRE(d_in <= SBL_MAX_DIM && d_out <= SBL_MAX_DIM, SBL_ERR_SHAPE, "d_in/d_out above %lld",
              (long long)SBL_MAX_DIM);
  SBL_REQUIRE(d_in * d_out <= SBL_MAX_WEIGHTS, SBL_ERR_SHAPE, "d_out*d_in above %lld", (long long)SBL_MAX_WEIGHTS);
  return SBL_OK;
}

static int check_tokens(int64_t T) {
  SBL_REQUIRE(T >= 0 && T <= SBL_MAX_DIM, SBL_ERR_SHAPE, "T=%lld outside [0, %lld]", (long long)T,
              (long long)SBL_MAX_DIM);
  return SBL_OK;
}

// Scratch of sbl_quant_mask_pack_noalloc: the per-block partial sums of the
// gamma reduction for the largest grid that reduction launches
// (kAbsumMaxBlocks blocks, whatever the matrix size).  Each GPU holds its own
// copy until the process ends.  Every block writes its partial (and its
// histogram when it has one) before the finalize reads it, so nothing needs
// clearing between calls.
constexpr size_t kPackScratchBytes =
    (size_t)kAbsumMaxBlocks * (sizeof(AbsumPartial) + 256 * sizeof(unsigned long long));
static __device__ __align__(256) unsigned char scratch[kPackScratchBytes];

// Device address of `scratch` on the current device, looked up once per
// device (the host-side name is only a handle for the runtime).
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

static int pack_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  SBL_REQUIRE(dev >= 0 && dev < kMaxDevices, SBL_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    SBL_REQUIRE(p != nullptr, SBL_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SBL_OK;
}

}  // namespace sbl

using namespace sbl;

extern "C" {

SBL_API const char* sbl_version(void) { return "sbl 0.1.0 (gfx950)"; }

SBL_API const char* sbl_status_string(int status) {
  switch (status) {
    case SBL_OK: return "ok";
    case SBL_ERR_INVALID_ARG: return "invalid argument";
    case SBL_ERR_SHAPE: return "unsupported shape";
    case SBL_ERR_UNSUPPORTED: return "unsupported option";
    case SBL_ERR_WORKSPACE: return "workspace missing or too small";
    case SBL_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

SBL_API const char* sbl_last_error(void) { return g_last_error; }

SBL_API size_t sbl_quant_mask_pack_workspace_size(int64_t d_out, int64_t d_in) {
  if (check_dims(d_out, d_in) != SBL_OK) return 0;
  return quant_workspace_bytes(d_out, d_in);
}

SBL_API int sbl_quant_mask_pack_nm(const uint16_t* W_bf16, int64_t d_out, int64_t d_in, int n_keep, int m_group,
                                   int flags, uint16_t* codes, uint8_t* mask, float* gamma, void* workspace,
                                   size_t workspace_bytes, void* hip_stream) {
  int rc = check_dims(d_out, d_in);
  if (rc != SBL_OK) return rc;
  SBL_REQUIRE(flags == 0 || flags == SBL_MASK_FROM_QUANTIZED, SBL_ERR_INVALID_ARG, "flags=%d: unknown flag bits",
              flags);
  SBL_REQUIRE(mask_pattern_supported(n_keep, m_group), SBL_ERR_UNSUPPORTED,
              "n_keep=%d, m_group=%d: supported patterns are N:8 and N:4 with 1 <= N <= M", n_keep, m_group);
  SBL_REQUIRE(W_bf16 && codes && gamma, SBL_ERR_INVALID_ARG, "W, codes and gamma must be non-NULL");
  SBL_REQUIRE(aligned(W_bf16, 16) && aligned(codes, 16) && aligned(gamma, 4), SBL_ERR_INVALID_ARG,
              "W and codes must be 16-byte aligned, gamma 4-byte aligned");
  const size_t need = quant_workspace_bytes(d_out, d_in);
  SBL_REQUIRE(workspace && workspace_bytes >= need && aligned(workspace, 16), SBL_ERR_WORKSPACE,
              "workspace of %zu bytes (16-byte aligned) required, got %zu", need,
              workspace ? workspace_bytes : (size_t)0);
  hipError_t e = launch_quant_mask_pack(W_bf16, d_out, d_in, n_keep, m_group, flags == SBL_MASK_FROM_QUANTIZED,
                                        codes, mask, gamma, workspace, (hipStream_t)hip_stream);
  if (e != hipSuccess) return hip_fail(e, "sbl_quant_mask_pack launch");
  return SBL_OK;
}

SBL_API int sbl_quant_mask_pack(const uint16_t* W_bf16, int64_t d_out, int64_t d_in, int n_keep, uint16_t* codes,
                                uint8_t* mask, float* gamma, void* workspace, size_t workspace_bytes,
                                void* hip_stream) {
  return sbl_quant_mask_pack_nm(W_bf16, d_out, d_in, n_keep, 8, 0, codes, mask, gamma, workspace, workspace_bytes,
                                hip_stream);
}

SBL_API int sbl_quant_mask_pack_noalloc(const uint16_t* W_bf16, int64_t d_out, int64_t d_in, int n_keep,
                                        uint16_t* codes, uint8_t* mask, float* gamma, void* hip_stream) {
  int rc = check_dims(d_out, d_in);
  if (rc != SBL_OK) return rc;
  SBL_REQUIRE(mask_pattern_supported(n_keep, 8), SBL_ERR_UNSUPPORTED, "n_keep=%d: supported are 1 <= N <= 8",
              n_keep);
  SBL_REQUIRE(W_bf16 && codes && gamma, SBL_ERR_INVALID_ARG, "W, codes and gamma must be non-NULL");
  SBL_REQUIRE(aligned(W_bf16, 16) && aligned(codes, 16) && aligned(gamma, 4), SBL_ERR_INVALID_ARG,
              "W and codes must be 16-byte aligned, gamma 4-byte aligned");
  const size_t need = quant_workspace_bytes(d_out, d_in);
  SBL_REQUIRE(need <= kPackScratchBytes, SBL_ERR_WORKSPACE,
              "d_out=%lld, d_in=%lld needs %zu bytes of scratch; the static scratch holds %zu",
              (long long)d_out, (long long)d_in, need, kPackScratchBytes);
  void* ws = nullptr;
  rc = pack_scratch(&ws);
  if (rc != SBL_OK) return rc;
  hipError_t e = launch_quant_mask_pack(W_bf16, d_out, d_in, n_keep, 8, false, codes, mask, gamma, ws,
                                        (hipStream_t)hip_stream);
  if (e != hipSuccess) return hip_fail(e, "sbl_quant_mask_pack_noalloc launch");
  return SBL_OK;
}

SBL_API size_t sbl_quant_mask_pack_noalloc_scratch_bytes(void) { return kPackScratchBytes; }

static_assert(SBL_PACK_BATCH_MAX == kPackBatchMax, "batch limit");

SBL_API size_t sbl_quant_mask_pack_batch_workspace_size(int count, const sbl_pack_item* items) {
  if (count < 1 || count > SBL_PACK_BATCH_MAX || !items) return 0;
  int64_t nw[SBL_PACK_BATCH_MAX];
  for (int i = 0; i < count; ++i) {
    if (check_dims(items[i].d_out, items[i].d_in) != SBL_OK) return 0;
    nw[i] = items[i].d_out * items[i].d_in;
  }
  return quant_batch_workspace_bytes(count, nw);
}

SBL_API int sbl_quant_mask_pack_batch(int count, const sbl_pack_item* items, int n_keep, int m_group, int flags,
                                      void* workspace, size_t workspace_bytes, void* hip_stream) {
  SBL_REQUIRE(items && count >= 1 && count <= SBL_PACK_BATCH_MAX, SBL_ERR_INVALID_ARG,
              "count=%d: 1..%d items (host array) required", count, SBL_PACK_BATCH_MAX);
  SBL_REQUIRE(flags == 0 || flags == SBL_MASK_FROM_QUANTIZED, SBL_ERR_INVALID_ARG, "flags=%d: unknown flag bits",
              flags);
  SBL_REQUIRE(mask_pattern_supported(n_keep, m_group), SBL_ERR_UNSUPPORTED,
              "n_keep=%d, m_group=%d: supported patterns are N:8 and N:4 with 1 <= N <= M", n_keep, m_group);
  PackItem it[SBL_PACK_BATCH_MAX];
  int64_t nw[SBL_PACK_BATCH_MAX];
  for (int i = 0; i < count; ++i) {
    const sbl_pack_item& q = items[i];
    const int rc = check_dims(q.d_out, q.d_in);
    if (rc != SBL_OK) return rc;
    SBL_REQUIRE(q.W_bf16 && q.codes && q.gamma, SBL_ERR_INVALID_ARG, "item %d: W, codes and gamma must be non-NULL",
                i);
    SBL_REQUIRE(aligned(q.W_bf16, 16) && aligned(q.codes, 16) && aligned(q.gamma, 4), SBL_ERR_INVALID_ARG,
                "item %d: W and codes must be 16-byte aligned, gamma 4-byte aligned", i);
    it[i] = PackItem{q.W_bf16, q.d_out, q.d_in, q.codes, q.mask, q.gamma};
    nw[i] = q.d_out * q.d_in;
  }
  const size_t need = quant_batch_workspace_bytes(count, nw);
  SBL_REQUIRE(workspace && workspace_bytes >= need && aligned(workspace, 16), SBL_ERR_WORKSPACE,
              "workspace of %zu bytes (16-byte aligned) required, got %zu", need,
              workspace ? workspace_bytes : (size_t)0);
  hipError_t e = launch_quant_mask_pack_batch(count, it, n_keep, m_group, flags == SBL_MASK_FROM_QUANTIZED,
                                              workspace, (hipStream_t)hip_stream);
  if (e != hipSuccess) return hip_fail(e, "sbl_quant_mask_pack_batch launch");
  return SBL_OK;
}

SBL_API int sbl_mask_grad(float* dW, const uint8_t* mask, int64_t d_out, int64_t d_in, void* hip_stream) {
  int rc = check_dims(d_out, d_in);
  if (rc != SBL_OK) return rc;
  SBL_REQUIRE(dW && mask, SBL_ERR_INVALID_ARG, "dW and mask must be non-NULL");
  SBL_REQUIRE(aligned(dW, 16), SBL_ERR_INVALID_ARG, "dW must be 16-byte aligned");
  hipError_t e = launch_mask_grad(dW, mask, d_out, d_in, (hipStream_t)hip_stream);
  if (e != hipSuccess) return hip_fail(e, "sbl_mask_grad launch");
  return SBL_OK;
}

SBL_API size_t sbl_adamw_repack_workspace_size(int64_t d_out, int64_t d_in) {
  if (check_dims(d_out, d_in) != SBL_OK) return 0;
  return quant_workspace_bytes(d_out, d_in);
}

SBL_API int sbl_adamw_repack(uint16_t* W_bf16, const float* dW, float* m, float* v, int64_t d_out, int64_t d_in,
                             const sbl_adamw_params* hp, int n_keep, int m_group, const uint8_t* mask_prev,
                             uint8_t* mask, uint16_t* codes, float* gamma, uint64_t* flips, void* workspace,
                             size_t workspace_bytes, void* hip_stream) {
  int rc = check_dims(d_out, d_in);
  if (rc != SBL_OK) return rc;
  SBL_REQUIRE(hp, SBL_ERR_INVALID_ARG, "hp (host pointer) must be non-NULL");
  const bool fin = std::isfinite(hp->lr) && std::isfinite(hp->beta1) && std::isfinite(hp->beta2) &&
                   std::isfinite(hp->eps) && std::isfinite(hp->weight_decay) && std::isfinite(hp->grad_scale);
  SBL_REQUIRE(fin && hp->step >= 1 && hp->beta1 >= 0.0f && hp->beta1 < 1.0f && hp->beta2 >= 0.0f &&
                  hp->beta2 < 1.0f && hp->eps > 0.0f && hp->lr >= 0.0f && hp->weight_decay >= 0.0f &&
                  hp->grad_scale >= 0.0f,
              SBL_ERR_INVALID_ARG, "AdamW parameters out of range (step >= 1, 0 <= beta < 1, eps > 0, lr, wd, "
              "grad_scale >= 0, all finite)");
  SBL_REQUIRE(mask_pattern_supported(n_keep, m_group), SBL_ERR_UNSUPPORTED,
              "n_keep=%d, m_group=%d: supported patterns are N:8 and N:4 with 1 <= N <= M", n_keep, m_group);
  SBL_REQUIRE(W_bf16 && dW && m && v && mask && codes && gamma, SBL_ERR_INVALID_ARG,
              "W, dW, m, v, mask, codes and gamma must be non-NULL");
  SBL_REQUIRE(aligned(W_bf16, 16) && aligned(dW, 16) && aligned(m, 16) && aligned(v, 16) && aligned(codes, 16) &&
                  aligned(gamma, 4) && (!flips || aligned(flips, 8)),
              SBL_ERR_INVALID_ARG, "W, dW, m, v, codes must be 16-byte aligned; gamma 4-byte, flips 8-byte");
  const size_t need = quant_workspace_bytes(d_out, d_in);
  SBL_REQUIRE(workspace && workspace_bytes >= need && aligned(workspace, 16), SBL_ERR_WORKSPACE,
              "workspace of %zu bytes (16-byte aligned) required, got %zu", need,
              workspace ? workspace_bytes : (size_t)0);
  AdamwArgs a{hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay, hp->grad_scale, hp->step};
  hipError_t e = launch_adamw_repack(W_bf16, dW, m, v, d_out, d_in, a, n_keep, m_group, mask_prev, mask, codes,
                                     gamma, (unsigned long long*)flips, workspace, (hipStream_t)hip_stream);
  if (e != hipSuccess) return hip_fail(e, "sbl_adamw_repack launch");
  return SBL_OK;
}

SBL_API int sbl_act_quant(const uint16_t* x_bf16, int64_t T, int64_t d_in, int8_t* x_q, float* absmax,
                          void* hip_stream) {
  int rc = check_tokens(T);
  if (rc != SBL_OK) return rc;
  rc = check_dims(1, d_in);
  if (rc != SBL_OK) return rc;
  if (T == 0) return SBL_OK;
  SBL_REQUIRE(x_bf16 && x_q && absmax, SBL_ERR_INVALID_ARG, "x, x_q and absmax must be non-NULL");
  SBL_REQUIRE(aligned(x_bf16, 16) && aligned(x_q, 16) && aligned(absmax, 4), SBL_ERR_INVALID_ARG,
              "x and x_q must be 16-byte aligned, absmax 4-byte aligned");
  SBL_REQUIRE(T * d_in <= SBL_MAX_WEIGHTS * 16, SBL_ERR_SHAPE, "T*d_in too large");
  hipError_t e = launch_act_quant(x_bf16, T, d_in, x_q, absmax, (hipStream_t)hip_stream);
  if (e != hipSuccess) return hip_fail(e, "sbl_act_quant launch");
  return SBL_OK;
}

SBL_API int sbl_rmsnorm_act_quant(const uint16_t* x_bf16, const uint16_t* g_bf16, float eps, int64_t T, int64_t d_in,
                                  int8_t* x_q, float* absmax, float* rstd, void* hip_stream) {
  int rc = check_tokens(T);
  if (rc != SBL_OK) return rc;
  SBL_REQUIRE(d_in >= 8 && d_in % 8 == 0, SBL_ERR_SHAPE, "d_in=%lld must be a positive multiple of 8",
              (long long)d_in);
  SBL_REQUIRE(rmsnorm_supported(d_in), SBL_ERR_UNSUPPORTED, "d_in=%lld: rows up to 16384 are supported",
              (long long)d_in);
  SBL_REQUIRE(std::isfinite(eps) && eps > 0.0f, SBL_ERR_INVALID_ARG, "eps must be finite and > 0");
  if (T == 0) return SBL_OK;
  SBL_REQUIRE(x_bf16 && x_q && absmax, SBL_ERR_INVALID_ARG, "x, x_q and absmax must be non-NULL");
  SBL_REQUIRE(aligned(x_bf16, 16) && aligned(x_q, 16) && aligned(absmax, 4) && (!g_bf16 || aligned(g_bf16, 16)) &&
                  aligned(rstd, 4),
              SBL_ERR_INVALID_ARG, "x, g, x_q must be 16-byte aligned; absmax and rstd 4-byte aligned");
  hipError_t e =
      launch_rmsnorm_act_quant(x_bf16, g_bf16, eps, T, d_in, x_q, absmax, rstd, (hipStream_t)hip_stream);
  if (e != hipSuccess) return hip_fail(e, "sbl_rmsnorm_act_quant launch");
  return SBL_OK;
}

SBL_API int sbl_forward(const uint16_t* codes, const float* gamma, const int8_t* x_q, const float* absmax, int64_t T,
                        int64_t d_in, int64_t d_out, void* y, int y_dtype, void* hip_stream) {
  int rc = check_tokens(T);
  if (rc != SBL_OK) return rc;
  rc = check_dims(d_out, d_in);
  if (rc != SBL_OK) return rc;
  SBL_REQUIRE(y_dtype == SBL_F32 || y_dtype == SBL_BF16 || y_dtype == SBL_I32, SBL_ERR_INVALID_ARG,
              "y_dtype=%d is not SBL_F32, SBL_BF16 or SBL_I32", y_dtype);
  if (T == 0) return SBL_OK;
  SBL_REQUIRE(codes && gamma && x_q && absmax && y, SBL_ERR_INVALID_ARG, "NULL pointer argument");
  SBL_REQUIRE(aligned(codes, 16) && aligned(x_q, 16) && aligned(y, 16) && aligned(gamma, 4) && aligned(absmax, 4),
              SBL_ERR_INVALID_ARG, "codes, x_q, y must be 16-byte aligned; gamma, absmax 4-byte aligned");
  hipError_t e = launch_forward(codes, gamma, x_q, absmax, T, d_in, d_out, y, y_dtype, (hipStream_t)hip_stream);
  if (e != hipSuccess) return hip_fail(e, "sbl_forward launch");
  return SBL_OK;
}

SBL_API int sbl_decode_supported(int64_t T, int64_t d_in) { return decode_fused_supported(T, d_in) ? 1 : 0; }

SBL_API int sbl_decode(const uint16_t* codes, const float* gamma, const uint16_t* x_bf16, int64_t T, int64_t d_in,
                       int64_t d_out, void* y, int y_dtype, void* hip_stream) {
  int rc = check_tokens(T);
  if (rc != SBL_OK) return rc;
  rc = check_dims(d_out, d_in);
  if (rc != SBL_OK) return rc;
  SBL_REQUIRE(y_dtype == SBL_F32 || y_dtype == SBL_BF16 || y_dtype == SBL_I32, SBL_ERR_INVALID_ARG,
              "y_dtype=%d is not SBL_F32, SBL_BF16 or SBL_I32", y_dtype);
  if (T == 0) return SBL_OK;
  SBL_REQUIRE(decode_fused_supported(T, d_in), SBL_ERR_UNSUPPORTED,
              "sbl_decode takes 1 <= T <= 16, d_in %% 64 == 0, T * d_in <= 65536, T * (d_in + 16) <= 56832 "
              "(got T=%lld, d_in=%lld); "
              "use sbl_act_quant + sbl_forward",
              (long long)T, (long long)d_in);
  SBL_REQUIRE(codes && gamma && x_bf16 && y, SBL_ERR_INVALID_ARG, "NULL pointer argument");
  SBL_REQUIRE(aligned(codes, 16) && aligned(x_bf16, 16) && aligned(y, 16) && aligned(gamma, 4), SBL_ERR_INVALID_ARG,
              "codes, x, y must be 16-byte aligned; gamma 4-byte aligned");
  const DecodeItem it{codes, gamma, d_out, y};
  hipError_t e = launch_decode_plane(SBL_PLANE_CODES, 1, &it, true, x_bf16, nullptr, T, d_in, y_dtype,
                                     (hipStream_t)hip_stream);
  if (e != hipSuccess) return hip_fail(e, "sbl_decode launch");
  return SBL_OK;
}

static_assert(SBL_DECODE_MULTI_MAX == kDecodeMultiMax, "decode group limit");

// Shared checks of the multi-matrix decode entry points; fills it[].
static int check_decode_items(int count, const sbl_decode_item* items, int64_t d_in, int y_dtype, DecodeItem* it) {
  SBL_REQUIRE(items && count >= 1 && count <= SBL_DECODE_MULTI_MAX, SBL_ERR_INVALID_ARG,
              "count=%d: 1..%d items (host array) required", count, SBL_DECODE_MULTI_MAX);
  SBL_REQUIRE(y_dtype == SBL_F32 || y_dtype == SBL_BF16 || y_dtype == SBL_I32, SBL_ERR_INVALID_ARG,
              "y_dtype=%d is not SBL_F32, SBL_BF16 or SBL_I32", y_dtype);
  for (int i = 0; i < count; ++i) {
    const sbl_decode_item& q = items[i];
    const int rc = check_dims(q.d_out, d_in);
    if (rc != SBL_OK) return rc;
    SBL_REQUIRE(q.codes && q.gamma && q.y, SBL_ERR_INVALID_ARG, "item %d: codes, gamma and y must be non-NULL", i);
    SBL_REQUIRE(aligned(q.codes, 16) && aligned(q.y, 16) && aligned(q.gamma, 4), SBL_ERR_INVALID_ARG,
                "item %d: codes and y must be 16-byte aligned, gamma 4-byte aligned", i);
    it[i] = DecodeItem{q.codes, q.gamma, q.d_out, q.y};
  }
  return SBL_OK;
}

SBL_API int sbl_decode_multi(int count, const sbl_decode_item* items, const uint16_t* x_bf16, int64_t T,
                             int64_t d_in, int y_dtype, void* hip_stream) {
  DecodeItem it[SBL_DECODE_MULTI_MAX];
  int rc = check_tokens(T);
  if (rc != SBL_OK) return rc;
  rc = check_decode_items(count, items, d_in, y_dtype, it);
  if (rc != SBL_OK) return rc;
  if (T == 0) return SBL_OK;
  SBL_REQUIRE(decode_fused_supported(T, d_in), SBL_ERR_UNSUPPORTED,
              "sbl_decode_multi takes what sbl_decode takes (got T=%lld, d_in=%lld); "
              "use sbl_act_quant + sbl_forward_decode_multi",
              (long long)T, (long long)d_in);
  SBL_REQUIRE(x_bf16 && aligned(x_bf16, 16), SBL_ERR_INVALID_ARG, "x must be non-NULL and 16-byte aligned");
  hipError_t e = launch_decode_plane(SBL_PLANE_CODES, count, it, true, x_bf16, nullptr, T, d_in, y_dtype,
                                     (hipStream_t)hip_stream);
  if (e != hipSuccess) return hip_fail(e, "sbl_decode_multi launch");
  return SBL_OK;
}

SBL_API int sbl_forward_decode_multi(int count, const sbl_decode_item* items, const int8_t* x_q, const float* absmax,
                                     int64_t T, int64_t d_in, int y_dtype, void* hip_stream) {
  DecodeItem it[SBL_DECODE_MULTI_MAX];
  int rc = check_tokens(T);
  if (rc != SBL_OK) return rc;
  rc = check_decode_items(count, items, d_in, y_dtype, it);
  if (rc != SBL_OK) return rc;
  SBL_REQUIRE(T <= 64 && d_in % 64 == 0, SBL_ERR_UNSUPPORTED,
              "sbl_forward_decode_multi takes T <= 64 and d_in %% 64 == 0 (got T=%lld, d_in=%lld); use sbl_forward",
              (long long)T, (long long)d_in);
  if (T == 0) return SBL_OK;
  SBL_REQUIRE(x_q && absmax && aligned(x_q, 16) && aligned(absmax, 4), SBL_ERR_INVALID_ARG,
              "x_q (16-byte aligned) and absmax (4-byte aligned) must be non-NULL");
  hipError_t e = launch_decode_plane(SBL_PLANE_CODES, count, it, false, x_q, absmax, T, d_in, y_dtype,
                                     (hipStream_t)hip_stream);
  if (e != hipSuccess) return hip_fail(e, "sbl_forward_decode_multi launch");
  return SBL_OK;
}

SBL_API int sbl_pack_pairs(const uint16_t* codes, int64_t d_out, int64_t d_in, uint8_t* plane, uint64_t* bad,
                           void* hip_stream) {
  int rc = check_dims(d_out, d_in);
  if (rc != SBL_OK) return rc;
  SBL_REQUIRE(codes && plane, SBL_ERR_INVALID_ARG, "codes and plane must be non-NULL");
  SBL_REQUIRE(aligned(codes, 16) && aligned(plane, 16) && (!bad || aligned(bad, 8)), SBL_ERR_INVALID_ARG,
              "codes and plane must be 16-byte aligned, bad 8-byte aligned");
  hipError_t e = launch_pack_pairs(codes, d_out, d_in, plane, (unsigned long long*)bad, (hipStream_t)hip_stream);
  if (e != hipSuccess) return hip_fail(e, "sbl_pack_pairs launch");
  return SBL_OK;
}

SBL_API int sbl_decode_plane_supported(int format, int64_t T, int64_t d_in) {
  return (format == SBL_PLANE_CODES || format == SBL_PLANE_PAIRS) && decode_fused_plane_supported(format, T, d_in);
}

SBL_API int sbl_forward_plane_multi(int format, int count, const sbl_decode_item* items, const int8_t* x_q,
                                    const float* absmax, const uint16_t* x_bf16, int64_t T, int64_t d_in,
                                    int y_dtype, void* hip_stream) {
  DecodeItem it[SBL_DECODE_MULTI_MAX];
  SBL_REQUIRE(format == SBL_PLANE_CODES || format == SBL_PLANE_PAIRS, SBL_ERR_INVALID_ARG,
              "format=%d is not SBL_PLANE_CODES or SBL_PLANE_PAIRS", format);
  int rc = check_tokens(T);
  if (rc != SBL_OK) return rc;
  rc = check_decode_items(count, items, d_in, y_dtype, it);
  if (rc != SBL_OK) return rc;
  const bool fused = x_bf16 != nullptr;
  SBL_REQUIRE(fused != (x_q != nullptr) && (fused || absmax), SBL_ERR_INVALID_ARG,
              "give either x_bf16 (quantization fused in) or x_q and absmax");
  SBL_REQUIRE(decode_plane_supported(format, T, d_in), SBL_ERR_UNSUPPORTED,
              "T=%lld, d_in=%lld: T <= 64 and d_in a multiple of %d are required", (long long)T, (long long)d_in,
              format == SBL_PLANE_PAIRS ? 128 : 64);
  SBL_REQUIRE(!fused || T == 0 || decode_fused_plane_supported(format, T, d_in), SBL_ERR_UNSUPPORTED,
              "T=%lld, d_in=%lld: outside the fused form's range", (long long)T, (long long)d_in);
  if (T == 0) return SBL_OK;
  SBL_REQUIRE(fused ? aligned(x_bf16, 16) : (aligned(x_q, 16) && aligned(absmax, 4)), SBL_ERR_INVALID_ARG,
              "x_bf16 and x_q must be 16-byte aligned, absmax 4-byte aligned");
  hipError_t e = launch_decode_plane(format, count, it, fused, fused ? (const void*)x_bf16 : (const void*)x_q,
                                     absmax, T, d_in, y_dtype, (hipStream_t)hip_stream);
  if (e != hipSuccess) return hip_fail(e, "sbl_forward_plane_multi launch");
  return SBL_OK;
}

SBL_API int sbl_pack_sparse24(const uint16_t* codes, int64_t d_out, int64_t d_in, uint8_t* plane, uint64_t* bad,
                              void* hip_stream) {
  int rc = check_dims(d_out, d_in);
  if (rc != SBL_OK) return rc;
  SBL_REQUIRE(d_in % 64 == 0, SBL_ERR_SHAPE, "d_in=%lld must be a multiple of 64", (long long)d_in);
  SBL_REQUIRE(codes && plane, SBL_ERR_INVALID_ARG, "codes and plane must be non-NULL");
  SBL_REQUIRE(aligned(codes, 16) && aligned(plane, 16) && (!bad || aligned(bad, 8)), SBL_ERR_INVALID_ARG,
              "codes and plane must be 16-byte aligned, bad 8-byte aligned");
  hipError_t e = launch_pack_sparse24(codes, d_out, d_in, plane, (unsigned long long*)bad, (hipStream_t)hip_stream);
  if (e != hipSuccess) return hip_fail(e, "sbl_pack_sparse24 launch");
  return SBL_OK;
}

SBL_API int sbl_forward_sparse24(const uint8_t* plane, const float* gamma, const int8_t* x_q, const float* absmax,
                                 int64_t T, int64_t d_in, int64_t d_out, void* y, int y_dtype, void* hip_stream) {
  int rc = check_tokens(T);
  if (rc != SBL_OK) return rc;
  rc = check_dims(d_out, d_in);
  if (rc != SBL_OK) return rc;
  SBL_REQUIRE(y_dtype == SBL_F32 || y_dtype == SBL_BF16 || y_dtype == SBL_I32, SBL_ERR_INVALID_ARG,
              "y_dtype=%d is not SBL_F32, SBL_BF16 or SBL_I32", y_dtype);
  SBL_REQUIRE(forward_sparse24_supported(d_in), SBL_ERR_UNSUPPORTED, "d_in=%lld: a multiple of 128 is required",
              (long long)d_in);
  if (T == 0) return SBL_OK;
  SBL_REQUIRE(plane && gamma && x_q && absmax && y, SBL_ERR_INVALID_ARG, "NULL pointer argument");
  SBL_REQUIRE(aligned(plane, 16) && aligned(x_q, 16) && aligned(y, 16) && aligned(gamma, 4) && aligned(absmax, 4),
              SBL_ERR_INVALID_ARG, "plane, x_q, y must be 16-byte aligned; gamma, absmax 4-byte aligned");
  hipError_t e = launch_forward_sparse24(plane, gamma, x_q, absmax, T, d_in, d_out, y, y_dtype,
                                         (hipStream_t)hip_stream);
  if (e != hipSuccess) return hip_fail(e, "sbl_forward_sparse24 launch");
  return SBL_OK;
}

SBL_API size_t sbl_backward_workspace_size(int64_t T, int64_t d_in, int64_t d_out, int flags) {
  if (check_tokens(T) != SBL_OK || check_dims(d_out, d_in) != SBL_OK) return 0;
  return backward_workspace_bytes(T, d_in, d_out, flags);
}

SBL_API int sbl_backward(const uint16_t* codes, const float* gamma, const int8_t* x_q, const float* absmax,
                         const uint16_t* dY_bf16, int64_t T, int64_t d_in, int64_t d_out, void* dX, int dx_dtype,
                         float* dW, int flags, void* workspace, size_t workspace_bytes, void* hip_stream) {
  int rc = check_tokens(T);
  if (rc != SBL_OK) return rc;
  rc = check_dims(d_out, d_in);
  if (rc != SBL_OK) return rc;
  SBL_REQUIRE(flags >= 1 && flags <= (SBL_BWD_DX | SBL_BWD_DW), SBL_ERR_INVALID_ARG,
              "flags=%d must be a non-empty combination of SBL_BWD_DX and SBL_BWD_DW", flags);
  if (flags & SBL_BWD_DX) {
    SBL_REQUIRE(dx_dtype == SBL_F32 || dx_dtype == SBL_BF16, SBL_ERR_INVALID_ARG,
                "dx_dtype=%d is not SBL_F32 or SBL_BF16", dx_dtype);
    if (T > 0) {
      SBL_REQUIRE(dX && codes && gamma && dY_bf16, SBL_ERR_INVALID_ARG, "dX, codes, gamma, dY must be non-NULL");
      SBL_REQUIRE(aligned(dX, 16) && aligned(codes, 16) && aligned(dY_bf16, 16) && aligned(gamma, 4),
                  SBL_ERR_INVALID_ARG, "dX, codes, dY must be 16-byte aligned; gamma 4-byte aligned");
    }
  }
  if (flags & SBL_BWD_DW) {
    SBL_REQUIRE(dW && aligned(dW, 16), SBL_ERR_INVALID_ARG, "dW must be non-NULL and 16-byte aligned");
    if (T > 0) {
      SBL_REQUIRE(x_q && absmax && dY_bf16, SBL_ERR_INVALID_ARG, "x_q, absmax, dY must be non-NULL");
      SBL_REQUIRE(aligned(x_q, 16) && aligned(absmax, 4) && aligned(dY_bf16, 16), SBL_ERR_INVALID_ARG,
                  "x_q, dY must be 16-byte aligned; absmax 4-byte aligned");
    }
  }
  const size_t need = backward_workspace_bytes(T, d_in, d_out, flags);
  if (need > 0) {
    SBL_REQUIRE(workspace && workspace_bytes >= need && aligned(workspace, 16), SBL_ERR_WORKSPACE,
                "workspace of %zu bytes (16-byte aligned) required, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  }
  if (T == 0 && !(flags & SBL_BWD_DW)) return SBL_OK;
  hipError_t e = launch_backward(codes, gamma, x_q, absmax, dY_bf16, T, d_in, d_out, dX, dx_dtype, dW, flags,
                                 workspace, (hipStream_t)hip_stream);
  if (e != hipSuccess) return hip_fail(e, "sbl_backward launch");
  return SBL_OK;
}

SBL_API int sbl_test_round_mean(const uint32_t* S_words, int n_words, int64_t count, float* out) {
  SBL_REQUIRE(S_words && out && n_words >= 1 && n_words <= 10, SBL_ERR_INVALID_ARG, "bad arguments");
  SBL_REQUIRE(count >= 1 && count <= SBL_MAX_WEIGHTS, SBL_ERR_SHAPE, "count outside [1, 2^36]");
  uint32_t w[10] = {0};
  for (int i = 0; i < n_words; ++i) w[i] = S_words[i];
  *out = round_mean_words(w, 10, (unsigned long long)count);
  return SBL_OK;
}

SBL_API int sbl_peak_mfma(int kind, int64_t iters, int blocks, float* sink, void* hip_stream) {
  SBL_REQUIRE(kind == 0 || kind == 1, SBL_ERR_INVALID_ARG, "kind=%d: 0 (int8) or 1 (bf16)", kind);
  SBL_REQUIRE(iters >= 1 && iters <= ((int64_t)1 << 40), SBL_ERR_INVALID_ARG, "iters=%lld out of range",
              (long long)iters);
  SBL_REQUIRE(blocks >= 1 && blocks <= 65536, SBL_ERR_INVALID_ARG, "blocks=%d out of [1, 65536]", blocks);
  SBL_REQUIRE(sink && aligned(sink, 4), SBL_ERR_INVALID_ARG, "sink must be a non-NULL float buffer of blocks");
  hipError_t e = launch_mfma_peak(kind, iters, blocks, sink, (hipStream_t)hip_stream);
  if (e != hipSuccess) return hip_fail(e, "sbl_peak_mfma launch");
  return SBL_OK;
}

SBL_API int sbl_peak_read(const void* src, int64_t bytes, uint32_t* sink, void* hip_stream) {
  SBL_REQUIRE(src && aligned(src, 16) && bytes >= 16 && bytes % 16 == 0, SBL_ERR_INVALID_ARG,
              "src must be 16-byte aligned and bytes a positive multiple of 16");
  SBL_REQUIRE(sink && aligned(sink, 4), SBL_ERR_INVALID_ARG, "sink must be a non-NULL uint32");
  hipError_t e = launch_read_peak(src, bytes, sink, (hipStream_t)hip_stream);
  if (e != hipSuccess) return hip_fail(e, "sbl_peak_read launch");
  return SBL_OK;
}

}  // extern "C"
