// C ABI: argument validation, error reporting and dispatch to the HIP kernels.
// Every check runs on the host before anything is launched; the device is only
// queried (once per device, for its architecture) after the arguments pass.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/mxfp8.h"

hipError_t mx_launch_dim0(const uint16_t*, int64_t, int64_t, int64_t, uint8_t*, uint8_t*, int, hipStream_t);
hipError_t mx_launch_dim1(const uint16_t*, int64_t, int64_t, int64_t, int64_t, uint8_t*, uint8_t*, int, hipStream_t);
hipError_t mx_launch_both(const uint16_t*, int64_t, int64_t, int64_t, int64_t, uint8_t*, uint8_t*, uint8_t*, uint8_t*,
                          int, int, hipStream_t);
hipError_t mx_launch_w32(const uint16_t*, int64_t, int64_t, int64_t, int64_t, uint8_t*, uint8_t*, uint8_t*, uint8_t*,
                         hipStream_t);
hipError_t mx_launch_pad(const uint16_t*, int64_t, int64_t, int64_t, const int32_t*, int, uint16_t*, int64_t, int32_t*,
                         hipStream_t);
hipError_t mx_launch_unpad(const void*, int64_t, int64_t, int64_t, const int32_t*, int, void*, int64_t, int64_t,
                           hipStream_t);
hipError_t mx_launch_dequant(const uint8_t*, const uint8_t*, int64_t, int64_t, int64_t, int, uint16_t*, hipStream_t);
hipError_t mx_launch_transpose_bf16(const uint16_t*, int64_t, int64_t, int64_t, int64_t, uint16_t*, hipStream_t);
hipError_t mx_launch_scales_logical(const uint8_t*, int64_t, int64_t, uint8_t*, hipStream_t);
hipError_t mx_launch_gemm_bf16_mgroup(const uint16_t*, const uint16_t*, const int32_t*, int, int64_t, int64_t, int64_t,
                                      void*, int, hipStream_t);
hipError_t mx_launch_gemm_bf16_kgroup(const uint16_t*, const uint16_t*, const int32_t*, int, int64_t, int64_t, int64_t,
                                      void*, int, void*, int64_t, hipStream_t);
hipError_t mx_launch_gemm_mgroup(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, const int32_t*,
                                 const int32_t*, int, int64_t, int64_t, int64_t, int64_t, void*, int, hipStream_t);
hipError_t mx_launch_check_offs(const int32_t*, int, int64_t, int, int32_t*, hipStream_t);
hipError_t mx_launch_probe_mfma(int64_t, float*, hipStream_t);
hipError_t mx_launch_probe_dot(int, const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, const float*, float*,
                               hipStream_t);
hipError_t mx_launch_pad_both(const uint16_t*, int64_t, int64_t, int64_t, const int32_t*, int, int64_t, uint8_t*,
                              uint8_t*, uint8_t*, uint8_t*, int32_t*, int, hipStream_t);
hipError_t mx_launch_gemm_kgroup(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, const int32_t*, int,
                                 int64_t, int64_t, int64_t, void*, int, void*, int64_t, hipStream_t);
int64_t mx_kgroup_workspace_bytes(int, int64_t, int64_t, int64_t, int);
int64_t mx_noalloc_scratch_bytes();
hipError_t mx_noalloc_scratch(void**);

namespace {

thread_local char g_err[512] = "";

// Largest size accepted for any dimension: keeps every byte offset far inside int64.
constexpr int64_t kMaxDim = (int64_t)1 << 31;
constexpr int64_t kMaxContraction = (int64_t)1 << 22;

mx_status fail(mx_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
mx_status fail(mx_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Architecture check, cached per device ordinal.
mx_status check_device() {
  static std::mutex mu;
  static int state[64] = {0};  // 0 unknown, 1 ok, -1 not gfx950
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return fail(MX_E_DEVICE, "no HIP device is available");
  if (dev >= 64) return fail(MX_E_DEVICE, "device ordinal %d out of range", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (state[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return fail(MX_E_DEVICE, "cannot query device %d", dev);
    state[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    if (state[dev] < 0) return fail(MX_E_DEVICE, "device %d is %s; this library runs on gfx950 only", dev, prop.gcnArchName);
  }
  if (state[dev] < 0) return fail(MX_E_DEVICE, "device %d is not gfx950", dev);
  return MX_OK;
}

mx_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MX_E_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  g_err[0] = 0;
  return MX_OK;
}

mx_status check_dim(const char* name, int64_t v, int64_t lo) {
  if (v < lo || v > kMaxDim) return fail(MX_E_SHAPE, "%s = %lld is outside [%lld, 2^31]", name, (long long)v, (long long)lo);
  return MX_OK;
}

#define TRY(x)                  \
  do {                          \
    mx_status _s = (x);         \
    if (_s != MX_OK) return _s; \
  } while (0)

mx_status check_ptr(const char* name, const void* p) {
  if (!p) return fail(MX_E_NULL, "%s is NULL", name);
  if (!aligned16(p)) return fail(MX_E_ALIGN, "%s is not 16-byte aligned", name);
  return MX_OK;
}

// A buffer of zero rows may be NULL (nothing is read or written there).
mx_status check_rows_ptr(const char* name, const void* p, int64_t rows) {
  if (!p && rows == 0) return MX_OK;
  return check_ptr(name, p);
}

mx_status check_pitch(const char* name, int64_t ld, int64_t cols) {
  if (ld < cols) return fail(MX_E_LAYOUT, "%s = %lld is smaller than the row length %lld", name, (long long)ld, (long long)cols);
  if (ld % 8 != 0) return fail(MX_E_ALIGN, "%s = %lld: bf16 rows must start 16-byte aligned (pitch %% 8 == 0)", name, (long long)ld);
  if (ld > kMaxDim) return fail(MX_E_SHAPE, "%s = %lld is too large", name, (long long)ld);
  return MX_OK;
}

// The one-pass cast reads a 32-row sub-tile and writes four q_t rows at a time through
// 32-bit buffer offsets from a per-sub-tile base: the row pitch must stay below 2^25
// elements and the rows (q_t's row length) below 2^29.
mx_status check_one_pass(int64_t ld, int64_t rows) {
  if (ld >= ((int64_t)1 << 25))
    return fail(MX_E_SHAPE, "ld_x = %lld: the one-pass cast needs a row pitch below 2^25 elements", (long long)ld);
  if (rows >= ((int64_t)1 << 29))
    return fail(MX_E_SHAPE, "rows = %lld: the one-pass cast needs fewer than 2^29 rows", (long long)rows);
  return MX_OK;
}

mx_status check_mul32(const char* name, int64_t v) {
  if (v % 32 != 0) return fail(MX_E_SHAPE, "%s = %lld must be a multiple of 32 (one MX block)", name, (long long)v);
  return MX_OK;
}

// a_rows / b_rows / out_rows: 0 when that buffer holds no element (it may be NULL)
mx_status check_gemm_common(const void* a, const void* a_s, const void* b, const void* b_s, const void* out,
                            int out_dtype, int32_t groups, const int32_t* offs, int64_t a_elems, int64_t b_elems,
                            int64_t out_elems) {
  TRY(check_rows_ptr("a", a, a_elems));
  TRY(check_rows_ptr("a_scale", a_s, a_elems));
  TRY(check_rows_ptr("b", b, b_elems));
  TRY(check_rows_ptr("b_scale", b_s, b_elems));
  TRY(check_rows_ptr("out", out, out_elems));
  if (out_dtype != MX_OUT_F32 && out_dtype != MX_OUT_BF16)
    return fail(MX_E_DTYPE, "out_dtype = %d is neither MX_OUT_F32 (0) nor MX_OUT_BF16 (1)", out_dtype);
  if (groups < 1 || groups > 65536) return fail(MX_E_SHAPE, "groups = %d is outside [1, 65536]", groups);
  if (!offs && groups != 1) return fail(MX_E_SHAPE, "offs is NULL (dense) but groups = %d", groups);
  if (offs && ((uintptr_t)offs & 3)) return fail(MX_E_ALIGN, "offs is not 4-byte aligned");
  return MX_OK;
}

}  // namespace

extern "C" {

int64_t mx_scale_bytes(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0 || cols % 32 != 0) return -1;
  const int64_t kb = cols / 32;
  return ((rows + 31) / 32) * ((kb + 7) / 8) * 256;
}

const char* mx_status_string(mx_status s) {
  switch (s) {
    case MX_OK: return "MX_OK";
    case MX_E_NULL: return "MX_E_NULL";
    case MX_E_SHAPE: return "MX_E_SHAPE";
    case MX_E_ALIGN: return "MX_E_ALIGN";
    case MX_E_LAYOUT: return "MX_E_LAYOUT";
    case MX_E_DTYPE: return "MX_E_DTYPE";
    case MX_E_DEVICE: return "MX_E_DEVICE";
    case MX_E_LAUNCH: return "MX_E_LAUNCH";
    default: return "MX_E_UNKNOWN";
  }
}

const char* mx_last_error(void) { return g_err; }

mx_status mx_quantize_dim0(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q, uint8_t* scale,
                           void* stream) {
  TRY(check_dim("rows", rows, 0));
  TRY(check_dim("cols", cols, 32));
  TRY(check_mul32("cols", cols));
  TRY(check_pitch("ld_x", ld_x, cols));
  TRY(check_rows_ptr("x", x, rows));
  TRY(check_rows_ptr("q", q, rows));
  TRY(check_rows_ptr("scale", scale, rows));
  TRY(check_device());
  return launched(mx_launch_dim0(x, rows, cols, ld_x, q, scale, 0, (hipStream_t)stream), "mx_quantize_dim0");
}

mx_status mx_quantize_dim1(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q_t,
                           uint8_t* scale_t, void* stream) {
  TRY(check_dim("batch", batch, 1));
  TRY(check_dim("rows", rows, 32));
  TRY(check_dim("cols", cols, 32));
  TRY(check_mul32("rows", rows));
  TRY(check_mul32("cols", cols));
  TRY(check_pitch("ld_x", ld_x, cols));
  if (batch * rows > kMaxDim || batch * cols > kMaxDim) return fail(MX_E_SHAPE, "batch * rows or batch * cols exceeds 2^31");
  TRY(check_ptr("x", x));
  TRY(check_ptr("q_t", q_t));
  TRY(check_ptr("scale_t", scale_t));
  TRY(check_device());
  return launched(mx_launch_dim1(x, batch, rows, cols, ld_x, q_t, scale_t, 0, (hipStream_t)stream), "mx_quantize_dim1");
}

mx_status mx_quantize_dim0_dim1(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, int64_t ld_x,
                                uint8_t* q, uint8_t* scale, uint8_t* q_t, uint8_t* scale_t, void* stream) {
  TRY(check_dim("batch", batch, 1));
  TRY(check_dim("rows", rows, 32));
  TRY(check_dim("cols", cols, 32));
  TRY(check_mul32("rows", rows));
  TRY(check_mul32("cols", cols));
  TRY(check_pitch("ld_x", ld_x, cols));
  TRY(check_one_pass(ld_x, rows));
  if (batch * rows > kMaxDim || batch * cols > kMaxDim) return fail(MX_E_SHAPE, "batch * rows or batch * cols exceeds 2^31");
  TRY(check_ptr("x", x));
  TRY(check_ptr("q", q));
  TRY(check_ptr("scale", scale));
  TRY(check_ptr("q_t", q_t));
  TRY(check_ptr("scale_t", scale_t));
  TRY(check_device());
  return launched(mx_launch_both(x, batch, rows, cols, ld_x, q, scale, q_t, scale_t, 0, 0, (hipStream_t)stream),
                  "mx_quantize_dim0_dim1");
}

mx_status mx_quantize_ex(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, int64_t ld_x, int forms,
                         int scale_mode, uint8_t* q, uint8_t* scale, uint8_t* q_t, uint8_t* scale_t, void* stream) {
  const int stream_t = (forms & MX_FORM_STREAM_T) != 0;
  if (stream_t) forms &= ~MX_FORM_STREAM_T;
  if (forms != MX_FORM_DIM0 && forms != MX_FORM_DIM1 && forms != (MX_FORM_DIM0 | MX_FORM_DIM1))
    return fail(MX_E_DTYPE, "forms = %d must be MX_FORM_DIM0, MX_FORM_DIM1 or both (plus MX_FORM_STREAM_T)", forms);
  if (stream_t && forms != (MX_FORM_DIM0 | MX_FORM_DIM1))
    return fail(MX_E_DTYPE, "MX_FORM_STREAM_T applies to the one-pass cast (both forms) only");
  if (scale_mode != MX_SCALE_RCEIL && scale_mode != MX_SCALE_FLOOR)
    return fail(MX_E_DTYPE, "scale_mode = %d must be MX_SCALE_RCEIL or MX_SCALE_FLOOR", scale_mode);
  const bool d0 = forms & MX_FORM_DIM0, d1 = forms & MX_FORM_DIM1;
  TRY(check_dim("batch", batch, 1));
  TRY(check_dim("rows", rows, d1 ? 32 : 0));
  TRY(check_dim("cols", cols, 32));
  if (d1) TRY(check_mul32("rows", rows));
  TRY(check_mul32("cols", cols));
  TRY(check_pitch("ld_x", ld_x, cols));
  if (d0 && d1) TRY(check_one_pass(ld_x, rows));
  if (batch * rows > kMaxDim || batch * cols > kMaxDim) return fail(MX_E_SHAPE, "batch * rows or batch * cols exceeds 2^31");
  TRY(check_rows_ptr("x", x, batch * rows));
  if (d0) {
    TRY(check_rows_ptr("q", q, batch * rows));
    TRY(check_rows_ptr("scale", scale, batch * rows));
  }
  if (d1) {
    TRY(check_ptr("q_t", q_t));
    TRY(check_ptr("scale_t", scale_t));
  }
  TRY(check_device());
  const int fl = scale_mode == MX_SCALE_FLOOR;
  hipError_t e;
  if (d0 && d1)
    e = mx_launch_both(x, batch, rows, cols, ld_x, q, scale, q_t, scale_t, fl, stream_t, (hipStream_t)stream);
  else if (d0)  // batches are contiguous with the row pitch: one stacked matrix
    e = mx_launch_dim0(x, batch * rows, cols, ld_x, q, scale, fl, (hipStream_t)stream);
  else
    e = mx_launch_dim1(x, batch, rows, cols, ld_x, q_t, scale_t, fl, (hipStream_t)stream);
  return launched(e, "mx_quantize_ex");
}

mx_status mx_quantize_weight_32x32(const uint16_t* w, int64_t batch, int64_t n, int64_t k, int64_t ld_w, uint8_t* q,
                                   uint8_t* q_t, uint8_t* scale_row, uint8_t* scale_col, void* stream) {
  TRY(check_dim("batch", batch, 1));
  TRY(check_dim("n", n, 32));
  TRY(check_dim("k", k, 32));
  TRY(check_mul32("n", n));
  TRY(check_mul32("k", k));
  TRY(check_pitch("ld_w", ld_w, k));
  if (batch * n > kMaxDim || batch * k > kMaxDim) return fail(MX_E_SHAPE, "batch * n or batch * k exceeds 2^31");
  TRY(check_ptr("w", w));
  TRY(check_ptr("q", q));
  TRY(check_ptr("scale_row", scale_row));
  if ((q_t == nullptr) != (scale_col == nullptr))
    return fail(MX_E_NULL, "q_t and scale_col must both be given or both be NULL");
  if (q_t) {
    TRY(check_ptr("q_t", q_t));
    TRY(check_ptr("scale_col", scale_col));
  }
  TRY(check_device());
  return launched(mx_launch_w32(w, batch, n, k, ld_w, q, q_t, scale_row, scale_col, (hipStream_t)stream),
                  "mx_quantize_weight_32x32");
}

// The GEMM addresses a 256-row window of an operand and a whole scale buffer
// through 32-bit buffer offsets, so the contraction is capped at 2^22 bytes per
// row and each operand's scale buffer below 2^31 bytes.
mx_status check_gemm_extent(const char* name, int64_t contraction, int64_t a_rows, int64_t b_rows) {
  if (contraction > kMaxContraction)
    return fail(MX_E_SHAPE, "%s = %lld exceeds the contraction limit 2^22", name, (long long)contraction);
  if (mx_scale_bytes(a_rows, contraction) >= kMaxDim || mx_scale_bytes(b_rows, contraction) >= kMaxDim)
    return fail(MX_E_SHAPE, "an operand's scale buffer would reach 2^31 bytes");
  return MX_OK;
}

mx_status mx_grouped_mm_fwd(const uint8_t* a, const uint8_t* a_s, const uint8_t* b, const uint8_t* b_s,
                            const int32_t* offs, int32_t groups, int64_t m, int64_t n, int64_t k, void* out,
                            int out_dtype, void* stream) {
  TRY(check_gemm_common(a, a_s, b, b_s, out, out_dtype, groups, offs, m * k, n * k, m * n));
  TRY(check_dim("m", m, 0));
  TRY(check_dim("n", n, 1));
  TRY(check_dim("k", k, 32));
  TRY(check_mul32("k", k));
  if (groups > 1 && n % 32 != 0) return fail(MX_E_SHAPE, "n = %lld must be a multiple of 32 when groups > 1", (long long)n);
  if ((int64_t)groups * n > kMaxDim) return fail(MX_E_SHAPE, "groups * n exceeds 2^31");
  TRY(check_gemm_extent("k", k, m, (int64_t)groups * n));
  TRY(check_device());
  return launched(mx_launch_gemm_mgroup(a, a_s, b, b_s, offs, nullptr, groups, m, m, n, k, out, out_dtype,
                                        (hipStream_t)stream),
                  "mx_grouped_mm_fwd");
}

mx_status mx_grouped_mm_dgrad(const uint8_t* dy, const uint8_t* dy_s, const uint8_t* w_t, const uint8_t* w_t_s,
                              const int32_t* offs, int32_t groups, int64_t m, int64_t n, int64_t k, void* dx,
                              int out_dtype, void* stream) {
  TRY(check_gemm_common(dy, dy_s, w_t, w_t_s, dx, out_dtype, groups, offs, m * n, k * n, m * k));
  TRY(check_dim("m", m, 0));
  TRY(check_dim("n", n, 32));
  TRY(check_dim("k", k, 1));
  TRY(check_mul32("n", n));
  if (groups > 1 && k % 32 != 0) return fail(MX_E_SHAPE, "k = %lld must be a multiple of 32 when groups > 1", (long long)k);
  if ((int64_t)groups * k > kMaxDim) return fail(MX_E_SHAPE, "groups * k exceeds 2^31");
  TRY(check_gemm_extent("n", n, m, (int64_t)groups * k));
  TRY(check_device());
  // dX[m x k] = dY[m x n] . (W_g^T [k x n])^T : the M-grouped core with contraction n
  return launched(mx_launch_gemm_mgroup(dy, dy_s, w_t, w_t_s, offs, nullptr, groups, m, m, k, n, dx, out_dtype,
                                        (hipStream_t)stream),
                  "mx_grouped_mm_dgrad");
}

namespace {

mx_status check_workspace(const void* workspace, int64_t workspace_bytes) {
  if (workspace_bytes < 0) return fail(MX_E_SHAPE, "workspace_bytes = %lld is negative", (long long)workspace_bytes);
  if (workspace && !aligned16(workspace)) return fail(MX_E_ALIGN, "workspace is not 16-byte aligned");
  return MX_OK;
}

mx_status check_wgrad(const uint8_t* dy_t, const uint8_t* dy_t_s, const uint8_t* x_t, const uint8_t* x_t_s,
                      const int32_t* offs, int32_t groups, int64_t m, int64_t n, int64_t k, void* dw, int out_dtype) {
  TRY(check_gemm_common(dy_t, dy_t_s, x_t, x_t_s, dw, out_dtype, groups, offs, n * m, k * m, n * k));
  TRY(check_dim("m", m, 0));
  TRY(check_dim("n", n, 1));
  TRY(check_dim("k", k, 1));
  TRY(check_mul32("m", m));
  if ((int64_t)groups * n > kMaxDim) return fail(MX_E_SHAPE, "groups * n exceeds 2^31");
  TRY(check_gemm_extent("m", m, n, k));
  return MX_OK;
}

}  // namespace

int64_t mx_grouped_mm_wgrad_workspace_bytes(int32_t groups, int64_t m, int64_t n, int64_t k, int bf16_operands) {
  if (groups < 1 || groups > 65536 || m < 0 || n < 1 || k < 1 || m > kMaxDim || n > kMaxDim || k > kMaxDim) return -1;
  if ((int64_t)groups * n > kMaxDim) return -1;
  return mx_kgroup_workspace_bytes(groups, m, n, k, bf16_operands ? 1 : 0);
}

mx_status mx_grouped_mm_wgrad(const uint8_t* dy_t, const uint8_t* dy_t_s, const uint8_t* x_t, const uint8_t* x_t_s,
                              const int32_t* offs, int32_t groups, int64_t m, int64_t n, int64_t k, void* dw,
                              int out_dtype, void* workspace, int64_t workspace_bytes, void* stream) {
  TRY(check_wgrad(dy_t, dy_t_s, x_t, x_t_s, offs, groups, m, n, k, dw, out_dtype));
  TRY(check_workspace(workspace, workspace_bytes));
  TRY(check_device());
  // dW_g[n x k] = dY^T[n x m] . (X^T[k x m])^T over group g's range of m
  return launched(mx_launch_gemm_kgroup(dy_t, dy_t_s, x_t, x_t_s, offs, groups, n, k, m, dw, out_dtype,
                                        workspace_bytes ? workspace : nullptr, workspace_bytes, (hipStream_t)stream),
                  "mx_grouped_mm_wgrad");
}

mx_status mx_grouped_mm_wgrad_noalloc(const uint8_t* dy_t, const uint8_t* dy_t_s, const uint8_t* x_t,
                                      const uint8_t* x_t_s, const int32_t* offs, int32_t groups, int64_t m, int64_t n,
                                      int64_t k, void* dw, int out_dtype, void* stream) {
  TRY(check_wgrad(dy_t, dy_t_s, x_t, x_t_s, offs, groups, m, n, k, dw, out_dtype));
  const int64_t need = mx_kgroup_workspace_bytes(groups, m, n, k, 0);
  const int64_t cap = mx_noalloc_scratch_bytes();
  if (need > cap)
    return fail(MX_E_SHAPE,
                "this wgrad splits its contraction into %lld bytes of fp32 partials; the library's fixed scratch "
                "holds %lld (use mx_grouped_mm_wgrad with a workspace)",
                (long long)need, (long long)cap);
  TRY(check_device());
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = mx_noalloc_scratch(&ws);
    if (e != hipSuccess)
      return fail(MX_E_LAUNCH, "mx_grouped_mm_wgrad_noalloc: scratch address: %s", hipGetErrorString(e));
  }
  return launched(mx_launch_gemm_kgroup(dy_t, dy_t_s, x_t, x_t_s, offs, groups, n, k, m, dw, out_dtype, ws, need,
                                        (hipStream_t)stream),
                  "mx_grouped_mm_wgrad_noalloc");
}

// ---- backward override arms: conversions and bf16 grouped GEMMs ----

mx_status mx_dequantize(const uint8_t* q, const uint8_t* scale, int64_t batch, int64_t rows, int64_t cols,
                        int transpose, uint16_t* out, void* stream) {
  if (transpose != 0 && transpose != 1) return fail(MX_E_DTYPE, "transpose = %d must be 0 or 1", transpose);
  TRY(check_dim("batch", batch, 1));
  TRY(check_dim("rows", rows, 0));
  TRY(check_dim("cols", cols, 32));
  TRY(check_mul32("cols", cols));
  if (batch * rows > kMaxDim) return fail(MX_E_SHAPE, "batch * rows exceeds 2^31");
  if (transpose && rows % 8 != 0)
    return fail(MX_E_SHAPE, "rows = %lld: a transposed output needs rows %% 8 == 0 (16-byte rows)", (long long)rows);
  TRY(check_rows_ptr("q", q, batch * rows));
  TRY(check_rows_ptr("out", out, batch * rows));
  if (!scale && batch * rows) return fail(MX_E_NULL, "scale is NULL");
  TRY(check_device());
  return launched(mx_launch_dequant(q, scale, batch, rows, cols, transpose, out, (hipStream_t)stream), "mx_dequantize");
}

mx_status mx_scales_to_logical(const uint8_t* scale, int64_t rows, int64_t cols, uint8_t* logical, void* stream) {
  TRY(check_dim("rows", rows, 0));
  TRY(check_dim("cols", cols, 32));
  TRY(check_mul32("cols", cols));
  if (rows && (!scale || !logical)) return fail(MX_E_NULL, "scale or logical is NULL");
  TRY(check_device());
  return launched(mx_launch_scales_logical(scale, rows, cols, logical, (hipStream_t)stream), "mx_scales_to_logical");
}

mx_status mx_transpose_bf16(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, int64_t ld_x, uint16_t* out,
                            void* stream) {
  TRY(check_dim("batch", batch, 1));
  TRY(check_dim("rows", rows, 0));
  TRY(check_dim("cols", cols, 8));
  if (rows % 8 != 0 || cols % 8 != 0)
    return fail(MX_E_SHAPE, "rows = %lld, cols = %lld: both must be multiples of 8 (16-byte rows in and out)",
                (long long)rows, (long long)cols);
  TRY(check_pitch("ld_x", ld_x, cols));
  if (batch * rows > kMaxDim || batch * cols > kMaxDim) return fail(MX_E_SHAPE, "batch * rows or batch * cols exceeds 2^31");
  TRY(check_rows_ptr("x", x, batch * rows));
  TRY(check_rows_ptr("out", out, batch * rows));
  TRY(check_device());
  return launched(mx_launch_transpose_bf16(x, batch, rows, cols, ld_x, out, (hipStream_t)stream), "mx_transpose_bf16");
}

namespace {

// bf16 operands: 16-byte rows along the contraction, which is at most 2^21
// elements (2^22 bytes, the byte limit of the MXFP8 GEMM).
mx_status check_bf16_gemm(const void* a, const void* b, const void* out, int out_dtype, int32_t groups,
                          const int32_t* offs, const char* cname, int64_t contraction, int64_t a_rows,
                          int64_t b_rows, int64_t out_elems) {
  TRY(check_rows_ptr("a", a, a_rows * contraction));
  TRY(check_rows_ptr("b", b, b_rows * contraction));
  TRY(check_rows_ptr("out", out, out_elems));
  if (out_dtype != MX_OUT_F32 && out_dtype != MX_OUT_BF16)
    return fail(MX_E_DTYPE, "out_dtype = %d is neither MX_OUT_F32 (0) nor MX_OUT_BF16 (1)", out_dtype);
  if (groups < 1 || groups > 65536) return fail(MX_E_SHAPE, "groups = %d is outside [1, 65536]", groups);
  if (!offs && groups != 1) return fail(MX_E_SHAPE, "offs is NULL (dense) but groups = %d", groups);
  if (offs && ((uintptr_t)offs & 3)) return fail(MX_E_ALIGN, "offs is not 4-byte aligned");
  if (contraction % 8 != 0)
    return fail(MX_E_SHAPE, "%s = %lld must be a multiple of 8 (16-byte bf16 rows)", cname, (long long)contraction);
  if (contraction > ((int64_t)1 << 21))
    return fail(MX_E_SHAPE, "%s = %lld exceeds the bf16 contraction limit 2^21", cname, (long long)contraction);
  if (a_rows > kMaxDim || b_rows > kMaxDim) return fail(MX_E_SHAPE, "operand rows exceed 2^31");
  return MX_OK;
}

}  // namespace

mx_status mx_grouped_mm_bf16_fwd(const uint16_t* a, const uint16_t* b, const int32_t* offs, int32_t groups, int64_t m,
                                 int64_t n, int64_t k, void* out, int out_dtype, void* stream) {
  TRY(check_dim("m", m, 0));
  TRY(check_dim("n", n, 1));
  TRY(check_dim("k", k, 8));
  TRY(check_bf16_gemm(a, b, out, out_dtype, groups, offs, "k", k, m, (int64_t)groups * n, m * n));
  TRY(check_device());
  return launched(mx_launch_gemm_bf16_mgroup(a, b, offs, groups, m, n, k, out, out_dtype, (hipStream_t)stream),
                  "mx_grouped_mm_bf16_fwd");
}

mx_status mx_grouped_mm_bf16_dgrad(const uint16_t* dy, const uint16_t* w_t, const int32_t* offs, int32_t groups,
                                   int64_t m, int64_t n, int64_t k, void* dx, int out_dtype, void* stream) {
  TRY(check_dim("m", m, 0));
  TRY(check_dim("n", n, 8));
  TRY(check_dim("k", k, 1));
  TRY(check_bf16_gemm(dy, w_t, dx, out_dtype, groups, offs, "n", n, m, (int64_t)groups * k, m * k));
  TRY(check_device());
  return launched(mx_launch_gemm_bf16_mgroup(dy, w_t, offs, groups, m, k, n, dx, out_dtype, (hipStream_t)stream),
                  "mx_grouped_mm_bf16_dgrad");
}

mx_status mx_grouped_mm_bf16_wgrad(const uint16_t* dy_t, const uint16_t* x_t, const int32_t* offs, int32_t groups,
                                   int64_t m, int64_t n, int64_t k, void* dw, int out_dtype, void* workspace,
                                   int64_t workspace_bytes, void* stream) {
  TRY(check_dim("m", m, 0));
  TRY(check_dim("n", n, 1));
  TRY(check_dim("k", k, 1));
  TRY(check_bf16_gemm(dy_t, x_t, dw, out_dtype, groups, offs, "m", m, n, k, (int64_t)groups * n * k));
  if ((int64_t)groups * n > kMaxDim) return fail(MX_E_SHAPE, "groups * n exceeds 2^31");
  TRY(check_workspace(workspace, workspace_bytes));
  TRY(check_device());
  return launched(mx_launch_gemm_bf16_kgroup(dy_t, x_t, offs, groups, n, k, m, dw, out_dtype,
                                             workspace_bytes ? workspace : nullptr, workspace_bytes, (hipStream_t)stream),
                  "mx_grouped_mm_bf16_wgrad");
}

// ---- token-group padding ----

namespace {

constexpr int32_t kPadMaxGroups = 1024;
constexpr int64_t kInt32Max = 2147483647;

mx_status check_pad_common(int64_t rows, int32_t groups, int64_t rows_pad, const int32_t* offs) {
  if (groups < 1 || groups > kPadMaxGroups)
    return fail(MX_E_SHAPE, "groups = %d is outside [1, %d]", groups, kPadMaxGroups);
  if (rows < 0 || rows + 31 * (int64_t)groups > kInt32Max)
    return fail(MX_E_SHAPE, "rows = %lld: rows + 31 * groups must stay below 2^31 (int32 offsets)", (long long)rows);
  const int64_t need = mx_padded_rows(rows, groups);
  if (rows_pad < need || rows_pad > kInt32Max)
    return fail(MX_E_SHAPE, "rows_pad = %lld: the padded buffer needs mx_padded_rows(%lld, %d) = %lld rows (and < 2^31)",
                (long long)rows_pad, (long long)rows, groups, (long long)need);
  if (!offs) return fail(MX_E_NULL, "offs is NULL");
  if ((uintptr_t)offs & 3) return fail(MX_E_ALIGN, "offs is not 4-byte aligned");
  return MX_OK;
}

}  // namespace

int64_t mx_padded_rows(int64_t rows, int32_t groups) {
  if (rows < 0 || groups < 1 || rows > kMaxDim) return -1;
  return ((rows + 31 * (int64_t)groups + 255) / 256) * 256;
}

mx_status mx_check_offs(const int32_t* offs, int32_t groups, int64_t m, int32_t multiple, int32_t* result,
                        void* stream) {
  if (groups < 1) return fail(MX_E_SHAPE, "groups = %d must be >= 1", groups);
  if (m < 0 || m > kMaxDim) return fail(MX_E_SHAPE, "m = %lld must be in [0, 2^31)", (long long)m);
  if (multiple < 1) return fail(MX_E_SHAPE, "multiple = %d must be >= 1", multiple);
  if (!offs) return fail(MX_E_NULL, "offs is NULL");
  if ((uintptr_t)offs & 3) return fail(MX_E_ALIGN, "offs is not 4-byte aligned");
  if (!result) return fail(MX_E_NULL, "result is NULL");
  if ((uintptr_t)result & 3) return fail(MX_E_ALIGN, "result is not 4-byte aligned");
  TRY(check_device());
  return launched(mx_launch_check_offs(offs, groups, m, multiple, result, (hipStream_t)stream), "mx_check_offs");
}

mx_status mx_probe_mfma(int64_t iters, float* sink, void* stream) {
  if (iters < 1 || iters > kInt32Max) return fail(MX_E_SHAPE, "iters = %lld must be in [1, 2^31)", (long long)iters);
  if (!sink) return fail(MX_E_NULL, "sink is NULL");
  if ((uintptr_t)sink & 3) return fail(MX_E_ALIGN, "sink is not 4-byte aligned");
  TRY(check_device());
  return launched(mx_launch_probe_mfma(iters, sink, (hipStream_t)stream), "mx_probe_mfma");
}

mx_status mx_probe_mfma_dot(int form, const uint8_t* a, const uint8_t* a_scale, const uint8_t* b,
                            const uint8_t* b_scale, const float* c, float* d, void* stream) {
  if (form < 0 || form > 3) return fail(MX_E_DTYPE, "form = %d must be in [0, 3]", form);
  if (!a || !a_scale || !b || !b_scale || !c || !d) return fail(MX_E_NULL, "a NULL operand, scale or accumulator");
  if (((uintptr_t)c & 3) || ((uintptr_t)d & 3)) return fail(MX_E_ALIGN, "c and d must be 4-byte aligned");
  TRY(check_device());
  return launched(mx_launch_probe_dot(form, a, a_scale, b, b_scale, c, d, (hipStream_t)stream), "mx_probe_mfma_dot");
}

mx_status mx_pad_token_groups(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, const int32_t* offs,
                              int32_t groups, uint16_t* x_pad, int64_t rows_pad, int32_t* offs_pad, void* stream) {
  TRY(check_pad_common(rows, groups, rows_pad, offs));
  TRY(check_dim("cols", cols, 8));
  if (cols % 8 != 0) return fail(MX_E_SHAPE, "cols = %lld must be a multiple of 8 (16-byte bf16 rows)", (long long)cols);
  TRY(check_pitch("ld_x", ld_x, cols));
  TRY(check_rows_ptr("x", x, rows));
  TRY(check_rows_ptr("x_pad", x_pad, rows_pad));
  if (!offs_pad) return fail(MX_E_NULL, "offs_pad is NULL");
  if ((uintptr_t)offs_pad & 3) return fail(MX_E_ALIGN, "offs_pad is not 4-byte aligned");
  TRY(check_device());
  return launched(mx_launch_pad(x, rows, cols, ld_x, offs, groups, x_pad, rows_pad, offs_pad, (hipStream_t)stream),
                  "mx_pad_token_groups");
}

mx_status mx_unpad_token_groups(const void* y_pad, int64_t rows_pad, int64_t cols, int64_t ld_pad,
                                const int32_t* offs, int32_t groups, void* y, int64_t rows, int64_t ld_y, int dtype,
                                void* stream) {
  if (dtype != MX_OUT_F32 && dtype != MX_OUT_BF16)
    return fail(MX_E_DTYPE, "dtype = %d is neither MX_OUT_F32 (0) nor MX_OUT_BF16 (1)", dtype);
  TRY(check_pad_common(rows, groups, rows_pad, offs));
  const int64_t es = dtype == MX_OUT_F32 ? 4 : 2;
  TRY(check_dim("cols", cols, 1));
  if ((cols * es) % 16 != 0)
    return fail(MX_E_SHAPE, "cols = %lld: rows must be a whole number of 16-byte chunks", (long long)cols);
  if (ld_pad < cols || ld_y < cols)
    return fail(MX_E_LAYOUT, "ld_pad = %lld / ld_y = %lld is smaller than cols = %lld", (long long)ld_pad,
                (long long)ld_y, (long long)cols);
  if ((ld_pad * es) % 16 != 0 || (ld_y * es) % 16 != 0)
    return fail(MX_E_ALIGN, "row pitches must be multiples of 16 bytes");
  if (ld_pad > kMaxDim || ld_y > kMaxDim) return fail(MX_E_SHAPE, "row pitch too large");
  TRY(check_rows_ptr("y_pad", y_pad, rows_pad));
  TRY(check_rows_ptr("y", y, rows));
  TRY(check_device());
  return launched(mx_launch_unpad(y_pad, rows_pad, cols * es, ld_pad * es, offs, groups, y, rows, ld_y * es,
                                  (hipStream_t)stream),
                  "mx_unpad_token_groups");
}

// ---- token-group padding fused into the cast and the GEMM outputs ----

mx_status mx_pad_quantize_ex(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, const int32_t* offs,
                             int32_t groups, int64_t rows_pad, int flags, uint8_t* q, uint8_t* scale, uint8_t* q_t,
                             uint8_t* scale_t, int32_t* offs_pad, void* stream) {
  if (flags != 0 && flags != MX_FORM_STREAM_T)
    return fail(MX_E_DTYPE, "flags = %d must be 0 or MX_FORM_STREAM_T", flags);
  TRY(check_pad_common(rows, groups, rows_pad, offs));
  if (rows_pad % 32 != 0) return fail(MX_E_SHAPE, "rows_pad = %lld must be a multiple of 32", (long long)rows_pad);
  TRY(check_dim("cols", cols, 32));
  TRY(check_mul32("cols", cols));
  TRY(check_pitch("ld_x", ld_x, cols));
  TRY(check_one_pass(ld_x, rows_pad));
  if (rows_pad * cols > ((int64_t)1 << 40)) return fail(MX_E_SHAPE, "rows_pad * cols is too large");
  TRY(check_rows_ptr("x", x, rows));
  TRY(check_ptr("q", q));
  TRY(check_ptr("scale", scale));
  TRY(check_ptr("q_t", q_t));
  TRY(check_ptr("scale_t", scale_t));
  if (!offs_pad) return fail(MX_E_NULL, "offs_pad is NULL");
  if ((uintptr_t)offs_pad & 3) return fail(MX_E_ALIGN, "offs_pad is not 4-byte aligned");
  TRY(check_device());
  return launched(mx_launch_pad_both(x, rows, cols, ld_x, offs, groups, rows_pad, q, scale, q_t, scale_t, offs_pad,
                                     flags == MX_FORM_STREAM_T, (hipStream_t)stream),
                  "mx_pad_quantize_ex");
}

mx_status mx_pad_quantize_dim0_dim1(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                                    const int32_t* offs, int32_t groups, int64_t rows_pad, uint8_t* q,
                                    uint8_t* scale, uint8_t* q_t, uint8_t* scale_t, int32_t* offs_pad,
                                    void* stream) {
  return mx_pad_quantize_ex(x, rows, cols, ld_x, offs, groups, rows_pad, 0, q, scale, q_t, scale_t, offs_pad, stream);
}

namespace {

mx_status check_padded_gemm(const int32_t* offs_pad, const int32_t* offs, int32_t groups, int64_t m_pad, int64_t m) {
  if (!offs_pad || !offs) return fail(MX_E_NULL, "offs_pad and offs must both be given");
  if (((uintptr_t)offs_pad & 3) || ((uintptr_t)offs & 3)) return fail(MX_E_ALIGN, "offs arrays must be 4-byte aligned");
  if (groups < 1 || groups > 65536) return fail(MX_E_SHAPE, "groups = %d is outside [1, 65536]", groups);
  TRY(check_dim("m", m, 0));
  TRY(check_dim("m_pad", m_pad, 0));
  if (m > m_pad) return fail(MX_E_SHAPE, "m = %lld exceeds m_pad = %lld", (long long)m, (long long)m_pad);
  return MX_OK;
}

}  // namespace

mx_status mx_grouped_mm_fwd_padded(const uint8_t* a, const uint8_t* a_s, const uint8_t* b, const uint8_t* b_s,
                                   const int32_t* offs_pad, const int32_t* offs, int32_t groups, int64_t m_pad,
                                   int64_t m, int64_t n, int64_t k, void* out, int out_dtype, void* stream) {
  TRY(check_padded_gemm(offs_pad, offs, groups, m_pad, m));
  TRY(check_gemm_common(a, a_s, b, b_s, out, out_dtype, groups, offs_pad, m_pad * k, n * k, m * n));
  TRY(check_dim("n", n, 1));
  TRY(check_dim("k", k, 32));
  TRY(check_mul32("k", k));
  if (groups > 1 && n % 32 != 0) return fail(MX_E_SHAPE, "n = %lld must be a multiple of 32 when groups > 1", (long long)n);
  if ((int64_t)groups * n > kMaxDim) return fail(MX_E_SHAPE, "groups * n exceeds 2^31");
  TRY(check_gemm_extent("k", k, m_pad, (int64_t)groups * n));
  TRY(check_device());
  return launched(mx_launch_gemm_mgroup(a, a_s, b, b_s, offs_pad, offs, groups, m_pad, m, n, k, out, out_dtype,
                                        (hipStream_t)stream),
                  "mx_grouped_mm_fwd_padded");
}

mx_status mx_grouped_mm_dgrad_padded(const uint8_t* dy, const uint8_t* dy_s, const uint8_t* w_t, const uint8_t* w_t_s,
                                     const int32_t* offs_pad, const int32_t* offs, int32_t groups, int64_t m_pad,
                                     int64_t m, int64_t n, int64_t k, void* dx, int out_dtype, void* stream) {
  TRY(check_padded_gemm(offs_pad, offs, groups, m_pad, m));
  TRY(check_gemm_common(dy, dy_s, w_t, w_t_s, dx, out_dtype, groups, offs_pad, m_pad * n, k * n, m * k));
  TRY(check_dim("n", n, 32));
  TRY(check_dim("k", k, 1));
  TRY(check_mul32("n", n));
  if (groups > 1 && k % 32 != 0) return fail(MX_E_SHAPE, "k = %lld must be a multiple of 32 when groups > 1", (long long)k);
  if ((int64_t)groups * k > kMaxDim) return fail(MX_E_SHAPE, "groups * k exceeds 2^31");
  TRY(check_gemm_extent("n", n, m_pad, (int64_t)groups * k));
  TRY(check_device());
  return launched(mx_launch_gemm_mgroup(dy, dy_s, w_t, w_t_s, offs_pad, offs, groups, m_pad, m, k, n, dx, out_dtype,
                                        (hipStream_t)stream),
                  "mx_grouped_mm_dgrad_padded");
}

}  // extern "C"
