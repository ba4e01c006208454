// C ABI of libvq: host-side validation, then kernel launches on the caller's
// stream.  Every check runs before the first HIP call, so invalid arguments
// never reach the device and every error path is reachable without a GPU.
#include "vq_internal.h"

#include <atomic>
#include <initializer_list>
#include <mutex>
#include <cmath>
#include <cstdarg>
#include <cstdio>

namespace vq {

namespace {
thread_local char g_last_error[512] = "";

int device_count() {
  // -1 = not probed yet.  Devices do not appear during a process's life.
  static std::atomic<int> cached{-1};
  int n = cached.load(std::memory_order_acquire);
  if (n < 0) {
    int c = 0;
    if (hipGetDeviceCount(&c) != hipSuccess) {
      (void)hipGetLastError();
      c = 0;
    }
    cached.store(c, std::memory_order_release);
    n = c;
  }
  return n;
}

bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

bool supported_head_dim(int D) { return D == 32 || D == 64 || D == 128 || D == 256; }

bool supported_sub_dim(int d) { return d == 1 || d == 2 || d == 4 || d == 8 || d == 16; }

int check_quantizer(const char* what, int D, int n_c, int sub_dim) {
  if (D <= 0) return fail(VQ_ERR_INVALID_ARGUMENT, "%s: D must be positive (got %d)", what, D);
  if (sub_dim <= 0) return fail(VQ_ERR_INVALID_ARGUMENT, "%s: sub_dim must be positive (got %d)", what, sub_dim);
  if (D % sub_dim != 0)
    return fail(VQ_ERR_INVALID_ARGUMENT, "%s: D (%d) is not divisible by sub_dim (%d)", what, D, sub_dim);
  if (n_c <= 0) return fail(VQ_ERR_INVALID_ARGUMENT, "%s: n_centroids must be positive (got %d)", what, n_c);
  if (n_c > 256)
    return fail(VQ_ERR_INVALID_ARGUMENT, "%s: n_centroids %d does not fit uint8 codes (max 256)", what, n_c);
  if (!vq_supports_shape(n_c, D / sub_dim, D))
    return fail(VQ_ERR_UNSUPPORTED, "%s: (n_centroids=%d, n_sub=%d, head_dim=%d) is outside the compiled caps",
                what, n_c, D / sub_dim, D);
  return VQ_OK;
}

int check_smooth(const char* what, const float* smooth, int smooth_rows, int H) {
  if (smooth && smooth_rows != 1 && smooth_rows != H)
    return fail(VQ_ERR_INVALID_ARGUMENT, "%s: smooth_rows must be 1 or %d (got %d)", what, H, smooth_rows);
  return VQ_OK;
}

// transform 0 (none), 1 (Sylvester Walsh-Hadamard, power-of-two D) or 2
// (the explicit matrices; `need` bit 1: mat, bit 2: mat_inv), head dims <= 128.
int check_transform(const char* what, int transform, int D, const float* mat, const float* mat_inv,
                    int need) {
  if (transform < 0 || transform > 2)
    return fail(VQ_ERR_INVALID_ARGUMENT, "%s: transform must be 0, 1 or 2 (got %d)", what, transform);
  if (transform == 1 && !is_pow2(D))
    return fail(VQ_ERR_UNSUPPORTED, "%s: the Walsh-Hadamard transform needs a power-of-two D (got %d)", what, D);
  if (transform == 2) {
    if (D > 128)
      return fail(VQ_ERR_UNSUPPORTED, "%s: an explicit transform matrix needs D <= 128 (got %d)", what, D);
    if (((need & 1) && !mat) || ((need & 2) && !mat_inv))
      return fail(VQ_ERR_INVALID_ARGUMENT, "%s: transform 2 needs the %s matrix", what,
                  (need & 1) && !mat ? "mat" : "mat_inv");
  }
  return VQ_OK;
}

// 8-bit codes (one byte each) or 4-bit codes (two per byte: n_c <= 16 and an
// even number of sub-vectors; `multiple` more for kernels that read whole words).
int check_code_bits(const char* what, int code_bits, int n_c, int n_sub, int multiple) {
  if (code_bits == 8) return VQ_OK;
  if (code_bits != 4)
    return fail(VQ_ERR_INVALID_ARGUMENT, "%s: code_bits must be 8 or 4 (got %d)", what, code_bits);
  if (n_c > 16)
    return fail(VQ_ERR_INVALID_ARGUMENT, "%s: 4-bit codes hold at most 16 centroids (got %d)", what, n_c);
  if (n_sub % multiple != 0)
    return fail(VQ_ERR_INVALID_ARGUMENT, "%s: 4-bit codes need a multiple of %d sub-vectors (got %d)", what,
                multiple, n_sub);
  return VQ_OK;
}

// Device buffers are read and written with 16-byte vector accesses.
int check_aligned(const char* what, std::initializer_list<const void*> ptrs) {
  for (const void* ptr : ptrs)
    if (ptr && (reinterpret_cast<uintptr_t>(ptr) & 15u) != 0)
      return fail(VQ_ERR_INVALID_ARGUMENT, "%s: device pointers must be 16-byte aligned", what);
  return VQ_OK;
}

int check_device(const char* what) {
  if (device_count() <= 0) return fail(VQ_ERR_NO_DEVICE, "%s: no HIP device is visible", what);
  return VQ_OK;
}

int hip_status(const char* what, hipError_t e) {
  if (e == hipSuccess) return VQ_OK;
  return fail(VQ_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

// The encode and decode kernels index token-heads (b, h, t) with 32-bit
// arithmetic.
int check_token_heads(const char* what, int B, int H, int S) {
  if ((long long)B * H * S >= (1LL << 31))
    return fail(VQ_ERR_INVALID_ARGUMENT, "%s: B * H * S = %lld token-heads, need fewer than 2^31", what,
                (long long)B * H * S);
  return VQ_OK;
}

// Shared validation of vq_encode / vq_encode_decode.
int check_encode(const char* what, const void* keys, int B, int H, int S, int D,
                 const float* codebook, int n_c, int sub_dim, int code_bits, const float* smooth,
                 int smooth_rows, int transform, const float* mat, const float* mat_inv, int need,
                 const uint8_t* codes, int S_cap, int S_off, const int32_t* row_offsets) {
  if (B < 0 || H <= 0 || S < 0)
    return fail(VQ_ERR_INVALID_ARGUMENT, "%s: need B >= 0, H > 0, S >= 0 (got %d, %d, %d)", what, B, H, S);
  if (!keys || !codebook || !codes)
    return fail(VQ_ERR_INVALID_ARGUMENT, "%s: keys, codebook and codes must be non-null", what);
  int st = check_token_heads(what, B, H, S);
  if (st) return st;
  if ((st = check_quantizer(what, D, n_c, sub_dim))) return st;
  if (st) return st;
  if ((st = check_code_bits(what, code_bits, n_c, D / sub_dim, 2))) return st;
  if ((st = check_smooth(what, smooth, smooth_rows, H))) return st;
  if ((st = check_transform(what, transform, D, mat, mat_inv, need))) return st;
  if ((st = check_aligned(what, {keys, codebook, smooth, mat, mat_inv}))) return st;
  if (S_cap <= 0) return fail(VQ_ERR_INVALID_ARGUMENT, "%s: S_cap must be positive (got %d)", what, S_cap);
  if (row_offsets) {
    if (B > VQ_MAX_ROW_OFFSETS)
      return fail(VQ_ERR_INVALID_ARGUMENT, "%s: per-row offsets support B <= %d (got %d)", what,
                  VQ_MAX_ROW_OFFSETS, B);
    for (int b = 0; b < B; ++b) {
      const long long o = row_offsets[b];
      if (o < 0 || o + S > S_cap)
        return fail(VQ_ERR_INVALID_ARGUMENT, "%s: row %d writes slots [%lld, %lld) outside [0, %d)", what, b, o,
                    o + S, S_cap);
    }
  } else if (S_off < 0 || (long long)S_off + S > S_cap) {
    return fail(VQ_ERR_INVALID_ARGUMENT, "%s: slots [%d, %lld) fall outside [0, %d)", what, S_off,
                (long long)S_off + S, S_cap);
  }
  return VQ_OK;
}

int run_encode(const char* what, const void* keys, const uint8_t* codes_in, int B, int H, int S,
               int D, const float* codebook, int n_c, int sub_dim, int code_bits, const float* smooth,
               int smooth_rows, int transform, const float* mat, const float* mat_inv,
               uint8_t* codes, int S_cap, int S_off,
               const int32_t* row_offsets, void* recon, int out_dtype, int mode, void* stream) {
  if (B == 0 || S == 0) return VQ_OK;
  int st = check_device(what);
  if (st) return st;
  EncodeArgs a{};
  a.keys = reinterpret_cast<const __half*>(keys);
  a.codes_in = codes_in;
  a.codebook = codebook;
  a.smooth = smooth;
  a.codes = codes;
  a.recon = recon;
  a.B = B; a.H = H; a.S = S; a.D = D; a.n_c = n_c; a.sub_dim = sub_dim; a.code_bits = code_bits;
  a.smooth_rows = smooth_rows; a.transform = transform;
  a.rot = mat; a.rot_inv = mat_inv;
  a.S_cap = S_cap; a.S_off = S_off; a.use_row_offsets = row_offsets != nullptr;
  a.recon_dtype = out_dtype;
  RowOffsets offs{};
  if (row_offsets)
    for (int b = 0; b < B; ++b) offs.v[b] = row_offsets[b];
  return hip_status(what, launch_encode(a, row_offsets ? &offs : nullptr, mode,
                                        reinterpret_cast<hipStream_t>(stream)));
}

// Device scratch of vq_attend_noalloc: the split partials of the attention
// kernels live here instead of in a caller's workspace.  Every GPU the
// library runs on holds its own copy until the process ends.
static __device__ __align__(256) unsigned char scratch[VQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device.  In host code the
// array's name is only a stand-in; the address is looked up once per device
// (with that device current) and kept.
int scratch_address(const char* what, void** out) {
  static std::once_flag once[kMaxDevices];
  static std::atomic<void*> addr[kMaxDevices];
  static std::atomic<int> err[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(what, e);
  if (dev < 0 || dev >= kMaxDevices)
    return fail(VQ_ERR_UNSUPPORTED, "%s: device index %d is beyond %d", what, dev, kMaxDevices);
  std::call_once(once[dev], [dev] {
    void* ptr = nullptr;
    const hipError_t r = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    err[dev].store((int)r, std::memory_order_relaxed);
    addr[dev].store(r == hipSuccess ? ptr : nullptr, std::memory_order_release);
  });
  void* ptr = addr[dev].load(std::memory_order_acquire);
  if (!ptr)
    return fail(VQ_ERR_HIP, "%s: the scratch array's device address is unavailable (HIP error %d)", what,
                err[dev].load(std::memory_order_relaxed));
  *out = ptr;
  return VQ_OK;
}

// vq_attend and vq_attend_noalloc: the workspace is the caller's buffer, or
// (workspace == nullptr and noalloc) the device's scratch array.
int attend_impl(const char* what, const void* q_f16, int B, int H_q, int S_q, int D,
                const uint8_t* k_codes, const float* k_codebook, int k_sub_dim, const float* smooth,
                int smooth_rows, int transform, const float* mat, const float* mat_inv,
                const uint8_t* v_codes, const float* v_codebook,
                int v_sub_dim, int n_centroids, int code_bits, int H_kv, int S_cap,
                const int32_t* kv_lens, float scale, int causal, int sliding_window, void* out_f16,
                void* workspace, size_t workspace_bytes, bool noalloc, void* stream,
                const void* k_new = nullptr, const void* v_new = nullptr) {
  if (B < 0 || S_q < 0)
    return fail(VQ_ERR_INVALID_ARGUMENT, "%s: need B >= 0 and S_q >= 0 (got %d, %d)", what, B, S_q);
  if (H_q <= 0 || H_kv <= 0 || S_cap <= 0)
    return fail(VQ_ERR_INVALID_ARGUMENT, "%s: need H_q, H_kv, S_cap > 0 (got %d, %d, %d)", what, H_q, H_kv,
                S_cap);
  if (!q_f16 || !k_codes || !k_codebook || !v_codes || !v_codebook || !out_f16)
    return fail(VQ_ERR_INVALID_ARGUMENT, "%s: q, codes, codebooks and out must be non-null", what);
  if (H_q % H_kv != 0)
    return fail(VQ_ERR_INVALID_ARGUMENT, "%s: H_q (%d) is not a multiple of H_kv (%d)", what, H_q, H_kv);
  int st = check_quantizer(what, D, n_centroids, k_sub_dim);
  if (st) return st;
  if ((st = check_quantizer(what, D, n_centroids, v_sub_dim))) return st;
  if ((D / k_sub_dim) % 4 != 0 || (D / v_sub_dim) % 4 != 0)
    return fail(VQ_ERR_UNSUPPORTED, "%s: the number of key and value sub-vectors must be multiples of 4", what);
  if ((st = check_code_bits(what, code_bits, n_centroids, D / k_sub_dim, 8))) return st;
  if ((st = check_code_bits(what, code_bits, n_centroids, D / v_sub_dim, 8))) return st;
  if ((st = check_smooth(what, smooth, smooth_rows, H_kv))) return st;
  if ((st = check_transform(what, transform, D, mat, mat_inv, 2))) return st;
  if (causal != 0 && causal != 1)
    return fail(VQ_ERR_INVALID_ARGUMENT, "%s: causal must be 0 or 1 (got %d)", what, causal);
  if (sliding_window < 0)
    return fail(VQ_ERR_INVALID_ARGUMENT, "%s: sliding_window must be >= 0 (got %d)", what, sliding_window);
  if (!std::isfinite(scale)) return fail(VQ_ERR_INVALID_ARGUMENT, "%s: scale must be finite", what);
  if ((st = check_aligned(what, {q_f16, k_codes, k_codebook, smooth, v_codes, v_codebook, kv_lens,
                                 out_f16, workspace, mat_inv})))
    return st;
  const bool append = k_new != nullptr || v_new != nullptr;
  if (append) {
    if (!k_new || !v_new || !kv_lens)
      return fail(VQ_ERR_INVALID_ARGUMENT, "%s: k_new, v_new and kv_lens must be non-null", what);
    if ((st = check_aligned(what, {k_new, v_new}))) return st;
    if (B > 0 && (S_q != 1 || transform == 2 || k_sub_dim != 8 || v_sub_dim != 4 ||
                  attend_path(B, H_q, S_q, D, H_kv, S_cap, sliding_window, k_sub_dim, v_sub_dim,
                              n_centroids, code_bits, transform) != VQ_PATH_STREAM))
      return fail(VQ_ERR_UNSUPPORTED,
                  "%s: the fused append runs on the streaming kernel only (one new token per row, "
                  "head dim 128, key / value sub_dim 8 / 4, transform 0 or 1, enough keys); call "
                  "vq_encode_kv and vq_attend instead",
                  what);
  }
  if (B == 0 || S_q == 0) return VQ_OK;
  AttendPlan plan;
  if (!plan_attend(B, H_q, S_q, D, H_kv, S_cap, sliding_window, &plan))
    return fail(VQ_ERR_INVALID_ARGUMENT, "%s: no launch plan for this shape", what);
  size_t lds = 0;
  if (!attend_pick_rows(plan.rows, D / k_sub_dim, n_centroids, v_sub_dim, D / v_sub_dim, D, &lds))
    return fail(VQ_ERR_UNSUPPORTED, "%s: the query LUT does not fit in LDS for this shape", what);
  if (noalloc) {
    if (plan.workspace_bytes > (size_t)VQ_NOALLOC_SCRATCH_BYTES)
      return fail(VQ_ERR_WORKSPACE,
                  "%s: this shape needs %zu bytes of scratch, above the %zu-byte device array; "
                  "call vq_attend with a workspace instead",
                  what, plan.workspace_bytes, (size_t)VQ_NOALLOC_SCRATCH_BYTES);
  } else if (!workspace || workspace_bytes < plan.workspace_bytes) {
    return fail(VQ_ERR_WORKSPACE, "%s: workspace needs %zu bytes (got %zu)", what, plan.workspace_bytes,
                workspace ? workspace_bytes : (size_t)0);
  }
  if ((st = check_device(what))) return st;
  if (noalloc && (st = scratch_address(what, &workspace))) return st;
  AttendArgs a{};
  a.q = reinterpret_cast<const __half*>(q_f16);
  a.k_codes = k_codes; a.k_codebook = k_codebook; a.smooth = smooth;
  a.v_codes = v_codes; a.v_codebook = v_codebook; a.kv_lens = kv_lens;
  a.out = reinterpret_cast<__half*>(out_f16);
  a.partials = reinterpret_cast<float*>(workspace);
  a.B = B; a.Hq = H_q; a.Sq = S_q; a.D = D; a.Hkv = H_kv; a.S_cap = S_cap;
  a.dk = k_sub_dim; a.dv = v_sub_dim; a.n_c = n_centroids; a.code_bits = code_bits;
  a.smooth_rows = smooth_rows; a.transform = transform;
  a.rot_inv = transform == 2 ? mat_inv : nullptr;
  a.scale_log2e = scale * 1.4426950408889634f;
  a.causal = causal; a.window = sliding_window;
  a.k_new = reinterpret_cast<const __half*>(k_new);
  a.v_new = reinterpret_cast<const __half*>(v_new);
  return hip_status(what, launch_attend(a, plan, reinterpret_cast<hipStream_t>(stream)));
}

}  // namespace

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return status;
}

}  // namespace vq

using namespace vq;

extern "C" {

const char* vq_status_string(int status) {
  switch (status) {
    case VQ_OK: return "ok";
    case VQ_ERR_INVALID_ARGUMENT: return "invalid argument";
    case VQ_ERR_UNSUPPORTED: return "unsupported shape";
    case VQ_ERR_NO_DEVICE: return "no HIP device";
    case VQ_ERR_HIP: return "HIP runtime error";
    case VQ_ERR_WORKSPACE: return "workspace missing or too small";
  }
  return "unknown status";
}

const char* vq_last_error(void) { return g_last_error; }

int vq_version(void) { return 100; }

int vq_supports_shape(int n_centroids, int n_sub, int head_dim) {
  if (n_centroids < 1 || n_centroids > 256) return 0;
  if (!supported_head_dim(head_dim)) return 0;
  if (n_sub < 1 || n_sub > 64 || head_dim % n_sub != 0) return 0;
  return supported_sub_dim(head_dim / n_sub) ? 1 : 0;
}

int vq_encode(const void* keys_f16, int B, int H, int S, int D, const float* codebook,
              int n_centroids, int sub_dim, int code_bits, const float* smooth, int smooth_rows,
              int transform, const float* mat, const float* mat_inv, uint8_t* codes, int S_cap,
              int S_off, const int32_t* row_offsets, void* stream) {
  g_last_error[0] = 0;
  int st = check_encode("vq_encode", keys_f16, B, H, S, D, codebook, n_centroids, sub_dim, code_bits,
                        smooth, smooth_rows, transform, mat, mat_inv, 1, codes, S_cap, S_off,
                        row_offsets);
  if (st) return st;
  return run_encode("vq_encode", keys_f16, nullptr, B, H, S, D, codebook, n_centroids, sub_dim,
                    code_bits, smooth, smooth_rows, transform, mat, mat_inv, codes, S_cap, S_off,
                    row_offsets, nullptr, 0, 0, stream);
}

int vq_encode_kv(const void* keys_f16, const void* values_f16, int B, int H, int S, int D,
                 const float* k_codebook, int k_n_centroids, int k_sub_dim, const float* smooth,
                 int smooth_rows, int transform, const float* mat, const float* mat_inv,
                 const float* v_codebook, int v_n_centroids, int v_sub_dim, int code_bits,
                 uint8_t* k_codes, uint8_t* v_codes, int S_cap, int S_off,
                 const int32_t* row_offsets, void* stream) {
  g_last_error[0] = 0;
  const char* what = "vq_encode_kv";
  int st = check_encode(what, keys_f16, B, H, S, D, k_codebook, k_n_centroids, k_sub_dim, code_bits,
                        smooth, smooth_rows, transform, mat, mat_inv, 1, k_codes, S_cap, S_off,
                        row_offsets);
  if (st) return st;
  if ((st = check_encode(what, values_f16, B, H, S, D, v_codebook, v_n_centroids, v_sub_dim, code_bits,
                         nullptr, 1, 0, nullptr, nullptr, 0, v_codes, S_cap, S_off, row_offsets)))
    return st;
  if (B == 0 || S == 0) return VQ_OK;
  if ((st = check_device(what))) return st;
  EncodeArgs k{}, v{};
  k.keys = reinterpret_cast<const __half*>(keys_f16);
  k.codebook = k_codebook;
  k.smooth = smooth;
  k.codes = k_codes;
  k.B = B; k.H = H; k.S = S; k.D = D; k.n_c = k_n_centroids; k.sub_dim = k_sub_dim;
  k.code_bits = code_bits;
  k.smooth_rows = smooth_rows; k.transform = transform;
  k.rot = mat; k.rot_inv = mat_inv;
  k.S_cap = S_cap; k.S_off = S_off; k.use_row_offsets = row_offsets != nullptr;
  v = k;
  v.keys = reinterpret_cast<const __half*>(values_f16);
  v.codebook = v_codebook;
  v.smooth = nullptr;
  v.smooth_rows = 1;
  v.transform = 0;
  v.rot = v.rot_inv = nullptr;
  v.codes = v_codes;
  v.n_c = v_n_centroids;
  v.sub_dim = v_sub_dim;
  RowOffsets offs{};
  if (row_offsets)
    for (int b = 0; b < B; ++b) offs.v[b] = row_offsets[b];
  return hip_status(what, launch_encode_kv(k, v, row_offsets ? &offs : nullptr,
                                           reinterpret_cast<hipStream_t>(stream)));
}

int vq_encode_decode(const void* keys_f16, int B, int H, int S, int D, const float* codebook,
                     int n_centroids, int sub_dim, int code_bits, const float* smooth,
                     int smooth_rows, int transform, const float* mat, const float* mat_inv,
                     uint8_t* codes, int S_cap, int S_off, const int32_t* row_offsets, void* recon,
                     int out_dtype, void* stream) {
  g_last_error[0] = 0;
  int st = check_encode("vq_encode_decode", keys_f16, B, H, S, D, codebook, n_centroids, sub_dim,
                        code_bits, smooth, smooth_rows, transform, mat, mat_inv, 3, codes, S_cap,
                        S_off, row_offsets);
  if (st) return st;
  if (!recon) return fail(VQ_ERR_INVALID_ARGUMENT, "vq_encode_decode: recon must be non-null");
  if ((st = check_aligned("vq_encode_decode", {recon}))) return st;
  if (out_dtype != 0 && out_dtype != 1)
    return fail(VQ_ERR_INVALID_ARGUMENT, "vq_encode_decode: out_dtype must be 0 (fp32) or 1 (fp16)");
  return run_encode("vq_encode_decode", keys_f16, nullptr, B, H, S, D, codebook, n_centroids,
                    sub_dim, code_bits, smooth, smooth_rows, transform, mat, mat_inv, codes, S_cap,
                    S_off, row_offsets, recon, out_dtype, 1, stream);
}

int vq_decode(const uint8_t* codes, int B, int H, int S, int S_cap, int S_off,
              const float* codebook, int n_centroids, int sub_dim, int code_bits,
              const float* smooth, int smooth_rows, int transform, const float* mat,
              const float* mat_inv, int D, void* out, int out_dtype, void* stream) {
  g_last_error[0] = 0;
  const char* what = "vq_decode";
  if (B < 0 || H <= 0 || S < 0)
    return fail(VQ_ERR_INVALID_ARGUMENT, "%s: need B >= 0, H > 0, S >= 0 (got %d, %d, %d)", what, B, H, S);
  if (!codes || !codebook || !out)
    return fail(VQ_ERR_INVALID_ARGUMENT, "%s: codes, codebook and out must be non-null", what);
  int st = check_token_heads(what, B, H, S);
  if (st) return st;
  if ((st = check_quantizer(what, D, n_centroids, sub_dim))) return st;
  if (st) return st;
  if ((st = check_code_bits(what, code_bits, n_centroids, D / sub_dim, 2))) return st;
  if ((st = check_smooth(what, smooth, smooth_rows, H))) return st;
  if ((st = check_transform(what, transform, D, mat, mat_inv, 2))) return st;
  if (out_dtype != 0 && out_dtype != 1)
    return fail(VQ_ERR_INVALID_ARGUMENT, "%s: out_dtype must be 0 (fp32) or 1 (fp16)", what);
  if ((st = check_aligned(what, {codebook, smooth, out, mat_inv}))) return st;
  if (S_cap <= 0 || S_off < 0 || (long long)S_off + S > S_cap)
    return fail(VQ_ERR_INVALID_ARGUMENT, "%s: slots [%d, %lld) fall outside [0, %d)", what, S_off,
                (long long)S_off + S, S_cap);
  return run_encode(what, nullptr, codes, B, H, S, D, codebook, n_centroids, sub_dim, code_bits,
                    smooth, smooth_rows, transform, mat, mat_inv, nullptr, S_cap, S_off, nullptr, out,
                    out_dtype, 2, stream);
}

size_t vq_attend_workspace_bytes(int B, int H_q, int S_q, int D, int H_kv, int S_cap,
                                 int sliding_window) {
  AttendPlan p;
  if (!plan_attend(B, H_q, S_q, D, H_kv, S_cap, sliding_window, &p)) return 0;
  return p.workspace_bytes;
}

int vq_attend_path(int B, int H_q, int S_q, int D, int k_sub_dim, int v_sub_dim,
                   int n_centroids, int code_bits, int transform, int H_kv, int S_cap,
                   int sliding_window) {
  g_last_error[0] = 0;
  const char* what = "vq_attend_path";
  if (B <= 0 || H_q <= 0 || S_q <= 0 || H_kv <= 0 || S_cap <= 0) {
    fail(VQ_ERR_INVALID_ARGUMENT, "%s: sizes must be positive", what);
    return 0;
  }
  if (H_q % H_kv != 0 || sliding_window < 0) {
    fail(VQ_ERR_INVALID_ARGUMENT, "%s: H_q %% H_kv != 0 or sliding_window < 0", what);
    return 0;
  }
  if (check_quantizer("vq_attend_path (keys)", D, n_centroids, k_sub_dim) ||
      check_quantizer("vq_attend_path (values)", D, n_centroids, v_sub_dim))
    return 0;
  if ((D / k_sub_dim) % 4 != 0 || (D / v_sub_dim) % 4 != 0) {
    fail(VQ_ERR_UNSUPPORTED, "%s: the numbers of key and value sub-vectors must be multiples of 4", what);
    return 0;
  }
  if (check_code_bits(what, code_bits, n_centroids, D / k_sub_dim, 8) ||
      check_code_bits(what, code_bits, n_centroids, D / v_sub_dim, 8))
    return 0;
  if (transform < 0 || transform > 2 || (transform == 2 && D > 128)) {
    fail(VQ_ERR_UNSUPPORTED, "%s: transform %d with head dim %d", what, transform, D);
    return 0;
  }
  const int path = attend_path(B, H_q, S_q, D, H_kv, S_cap, sliding_window, k_sub_dim, v_sub_dim,
                               n_centroids, code_bits, transform);
  if (!path) fail(VQ_ERR_UNSUPPORTED, "%s: no kernel fits this shape", what);
  return path;
}

int vq_attend(const void* q_f16, int B, int H_q, int S_q, int D, const uint8_t* k_codes,
              const float* k_codebook, int k_sub_dim, const float* smooth, int smooth_rows,
              int transform, const float* mat, const float* mat_inv, const uint8_t* v_codes,
              const float* v_codebook, int v_sub_dim, int n_centroids, int code_bits, int H_kv,
              int S_cap, const int32_t* kv_lens, float scale, int causal, int sliding_window,
              void* out_f16, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  return attend_impl("vq_attend", q_f16, B, H_q, S_q, D, k_codes, k_codebook, k_sub_dim, smooth,
                     smooth_rows, transform, mat, mat_inv, v_codes, v_codebook, v_sub_dim, n_centroids, code_bits,
                     H_kv, S_cap, kv_lens, scale, causal, sliding_window, out_f16, workspace,
                     workspace_bytes, false, stream);
}

int vq_decode_step(const void* q_f16, const void* k_new_f16, const void* v_new_f16, int B, int H_q,
                   int D, uint8_t* k_codes, const float* k_codebook, int k_sub_dim, const float* smooth,
                   int smooth_rows, int transform, uint8_t* v_codes, const float* v_codebook,
                   int v_sub_dim, int n_centroids, int code_bits, int H_kv, int S_cap,
                   const int32_t* kv_lens, float scale, int causal, int sliding_window, void* out_f16,
                   void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  return attend_impl("vq_decode_step", q_f16, B, H_q, 1, D, k_codes, k_codebook, k_sub_dim, smooth,
                     smooth_rows, transform, nullptr, nullptr, v_codes, v_codebook, v_sub_dim, n_centroids,
                     code_bits, H_kv, S_cap, kv_lens, scale, causal, sliding_window, out_f16, workspace,
                     workspace_bytes, false, stream, k_new_f16, v_new_f16);
}

int vq_attend_noalloc(const void* q_f16, int B, int H_q, int S_q, int D, const uint8_t* k_codes,
                      const float* k_codebook, int k_sub_dim, const float* smooth, int smooth_rows,
                      int transform, const float* mat, const float* mat_inv, const uint8_t* v_codes,
                      const float* v_codebook, int v_sub_dim, int n_centroids, int code_bits,
                      int H_kv, int S_cap, const int32_t* kv_lens, float scale, int causal,
                      int sliding_window, void* out_f16, void* stream) {
  g_last_error[0] = 0;
  return attend_impl("vq_attend_noalloc", q_f16, B, H_q, S_q, D, k_codes, k_codebook, k_sub_dim,
                     smooth, smooth_rows, transform, mat, mat_inv, v_codes, v_codebook, v_sub_dim, n_centroids,
                     code_bits, H_kv, S_cap, kv_lens, scale, causal, sliding_window, out_f16, nullptr, 0,
                     true, stream);
}

int vq_transform(const void* keys_f16, int B, int H, int S, int D, const float* smooth,
                 int smooth_rows, int transform, const float* mat, float* out, void* stream) {
  g_last_error[0] = 0;
  const char* what = "vq_transform";
  if (B < 0 || H <= 0 || S < 0)
    return fail(VQ_ERR_INVALID_ARGUMENT, "%s: need B >= 0, H > 0, S >= 0 (got %d, %d, %d)", what, B, H, S);
  if (!keys_f16 || !out) return fail(VQ_ERR_INVALID_ARGUMENT, "%s: keys and out must be non-null", what);
  if (!supported_head_dim(D))
    return fail(VQ_ERR_UNSUPPORTED, "%s: head_dim must be 32, 64, 128 or 256 (got %d)", what, D);
  int st = check_smooth(what, smooth, smooth_rows, H);
  if (st) return st;
  if ((st = check_transform(what, transform, D, mat, nullptr, 1))) return st;
  if ((st = check_aligned(what, {keys_f16, smooth, mat, out}))) return st;
  // the transform-only kernels use an 8-wide lane layout (the result does
  // not depend on it)
  return run_encode(what, keys_f16, nullptr, B, H, S, D, nullptr, 1, 8, 8, smooth, smooth_rows,
                    transform, mat, nullptr, nullptr, S, 0, nullptr, out, 0, 3, stream);
}

size_t vq_kmeans_workspace_bytes(long long N, int sub_dim, int n_centroids) {
  if (N < 0 || !supported_sub_dim(sub_dim) || n_centroids < 1 || n_centroids > 256) return 0;
  return kmeans_workspace_bytes(N, sub_dim, n_centroids);
}

int vq_kmeans(const float* vectors, long long N, int sub_dim, float* centroids, int n_centroids,
              int iters, uint8_t* labels, double* inertia, void* workspace, size_t workspace_bytes,
              void* stream) {
  g_last_error[0] = 0;
  const char* what = "vq_kmeans";
  if (N < 0 || N > (1LL << 48))
    return fail(VQ_ERR_INVALID_ARGUMENT, "%s: N must be in [0, 2^48] (got %lld)", what, N);
  if (!supported_sub_dim(sub_dim))
    return fail(VQ_ERR_UNSUPPORTED, "%s: sub_dim must be 1, 2, 4, 8 or 16 (got %d)", what, sub_dim);
  if (n_centroids < 1 || n_centroids > 256)
    return fail(VQ_ERR_INVALID_ARGUMENT, "%s: n_centroids must be in [1, 256] (got %d)", what, n_centroids);
  if (iters < 0) return fail(VQ_ERR_INVALID_ARGUMENT, "%s: iters must be >= 0 (got %d)", what, iters);
  if (!centroids || (N > 0 && !vectors))
    return fail(VQ_ERR_INVALID_ARGUMENT, "%s: centroids (and vectors when N > 0) must be non-null", what);
  int st = check_aligned(what, {vectors, centroids, workspace});
  if (st) return st;
  if (iters == 0) return VQ_OK;
  const size_t need = kmeans_workspace_bytes(N, sub_dim, n_centroids);
  if (!workspace || workspace_bytes < need)
    return fail(VQ_ERR_WORKSPACE, "%s: workspace needs %zu bytes (got %zu)", what, need,
                workspace ? workspace_bytes : (size_t)0);
  if ((st = check_device(what))) return st;
  KmeansArgs a{};
  a.vectors = vectors; a.N = N; a.sub_dim = sub_dim; a.n_c = n_centroids; a.iters = iters;
  a.centroids = centroids; a.labels = labels; a.inertia = inertia;
  a.partials = reinterpret_cast<double*>(workspace);
  return hip_status(what, launch_kmeans(a, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
