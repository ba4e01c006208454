/*
 * vq.h - C ABI of the MI355X (gfx950) product-VQ KV-cache hot path.
 *
 * Method: VecInfer-style product vector quantization of attention keys and
 * values, as described on the "veloxquant_mlx.cache.vecinfer_cache module"
 * page (module description: per-(head, channel) smoothing and a
 * Walsh-Hadamard rotation of the keys, product-VQ encoding against a
 * codebook, dequantization; per-token storage (D / d_k) * b_k / 8 bytes) and
 * on the "Metal Kernels API" page (sections "VecInfer kernels" and
 * "Fused SDPA").
 *
 * Conventions shared by every entry point
 *   - All tensors are dense, row-major (last index fastest), device
 *     pointers, unless stated otherwise.  fp16 means IEEE binary16.
 *   - Codes are code_bits = 8 bits wide (one uint8 per sub-vector,
 *     n_centroids <= 256) or code_bits = 4 (two per byte, n_centroids <= 16:
 *     sub-vector 2k in the low nibble and 2k + 1 in the high nibble of byte
 *     k, the packing of rabitq_pack_values on the "Metal Kernels API" page;
 *     per-token storage (D / sub_dim) * code_bits / 8 bytes, the storage
 *     formula on the "veloxquant_mlx.cache.vecinfer_cache module" page).  A
 *     code buffer has shape [B, H, S_cap, row_bytes], row_bytes =
 *     (D / sub_dim) * code_bits / 8: token slot t of (b, h) starts at byte
 *     ((b * H + h) * S_cap + t) * row_bytes.  4-bit codes need an even
 *     number of sub-vectors (a multiple of 8 for vq_attend).
 *   - Sub-vector j of a D-vector covers dims [j * sub_dim, (j+1) * sub_dim).
 *     One codebook [n_centroids, sub_dim] (fp32) serves every sub-vector,
 *     head and batch row.
 *   - smooth is NULL (no smoothing) or fp32 [smooth_rows, D] with
 *     smooth_rows = 1 (one row shared by all heads) or H (one row per head;
 *     for attention, per kv head).  Encode divides by it, decode multiplies.
 *     Its entries must be finite and nonzero; they are not inspected.
 *   - transform = 1 applies the normalized Sylvester Walsh-Hadamard matrix
 *     H[i][k] = (-1)^popcount(i & k) / sqrt(D) (symmetric, its own inverse);
 *     transform = 0 applies none (the value path); transform = 2 applies an
 *     explicit invertible matrix M (the H_mat [D, D] argument of
 *     vecinfer_encode_decode_metal, "Metal Kernels API", "VecInfer
 *     kernels"), given by the arguments mat = M and mat_inv = M^-1, both
 *     fp32 [D, D] row-major device arrays (head dims up to 128): encode
 *     rotates a row vector as x . M, decode as x~ . M^-1, and the query's
 *     dual transform is (q * s) . (M^-1)^T.  An entry point reads only the
 *     matrices its steps use (encode: mat; decode: mat_inv; attention:
 *     mat_inv); the others may be NULL, and both are ignored unless
 *     transform = 2.  The matrices are not inspected: mat_inv must be the
 *     inverse of mat.
 *   - A randomized Hadamard rotation M = diag(sigma) . H, sigma in {-1, +1}^D
 *     (an orthonormal choice of the fused encode-decode kernel's H_mat,
 *     "Metal Kernels API", "VecInfer kernels"), is given as transform = 1
 *     with smooth factors s * sigma: dividing by s * sigma is smoothing by s
 *     followed by the sign flips, decode's multiply undoes both, and the
 *     query's multiply by s * sigma is the dual transform (q * s) . M.
 *   - Device pointers must be 16-byte aligned (the kernels use 16-byte
 *     vector accesses); a misaligned pointer is rejected as an invalid
 *     argument.
 *   - Every call is enqueued on `stream` (a hipStream_t; NULL = the null
 *     stream) and returns without synchronizing.  The caller owns every
 *     buffer; the library allocates no device memory and keeps no state
 *     between calls other than cached device attributes.
 *   - A call enqueues kernel launches only (no memset, copy or allocation),
 *     so calls may be captured into a HIP graph and replayed; a replay
 *     reuses the arguments of the captured call, including per-row offsets.
 *   - Errors: arguments are validated on the host before any HIP call; on
 *     failure nothing is enqueued and a nonzero status is returned, with a
 *     message available from vq_last_error().  Device data (codes, lengths)
 *     is not validated: kv lengths are clamped to [0, S_cap].  A failed
 *     kernel launch returns VQ_ERR_HIP; faults during execution surface at
 *     the caller's next synchronization.  The library never aborts.
 */
#ifndef VQ_H
#define VQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  VQ_OK = 0,
  VQ_ERR_INVALID_ARGUMENT = 1, /* inconsistent shapes, null pointers, ranges */
  VQ_ERR_UNSUPPORTED = 2,      /* outside the compiled caps (see vq_supports_shape) */
  VQ_ERR_NO_DEVICE = 3,        /* no HIP device is visible */
  VQ_ERR_HIP = 4,              /* a HIP runtime call or kernel launch failed */
  VQ_ERR_WORKSPACE = 5         /* attention workspace missing or too small */
};

/* Upper bound on B for the per-row write offsets of vq_encode. */
#define VQ_MAX_ROW_OFFSETS 256

/* Static description of a status code. */
const char* vq_status_string(int status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* vq_last_error(void);

/* Library version as major * 10000 + minor * 100 + patch. */
int vq_version(void);

/*
 * 1 if (n_centroids, n_sub, head_dim) fits the compiled kernels, else 0.
 * Mirrors supports_shape of the fused attention ("Metal Kernels API", "Fused
 * SDPA": a check of the codebook size, the number of sub-vectors and the
 * head dimension, not of batch or sequence sizes; head_dim a multiple of 32).
 * Caps: 1 <= n_centroids <= 256; head_dim in {32, 64, 128, 256};
 * n_sub divides head_dim, head_dim / n_sub in {1, 2, 4, 8, 16}, n_sub <= 64.
 * vq_attend additionally needs n_sub to be a multiple of 4 for both codes.
 */
int vq_supports_shape(int n_centroids, int n_sub, int head_dim);

/*
 * Key (or value) encode: smooth -> rotate -> nearest centroid, written into
 * a code buffer ("Metal Kernels API", "VecInfer kernels",
 * vecinfer_quantize_metal and the first three steps of
 * vecinfer_encode_decode_metal; the cache appends codes into index buffers,
 * "veloxquant_mlx.cache.vecinfer_cache module", update_and_fetch).
 *
 *   keys_f16    [B, H, S, D] fp16
 *   codebook    [n_centroids, sub_dim] fp32
 *   smooth      NULL or [smooth_rows, D] fp32 (see conventions)
 *   transform   0, 1 or 2; mat, mat_inv as in the conventions
 *   code_bits   8 or 4 (see conventions)
 *   codes       [B, H, S_cap, row_bytes] uint8; token t of row b is
 *               written to slot off_b + t, off_b = row_offsets[b] if
 *               row_offsets != NULL else S_off.  Other slots are untouched.
 *   row_offsets NULL or HOST array of B int32 (B <= VQ_MAX_ROW_OFFSETS),
 *               each with 0 <= off_b and off_b + S <= S_cap.
 * The centroid index minimizes the fp32 squared distance summed over the
 * sub-vector; exact ties resolve to the lowest index.
 * Errors: INVALID_ARGUMENT for null pointers, nonpositive sizes, B * H * S
 * of 2^31 or more, S_off or offsets out of range, D % sub_dim != 0,
 * smooth_rows not in {1, H},
 * code_bits not in {8, 4}, n_centroids > 16 or an odd number of
 * sub-vectors with 4-bit codes; UNSUPPORTED outside the caps.  S = 0 or
 * B = 0 is a no-op returning VQ_OK.
 */
int vq_encode(const void* keys_f16, int B, int H, int S, int D,
              const float* codebook, int n_centroids, int sub_dim, int code_bits,
              const float* smooth, int smooth_rows, int transform,
              const float* mat, const float* mat_inv,
              uint8_t* codes, int S_cap, int S_off, const int32_t* row_offsets,
              void* stream);

/*
 * Encode of the keys and the values of one cache append together (the
 * cache's update_and_fetch encodes both into their index buffers,
 * "veloxquant_mlx.cache.vecinfer_cache module").  Same result as
 *   vq_encode(keys_f16 -> k_codes, k_codebook, smooth, transform) and then
 *   vq_encode(values_f16 -> v_codes, v_codebook, no smooth, transform 0),
 * with the same B, H, S, D, S_cap, S_off and row_offsets for both; short
 * appends (few token-heads) run as one launch.
 *
 *   keys_f16, values_f16   [B, H, S, D] fp16
 *   k_codebook [k_n_centroids, k_sub_dim], v_codebook [v_n_centroids,
 *   v_sub_dim] fp32; smooth, smooth_rows, transform as for vq_encode (keys)
 *   code_bits 8 or 4, for both halves
 *   k_codes [B, H, S_cap, row bytes of k_sub_dim], v_codes [B, H, S_cap,
 *   row bytes of v_sub_dim]
 * Errors: those of vq_encode for either half, checked before anything is
 * enqueued.
 */
int vq_encode_kv(const void* keys_f16, const void* values_f16, int B, int H, int S, int D,
                 const float* k_codebook, int k_n_centroids, int k_sub_dim,
                 const float* smooth, int smooth_rows, int transform,
                 const float* mat, const float* mat_inv,
                 const float* v_codebook, int v_n_centroids, int v_sub_dim, int code_bits,
                 uint8_t* k_codes, uint8_t* v_codes, int S_cap, int S_off,
                 const int32_t* row_offsets, void* stream);

/*
 * Decode: codebook gather -> inverse rotation -> inverse smoothing ("Metal
 * Kernels API", "VecInfer kernels", vecinfer_dequant_metal and the last three
 * steps of vecinfer_encode_decode_metal).
 *
 *   codes       [B, H, S_cap, row_bytes] uint8 of code_bits-wide codes;
 *               slots [S_off, S_off + S) are read.  Codes >= n_centroids
 *               are undefined behaviour.
 *   out         [B, H, S, D]; out_dtype 0 = fp32, 1 = fp16 (round to
 *               nearest even).
 * Errors as vq_encode.
 */
int vq_decode(const uint8_t* codes, int B, int H, int S, int S_cap, int S_off,
              const float* codebook, int n_centroids, int sub_dim, int code_bits,
              const float* smooth, int smooth_rows, int transform,
              const float* mat, const float* mat_inv, int D,
              void* out, int out_dtype, void* stream);

/*
 * Fused round trip in one kernel: the codes of vq_encode and the
 * reconstruction of vq_decode of those codes ("Metal Kernels API",
 * "VecInfer kernels", vecinfer_encode_decode_metal: smooth -> WHT -> VQ
 * encode -> dequant -> inverse WHT -> inverse smooth in one dispatch).
 *
 *   recon       [B, H, S, D]; out_dtype 0 = fp32, 1 = fp16.
 * Other arguments and errors as vq_encode.
 */
int vq_encode_decode(const void* keys_f16, int B, int H, int S, int D,
                     const float* codebook, int n_centroids, int sub_dim, int code_bits,
                     const float* smooth, int smooth_rows, int transform,
                     const float* mat, const float* mat_inv,
                     uint8_t* codes, int S_cap, int S_off, const int32_t* row_offsets,
                     void* recon, int out_dtype, void* stream);

/*
 * Forward transform only: out = (x / s) . M in fp32, the first two steps of
 * vecinfer_encode_decode_metal ("Metal Kernels API", "VecInfer kernels"),
 * i.e. the vectors the encode searches.  Viewed as [B * H * S * D / d, d],
 * out holds the pooled sub-vectors a codebook of sub-vector width d is
 * trained on (sub-vector j of a row covers dims [j * d, (j + 1) * d)).
 *
 *   keys_f16    [B, H, S, D] fp16
 *   smooth, smooth_rows, transform, mat   as in vq_encode (mat_inv unused)
 *   out         [B, H, S, D] fp32, written in full
 * The arithmetic is that of the per-lane encode kernels (x / s in fp32,
 * then the butterflies or the fp32 matrix product in index order).
 * Errors: INVALID_ARGUMENT for null pointers, negative sizes, smooth_rows
 * not in {1, H}, a bad transform or a missing mat; UNSUPPORTED for head
 * dims other than 32, 64, 128, 256 (transform 2: up to 128).  B = 0 or
 * S = 0 is a no-op.
 */
int vq_transform(const void* keys_f16, int B, int H, int S, int D, const float* smooth,
                 int smooth_rows, int transform, const float* mat, float* out, void* stream);

/*
 * Bytes of device workspace vq_kmeans needs (0 on invalid arguments).
 * Depends only on its arguments.
 */
size_t vq_kmeans_workspace_bytes(long long N, int sub_dim, int n_centroids);

/*
 * Codebook training: `iters` iterations of Lloyd's k-means over N vectors.
 * The pages encode keys against a pre-trained codebook ("veloxquant_mlx.
 * cache.vecinfer_cache module" page, module description) and say no more;
 * this is the plain k-means reading of that training.  Each iteration
 * assigns every vector to its nearest centroid by the encode's rules (fp32
 * squared distance summed over the sub-vector in index order, lowest index
 * on exact ties; from 65,536 vectors of sub_dim 8, the matrix-core encode's
 * fp32-accurate argmin of |c|^2 - 2 c.x, which can differ from the former
 * only at near-ties), then moves every centroid to the mean of its members
 * (summed in fp64, rounded to fp32); a centroid with no member keeps its
 * value.  The inertia adds the direct fp32 distances.
 *
 *   vectors     [N, sub_dim] fp32 (e.g. vq_transform's output of the keys,
 *               or raw values converted to fp32); NULL allowed when N = 0
 *   centroids   [n_centroids, sub_dim] fp32: the initial centroids on
 *               entry, the trained ones on return (updated in place)
 *   labels      NULL or [N] uint8: the last iteration's assignment (made
 *               against the centroids that iteration started from)
 *   inertia     NULL or [iters] fp64: for each iteration, the sum over
 *               vectors of the smallest squared distance to the centroids it
 *               started from (non-increasing up to rounding)
 *   workspace   DEVICE buffer of >= vq_kmeans_workspace_bytes(...) bytes;
 *               calls that may run concurrently need distinct workspaces
 * sub_dim in {1, 2, 4, 8, 16}; 1 <= n_centroids <= 256.  Two kernel launches
 * per iteration, no host synchronization; vectors, centroids and workspace
 * must be 16-byte aligned.
 * Errors: INVALID_ARGUMENT for negative N or iters, n_centroids outside
 * [1, 256], null pointers; UNSUPPORTED for other sub_dim; WORKSPACE when the
 * workspace is missing or too small.  iters = 0 is a no-op.
 */
int vq_kmeans(const float* vectors, long long N, int sub_dim, float* centroids, int n_centroids,
              int iters, uint8_t* labels, double* inertia, void* workspace, size_t workspace_bytes,
              void* stream);

/*
 * Bytes of device workspace vq_attend needs for this shape (0 on invalid
 * sizes).  Depends only on its arguments, not on the device.
 */
size_t vq_attend_workspace_bytes(int B, int H_q, int S_q, int D, int H_kv,
                                 int S_cap, int sliding_window);

/* Kernel families of vq_attend (see vq_attend_path). */
enum {
  VQ_PATH_STREAM = 1,   /* persistent streaming kernel: decode, many keys */
  VQ_PATH_TILE = 2,     /* many-query tile kernel: >= 64 query rows per kv head */
  VQ_PATH_LUT_MFMA = 3, /* per-unit query-LUT kernel with matrix-core values */
  VQ_PATH_LUT_VALU = 4  /* per-unit query-LUT kernel on vector ALUs */
};

/*
 * The kernel family vq_attend runs for this shape (the fused attention of
 * "Metal Kernels API", "Fused SDPA"): one of VQ_PATH_*, or 0 when vq_attend
 * would reject the shape (the reason is left in vq_last_error).  The choice
 * depends only on these sizes, never on device data, and every family
 * computes the same attention.  Host-only; needs no device.
 */
int vq_attend_path(int B, int H_q, int S_q, int D, int k_sub_dim, int v_sub_dim,
                   int n_centroids, int code_bits, int transform, int H_kv, int S_cap,
                   int sliding_window);

/*
 * Fused attention read directly from key and value codes ("Metal Kernels
 * API", "Fused SDPA", metal_fused_sdpa; with the raw query and the dual
 * transform applied inside as in "veloxquant_mlx.cache.vecinfer_cache
 * module", fused_sdpa).  The result equals softmax attention over the
 * decoded keys K_hat = ((C_k[k_codes]) . H) * s and values C_v[v_codes]:
 *
 *   out[b, h, i] = sum_t p_t V_hat[b, g, t],
 *   p = softmax_t(scale * q[b, h, i] . K_hat[b, g, t]) over the valid t,
 *   g = h / (H_q / H_kv),
 *   q_abs = len_b - S_q + i (queries align to the tail of the key axis),
 *   t valid iff t < len_b, and (causal => t <= q_abs), and
 *              (sliding_window > 0 => t > q_abs - sliding_window).
 * A query row with no valid key gets zeros.
 *
 *   q_f16       [B, H_q, S_q, D] fp16 raw queries
 *   k_codes     [B, H_kv, S_cap, row bytes] uint8 (code_bits wide codes)
 *   k_codebook  [n_centroids, k_sub_dim] fp32
 *   smooth      NULL or [smooth_rows, D] fp32 smooth factors of the keys
 *               (smooth_rows 1 or H_kv); transform (and mat_inv) as for
 *               vq_encode; with transform = 2 the dual transform of the
 *               query rows is computed first into the workspace
 *   v_codes     [B, H_kv, S_cap, row bytes] uint8 (no smooth, no rotation)
 *   code_bits   8 or 4, the width of both the key and the value codes; 4-bit
 *               codes need n_centroids <= 16 and numbers of key and value
 *               sub-vectors that are multiples of 8.  Codes >= n_centroids
 *               are undefined behaviour.
 *   v_codebook  [n_centroids, v_sub_dim] fp32
 *   kv_lens     NULL (every row holds S_cap keys) or DEVICE int32 [B];
 *               values are clamped to [0, S_cap]
 *   out_f16     [B, H_q, S_q, D] fp16
 *   workspace   DEVICE buffer of >= vq_attend_workspace_bytes(...) bytes
 *               for the split partials; its contents on entry are ignored.
 *               Calls that may run concurrently need distinct workspaces.
 * Errors: INVALID_ARGUMENT for null pointers, nonpositive sizes,
 * H_q % H_kv != 0, D % sub_dim != 0, smooth_rows not in {1, H_kv},
 * sliding_window < 0, code_bits not in {8, 4} or a 4-bit shape outside its
 * limits; UNSUPPORTED outside the caps; WORKSPACE when the workspace is
 * NULL or smaller than required.
 */
int vq_attend(const void* q_f16, int B, int H_q, int S_q, int D,
              const uint8_t* k_codes, const float* k_codebook, int k_sub_dim,
              const float* smooth, int smooth_rows, int transform,
              const float* mat, const float* mat_inv,
              const uint8_t* v_codes, const float* v_codebook, int v_sub_dim,
              int n_centroids, int code_bits, int H_kv, int S_cap, const int32_t* kv_lens,
              float scale, int causal, int sliding_window,
              void* out_f16, void* workspace, size_t workspace_bytes, void* stream);

/*
 * One decode step of a code cache in one launch: the append of one new
 * token per row (the cache's update_and_fetch, "veloxquant_mlx.cache.
 * vecinfer_cache module") followed by the fused attention of vq_attend with
 * S_q = 1 (fused_sdpa on the same page, "Metal Kernels API", "Fused SDPA").
 * Same result as
 *   vq_encode_kv(k_new, v_new -> k_codes, v_codes at per-row offsets
 *                kv_lens[b] - 1, the same codebooks, smooth and transform)
 *   vq_attend(q over the updated caches, kv_lens)
 * (the same codes byte for byte, the same output), with the encode done by
 * the attention kernel's workgroups while they set up, before any of them
 * reads the new slots.
 *
 *   q_f16       [B, H_q, 1, D] fp16 raw queries
 *   k_new_f16, v_new_f16   [B, H_kv, 1, D] fp16: the new token's key and
 *               value of every (row, kv head)
 *   k_codes, v_codes       the caches as in vq_attend; slot kv_lens[b] - 1
 *               of row b is written (rows with kv_lens[b] <= 0 get no
 *               append), every other slot is only read
 *   kv_lens     DEVICE int32 [B], required: the lengths after the append,
 *               clamped to [0, S_cap]
 *   other arguments as for vq_attend (n_centroids for both codebooks,
 *   code_bits 8 or 4, transform 0 or 1)
 * Errors: those of vq_attend; INVALID_ARGUMENT when k_new, v_new or kv_lens
 * is NULL; UNSUPPORTED unless the shape runs on the streaming kernel
 * (vq_attend_path(...) == VQ_PATH_STREAM with S_q = 1) with head dim 128,
 * key / value sub_dim 8 / 4 and transform 0 or 1: for other shapes call
 * vq_encode_kv and vq_attend.
 */
int vq_decode_step(const void* q_f16, const void* k_new_f16, const void* v_new_f16,
                   int B, int H_q, int D,
                   uint8_t* k_codes, const float* k_codebook, int k_sub_dim,
                   const float* smooth, int smooth_rows, int transform,
                   uint8_t* v_codes, const float* v_codebook, int v_sub_dim,
                   int n_centroids, int code_bits, int H_kv, int S_cap, const int32_t* kv_lens,
                   float scale, int causal, int sliding_window,
                   void* out_f16, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the per-GPU device scratch array used by vq_attend_noalloc. */
#define VQ_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * vq_attend for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  Same
 * arguments, result and errors as vq_attend, without the workspace: the
 * split partials live in a file-scope device array of
 * VQ_NOALLOC_SCRATCH_BYTES bytes that the library holds on every GPU it
 * runs on until the process ends.  The call allocates nothing (no hipMalloc,
 * hipFree or allocating library routine); its first call on a device looks
 * up that device's array address once.  The stream must belong to the
 * current device.
 *
 * Shapes whose vq_attend_workspace_bytes(...) exceeds
 * VQ_NOALLOC_SCRATCH_BYTES are rejected with VQ_ERR_WORKSPACE (every decode
 * shape with S_q * H_q / H_kv < 64 query rows per kv head fits; a prefill
 * chunk such as 4 x 8 heads x 512 queries does not).  Every call on a GPU
 * shares that GPU's array: calls that may overlap on one GPU (concurrent
 * streams, or host threads) race and give undefined results; serialize them,
 * or use vq_attend with distinct workspaces.  The array's contents on entry
 * are ignored (nothing needs clearing).
 */
int vq_attend_noalloc(const void* q_f16, int B, int H_q, int S_q, int D,
                      const uint8_t* k_codes, const float* k_codebook, int k_sub_dim,
                      const float* smooth, int smooth_rows, int transform,
                      const float* mat, const float* mat_inv,
                      const uint8_t* v_codes, const float* v_codebook, int v_sub_dim,
                      int n_centroids, int code_bits, int H_kv, int S_cap, const int32_t* kv_lens,
                      float scale, int causal, int sliding_window,
                      void* out_f16, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VQ_H */
