// Internal declarations shared by the HIP translation units of libvq.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/vq.h"

namespace vq {

// Records a failure message for vq_last_error() and returns `status`.
int fail(int status, const char* fmt, ...);

// 1/sqrt(D) for the supported power-of-two head dims, rounded to fp32.
template <int D> struct WhtNorm;
template <> struct WhtNorm<32>  { static constexpr float value = 0.17677669529663688f; };
template <> struct WhtNorm<64>  { static constexpr float value = 0.125f; };
template <> struct WhtNorm<128> { static constexpr float value = 0.08838834764831845f; };
template <> struct WhtNorm<256> { static constexpr float value = 0.0625f; };

// Per-row write offsets passed by value in the kernel arguments.
struct RowOffsets { int32_t v[VQ_MAX_ROW_OFFSETS]; };

struct EncodeArgs {
  const __half* keys;      // [B, H, S, D]
  const uint8_t* codes_in; // decode: [B, H, S_cap, n_sub]
  const float* codebook;   // [n_c, sub_dim]
  const float* smooth;     // NULL or [smooth_rows, D]
  uint8_t* codes;          // encode: [B, H, S_cap, n_sub]
  void* recon;             // NULL or [B, H, S, D]
  int B, H, S, D, n_c, sub_dim, smooth_rows, transform;
  int S_cap, S_off, use_row_offsets, recon_dtype;  // recon_dtype 0 fp32, 1 fp16
  int code_bits;           // 8: one code per byte; 4: two per byte (low nibble first)
  const float* rot;        // transform == 2: [D, D] M (encode)
  const float* rot_inv;    // transform == 2: [D, D] M^-1 (decode)
};

// mode 0 = encode, 1 = encode + reconstruct, 2 = decode only, 3 = forward
// transform only (fp32 into recon; sub_dim must be 8).
hipError_t launch_encode(const EncodeArgs& a, const RowOffsets* offs, int mode, hipStream_t st);
// Keys (k) and values (v) of one append, same B, H, S, D and slots; one
// launch for short appends with a compiled sub_dim pair, else two encodes.
hipError_t launch_encode_kv(const EncodeArgs& k, const EncodeArgs& v, const RowOffsets* offs,
                            hipStream_t st);

struct AttendArgs {
  const __half* q;          // [B, H_q, S_q, D]
  const uint8_t* k_codes;   // [B, H_kv, S_cap, n_sub_k]
  const float* k_codebook;  // [n_c, dk]
  const float* smooth;      // NULL or [smooth_rows, D]
  const uint8_t* v_codes;   // [B, H_kv, S_cap, n_sub_v]
  const float* v_codebook;  // [n_c, dv]
  const int32_t* kv_lens;   // NULL or [B]
  __half* out;              // [B, H_q, S_q, D]
  float* partials;          // workspace: split partials
  int B, Hq, Sq, D, Hkv, S_cap, dk, dv, n_c, smooth_rows, transform;
  float scale_log2e;
  int causal, window;
  int code_bits;            // 8 or 4 (two codes per byte, low nibble first)
  const float* rot_inv;     // transform == 2: [D, D] M^-1 (the query uses its transpose)
  const float* q_pre;       // set by launch_attend for transform 2: [B, H_q, S_q, D] fp32
                            // dual-transformed, scale-free query rows in the workspace
  const __half* k_new;      // decode step: NULL, or [B, H_kv, 1, D] new keys and values whose
  const __half* v_new;      // codes the streaming kernel writes to slot kv_lens[b] - 1 first
};

struct AttendPlan {
  int G;            // query heads per kv head
  int rows;         // G * S_q query rows per kv head
  int R;            // rows handled by one workgroup (1, 2, 4 or 8)
  int n_rgroups;    // ceil(rows / R)
  int split_tokens; // keys per split
  int n_split;      // splits per (b, kv head, row group)
  size_t workspace_bytes; // split partials, then the transformed query rows
  size_t qpre_offset;     // byte offset of the transformed query rows
};

// Kernel-side parameters of one attention launch (by value).
struct AttParams {
  int B, Hq, Sq, Hkv, S_cap, dk, dv, n_c, nsk, nsv, smooth_rows, transform, code_bits;
  float fold;  // WHT normalization (if any) * scale * log2(e)
  int causal, window;
  int G, rows, R, n_rgroups, split_tokens, n_split;
};

// Split merge (log-sum-exp) of the partials into the fp16 output.
hipError_t launch_attend_merge(const AttendArgs& a, const AttParams& p, hipStream_t st);

// MFMA value-path kernel: rows per workgroup and LDS bytes if the shape fits
// (D in {64, 128}, value sub_dim 4, 8/16/32 key sub-vectors), else false.
bool attend_mfma_plan(int D, int dv, int nsk, int rows, int* R, size_t* lds_bytes);
hipError_t launch_attend_mfma(const AttendArgs& a, const AttParams& p, size_t lds_bytes,
                              hipStream_t st);

// Division of 0 <= n < 2^31 by a fixed divisor d >= 1 through a multiply
// (the round-up method of Granlund and Montgomery, "Division by invariant
// integers using multiplication", 1994): q = (umulhi(n, mul) + n) >> shift
// with shift = ceil(log2 d), mul = floor(2^32 (2^shift - d) / d) + 1.
struct FastDiv {
  uint32_t mul, shift;
};
inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  const uint64_t m = ((1ull << 32) * ((1ull << s) - d)) / d + 1;
  return FastDiv{(uint32_t)m, s};
}
__device__ __forceinline__ uint32_t fast_div(uint32_t n, FastDiv f) {
  return (__umulhi(n, f.mul) + n) >> f.shift;
}

// Persistent streaming kernel (head dim 128, key sub_dim 8, value sub_dim 4).
struct StreamParams {
  int B, Hq, Sq, Hkv, S_cap, n_c, smooth_rows, transform, causal, window;
  int G, GS, n_rg, U, cmin;
  int charge;  // virtual keys charged for a segment switch in the chunk plan
  int charge_end;  // virtual keys charged after each unit's last key (the fused append)
  FastDiv div_g, div_nrg, div_hkv;  // by G, n_rg and H_kv
  float fold;  // WHT normalization (if any) * scale * log2(e)
};
// True if the shape runs on the streaming kernel; fills its parameters, LDS
// bytes and workspace bytes.
bool stream_plan(int B, int Hq, int Sq, int D, int Hkv, int S_cap, int window, int dk, int dv, int n_c,
                 StreamParams* sp, size_t* lds_bytes, size_t* ws_bytes);
// Workspace of the streaming kernel for this shape (0 if D is not 128).
size_t stream_workspace_bytes(int B, int Hq, int Sq, int D, int Hkv);
hipError_t launch_attend_stream(const AttendArgs& a, StreamParams sp, size_t lds_bytes,
                                hipStream_t st);

// The VQ_PATH_* family launch_attend uses for a validated shape (0 if none).
int attend_path(int B, int Hq, int Sq, int D, int Hkv, int S_cap, int window, int dk, int dv,
                int n_c, int code_bits, int transform);

// Many-query kernel (prefill: at least 64 query rows per kv head; head dim
// 128, key sub_dim 8, value sub_dim 4).
struct TileParams {
  int B, Hq, Sq, Hkv, S_cap, n_c, smooth_rows, transform, causal, window;
  int G, GS, n_rt, n_split;
  float fold;  // WHT normalization (if any) * scale * log2(e)
};
bool tile_plan(int B, int Hq, int Sq, int D, int Hkv, int S_cap, int window, int dk, int dv, int n_c,
               TileParams* tp);
// Workspace of the many-query kernel for this shape (0 if it does not apply).
size_t tile_workspace_bytes(int B, int Hq, int Sq, int D, int Hkv, int S_cap, int window);
hipError_t launch_attend_tile(const AttendArgs& a, TileParams tp, hipStream_t st);

// Pure function of the shape: split count, row grouping, workspace size.
bool plan_attend(int B, int Hq, int Sq, int D, int Hkv, int S_cap, int window, AttendPlan* p);

// Rows per workgroup (1, 2, 4 or 8) whose LDS footprint fits; 0 if none does.
int attend_pick_rows(int rows, int nsk, int n_c, int dv, int nsv, int D, size_t* lds_bytes);

hipError_t launch_attend(const AttendArgs& a, const AttendPlan& p, hipStream_t st);

// Lloyd's k-means over vectors [N, sub_dim] fp32 (vq_kmeans.hip).
struct KmeansArgs {
  const float* vectors;
  long long N;
  int sub_dim, n_c, iters;
  float* centroids;         // [n_c, sub_dim], updated in place
  uint8_t* labels;          // NULL or [N]: the last iteration's assignment
  double* inertia;          // NULL or [iters]
  double* partials;         // kmeans_workspace_bytes(...) of scratch
};
int kmeans_blocks(long long N);
size_t kmeans_workspace_bytes(long long N, int sub_dim, int n_c);
hipError_t launch_kmeans(const KmeansArgs& a, hipStream_t st);
// The assignment step for sub-vectors of 8 on the matrix cores (vq_encode.hip):
// writes the same per-workgroup partial rows as the vector-ALU kernel.
hipError_t launch_kmeans_assign_f16(const float* vecs, long long N, const float* cb, int n_c,
                                    double* partials, int blocks, uint8_t* labels, hipStream_t st);

}  // namespace vq
