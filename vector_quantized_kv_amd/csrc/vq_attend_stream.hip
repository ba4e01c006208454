// Persistent streaming attention from product-VQ codes (gfx950): head dim
// 128, key sub_dim 8 (16 key codes per token), value sub_dim 4 (32 value
// codes per token).
//
// Method ("Metal Kernels API" page, "Fused SDPA", metal_fused_sdpa;
// "veloxquant_mlx.cache.vecinfer_cache module" page, fused_sdpa): the query
// gets the dual transform q~ = (q * s) . H, the score of key t is
// q~ . C_k[codes of t] (equal to q . K_hat_t), the softmax runs online in
// base 2 over split chunks, and the output accumulates p_t C_v[codes of t].
// Instead of a per-sub-vector lookup table of query-centroid dot products,
// the key sub-vectors are gathered from the codebook and contracted with the
// query on the matrix cores: on gfx950 that keeps the per-key work off the
// vector ALUs.
//
// Work split.  A unit is (batch row b, kv head g, group of 4 query rows);
// query row rho of a kv head is (position rho / G, head g * G + rho % G).
// A unit's keys are the union of its rows' valid ranges.  Units are laid
// end to end into one token space of T = sum of unit lengths, and the
// 16 * gridDim waves each take one equal chunk of it (at least 256 keys), so
// ragged lengths and masks cost no imbalance.  The unit prefix is computed
// on the device from kv_lens by every workgroup.  A wave writes one partial
// (m, l, acc) per (chunk c, unit u) it touches, into slot c + u (distinct
// for all overlapping pairs since chunks and units are both ordered), and
// the merge kernel combines the slots of each unit.
//
// LDS holds, for the whole persistent workgroup, the key codebook as fp16
// rows replicated 16 times ([code][replica][8 halves], 64 KiB) and the value
// codebook replicated 32 times ([code][replica][4 halves], 64 KiB).  A lane
// always reads replica (lane mod 16) for keys and (lane mod 32) for values,
// so the 16 (b128) or 32 (b64) lanes served together always hit distinct
// banks, whatever the codes.  The LDS byte address of a gathered row is the
// replica offset in byte 0 and the code in byte 1, so one v_perm per code
// both extracts the code byte and forms the address.
//
// Per 64-key block and wave (lane = key for the scores):
//   scores  16 b128 gathers and 32 v_mfma_f32_4x4x4_16b_f16: block b of the
//           instruction covers keys 4b..4b+3, K = 4 head dims; the query
//           operand comes from one block through the A-broadcast
//           (cbsz = 4, abid = k mod 16), so all of q~ lives in 4 VGPRs.
//           The scores land as lane = key, 4 registers = 4 rows.
//   softmax lazy: the running max m_r moves only when a score exceeds it by
//           more than 8 (log2 units), so p <= 256 is exact enough in fp16
//           and the usual block needs no cross-lane work.
//   values  8 x 2 v_mfma_f32_16x16x32_f16: M = (row, e), N = 16 value
//           sub-vectors (even / odd in two tiles), K = (2 keys, e') where
//           K group g of instruction q takes keys 4 (2q) + g, 4 (2q + 1) + g
//           (so each value-code load of the wave is one 128-byte span), with
//           A[(r,e)][(t,e')] = p_r(t) [e == e'] built by 4 v_perm from the
//           staged p, and B = two gathered value rows taken as they are.
#include "vq_internal.h"

#include <algorithm>
#include <utility>

namespace vq {
namespace {

constexpr int kW = 8;                  // waves per workgroup (2 per SIMD)
constexpr int kThreads = kW * 64;
constexpr int kD = 128;
constexpr int kRows = 4;               // query rows per unit
constexpr int kSlot = kRows * kD + 2 * kRows;  // floats per partial slot
constexpr uint32_t kKeyTab = 0;        // [256][16][8] fp16
constexpr uint32_t kValTab = 65536;    // [256][32][4] fp16
constexpr uint32_t kPStage = 131072;   // [wave][row][72] fp16
constexpr uint32_t kPRow = 144;        // bytes per staged row (64 fp16 + pad)
constexpr uint32_t kPWave = kRows * kPRow;
constexpr uint32_t kScan = kPStage + kW * kPWave;
constexpr uint32_t kPrefix = kScan + 64;  // int prefix[U + 1]
constexpr float kLazyMargin = 8.f;
constexpr int kMaxUnits = 4095;        // units whose prefix fits in LDS
constexpr int kUnitsPerThread = (kMaxUnits + kThreads) / kThreads;
constexpr int kMaxWaves = 256 * 16;    // partial slots reserved for chunks (>= 256 CUs * kW)

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ uint32_t pack_half2(float a, float b) {
  const __half2 h = __floats2half2_rn(a, b);
  return *reinterpret_cast<const uint32_t*>(&h);
}

__device__ __forceinline__ uint32_t pack_half2_rtz(float a, float b) {
  typedef __fp16 h2 __attribute__((ext_vector_type(2)));
  const h2 v = __builtin_amdgcn_cvt_pkrtz(a, b);
  return *reinterpret_cast<const uint32_t*>(&v);
}

// LDS accesses by byte address.  The kernel declares no static LDS, so the
// dynamic area it uses starts at LDS address 0.
typedef __attribute__((address_space(3))) uint8_t lds_byte;
template <typename T>
__device__ __forceinline__ T lds_ld(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) T*>(
      reinterpret_cast<const lds_byte*>((size_t)addr));
}

// Scores of the lane's key against the query rows: key sub-vector J (the
// gathered fp16 row kv[J]) is contracted with dims 8J..8J+7 of the query,
// which the A-broadcast takes from block (2J mod 16) / (2J+1 mod 16) of Aq.
// Even and odd halves accumulate separately to halve the dependent chain.
template <int J>
__device__ __forceinline__ void key_mfma(const half8_t (&kv)[16], const half4_t (&Aq)[2],
                                         float4_t& s0, float4_t& s1) {
  const half4_t lo = {kv[J][0], kv[J][1], kv[J][2], kv[J][3]};
  const half4_t hi = {kv[J][4], kv[J][5], kv[J][6], kv[J][7]};
  s0 = __builtin_amdgcn_mfma_f32_4x4x4f16(Aq[(2 * J) >> 4], lo, s0, 4, (2 * J) & 15, 0);
  s1 = __builtin_amdgcn_mfma_f32_4x4x4f16(Aq[(2 * J + 1) >> 4], hi, s1, 4, (2 * J + 1) & 15, 0);
}

template <int... J>
__device__ __forceinline__ void key_mfmas(std::integer_sequence<int, J...>, const half8_t (&kv)[16],
                                          const half4_t (&Aq)[2], float4_t& s0, float4_t& s1) {
  (key_mfma<J>(kv, Aq, s0, s1), ...);
}

__device__ __forceinline__ int kv_len(const StreamParams& p, const int32_t* kv_lens, int b) {
  if (!kv_lens) return p.S_cap;
  const int v = kv_lens[b];
  return v < 0 ? 0 : (v > p.S_cap ? p.S_cap : v);
}

// Valid key range [lo, hi) of query row rho (clamped to the rows that exist)
// in a batch row of len keys: the causal and sliding-window masks.
__device__ __forceinline__ void row_range(const StreamParams& p, int len, int rho, int& lo,
                                          int& hi) {
  rho = rho < p.GS ? rho : p.GS - 1;
  const int qa = len - p.Sq + rho / p.G;
  int h = p.causal ? (qa + 1 < len ? qa + 1 : len) : len;
  int l = p.window > 0 ? qa - p.window + 1 : 0;
  h = h > 0 ? h : 0;
  l = l > 0 ? l : 0;
  lo = l;
  hi = h > l ? h : l;
}

// Keys of unit u: from the first row's lower bound to the last row's upper
// bound (both are nondecreasing in rho).
__device__ __forceinline__ int unit_len(const StreamParams& p, const int32_t* kv_lens, int u,
                                        int* lo_out) {
  const int rg = u % p.n_rg;
  const int b = u / (p.n_rg * p.Hkv);
  const int len = kv_len(p, kv_lens, b);
  int lo0, hi0, lo3, hi3;
  row_range(p, len, 4 * rg, lo0, hi0);
  row_range(p, len, 4 * rg + 3, lo3, hi3);
  if (lo_out) *lo_out = lo0;
  return hi3 > lo0 ? hi3 - lo0 : 0;
}

__global__ __launch_bounds__(kThreads, 1) __attribute__((amdgpu_waves_per_eu(2, 2))) void attend_stream_kernel(
    const __half* __restrict__ q, const uint8_t* __restrict__ k_codes,
    const float* __restrict__ k_codebook, const float* __restrict__ smooth,
    const uint8_t* __restrict__ v_codes, const float* __restrict__ v_codebook,
    const int32_t* __restrict__ kv_lens, int* __restrict__ header, float* __restrict__ part,
    StreamParams p) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---- codebooks into LDS as replicated fp16 rows -------------------------
  // four threads per code: each writes a quarter of the code's replicas
  for (int code = tid >> 2; code < 256; code += kThreads / 4) {
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
    if (code < p.n_c) {
      a = reinterpret_cast<const float4*>(k_codebook)[2 * code];
      b = reinterpret_cast<const float4*>(k_codebook)[2 * code + 1];
    }
    const uint4 h = make_uint4(pack_half2(a.x, a.y), pack_half2(a.z, a.w), pack_half2(b.x, b.y),
                               pack_half2(b.z, b.w));
    const int r0 = (tid & 3) * 4;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      *reinterpret_cast<uint4*>(lds + kKeyTab + code * 256 + (r0 + k) * 16) = h;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (code < p.n_c) v = reinterpret_cast<const float4*>(v_codebook)[code];
    const uint2 hv = make_uint2(pack_half2(v.x, v.y), pack_half2(v.z, v.w));
    const int s0 = (tid & 3) * 8;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      *reinterpret_cast<uint2*>(lds + kValTab + code * 256 + (s0 + k) * 8) = hv;
  }

  // ---- unit prefix (exclusive) over the U <= kMaxUnits units --------------
  int* pre = reinterpret_cast<int*>(lds + kPrefix);
  int* scan = reinterpret_cast<int*>(lds + kScan);
  {
    int loc[kUnitsPerThread], sum = 0;
#pragma unroll
    for (int k = 0; k < kUnitsPerThread; ++k) {
      const int u = kUnitsPerThread * tid + k;
      loc[k] = sum;
      sum += u < p.U ? unit_len(p, kv_lens, u, nullptr) : 0;
    }
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    if (lane == 63) scan[wave] = incl;
    __syncthreads();
    int off = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kW; ++w) {
      const int s = scan[w];
      off += w < wave ? s : 0;
      total += s;
    }
    const int excl = off + incl - sum;
#pragma unroll
    for (int k = 0; k < kUnitsPerThread; ++k) {
      const int u = kUnitsPerThread * tid + k;
      if (u < p.U) pre[u] = excl + loc[k];
    }
    if (tid == 0) pre[p.U] = total;
    __syncthreads();
  }
  const int T = pre[p.U];
  const int NW = gridDim.x * kW;
  const int C = max(p.cmin, (T + NW - 1) / NW);
  if (blockIdx.x == 0) {
    for (int u = tid; u <= p.U; u += kThreads) header[1 + u] = pre[u];
    if (tid == 0) header[0] = C;
  }

  const int c = blockIdx.x * kW + wave;
  const int start = c * C;  // T <= U * S_cap < 2^30 is checked on the host
  const int end = min(T, start + C);
  // state of the wave's current unit segment; the last one is combined
  // across the workgroup at the end
  int u_last = -1;
  float m[kRows], lsum[kRows];
  float4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
#pragma unroll
  for (int r = 0; r < kRows; ++r) { m[r] = -INFINITY; lsum[r] = 0.f; }

  if (start < T) {
  // unit holding token position `start`: the largest u with pre[u] <= start
  int u = 0;
  {
    int lo = 0, hi = p.U - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre[mid] <= start) lo = mid; else hi = mid - 1;
    }
    u = lo;
  }

  // lane constants
  const uint32_t kbase = (uint32_t)(lane & 15) * 16u;                  // key replica
  const uint32_t vbase = (uint32_t)(lane & 31) * 8u | (1u << 16);      // value replica + 64 KiB
  const int e_a = lane & 3;          // A operand of the value MFMA: row (rA, e_a)
  const int rA = (lane & 15) >> 2;
  const int grp16 = lane >> 4;       // K group of the 16x16x32 operands
  const uint32_t sa0 = e_a == 0 ? 0x0c0c0100u : (e_a == 1 ? 0x01000c0cu : 0x0c0c0c0cu);
  const uint32_t sa1 = e_a == 2 ? 0x0c0c0100u : (e_a == 3 ? 0x01000c0cu : 0x0c0c0c0cu);
  const uint32_t sa2 = e_a == 0 ? 0x0c0c0302u : (e_a == 1 ? 0x03020c0cu : 0x0c0c0c0cu);
  const uint32_t sa3 = e_a == 2 ? 0x0c0c0302u : (e_a == 3 ? 0x03020c0cu : 0x0c0c0c0cu);
  uint8_t* const ps = lds + kPStage + wave * kPWave;

  int pos = start;
  while (true) {
    const int Pu = pre[u], Pn = pre[u + 1];
    const int seg_end = min(end, Pn);
    const int rg = u % p.n_rg;
    const int bg = u / p.n_rg;
    const int g = bg % p.Hkv;
    const int bb = bg / p.Hkv;
    const int len = kv_len(p, kv_lens, bb);
    int klo[kRows], khi[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) row_range(p, len, 4 * rg + r, klo[r], khi[r]);
    const int t0 = klo[0] + (pos - Pu);
    const int t1 = klo[0] + (seg_end - Pu);
    int full_lo = t0, full_hi = t1;
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      klo[r] = max(klo[r], t0);
      khi[r] = min(khi[r], t1);
      full_lo = max(full_lo, klo[r]);
      full_hi = min(full_hi, khi[r]);
    }

    // ---- query: dual transform into the broadcast A layout -------------
    // lane (bq = lane / 4, row ir = lane % 4) holds dims 4 bq + e and
    // 64 + 4 bq + e (e = 0..3) of row ir: Aq[k] serves dim chunk 16 k + bq.
    half4_t Aq[2];
    {
      const int bq = lane >> 2, ir = lane & 3;
      const int rho = 4 * rg + ir;
      const int rc = rho < p.GS ? rho : p.GS - 1;
      const int h = g * p.G + rc % p.G;
      const __half* qp = q + ((size_t)(bb * p.Hq + h) * p.Sq + rc / p.G) * kD;
      float x[8];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const uint2 w = *reinterpret_cast<const uint2*>(qp + 64 * k + 4 * bq);
        const float2 f0 = __half22float2(*reinterpret_cast<const __half2*>(&w.x));
        const float2 f1 = __half22float2(*reinterpret_cast<const __half2*>(&w.y));
        x[4 * k] = f0.x; x[4 * k + 1] = f0.y; x[4 * k + 2] = f1.x; x[4 * k + 3] = f1.y;
      }
      if (smooth) {
        const float* sp = smooth + (p.smooth_rows == 1 ? 0 : g) * kD;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const float4 s = *reinterpret_cast<const float4*>(sp + 64 * k + 4 * bq);
          x[4 * k] *= s.x; x[4 * k + 1] *= s.y; x[4 * k + 2] *= s.z; x[4 * k + 3] *= s.w;
        }
      }
      if (p.transform) {
        // in-register index bits 0, 1 (dims 0, 1) and 2 (dim bit 6)
#pragma unroll
        for (int m = 1; m < 8; m <<= 1) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            if (i & m) continue;
            const float a = x[i], b = x[i + m];
            x[i] = a + b;
            x[i + m] = a - b;
          }
        }
        // dim bits 2..5 are lane bits 2..5
#pragma unroll
        for (int m = 4; m < 64; m <<= 1) {
          const float sg = (lane & m) ? -1.f : 1.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) x[i] = fmaf(sg, x[i], __shfl_xor(x[i], m));
        }
      }
      const float f = rho < p.GS ? p.fold : 0.f;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        Aq[k] = half4_t{(_Float16)(x[4 * k] * f), (_Float16)(x[4 * k + 1] * f),
                        (_Float16)(x[4 * k + 2] * f), (_Float16)(x[4 * k + 3] * f)};
      }
    }

    float th[kRows], mref[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      m[r] = -INFINITY; th[r] = -INFINITY; mref[r] = 0.f; lsum[r] = 0.f;
    }
    acc0 = float4_t{0.f, 0.f, 0.f, 0.f};
    acc1 = acc0;

    const size_t row_tok = (size_t)bg * p.S_cap;
    const uint8_t* const kc_row = k_codes + row_tok * 16;
    const uint8_t* const vc_row = v_codes + row_tok * 32 + 2 * (lane & 15);
    const int tmax = p.S_cap - 1;

    // codes of one block: the lane's key (16 bytes) and, for the value
    // MFMA, the code pairs (2n, 2n+1) of keys 4 j + g, j = 0..15, kept as
    // loaded (one per register) so that the prefetch of the next block is
    // not waited for until that block is processed.  Load j of the wave
    // reads keys 4 j .. 4 j + 3: one contiguous 128-byte span.
    auto load_codes = [&](int tb, uint4& kc, uint32_t (&vr)[16]) {
      kc = *reinterpret_cast<const uint4*>(kc_row + (size_t)min(tb + lane, tmax) * 16);
      const int tv = tb + grp16;
      if (tb + 64 <= p.S_cap) {
        const uint16_t* vp = reinterpret_cast<const uint16_t*>(vc_row + (size_t)tv * 32);
#pragma unroll
        for (int k = 0; k < 16; ++k) vr[k] = vp[64 * k];
      } else {
#pragma unroll
        for (int k = 0; k < 16; ++k)
          vr[k] = *reinterpret_cast<const uint16_t*>(vc_row + (size_t)min(tv + 4 * k, tmax) * 32);
      }
    };

    // Software pipeline over 64-key blocks.  A block's key-row gathers and
    // score MFMAs run while the previous block's value rows (gathered at the
    // end of its own stage) go through the value MFMAs; the code buffers of
    // consecutive blocks alternate between two register sets, so the
    // prefetch of the next block is only waited for when it is used.
    u32x2_t vg[8][4];  // value rows of the block whose value MFMAs are pending
    uint32_t pp[8];    // that block's p, staged into the A operand layout

    auto value_mfmas = [&]() {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t x = pp[k];
        const uint4 au = make_uint4(__builtin_amdgcn_perm(0u, x, sa0), __builtin_amdgcn_perm(0u, x, sa1),
                                    __builtin_amdgcn_perm(0u, x, sa2), __builtin_amdgcn_perm(0u, x, sa3));
        const uint4 b0 = make_uint4(vg[k][0].x, vg[k][0].y, vg[k][1].x, vg[k][1].y);
        const uint4 b1 = make_uint4(vg[k][2].x, vg[k][2].y, vg[k][3].x, vg[k][3].y);
        const half8_t A = *reinterpret_cast<const half8_t*>(&au);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, *reinterpret_cast<const half8_t*>(&b0), acc0,
                                                      0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, *reinterpret_cast<const half8_t*>(&b1), acc1,
                                                      0, 0, 0);
      }
    };

    auto stage = [&](int tb, const uint4& kc, const uint32_t (&vr)[16], bool pending) {
      // key rows: address = replica offset | code << 8
      half8_t kv[16];
      {
        const uint32_t kw[4] = {kc.x, kc.y, kc.z, kc.w};
#pragma unroll
        for (int j = 0; j < 16; ++j)
          kv[j] = lds_ld<half8_t>(
              __builtin_amdgcn_perm(kw[j >> 2], kbase, 0x0c0c0000u | ((4u + (j & 3)) << 8)));
      }
      __builtin_amdgcn_sched_barrier(0);
      if (pending) value_mfmas();

      // ---- scores on the matrix cores ----------------------------------
      float4_t sc0 = {0.f, 0.f, 0.f, 0.f}, sc1 = sc0;
      key_mfmas(std::make_integer_sequence<int, 16>{}, kv, Aq, sc0, sc1);
      const float4_t sc = sc0 + sc1;

      // ---- masks and lazy online softmax -------------------------------
      float s[kRows] = {sc[0], sc[1], sc[2], sc[3]};
      if (!(tb >= full_lo && tb + 64 <= full_hi)) {
        const int t = tb + lane;
#pragma unroll
        for (int r = 0; r < kRows; ++r)
          if (!(t >= klo[r] && t < khi[r])) s[r] = -INFINITY;
      }
      bool over = false;
#pragma unroll
      for (int r = 0; r < kRows; ++r) over |= s[r] > th[r];
      if (__builtin_amdgcn_ballot_w64(over)) {
        float al[kRows];
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
          const float mn = fmaxf(m[r], wave_max(s[r]));
          al[r] = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m[r] - mn);
          m[r] = mn;
          th[r] = mn + kLazyMargin;
          mref[r] = mn == -INFINITY ? 0.f : mn;
          lsum[r] *= al[r];
        }
        const int rr = lane >> 4;
        const float a = rr == 0 ? al[0] : (rr == 1 ? al[1] : (rr == 2 ? al[2] : al[3]));
        acc0 *= a;
        acc1 *= a;
      }
      float pr[kRows];
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        pr[r] = __builtin_amdgcn_exp2f(s[r] - mref[r]);
        lsum[r] += pr[r];
      }

      // ---- p to the value operand layout through LDS -------------------
      wave_sync_lds();
      {
        const uint32_t p01 = pack_half2_rtz(pr[0], pr[1]);
        const uint32_t p23 = pack_half2_rtz(pr[2], pr[3]);
        // key 4 q + g is staged at position 16 g + q, so that lane group g
        // finds its keys 4 q + g (q = 0..15) contiguous
        uint8_t* const pw = ps + 2 * (16 * (lane & 3) + (lane >> 2));
        *reinterpret_cast<uint16_t*>(pw + 0 * kPRow) = (uint16_t)p01;
        *reinterpret_cast<uint16_t*>(pw + 1 * kPRow) = (uint16_t)(p01 >> 16);
        *reinterpret_cast<uint16_t*>(pw + 2 * kPRow) = (uint16_t)p23;
        *reinterpret_cast<uint16_t*>(pw + 3 * kPRow) = (uint16_t)(p23 >> 16);
      }
      wave_sync_lds();
      const uint4 P0 = *reinterpret_cast<const uint4*>(ps + rA * kPRow + 32 * grp16);
      const uint4 P1 = *reinterpret_cast<const uint4*>(ps + rA * kPRow + 32 * grp16 + 16);
      pp[0] = P0.x; pp[1] = P0.y; pp[2] = P0.z; pp[3] = P0.w;
      pp[4] = P1.x; pp[5] = P1.y; pp[6] = P1.z; pp[7] = P1.w;


      // ---- this block's value rows, consumed by the next stage ---------
      // rows of key pair k: [key 0 sub 2n, key 1 sub 2n, key 0 sub 2n+1, key 1 sub 2n+1]
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        // [code(key 0, 2n), code(key 0, 2n+1), code(key 1, 2n), code(key 1, 2n+1)]
        const uint32_t w = __builtin_amdgcn_perm(vr[2 * k + 1], vr[2 * k], 0x05040100u);
        vg[k][0] = lds_ld<u32x2_t>(__builtin_amdgcn_perm(w, vbase, 0x0c020400u));
        vg[k][1] = lds_ld<u32x2_t>(__builtin_amdgcn_perm(w, vbase, 0x0c020600u));
        vg[k][2] = lds_ld<u32x2_t>(__builtin_amdgcn_perm(w, vbase, 0x0c020500u));
        vg[k][3] = lds_ld<u32x2_t>(__builtin_amdgcn_perm(w, vbase, 0x0c020700u));
      }
    };

    uint4 kcA, kcB;
    uint32_t vrA[16], vrB[16];
    load_codes(t0, kcA, vrA);
    for (int tb = t0;;) {
      if (tb + 64 < t1) load_codes(tb + 64, kcB, vrB);
      stage(tb, kcA, vrA, tb != t0);
      tb += 64;
      if (tb >= t1) break;
      if (tb + 64 < t1) load_codes(tb + 64, kcA, vrA);
      stage(tb, kcB, vrB, true);
      tb += 64;
      if (tb >= t1) break;
    }
    value_mfmas();

    pos = seg_end;
    if (pos >= end) {
      u_last = u;
      break;
    }
    // ---- partial of (chunk c, unit u), not the chunk's last one ----------
    {
      float* sp = part + (size_t)(c + u) * kSlot;
      const int r = lane >> 4, n = lane & 15;
      *reinterpret_cast<float4*>(sp + r * kD + 8 * n) = make_float4(acc0[0], acc0[1], acc0[2], acc0[3]);
      *reinterpret_cast<float4*>(sp + r * kD + 8 * n + 4) =
          make_float4(acc1[0], acc1[1], acc1[2], acc1[3]);
      float l[kRows];
#pragma unroll
      for (int rr = 0; rr < kRows; ++rr) l[rr] = wave_sum(lsum[rr]);
      if (lane < kRows) {
        const float mm = lane == 0 ? m[0] : (lane == 1 ? m[1] : (lane == 2 ? m[2] : m[3]));
        const float ll = lane == 0 ? l[0] : (lane == 1 ? l[1] : (lane == 2 ? l[2] : l[3]));
        sp[kRows * kD + lane] = mm;
        sp[kRows * kD + kRows + lane] = ll;
      }
    }
    ++u;
    while (pre[u + 1] == pre[u]) ++u;  // skip empty units (pos < T, so one follows)
  }
  }

  // ---- combine the last partials of the workgroup's waves per unit -------
  // Consecutive waves hold consecutive chunks, so the waves whose last unit
  // is the same form one run; the run's first wave writes the combined
  // partial into its slot and marks the others' slots empty.
  __syncthreads();  // the codebook tables are no longer read
  float* red = reinterpret_cast<float*>(lds + kKeyTab);  // [kW][kSlot]
  int* ul = reinterpret_cast<int*>(lds + kScan);
  {
    const int r = lane >> 4, n = lane & 15;
    float* sp = red + wave * kSlot;
    float l[kRows];
#pragma unroll
    for (int rr = 0; rr < kRows; ++rr) l[rr] = wave_sum(lsum[rr]);
    if (u_last >= 0) {
      *reinterpret_cast<float4*>(sp + r * kD + 8 * n) = make_float4(acc0[0], acc0[1], acc0[2], acc0[3]);
      *reinterpret_cast<float4*>(sp + r * kD + 8 * n + 4) =
          make_float4(acc1[0], acc1[1], acc1[2], acc1[3]);
      if (lane < kRows) {
        sp[kRows * kD + lane] = lane == 0 ? m[0] : (lane == 1 ? m[1] : (lane == 2 ? m[2] : m[3]));
        sp[kRows * kD + kRows + lane] = lane == 0 ? l[0] : (lane == 1 ? l[1] : (lane == 2 ? l[2] : l[3]));
      }
    }
    if (lane == 0) ul[wave] = u_last;
  }
  __syncthreads();
  {
    const int uw = ul[wave];
    if (uw >= 0 && (wave == 0 || ul[wave - 1] != uw)) {
      int wb = wave;
      while (wb + 1 < kW && ul[wb + 1] == uw) ++wb;
      const int r = lane >> 4, n = lane & 15;
      float M = -INFINITY;
      for (int i = wave; i <= wb; ++i) M = fmaxf(M, red[i * kSlot + kRows * kD + r]);
      float L = 0.f;
      float4 a0 = make_float4(0.f, 0.f, 0.f, 0.f), a1 = a0;
      if (M != -INFINITY) {
        for (int i = wave; i <= wb; ++i) {
          const float* sp = red + i * kSlot;
          const float mi = sp[kRows * kD + r];
          if (mi == -INFINITY) continue;
          const float w = __builtin_amdgcn_exp2f(mi - M);
          L += w * sp[kRows * kD + kRows + r];
          const float4 x0 = *reinterpret_cast<const float4*>(sp + r * kD + 8 * n);
          const float4 x1 = *reinterpret_cast<const float4*>(sp + r * kD + 8 * n + 4);
          a0.x += w * x0.x; a0.y += w * x0.y; a0.z += w * x0.z; a0.w += w * x0.w;
          a1.x += w * x1.x; a1.y += w * x1.y; a1.z += w * x1.z; a1.w += w * x1.w;
        }
      }
      float* gp = part + (size_t)(c + uw) * kSlot;
      *reinterpret_cast<float4*>(gp + r * kD + 8 * n) = a0;
      *reinterpret_cast<float4*>(gp + r * kD + 8 * n + 4) = a1;
      if (n == 0) {
        gp[kRows * kD + r] = M;
        gp[kRows * kD + kRows + r] = L;
      }
      for (int i = wave + 1; i <= wb; ++i) {
        float* ep = part + (size_t)(blockIdx.x * kW + i + uw) * kSlot;
        if (lane < kRows) {
          ep[kRows * kD + lane] = -INFINITY;
          ep[kRows * kD + kRows + lane] = 0.f;
        }
      }
    }
  }
}

// One wave per output row: log-sum-exp merge of the unit's chunk partials.
__global__ __launch_bounds__(256) void stream_merge_kernel(const int* __restrict__ header,
                                                           const float* __restrict__ part,
                                                           __half* __restrict__ out,
                                                           StreamParams p) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= p.B * p.Hq * p.Sq) return;
  const int ip = row % p.Sq;
  const int bh = row / p.Sq;
  const int h = bh % p.Hq;
  const int bb = bh / p.Hq;
  const int g = h / p.G;
  const int rho = ip * p.G + h % p.G;
  const int r = rho & 3;
  const int u = (bb * p.Hkv + g) * p.n_rg + (rho >> 2);
  const int C = header[0];
  const int Pu = header[1 + u], Pn = header[2 + u];
  float2 acc = make_float2(0.f, 0.f);
  float L = 0.f;
  if (Pn > Pu) {
    const int c_lo = Pu / C, n_part = (Pn - 1) / C - c_lo + 1;
    const float* base = part + (size_t)(c_lo + u) * kSlot;
    // maxima of all partials, one lane per partial
    float M = -INFINITY;
    for (int j = lane; j < n_part; j += 64) M = fmaxf(M, base[(size_t)j * kSlot + kRows * kD + r]);
    M = wave_max(M);
    if (M != -INFINITY) {
      float Ls = 0.f;
      for (int j0 = 0; j0 < n_part; j0 += 64) {
        const int j = j0 + lane;
        const float mj = j < n_part ? base[(size_t)j * kSlot + kRows * kD + r] : -INFINITY;
        const bool ok = mj != -INFINITY;
        const float wj = ok ? __builtin_amdgcn_exp2f(mj - M) : 0.f;
        if (ok) Ls += wj * base[(size_t)j * kSlot + kRows * kD + kRows + r];
        // the few nonempty partials: four loads in flight at a time
        uint64_t mask = __builtin_amdgcn_ballot_w64(ok);
        while (mask) {
          int idx[4];
          float w[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int b = mask ? __builtin_ctzll(mask) : -1;
            if (mask) mask &= mask - 1;
            idx[k] = b;
            w[k] = __shfl(wj, b < 0 ? 0 : b);
          }
          float2 x[4];
#pragma unroll
          for (int k = 0; k < 4; ++k)
            x[k] = idx[k] >= 0 ? *reinterpret_cast<const float2*>(base + (size_t)(j0 + idx[k]) * kSlot +
                                                                   r * kD + 2 * lane)
                               : make_float2(0.f, 0.f);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float wk = idx[k] >= 0 ? w[k] : 0.f;
            acc.x += wk * x[k].x;
            acc.y += wk * x[k].y;
          }
        }
      }
      L = wave_sum(Ls);
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  *reinterpret_cast<__half2*>(out + (size_t)row * kD + 2 * lane) =
      __floats2half2_rn(acc.x * inv, acc.y * inv);
}

int cached_cu_count() {
  static int cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cus[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cus[dev] = n;
  }
  return cus[dev];
}

}  // namespace

bool stream_plan(int B, int Hq, int Sq, int D, int Hkv, int S_cap, int window, int dk, int dv, int n_c,
                 StreamParams* sp, size_t* lds_bytes, size_t* ws_bytes) {
  if (D != kD || dk != 8 || dv != 4 || n_c < 1 || n_c > 256) return false;
  if (B <= 0 || Hq <= 0 || Sq <= 0 || Hkv <= 0 || S_cap <= 0 || Hq % Hkv) return false;
  const long long G = Hq / Hkv, GS = G * Sq, n_rg = (GS + kRows - 1) / kRows;
  const long long U = (long long)B * Hkv * n_rg;
  if (U > kMaxUnits || U * (long long)S_cap >= (1LL << 30)) return false;
  // the persistent grid's fixed cost (table fill, unit prefix, merge) only
  // pays off with enough keys: small problems go to the per-unit kernel
  const long long max_range = window > 0 ? std::min<long long>(S_cap, (long long)Sq + window - 1) : S_cap;
  if (U * max_range < (1LL << 18)) return false;
  if (sp) {
    sp->B = B; sp->Hq = Hq; sp->Sq = Sq; sp->Hkv = Hkv; sp->S_cap = S_cap; sp->n_c = n_c;
    sp->G = (int)G; sp->GS = (int)GS; sp->n_rg = (int)n_rg; sp->U = (int)U; sp->cmin = 256;
  }
  if (lds_bytes) *lds_bytes = (kPrefix + (size_t)(U + 1) * 4 + 15) / 16 * 16;
  if (ws_bytes) *ws_bytes = stream_workspace_bytes(B, Hq, Sq, D, Hkv);
  return true;
}

size_t stream_workspace_bytes(int B, int Hq, int Sq, int D, int Hkv) {
  if (D != kD || B <= 0 || Hq <= 0 || Sq <= 0 || Hkv <= 0 || Hq % Hkv) return 0;
  const long long G = Hq / Hkv, GS = G * Sq, n_rg = (GS + kRows - 1) / kRows;
  const long long U = (long long)B * Hkv * n_rg;
  const size_t header = ((size_t)(U + 2) * 4 + 255) / 256 * 256;
  return header + (size_t)(kMaxWaves + U) * kSlot * sizeof(float);
}

hipError_t launch_attend_stream(const AttendArgs& a, StreamParams sp, size_t lds, hipStream_t st) {
  const int cus = cached_cu_count();
  if (cus <= 0) return hipErrorInvalidDevice;
  const int grid = cus < kMaxWaves / kW ? cus : kMaxWaves / kW;
  sp.smooth_rows = a.smooth_rows;
  sp.transform = a.transform;
  sp.causal = a.causal;
  sp.window = a.window;
  sp.fold = (a.transform ? WhtNorm<kD>::value : 1.f) * a.scale_log2e;
  const size_t header_bytes = ((size_t)(sp.U + 2) * 4 + 255) / 256 * 256;
  int* header = reinterpret_cast<int*>(a.partials);
  float* part = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(a.partials) + header_bytes);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(attend_stream_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attend_stream_kernel, dim3(grid), dim3(kThreads), lds, st, a.q, a.k_codes,
                     a.k_codebook, a.smooth, a.v_codes, a.v_codebook, a.kv_lens, header, part, sp);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long rows = (long long)a.B * a.Hq * a.Sq;
  hipLaunchKernelGGL(stream_merge_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, header,
                     part, a.out, sp);
  return hipGetLastError();
}

}  // namespace vq
